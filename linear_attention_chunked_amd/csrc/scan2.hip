// The inter-chunk state scan for bfloat16 storage on gfx950 (the fast path;
// float32 storage keeps the simpler kernel in scan.hip).
//
// Same recurrence and same per-column instruction sequence as scan.hip
// (kev pull request #259, opening section: one program per value block,
// serial over 64-token chunks), organised for latency:
//
//   * Buffer resources.  Every chunk gets scalar resource descriptors whose
//     base is the chunk's first token of this head and whose size ends at the
//     chunk's last valid token.  Per-lane offsets are fixed for the whole loop;
//     rows past a ragged tail read as zero and stores to them are dropped by
//     the hardware range check, so there is no per-lane masking and no 64-bit
//     address arithmetic in the loop.
//   * Row-major LDS tiles written straight from the 16-byte loads, rows padded
//     (W by 16 bytes, K and U by 32) so the two read patterns below hit distinct
//     banks and every operand address is a per-lane base plus an immediate.
//     The contraction over tokens needs K and U with the token index running
//     inside a lane; gfx950's ds_read_b64_tr_b16 delivers exactly that from the
//     row-major tile (within 16 lanes, lane j names 4 elements of a 4x16 block
//     and lane i receives its column i).
//   * The chunk's decay weights exp(g_last - g_t) (zero past the tail) and
//     exp(g_last) are computed once per chunk by the first wave and shared
//     through LDS.  With one wave per SIMD every wave64 VALU instruction costs
//     the SIMD four cycles, so the chunk step is kept lean in VALU work.
//   * Two LDS buffers and a register prefetch of PF chunks, one barrier per
//     chunk: the global loads of chunk c+PF are in flight while chunk c
//     computes.
//   * U enters the accumulator negated and the sign is folded into the decay
//     weights, so W needs no negation: acc = -U + W S = -D, v_new = -acc,
//     D' = acc * (-exp(g_last - g)).
//   * Segment summaries (MODE 1, 2) keep the state as a scalar multiple,
//     S = sig * S', so the chunk's decay e^{g_last} is folded into the 64
//     token weights (and the U tile into -1/sig) instead of multiplying all
//     DK x BV accumulators every chunk: S' <- S' + K^T (acc' * nd / e^{g_last})
//     with acc' = -U / sig + W S', sig <- sig e^{g_last}.  When sig would leave
//     [2^-40, 2^40] the chunk instead renormalises (S' <- sig e^{g_last} S',
//     weights nd * sig, sig <- 1), so no scale factor can overflow.  The
//     result is the same state up to where bfloat16 rounding falls; it is
//     still the same for every tile.  The plain pass (MODE 0) emits h from
//     the true state every chunk and keeps the direct form.
//   * Per-key-channel decay (KD): the caller passes the decayed keys
//     kg = K * e^{Gam_last - Gam} in place of K and the chunk's channel decays
//     e^{Gam_last} (one DK-vector per chunk and head); the weights are then
//     -1 (0 past the tail) and every state row is scaled by its own channel's
//     decay: S <- diag(decay) S + kg^T D.
//   * Dense form (DENSE, the staged plain pass of 64-column blocks with four
//     waves): three workgroups share a CU instead of two.  The full form
//     holds every W and K operand fragment of a chunk in registers at once
//     and stages h and v_new in LDS of their own (about 250 VGPRs and 73 KB:
//     two workgroups per CU).  The dense form reads the W fragments of one
//     contraction step and the K fragments of one token step at a time,
//     issues the fused output's Q loads after GEMM1, and stages h in the W
//     tile's place and v_new in the U tile's (dead once every wave holds its
//     W and U operands of the chunk; one more barrier there and one between
//     the staged stores leaving and the next tiles arriving): at most 168
//     VGPRs and 46 KB.  The products and their order are the same, so the
//     results are the same bits; the planner takes it when a launch has more
//     workgroups than two per CU (many short sequences), where the third
//     resident block shortens the tail of the last round.
//   * Fused chunk output (FO, staged plain pass with four waves): once every
//     wave has staged its h columns and v_new columns of the chunk, wave w
//     forms the output of token tile w over the block's BV columns,
//       o_t = scale (e^{gamma_t} q_t^T S_c + sum_{i <= t} e^{gamma_t - gamma_i} (q_t . k_i) v_new_i),
//     from the staged (bf16) S_c and v_new, the K tile still in LDS and Q
//     fragments read from HBM straight into registers, without reading h or
//     v_new back from HBM.  The products are output2.hip's with the operand
//     roles exchanged (O^T = S_c^T Q^T e^gamma + v_new^T P^T: the same
//     products in the same k order, so o is the same bits), which leaves
//     each lane four consecutive value columns of one token: 8-byte stores.
#include "gfx950.hpp"
#include "kernels.hpp"
#include "wy_core.hpp"

namespace gdr {

template <int DK, int BV, int NW, int PF, int MODE, int NBUF, bool KD, bool FO = false, bool DENSE = false,
          bool PREP = false>
struct Scan2 {
  using S = St<bf16_t>;
  using frag = S::frag;
  static constexpr int NT = NW * 64;
  static constexpr int NC = BV / (16 * NW);
  static constexpr int KS = DK / 32;
  static constexpr int DT = DK / 16;
  static constexpr int RBW = DK * 2;      // bytes per W / K row
  // MODE 2 (balanced summaries): a block holds BV/2 state columns (waves
  // 0..NW/2-1, which read U) and the same BV/2 columns of the transition
  // (the other waves), so every block of a (segment, head) does the same work
  // and reads the same K/W tiles at the same pace (shared through L2).
  static constexpr int UBV = (MODE == 2) ? BV / 2 : BV;  // U columns staged per block
  static constexpr int RBU = UBV * 2;     // bytes per U row (this block's columns)
  // Padded LDS row strides (bytes).  W rows are read as row fragments, two
  // 8-byte pieces 32 bytes apart that the compiler issues as one
  // ds_read2_b64: with a 24-byte pad those run at twice the rate of a
  // 16-byte pad on gfx950 (measured: 118 against 61 bytes per clock and CU).
  // The rows are then only 8-byte aligned, so the tile is stored in 8-byte
  // pieces.
  static constexpr int SW = RBW + 24;
  static constexpr int SK = RBW + 32;
  // The fused output (P^T) and the fused prepare (Gram) also read K by rows,
  // not only transposed: rows 8..15 of every 16 then sit 16 bytes further on
  // (KX), which keeps the transposed reads free of LDS bank conflicts and
  // makes the row reads free of them too (64 banks of 4 bytes: at the plain
  // 288-byte stride rows r and r + 8 of a row read share their banks).
  static constexpr int KX = (FO && DENSE) ? 16 : 0;
  static constexpr int SU = RBU + 32;
  static constexpr int CPW = RBW / 16;    // 16-byte chunks per W row
  static constexpr int CPU = RBU / 16;
  static constexpr int OFF_W = 0, OFF_K = kChunk * SW, OFF_U = OFF_K + kChunk * SK;
  // 64 negated decay weights, then exp(g_last) (SIG: the state multiplier,
  // the U scale -1/sig and sig after the chunk)
  static constexpr int OFF_D = OFF_U + kChunk * SU;
  static constexpr int OFF_DEC = OFF_D + (kChunk + 4) * 4;  // KD: the chunk's DK channel decays
  static constexpr bool SIG = (MODE != 0) && !KD;           // scaled-state form (summaries)
  static constexpr int OFF_GM = OFF_DEC + (KD ? DK * 4 : 0);  // FO: the chunk's gamma (zero past the tail)
  // PREP: the chunk's gamma, beta and beta e^gamma for the WY factors (the
  // A / T scratch takes the W tile's place until w replaces it)
  static constexpr int OFF_PG = OFF_GM + (FO ? kChunk * 4 : 0);
  static constexpr int BUF = OFF_PG + (PREP ? 3 * kChunk * 4 : 0);
  // Output staging (single-buffer loop, plain and segmented passes): the
  // chunk's h block and v_new tile are written to LDS in their memory layout
  // and leave the next iteration as whole 16-byte vectors per lane (the h
  // block of one (chunk, head, column block) is contiguous; v_new rows are BV
  // columns), instead of 8- and 2-byte pieces straight from the MFMA layout.
  static constexpr bool STAGE = (MODE == 0) && (NBUF == 1);
  static constexpr int SHS = DK * 2 + 16;           // staged h rows (one value column each)
  static constexpr int SVS = BV * 2 + 16;           // staged v_new rows (one token each)
  // DENSE: the h staging takes the W tile's place, v_new the U tile's
  static constexpr bool ALIAS = DENSE && STAGE && (BV * SHS <= kChunk * SW) && (SVS <= SU);
  static constexpr int OFF_HS = ALIAS ? OFF_W : BUF;
  static constexpr int OFF_VS = ALIAS ? OFF_U : OFF_HS + BV * SHS;
  static constexpr int SMEM = NBUF * BUF + ((STAGE && !ALIAS) ? BV * SHS + kChunk * SVS : 0);
  // the staged stores stream past L2 (kStreamStore), except in the fused
  // pass, whose own 8-byte output pieces share the lines' trip through L2
  // (non-temporal h / v_new there measured 0.5 us slower with cold caches)
  static constexpr int ST_POL = FO ? 0 : kStreamStore;
  // U is read by one column block only (K and W by every block of the
  // (sequence, head)): on long chains it is loaded non-temporally so its
  // stream does not push the shared K / W tiles out of L2 before the other
  // block reads them (new_states: 571 -> 509 MB fetched, 213 -> 199 us; the
  // 64K summaries 118 -> 114 us).  The dense form (short packed sequences)
  // keeps the default policy: there U written by the chunk prepare just
  // before is still in the Infinity Cache (non-temporal loads measured
  // 24.6 -> 30.6 us on back-to-back question_rows scans).
  static constexpr int U_POL = (DENSE || FO) ? 0 : kStreamStore;
  static constexpr int H_PT = BV * DK / 8 / NT;     // 16-byte h vectors per thread
  static constexpr int V_PT = kChunk * BV / 8 / NT; // 16-byte v_new vectors per thread
  static constexpr int W_PT = kChunk * CPW / NT;   // 16-byte vectors per thread (W, and K)
  static constexpr int U_PT = (kChunk * CPU + NT - 1) / NT;
  static_assert(NC >= 1 && BV % (16 * NW) == 0, "each wave owns whole 16-column tiles");
  static_assert((kChunk * CPW) % NT == 0, "W/K tiles split evenly over the threads");
  static_assert(!STAGE || ((BV * DK / 8) % NT == 0 && (kChunk * BV / 8) % NT == 0), "staged outputs split evenly");
  static_assert(!FO || (STAGE && NW == 4 && !KD), "the fused output runs on the staged plain pass, one token tile per wave");
  static_assert(!DENSE || ALIAS, "the dense form needs the staging to fit the W and U tiles");
  static_assert(!PREP || (FO && MODE == 0 && NBUF == 1 && NW == 4 && !KD && UBV % 16 == 0),
                "the prepare is fused into the staged plain pass with the chunk output, four waves");
  static_assert(!PREP || WyCore<DK>::kTri * 4 <= kChunk * SW, "the A / T scratch fits the W tile");

  struct Stage {
    u32x4_t w[PREP ? 1 : W_PT];
    u32x4_t k[W_PT];
    u32x4_t u[U_PT];  // PREP: the block's columns of v
    float g;          // g_cum (PREP: g) of token threadIdx.x
    float b;          // PREP: beta of token threadIdx.x
  };

  struct Ctx {
    const ScanArgs* a;
    int hd, col_blk, H, DV;
    bool has_u;
    // global byte offsets (row-relative) of this thread's first W/K and U
    // vectors; vector i sits i strides further on (NT / CPW rows, NT / CPU
    // rows), added at each load (off_at) rather than held in registers
    int vo_wk, vo_u;
    int st_wk, st_u;
  };

  // o + i s, formed next to the load that uses it: an asm add is not hoisted
  // out of the chunk loop, so the per-vector offsets never occupy registers
  // across it (holding them pushed the fused dense pass past its register
  // budget into scratch spills)
  __device__ static __forceinline__ int off_at(int o, int s, int i) {
    if (i == 0) return o;
    int r;
    asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(i * s), "v"(o));
    return r;
  }

  // Issues the loads of one chunk.  A chunk past the row's end (nvalid <= 0)
  // gets empty buffer ranges: the same instructions are issued and return
  // zeros, so every loop iteration issues the same number of loads and the
  // compiler's wait counts keep the younger prefetches in flight.
  __device__ static __forceinline__ void load(Stage& st, const Ctx& x, int64_t tok0, int nvalid, int64_t hrow) {
    const ScanArgs& a = *x.a;
    const int64_t H = x.H;
    const bool live = nvalid > 0;
    if (!live) tok0 = 0;
    const uint32_t wk_bytes = live ? static_cast<uint32_t>(((nvalid - 1) * H + 1) * DK * 2) : 0u;
    const uint16_t* wp = static_cast<const uint16_t*>(a.w) + (tok0 * H + x.hd) * DK;
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + (tok0 * H + x.hd) * DK;
    const rsrc_t rk = make_rsrc(kp, wk_bytes);
    if constexpr (PREP) {
#pragma unroll
      for (int i = 0; i < W_PT; ++i) st.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off_at(x.vo_wk, x.st_wk, i), 0, 0);
      const uint16_t* vp = static_cast<const uint16_t*>(a.v) + (tok0 * H + x.hd) * x.DV + x.col_blk;
      const rsrc_t rv = make_rsrc(vp, live ? static_cast<uint32_t>(((nvalid - 1) * H * x.DV + UBV) * 2) : 0u);
#pragma unroll
      for (int i = 0; i < U_PT; ++i) st.u[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, off_at(x.vo_u, x.st_u, i), 0, 0);
      const uint32_t gb = live ? static_cast<uint32_t>(((nvalid - 1) * H + 1) * 4) : 0u;
      const int go = static_cast<int>(threadIdx.x * H * 4);
      st.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.g + tok0 * H + x.hd, gb), go, 0, 0));
      st.b = __builtin_bit_cast(float,
                                __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.beta + tok0 * H + x.hd, gb), go, 0, 0));
      return;
    }
    const rsrc_t rw = make_rsrc(wp, wk_bytes);
#pragma unroll
    for (int i = 0; i < W_PT; ++i) st.w[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, off_at(x.vo_wk, x.st_wk, i), 0, 0);
#pragma unroll
    for (int i = 0; i < W_PT; ++i) st.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off_at(x.vo_wk, x.st_wk, i), 0, 0);
    if (MODE != 1 || x.has_u) {
      const uint16_t* up = static_cast<const uint16_t*>(a.u) + (tok0 * H + x.hd) * x.DV + x.col_blk;
      const rsrc_t ru = make_rsrc(up, live ? static_cast<uint32_t>(((nvalid - 1) * H * x.DV + UBV) * 2) : 0u);
#pragma unroll
      for (int i = 0; i < U_PT; ++i) st.u[i] = __builtin_amdgcn_raw_buffer_load_b128(ru, off_at(x.vo_u, x.st_u, i), 0, U_POL);
    }
    if constexpr (KD) {  // thread d < DK: channel d's decay over the chunk
      const float* dp = a.decay + (hrow * H + x.hd) * DK;
      const rsrc_t rd = make_rsrc(dp, live ? static_cast<uint32_t>(DK * 4) : 0u);
      st.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, static_cast<int>(threadIdx.x * 4), 0, 0));
    } else {
      const float* gp = a.g_cum + tok0 * H + x.hd;
      const rsrc_t rg = make_rsrc(gp, live ? static_cast<uint32_t>(((nvalid - 1) * H + 1) * 4) : 0u);
      st.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, static_cast<int>(threadIdx.x * H * 4), 0, 0));
    }
  }

  __device__ static __forceinline__ void store(const Stage& st, const Ctx& x, char* buf, int nvalid, float& sig,
                                               int64_t tok0 = 0) {
    const int tid = threadIdx.x;
    if constexpr (PREP) {  // K and V tiles; the first wave forms gamma, beta, the decay weights
#pragma unroll
      for (int i = 0; i < W_PT; ++i) {
        const int v = tid + i * NT;
        const int r = v / CPW, c = v % CPW;
        *reinterpret_cast<u32x4_t*>(buf + OFF_K + r * SK + KX * ((r >> 3) & 1) + c * 16) = st.k[i];
      }
#pragma unroll
      for (int i = 0; i < U_PT; ++i) {
        const int v = tid + i * NT;
        if ((kChunk * CPU) % NT == 0 || v < kChunk * CPU) {
          const int r = v / CPU, c = v % CPU;
          *reinterpret_cast<u32x4_t*>(buf + OFF_U + r * SU + c * 16) = st.u[i];
        }
      }
      if (tid < kChunk) {
        float* pg = reinterpret_cast<float*>(buf + OFF_PG);
        const float gam = WyCore<DK>::gamma_beta(st.g, st.b, nvalid, pg, pg + kChunk, pg + 2 * kChunk);
        const ScanArgs& a = *x.a;
        if (a.g_cum_out != nullptr && tid < nvalid) a.g_cum_out[(tok0 + tid) * x.H + x.hd] = gam;
        const float g_last = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gam), max(nvalid, 1) - 1));
        float* d = reinterpret_cast<float*>(buf + OFF_D);
        d[tid] = (tid < nvalid) ? -exp_fast(g_last - gam) : 0.f;
        if (tid == 0) d[kChunk] = exp_fast(g_last);
        reinterpret_cast<float*>(buf + OFF_GM)[tid] = (tid < nvalid) ? gam : 0.f;
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < W_PT; ++i) {
      const int v = tid + i * NT;
      const int r = v / CPW, c = v % CPW;
      u32x2_t* wd = reinterpret_cast<u32x2_t*>(buf + OFF_W + r * SW + c * 16);
      wd[0] = u32x2_t{st.w[i].x, st.w[i].y};
      wd[1] = u32x2_t{st.w[i].z, st.w[i].w};
      *reinterpret_cast<u32x4_t*>(buf + OFF_K + r * SK + KX * ((r >> 3) & 1) + c * 16) = st.k[i];
    }
    if (MODE != 1 || x.has_u) {
#pragma unroll
      for (int i = 0; i < U_PT; ++i) {
        const int v = tid + i * NT;
        if ((kChunk * CPU) % NT == 0 || v < kChunk * CPU) {
          const int r = v / CPU, c = v % CPU;
          *reinterpret_cast<u32x4_t*>(buf + OFF_U + r * SU + c * 16) = st.u[i];
        }
      }
    }
    if constexpr (KD) {
      if (tid < kChunk) reinterpret_cast<float*>(buf + OFF_D)[tid] = (tid < nvalid) ? -1.f : 0.f;
      if (tid < DK) reinterpret_cast<float*>(buf + OFF_DEC)[tid] = st.g;
    } else if (tid < kChunk) {  // first wave: decay weights of the chunk
      const float g_last = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, st.g), max(nvalid, 1) - 1));
      float* d = reinterpret_cast<float*>(buf + OFF_D);
      const float eg = exp_fast(g_last);
      if constexpr (SIG) {  // (sig is tracked by the first wave only)
        const float sn = sig * eg;
        const bool keep = (sn >= 0x1p-40f) && (sn <= 0x1p40f);
        const float f = keep ? 1.f / eg : sig;
        d[tid] = (tid < nvalid) ? -exp_fast(g_last - st.g) * f : 0.f;
        if (tid == 0) {
          d[kChunk] = keep ? 1.f : sn;
          d[kChunk + 1] = -1.f / sig;
          d[kChunk + 2] = keep ? sn : 1.f;
        }
        sig = keep ? sn : 1.f;
      } else {
        d[tid] = (tid < nvalid) ? -exp_fast(g_last - st.g) : 0.f;
        if (tid == 0) d[kChunk] = eg;
      }
      if constexpr (FO) reinterpret_cast<float*>(buf + OFF_GM)[tid] = (tid < nvalid) ? st.g : 0.f;
    }
  }

  // PREP: the chunk's w and u from the K and V tiles (wy_core.hpp), into the
  // W tile and the U tile (V's place) in the layout the loads give; the
  // A / T scratch sits in the W tile until w replaces it.  Starts after the
  // barrier that follows store(); ends with a barrier.
  __device__ static __forceinline__ void prep_wy(char* buf) {
    using W = WyCore<DK>;
    const int lane = threadIdx.x & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    float* t = reinterpret_cast<float*>(buf + OFF_W);
    const float* pg = reinterpret_cast<const float*>(buf + OFF_PG);
    W::gram_diag(buf + OFF_K, SK, KX, t, pg, pg + kChunk);
    __syncthreads();
    W::off_diag(t);
    frag hw[2], lw[2], hu[2], lu[2];
    W::row_frags(t, pg + 2 * kChunk, hw, lw);  // T diag(beta e^gamma)
    W::row_frags(t, pg + kChunk, hu, lu);      // T diag(beta)
    __syncthreads();  // T is read: w takes the W tile
    const int row = 16 * wave + c16;
    char* wrow = buf + OFF_W + row * SW + 8 * g4;
    W::template product<DK>(buf + OFF_K, SK, KX, hw, lw, [&](int dt, const f32x4_t& acc) {
      *reinterpret_cast<u32x2_t*>(wrow + 32 * dt) = u32x2_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    });
    f32x4_t uacc[UBV / 16];
    W::template product<UBV>(buf + OFF_U, SU, 0, hu, lu, [&](int dt, const f32x4_t& acc) { uacc[dt] = acc; });
    __syncthreads();  // every wave has read V: u takes the U tile
    char* urow = buf + OFF_U + row * SU + 8 * g4;
#pragma unroll
    for (int dt = 0; dt < UBV / 16; ++dt)
      *reinterpret_cast<u32x2_t*>(urow + 32 * dt) =
          u32x2_t{pack_bf16x2(uacc[dt][0], uacc[dt][1]), pack_bf16x2(uacc[dt][2], uacc[dt][3])};
    __syncthreads();
  }

  // FO: the chunk output of token tile `wave` over the block's BV columns
  // (fq: this wave's Q fragments of the chunk).  Called by every wave once
  // the chunk's h and v_new are staged; reads only LDS and registers, and
  // the K tile and the staging stay untouched until the next chunk's first
  // barrier.
  __device__ static __forceinline__ void fused_output(const Ctx& x, const Row& row, int c, const char* buf,
                                                      const char* so, const frag (&fq)[KS]) {
    const ScanArgs& a = *x.a;
    const int lane = threadIdx.x & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t H = x.H;
    const int DV = x.DV;
    const int64_t tok0 = static_cast<int64_t>(row.bos) + static_cast<int64_t>(c) * kChunk;
    const int nvalid = min(kChunk, row.len - c * kChunk);
    __syncthreads();  // every wave's h and v_new columns are staged

    // P^T[i][t] = k_i . q_t for t in tile `wave`, i tiles 0..wave
    const char* rowk = buf + OFF_K + c16 * SK + KX * (c16 >> 3) + 16 * g4;  // + 16 tile SK + 64 s
    f32x4_t pt[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) pt[it] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int it = 0; it < 4; ++it)
        if (it <= wave)
          S::mma(pt[it], lds_frag16(rowk, 16 * it * SK + 64 * s), fq[s]);
    const float* gm = reinterpret_cast<const float*>(buf + OFF_GM);
    const int t = 16 * wave + c16;
    const float gt = gm[t];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const f32x4_t gi = *reinterpret_cast<const f32x4_t*>(&gm[16 * it + 4 * g4]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * it + 4 * g4 + r;
        pt[it][r] = (i <= t && t < nvalid) ? pt[it][r] * exp_fast(gt - gi[r]) : 0.f;
      }
    }
    const float eg = exp_fast(gt);  // e^{gamma_t} of this lane's token

    // O^T = (S_c^T Q^T) e^{gamma} + v_new^T P^T, so that each lane ends with
    // four consecutive value columns of its token t = 16 wave + c16:
    // acc[ct][r] = O[t][16 ct + 4 g4 + r].  S_c^T is read from the staged h
    // rows (one value column each); v_new^T by transpose reads of the staged
    // v_new rows.
    constexpr int NCT = BV / 16;
    const char* rowh = so + c16 * SHS + 16 * g4;  // + 16 ct SHS + 64 s
    f32x4_t acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        S::mma(acc[ct], lds_frag16(rowh, 16 * ct * SHS + 64 * s), fq[s]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] *= eg;
    const char* vb = so + (OFF_VS - OFF_HS) + (4 * g4 + (c16 >> 2)) * SVS + 8 * (c16 & 3);  // + 32 s SVS (+16 SVS) + 32 ct
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (32 * s <= 16 * wave + 15) {
        const frag fp = S::frag_from_f32(pt[2 * s], pt[2 * s + 1]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          S::mma(acc[ct], S::frag_from_quads(lds_tr16(vb, 32 * s * SVS + 32 * ct), lds_tr16(vb, (32 * s + 16) * SVS + 32 * ct)),
                 fp);
      }
    }

    // o of the block's columns, 8 bytes per lane and column tile (rows past
    // the tail dropped by the range check)
    uint16_t* op = static_cast<uint16_t*>(a.o) + (tok0 * H + x.hd) * DV + x.col_blk;
    const rsrc_t ro = make_rsrc(op, static_cast<uint32_t>(((nvalid - 1) * H * DV + BV) * 2));
    const int voff = t * static_cast<int>(H * DV * 2) + 8 * g4;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(a.scale * acc[ct][0], a.scale * acc[ct][1]),
                                                    pack_bf16x2(a.scale * acc[ct][2], a.scale * acc[ct][3])},
                                            ro, voff, 32 * ct, 0);
  }

  // The staged outputs of chunk c (written before the last barrier) go to
  // global memory: the h block as one contiguous run, v_new as whole rows
  // (rows past the chunk's valid tokens fall outside the buffer range).
  __device__ static __forceinline__ void write_out(const Ctx& x, const Row& row, int c, const char* so) {
    const ScanArgs& a = *x.a;
    const int tid = threadIdx.x;
    const int64_t H = x.H;
    const int DV = x.DV;
    const int64_t tok0 = static_cast<int64_t>(row.bos) + static_cast<int64_t>(c) * kChunk;
    const int nvalid = min(kChunk, row.len - c * kChunk);
    uint16_t* hp = static_cast<uint16_t*>(a.h) + ((static_cast<int64_t>(row.chunk_off) + c) * H + x.hd) * DV * DK +
                   static_cast<int64_t>(x.col_blk) * DK;
    const rsrc_t rh = make_rsrc(hp, a.h != nullptr ? static_cast<uint32_t>(BV * DK * 2) : 0u);
#pragma unroll
    for (int i = 0; i < H_PT; ++i) {
      const int v = tid + NT * i;  // 16-byte vector of the block, row v / (DK / 8)
      const u32x4_t q = *reinterpret_cast<const u32x4_t*>(so + (v / (DK / 8)) * SHS + (v % (DK / 8)) * 16);
      __builtin_amdgcn_raw_buffer_store_b128(q, rh, 16 * v, 0, ST_POL);
    }
    uint16_t* vp = static_cast<uint16_t*>(a.v_new) + (tok0 * H + x.hd) * DV + x.col_blk;
    const rsrc_t rv =
        make_rsrc(vp, a.v_new != nullptr ? static_cast<uint32_t>(((nvalid - 1) * H * DV + BV) * 2) : 0u);
#pragma unroll
    for (int i = 0; i < V_PT; ++i) {
      const int v = tid + NT * i;  // token v / (BV / 8), 8 columns
      const int t = v / (BV / 8), p = v % (BV / 8);
      const u32x4_t q = *reinterpret_cast<const u32x4_t*>(so + (OFF_VS - OFF_HS) + t * SVS + p * 16);
      __builtin_amdgcn_raw_buffer_store_b128(q, rv, static_cast<int>(t * H * DV * 2) + 16 * p, 0, ST_POL);
    }
  }

  // One chunk.  The W operand reads are issued before the first matrix
  // instruction, the K operand reads while GEMM1 runs, and the accumulator
  // chains are interleaved, so the chunk pays the LDS and MFMA latencies about
  // once instead of once per product.  HASU: this wave's columns read U (the
  // state columns); the transition columns start GEMM1 from a zero
  // accumulator.  sig_out (SIG): the state's scale after the chunk.
  template <bool HASU>
  __device__ static __forceinline__ void compute(f32x4_t (&Sacc)[DT][NC], const Ctx& x, const Row& row, int c,
                                                 const char* buf, float& sig_out,
                                                 char* smem_out = nullptr) {  // smem_out: staging (STAGE)
    const ScanArgs& a = *x.a;
    const int lane = threadIdx.x & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int colw = wave * (BV / NW);
    const int64_t H = x.H;
    const int DV = x.DV;
    const int64_t tok0 = static_cast<int64_t>(row.bos) + static_cast<int64_t>(c) * kChunk;
    const int nvalid = min(kChunk, row.len - c * kChunk);

    // per-lane LDS bases (immediates carry the tile/step offsets)
    const char* wb = buf + OFF_W + c16 * SW + (g4 >> 1) * 16 + (g4 & 1) * 8;            // + 16 mt SW + 64 s (+32)
    const char* kb = buf + OFF_K + (4 * g4 + (c16 >> 2)) * SK + KX * (g4 >> 1) + (c16 & 3) * 8;  // + 32 s2 SK (+16 SK) + 32 dt
    // (MODE 2: the state waves' columns colw lie in the first BV/2, the staged U tile)
    const char* ub = buf + OFF_U + (4 * g4 + (c16 >> 2)) * SU + (colw + 4 * (c16 & 3)) * 2;  // + 16 mt SU + 32 ct
    const float* nd_l = reinterpret_cast<const float*>(buf + OFF_D) + 4 * g4;          // + 16 mt

    // FO: this wave's Q fragments (token tile `wave`), in flight during the chunk step
    frag fq[KS];
    auto load_q = [&]() {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (tok0 * H + x.hd) * DK;
      const rsrc_t rq = make_rsrc(qp, static_cast<uint32_t>(((nvalid - 1) * H + 1) * DK * 2));
      const int qo = static_cast<int>((16 * wave + c16) * H * DK * 2) + 16 * g4;  // contiguous k map
#pragma unroll
      for (int s = 0; s < KS; ++s)
        fq[s] = S::frag_from_quads(__builtin_amdgcn_raw_buffer_load_b64(rq, qo + 64 * s, 0, 0),
                                   __builtin_amdgcn_raw_buffer_load_b64(rq, qo + 64 * s + 8, 0, 0));
    };
    if constexpr (FO && !DENSE) load_q();
    u32x2_t uq[4][NC];
    if constexpr (HASU) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) uq[mt][ct] = lds_tr16(ub, 16 * mt * SU + 32 * ct);
    }
    auto w_frags = [&](frag (&f)[4], int s) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        f[mt] = S::frag_from_quads(lds_b64(wb, 16 * mt * SW + 64 * s), lds_b64(wb, 16 * mt * SW + 64 * s + 32));
    };
    frag aw[DENSE ? 1 : KS][4];
    if constexpr (!DENSE) {
#pragma unroll
      for (int s = 0; s < KS; ++s) w_frags(aw[s], s);
    }

    // ---- S as B operand; pre-chunk state h[c] ----
    frag Sb[KS][NC];
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) Sb[s][ct] = S::frag_from_f32(Sacc[2 * s][ct], Sacc[2 * s + 1][ct]);

    // ---- acc = -U + W S  (= -D; SIG: -U / sig + W S'); independent chains interleaved ----
    f32x4_t acc[4][NC];
    if constexpr (HASU) {
      const float us = SIG ? reinterpret_cast<const float*>(buf + OFF_D)[kChunk + 1] : -1.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
          const u32x2_t q = uq[mt][ct];
          if constexpr (SIG) {  // bf16 -> f32, times -1/sig
            acc[mt][ct] = f32x4_t{__builtin_bit_cast(float, q.x << 16) * us,
                                  __builtin_bit_cast(float, q.x & 0xffff0000u) * us,
                                  __builtin_bit_cast(float, q.y << 16) * us,
                                  __builtin_bit_cast(float, q.y & 0xffff0000u) * us};
          } else {  // bf16 -> f32 with the sign flipped in the same instruction
            acc[mt][ct] = f32x4_t{__builtin_bit_cast(float, (q.x << 16) + 0x80000000u),
                                  __builtin_bit_cast(float, (q.x & 0xffff0000u) ^ 0x80000000u),
                                  __builtin_bit_cast(float, (q.y << 16) + 0x80000000u),
                                  __builtin_bit_cast(float, (q.y & 0xffff0000u) ^ 0x80000000u)};
          }
        }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if constexpr (DENSE) w_frags(aw[0], s);
      const frag (&ws)[4] = aw[DENSE ? 0 : s];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
          if (!HASU && s == 0)
            acc[mt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ws[mt].v, Sb[s][ct].v,
                                                                  f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          else
            S::mma(acc[mt][ct], ws[mt], Sb[s][ct]);
        }
    }
    if constexpr (FO && DENSE) load_q();
    if constexpr (ALIAS) __syncthreads();  // every wave holds its W and U operands: their tiles become staging

    if (STAGE) {
      // h block: value column (colw + 16 ct + c16), rows 32 s + 4 g4 (+16)
      char* hs = smem_out + (colw + c16) * SHS + 8 * g4;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
          const u32x4_t q = __builtin_bit_cast(u32x4_t, Sb[s][ct].v);
          *reinterpret_cast<u32x2_t*>(hs + 16 * ct * SHS + 64 * s) = u32x2_t{q.x, q.y};
          *reinterpret_cast<u32x2_t*>(hs + 16 * ct * SHS + 64 * s + 32) = u32x2_t{q.z, q.w};
        }
    } else if (MODE == 0) {  // (a NULL output gets an empty range: the stores are dropped)
      uint16_t* hp = static_cast<uint16_t*>(a.h) +
                     ((static_cast<int64_t>(row.chunk_off) + c) * H + x.hd) * DV * DK +
                     static_cast<int64_t>(x.col_blk + colw) * DK;
      const rsrc_t rh = make_rsrc(hp, a.h != nullptr ? static_cast<uint32_t>((BV / NW) * DK * 2) : 0u);
      const int hoff = (c16 * DK + 4 * g4) * 2;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
          const u32x4_t q = __builtin_bit_cast(u32x4_t, Sb[s][ct].v);
          __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{q.x, q.y}, rh, hoff, (16 * ct * DK + 32 * s) * 2, 0);
          __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{q.z, q.w}, rh, hoff, (16 * ct * DK + 32 * s + 16) * 2, 0);
        }
    }

    // ---- K operand reads overlap GEMM1 ----
    auto k_frag = [&](int s2, int dt) {
      return S::frag_from_quads(lds_tr16(kb, 32 * s2 * SK + 32 * dt), lds_tr16(kb, (32 * s2 + 16) * SK + 32 * dt));
    };
    frag ak[DENSE ? 1 : 2][DENSE ? 1 : DT];
    if constexpr (!DENSE) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) ak[s2][dt] = k_frag(s2, dt);
    }
    f32x4_t nd[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) nd[mt] = *reinterpret_cast<const f32x4_t*>(nd_l + 16 * mt);
    const float eg = reinterpret_cast<const float*>(buf + OFF_D)[kChunk];

    // ---- v_new = -acc (tail rows dropped by the range check); D' = acc * nd ----
    if (STAGE) {
      // v_new tile: token 16 mt + 4 g4 + r, column colw + 16 ct + c16
      uint16_t* vs = reinterpret_cast<uint16_t*>(smem_out + (OFF_VS - OFF_HS)) + (4 * g4) * (SVS / 2) + colw + c16;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct)
#pragma unroll
          for (int r = 0; r < 4; r += 2) {
            const uint32_t pk = pack_bf16x2(-acc[mt][ct][r], -acc[mt][ct][r + 1]);
            vs[(16 * mt + r) * (SVS / 2) + 16 * ct] = static_cast<uint16_t>(pk);
            vs[(16 * mt + r + 1) * (SVS / 2) + 16 * ct] = static_cast<uint16_t>(pk >> 16);
          }
    } else if (MODE == 0) {
      uint16_t* vp = static_cast<uint16_t*>(a.v_new) + (tok0 * H + x.hd) * DV + x.col_blk + colw;
      const rsrc_t rv =
          make_rsrc(vp, a.v_new != nullptr ? static_cast<uint32_t>(((nvalid - 1) * H * DV + BV - colw) * 2) : 0u);
      const int rs = static_cast<int>(H * DV * 2);
      const int voff = (4 * g4) * rs + c16 * 2;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct)
#pragma unroll
          for (int r = 0; r < 4; r += 2) {
            const uint32_t pk = pack_bf16x2(-acc[mt][ct][r], -acc[mt][ct][r + 1]);
            const int so = (16 * mt + r) * rs + 32 * ct;
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(pk), rv, voff, so, 0);
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(pk >> 16), rv, voff, so + rs, 0);
          }
    }
    frag Db[2][NC];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) Db[s2][ct] = S::frag_from_f32(acc[2 * s2][ct] * nd[2 * s2], acc[2 * s2 + 1][ct] * nd[2 * s2 + 1]);

    // ---- S = exp(g_last) S + K^T D'  (KD: each state row by its channel's decay) ----
    if constexpr (KD) {
      const float* dec = reinterpret_cast<const float*>(buf + OFF_DEC) + 4 * g4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4_t dv4 = *reinterpret_cast<const f32x4_t*>(dec + 16 * dt);
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) Sacc[dt][ct] *= dv4;
      }
    } else if constexpr (SIG) {  // renormalising chunks only (eg holds the multiplier, 1 otherwise)
      sig_out = reinterpret_cast<const float*>(buf + OFF_D)[kChunk + 2];
      const float m = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, eg)));
      if (m != 1.f) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int ct = 0; ct < NC; ++ct) Sacc[dt][ct] *= m;
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) Sacc[dt][ct] *= eg;
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        if constexpr (DENSE) ak[0][0] = k_frag(s2, dt);
        const frag& kf = ak[DENSE ? 0 : s2][DENSE ? 0 : dt];
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) S::mma(Sacc[dt][ct], kf, Db[s2][ct]);
      }
    if constexpr (FO) fused_output(x, row, c, buf, smem_out, fq);
  }

  // The serial chunk loop of one block (HASU: this wave's columns read U).
  template <bool HASU>
  __device__ static __forceinline__ void chunk_loop(f32x4_t (&Sacc)[DT][NC], const Ctx& x, const Row& row, char* smem,
                                                    float& sig_out) {
    char* buf0 = smem;
    char* buf1 = smem + (NBUF == 2 ? BUF : 0);
    float sig = 1.f;  // SIG: scale of the staged chunks (first wave)
    auto step = [&](int c, const char* b, char* so) { compute<HASU>(Sacc, x, row, c, b, sig_out, so); };
    const int nchunks = (row.len + kChunk - 1) / kChunk;
    auto tok_of = [&](int c) { return static_cast<int64_t>(row.bos) + static_cast<int64_t>(c) * kChunk; };
    auto hr_of = [&](int c) { return static_cast<int64_t>(row.chunk_off) + c; };
    auto nv_of = [&](int c) { return min(kChunk, row.len - c * kChunk); };
    if (nchunks > 0) {
      if (NBUF == 1) {
        // one LDS buffer: fill, compute, and refill behind a second barrier;
        // the next chunk's loads are in flight during the compute
        Stage st;
        char* so = smem + OFF_HS;
        load(st, x, tok_of(0), nv_of(0), hr_of(0));
        for (int c = 0; c < nchunks; ++c) {
          __syncthreads();
          if (STAGE && c > 0) write_out(x, row, c - 1, so);
          if constexpr (ALIAS) __syncthreads();  // the staged outputs have left before the tiles refill them
          store(st, x, buf0, nv_of(c), sig, tok_of(c));
          __syncthreads();
          if (c + 1 < nchunks) load(st, x, tok_of(c + 1), nv_of(c + 1), hr_of(c + 1));
          if constexpr (PREP) prep_wy(buf0);
          step(c, buf0, so);
        }
        if (STAGE) {
          __syncthreads();
          write_out(x, row, nchunks - 1, so);
        }
      } else if (PF == 1) {
        Stage st;
        load(st, x, tok_of(0), nv_of(0), hr_of(0));
        store(st, x, buf0, nv_of(0), sig);
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
          char* cur = (c & 1) ? buf1 : buf0;
          char* nxt = (c & 1) ? buf0 : buf1;
          if (c + 1 < nchunks) load(st, x, tok_of(c + 1), nv_of(c + 1), hr_of(c + 1));
          step(c, cur, nullptr);
          if (c + 1 < nchunks) store(st, x, nxt, nv_of(c + 1), sig);
          __syncthreads();
        }
      } else {
        // two chunks in flight; loads and LDS fills are unconditional (chunks
        // past the end load as empty ranges and are never computed)
        Stage A, B;
        load(A, x, tok_of(0), nv_of(0), hr_of(0));
        load(B, x, tok_of(1), nv_of(1), hr_of(1));
        store(A, x, buf0, nv_of(0), sig);
        __syncthreads();
        for (int c = 0; c < nchunks; c += 2) {
          load(A, x, tok_of(c + 2), nv_of(c + 2), hr_of(c + 2));
          step(c, buf0, nullptr);
          store(B, x, buf1, nv_of(c + 1), sig);
          __syncthreads();
          if (c + 1 >= nchunks) break;
          load(B, x, tok_of(c + 3), nv_of(c + 3), hr_of(c + 3));
          step(c + 1, buf1, nullptr);
          store(A, x, buf0, nv_of(c + 2), sig);
          __syncthreads();
        }
      }
    }

  }

  __device__ static void run(const ScanArgs& a, char* smem) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int NJ = a.n_blk;
    const int bx = blockIdx.x;
    const int xcd = bx & 7, slot = bx >> 3;
    const int pair = 8 * (slot / NJ) + xcd;
    const int jb = slot % NJ;
    if (pair >= a.n_rows * a.H) return;
    const int ri = pair / a.H;
    const Row row = a.rows[ri];
    Ctx x;
    x.a = &a;
    x.hd = pair % a.H;
    x.H = a.H;
    x.DV = a.DV;
    x.col_blk = jb * UBV;
    const bool trans = (MODE == 1) && (x.col_blk >= x.DV);
    x.has_u = !trans;
    const int64_t H = a.H;
    // vector i of a thread is tid + i NT: row tid / CPW + i NT / CPW, column tid % CPW
    // (vectors past the U tile, if any, fall on rows past the chunk: the
    // buffer range check returns zero and the LDS store skips them)
    static_assert(NT % CPW == 0 && NT % CPU == 0, "whole rows per round of vectors");
    x.vo_wk = static_cast<int>((tid / CPW) * H * DK * 2 + (tid % CPW) * 16);
    x.st_wk = static_cast<int>((NT / CPW) * H * DK * 2);
    x.vo_u = static_cast<int>((tid / CPU) * H * x.DV * 2 + (tid % CPU) * 16);
    x.st_u = static_cast<int>((NT / CPU) * H * x.DV * 2);
    const int colw = wave * (BV / NW);
    const int DV = x.DV;
    const int hd = x.hd;
    // this wave's columns: of the transition (wtrans) or of the state / h_out,
    // first column colj
    const bool wtrans = (MODE == 2) ? (wave >= NW / 2) : trans;
    const int colj = (MODE == 2) ? x.col_blk + (wave % (NW / 2)) * (BV / NW)
                                 : x.col_blk + colw - (trans ? DV : 0);

    f32x4_t Sacc[DT][NC];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) Sacc[dt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (MODE == 0 && row.in_idx >= 0 && a.h_in != nullptr) {
      const float* base = a.h_in + (static_cast<int64_t>(row.in_idx) * H + hd) * DV * DK;
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        const int j = x.col_blk + colw + 16 * ct + c16;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int i0 = 16 * dt + 4 * g4;
          if (a.in_vk) {
            Sacc[dt][ct] = *reinterpret_cast<const f32x4_t*>(base + static_cast<int64_t>(j) * DK + i0);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) Sacc[dt][ct][r] = base[static_cast<int64_t>(i0 + r) * DV + j];
          }
        }
      }
    }
    if (MODE != 0 && wtrans) {
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        const int jj = colj + 16 * ct + c16;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) Sacc[dt][ct][r] = (16 * dt + 4 * g4 + r == jj) ? 1.f : 0.f;
      }
    }

    // wave-uniform: this wave's columns read U
    const bool use_u = (MODE == 0) || ((MODE == 2) ? (wave < NW / 2) : !trans);
    float sig_out = 1.f;  // SIG: the state's scale after the last chunk
    if (use_u)
      chunk_loop<true>(Sacc, x, row, smem, sig_out);
    else if constexpr (MODE != 0)
      chunk_loop<false>(Sacc, x, row, smem, sig_out);

    if (row.out_idx < 0) return;
    if constexpr (SIG) {  // the true state
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) Sacc[dt][ct] *= sig_out;
    }
    if (MODE == 0 || !wtrans) {
      if (a.h_out == nullptr) return;
      float* base = a.h_out + (static_cast<int64_t>(row.out_idx) * H + hd) * DV * DK;
      const bool vk = (MODE != 0) ? true : (a.out_vk != 0);
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        const int j = colj + 16 * ct + c16;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int i0 = 16 * dt + 4 * g4;
          if (vk) {
            *reinterpret_cast<f32x4_t*>(base + static_cast<int64_t>(j) * DK + i0) = Sacc[dt][ct];
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) base[static_cast<int64_t>(i0 + r) * DV + j] = Sacc[dt][ct][r];
          }
        }
      }
    } else {
      float* base = a.trans_out + (static_cast<int64_t>(row.out_idx) * H + hd) * DK * DK;
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        const int jj = colj + 16 * ct + c16;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) base[static_cast<int64_t>(16 * dt + 4 * g4 + r) * DK + jj] = Sacc[dt][ct][r];
      }
    }
  }
};

template <int DK, int BV, int NW, int PF, int MODE, int NBUF, bool KD, bool FO = false, bool DENSE = false,
          bool PREP = false>
__global__ __launch_bounds__(NW * 64, DENSE ? 3 : 1) void scan2_kernel(const ScanArgs a) {
  using K = Scan2<DK, BV, NW, PF, MODE, NBUF, KD, FO, DENSE, PREP>;
  __shared__ __align__(16) char smem[K::SMEM];
  K::run(a, smem);
}

template <int DK, int BV, int NW, int PF, int MODE, int NBUF, bool KD, bool FO = false, bool DENSE = false,
          bool PREP = false>
static hipError_t launch_scan2(const void* args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((scan2_kernel<DK, BV, NW, PF, MODE, NBUF, KD, FO, DENSE, PREP>), dim3(grid), dim3(NW * 64), 0,
                     stream,
                     *static_cast<const ScanArgs*>(args));
  return hipGetLastError();
}

// Built bf16 tiles (BV, waves, stages):
//   stages 2: one LDS buffer, the next chunk prefetched in registers (small LDS
//             footprint, several workgroups per CU: for many units)
//   stages 3: two LDS buffers, two chunks prefetched (for few, long units)
#define GDR_SCAN2_TILES(X, DK, MODE) \
  X(DK, 32, 2, 2, MODE, 1, 1)        \
  X(DK, 32, 2, 3, MODE, 2, 2)        \
  X(DK, 64, 2, 3, MODE, 2, 2)        \
  X(DK, 64, 4, 2, MODE, 1, 1)        \
  X(DK, 64, 4, 3, MODE, 2, 2)        \
  X(DK, 128, 4, 2, MODE, 1, 1)       \
  X(DK, 128, 4, 3, MODE, 2, 2)

#define GDR_SCAN2_CASE(DK, BV, NW, ST, MODE, PF, NBUF)                                        \
  if (dk == DK && bv == BV && waves == NW && stages == ST && mode == MODE)                      \
    return kd ? &launch_scan2<DK, BV, NW, PF, MODE, NBUF, true> : &launch_scan2<DK, BV, NW, PF, MODE, NBUF, false>;

LaunchFn find_scan2(int dk, int bv, int waves, int stages, int mode, bool kd) {
  GDR_SCAN2_TILES(GDR_SCAN2_CASE, 128, 0)
  GDR_SCAN2_TILES(GDR_SCAN2_CASE, 128, 1)
  GDR_SCAN2_TILES(GDR_SCAN2_CASE, 128, 2)
  GDR_SCAN2_TILES(GDR_SCAN2_CASE, 64, 0)
  GDR_SCAN2_TILES(GDR_SCAN2_CASE, 64, 1)
  GDR_SCAN2_TILES(GDR_SCAN2_CASE, 64, 2)
  // summaries only: one 8-wave block of all 256 columns of a (segment, head)
  GDR_SCAN2_CASE(128, 256, 8, 2, 2, 1, 1)
  return nullptr;
}

// The plain pass with the chunk output fused (tiles with stages 2 and four waves).
LaunchFn find_scan2_fused(int dk, int bv, int waves, int stages) {
  if (waves != 4 || stages != 2) return nullptr;
  if (dk == 128 && bv == 64) return &launch_scan2<128, 64, 4, 1, 0, 1, false, true>;
  if (dk == 128 && bv == 128) return &launch_scan2<128, 128, 4, 1, 0, 1, false, true>;
  if (dk == 64 && bv == 64) return &launch_scan2<64, 64, 4, 1, 0, 1, false, true>;
  if (dk == 64 && bv == 128) return &launch_scan2<64, 128, 4, 1, 0, 1, false, true>;
  return nullptr;
}

// The dense form of the staged plain pass (64-column blocks, four waves,
// stages 2): plain, per-channel decay (kd) or with the chunk output fused (fo).
LaunchFn find_scan2_dense(int dk, int bv, int waves, int stages, int mode, bool kd, bool fo) {
  if (bv != 64 || waves != 4 || stages != 2 || mode != 0 || (kd && fo)) return nullptr;
  if (dk == 128)
    return fo ? &launch_scan2<128, 64, 4, 1, 0, 1, false, true, true>
              : (kd ? &launch_scan2<128, 64, 4, 1, 0, 1, true, false, true> : &launch_scan2<128, 64, 4, 1, 0, 1, false, false, true>);
  if (dk == 64)
    return fo ? &launch_scan2<64, 64, 4, 1, 0, 1, false, true, true>
              : (kd ? &launch_scan2<64, 64, 4, 1, 0, 1, true, false, true> : &launch_scan2<64, 64, 4, 1, 0, 1, false, false, true>);
  return nullptr;
}

// The plain pass with the chunk prepare and the chunk output fused: the
// dense form only (with the prepare, the full form holds 253 VGPRs, one
// workgroup per CU).
LaunchFn find_scan2_prep(int dk) {
  if (dk == 128) return &launch_scan2<128, 64, 4, 1, 0, 1, false, true, true, true>;
  return nullptr;  // (DK = 64: the A / T scratch does not fit the W tile)
}

}  // namespace gdr
