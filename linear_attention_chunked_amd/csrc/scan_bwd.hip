// Reverse (gradient) state recurrence of the gated delta rule, bfloat16
// storage, gfx950 (flash-linear-attention fork issue #23, "Problem": the
// reverse kernel that walks the state chunk by chunk; "Proposed Dataflow",
// item 4: the reverse dH recurrence follows the forward one).
//
// With gamma = the chunk-local cumulative log decay, gamma_C its value at the
// chunk's last valid token, P[t][i] = (q_t . k_i) e^{gamma_t - gamma_i} for
// i <= t (zero otherwise), and dS the gradient with respect to the state
// after the chunk (dhT after a sequence's last chunk), every chunk, last to
// first:
//
//   dh[c]   = dS                                   (stored, storage dtype)
//   dv_new  = diag(e^{gamma_C - gamma}) K dS + scale P^T dO
//   dS      = e^{gamma_C} dS + scale Q^T diag(e^gamma) dO - W^T dv_new
//
// and dh0 = dS after the first chunk.  The chunk-local term scale P^T dO does
// not depend on dS: `dv_local_kernel` forms it for every chunk in parallel,
// and the serial `scan_bwd_kernel` adds the K dS part.  The serial kernel is
// the forward scan run backwards with the same gfx950 organisation: one
// workgroup per (sequence, head, 64 value columns), dS in FP32 MFMA
// accumulators for the whole loop, K as row fragments (K dS contracts over
// dk), Q and W through ds_read_b64_tr_b16 (Q^T and W^T contract over tokens),
// the next chunk's tiles prefetched in registers, dh and dv_new stored straight
// from the accumulators (no LDS staging, so two 128-key workgroups share a CU).
#include "gfx950.hpp"
#include "kernels.hpp"

namespace gdr {

// ---------------------------------------------------------------- scale P^T dO
// One workgroup per (chunk, head) for all DV value columns (Q and K read and
// P formed once per chunk-head); wave w owns key tile w.
template <int DK, int DV>
struct DvLocal {
  using S = St<bf16_t>;
  using frag = S::frag;
  static constexpr int NT = 256;
  static constexpr int BVO = DV;
  static constexpr int NCT = BVO / 16;
  static constexpr int SQ = DK * 2 + 16;   // Q, K rows (bytes)
  static constexpr int SD = BVO * 2 + 32;  // dO rows (transpose reads)
  static constexpr int KS = DK / 32;

  struct Smem {
    char q[kChunk * SQ];
    char k[kChunk * SQ];
    char d[kChunk * SD];
    float gam[kChunk];
  };

  __device__ static void run(const ChunkArgs& a, Smem& sm) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int NVB = DV / BVO;
    const int vb = blockIdx.x % NVB;
    const int rest = blockIdx.x / NVB;
    const int hd = rest % a.H;
    const int chunk = rest / a.H;
    if (chunk >= a.n_chunks) return;
    const Row row = row_of_chunk(a.rows, a.n_rows, chunk);
    const int cl = chunk - row.chunk_off;
    const int64_t tok0 = static_cast<int64_t>(row.bos) + static_cast<int64_t>(cl) * kChunk;
    const int nvalid = min(kChunk, row.len - cl * kChunk);
    const int64_t H = a.H;
    const int col0 = vb * BVO;
    {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (tok0 * H + hd) * DK;
      const uint16_t* kp = static_cast<const uint16_t*>(a.k) + (tok0 * H + hd) * DK;
      const uint16_t* dp = static_cast<const uint16_t*>(a.v) + (tok0 * H + hd) * DV + col0;  // dO
      const uint32_t qk_bytes = static_cast<uint32_t>(((nvalid - 1) * H + 1) * DK * 2);
      const rsrc_t rq = make_rsrc(qp, qk_bytes);
      const rsrc_t rk = make_rsrc(kp, qk_bytes);
      const rsrc_t rd = make_rsrc(dp, static_cast<uint32_t>(((nvalid - 1) * H * DV + BVO) * 2));
      constexpr int CQ = DK / 8, CD = BVO / 8;
#pragma unroll
      for (int i = 0; i < kChunk * CQ / NT; ++i) {
        const int vv = tid + i * NT, r = vv / CQ, c = vv % CQ;
        const int go = static_cast<int>(r * H * DK * 2 + c * 16);
        *reinterpret_cast<u32x4_t*>(sm.q + r * SQ + c * 16) = __builtin_amdgcn_raw_buffer_load_b128(rq, go, 0, 0);
        *reinterpret_cast<u32x4_t*>(sm.k + r * SQ + c * 16) = __builtin_amdgcn_raw_buffer_load_b128(rk, go, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kChunk * CD / NT; ++i) {
        const int vv = tid + i * NT, r = vv / CD, c = vv % CD;
        *reinterpret_cast<u32x4_t*>(sm.d + r * SD + c * 16) =
            __builtin_amdgcn_raw_buffer_load_b128(rd, static_cast<int>(r * H * DV * 2 + c * 16), 0, 0);
      }
      if (tid < kChunk) sm.gam[tid] = (tid < nvalid) ? a.g[(tok0 + tid) * H + hd] : 0.f;
    }
    __syncthreads();

    // P[t][i] for the wave's key tile i (C layout: rows t, column i), t tiles >= the key tile
    const char* rq = sm.q + c16 * SQ + 8 * g4;
    const char* rk = sm.k + c16 * SQ + 8 * g4;
    auto rfrag = [&](const char* base, int tile, int s) {
      return S::frag_from_quads(*reinterpret_cast<const u32x2_t*>(base + 16 * tile * SQ + 64 * s),
                                *reinterpret_cast<const u32x2_t*>(base + 16 * tile * SQ + 64 * s + 32));
    };
    f32x4_t p[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) p[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const frag fk = rfrag(rk, wave, s);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        if (tt >= wave) S::mma(p[tt], rfrag(rq, tt, s), fk);
    }
    const int i = 16 * wave + c16;
    const float gi = sm.gam[i];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const f32x4_t gt = *reinterpret_cast<const f32x4_t*>(&sm.gam[16 * tt + 4 * g4]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tt + 4 * g4 + r;
        p[tt][r] = (i <= t && t < nvalid) ? a.scale * p[tt][r] * exp_fast(gt[r] - gi) : 0.f;
      }
    }
    // dv_local rows i (the wave's key tile) = sum_t P[t][i] dO[t][:]
    f32x4_t acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const char* db = sm.d + (4 * g4 + (c16 >> 2)) * SD + 8 * (c16 & 3);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      if (32 * s2 + 31 >= 16 * wave) {
        const frag fa = S::frag_from_f32(p[2 * s2], p[2 * s2 + 1]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          S::mma(acc[ct], fa, S::frag_from_quads(lds_tr16(db, 32 * s2 * SD + 32 * ct),
                                                 lds_tr16(db, (32 * s2 + 16) * SD + 32 * ct)));
      }
    }
    uint16_t* op = static_cast<uint16_t*>(a.o) + (tok0 * H + hd) * DV + col0;  // dv_local
    const rsrc_t ro = make_rsrc(op, static_cast<uint32_t>(((nvalid - 1) * H * DV + BVO) * 2));
    const int rs = static_cast<int>(H * DV * 2);
    const int voff = (16 * wave + 4 * g4) * rs + c16 * 2;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const uint32_t pk = pack_bf16x2(acc[ct][r], acc[ct][r + 1]);
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(pk), ro, voff, r * rs + 32 * ct, 0);
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(pk >> 16), ro, voff, (r + 1) * rs + 32 * ct, 0);
      }
  }
};

template <int DK, int DV>
__global__ __launch_bounds__(256) void dv_local_kernel(const ChunkArgs a) {
  using K = DvLocal<DK, DV>;
  __shared__ __align__(16) typename K::Smem sm;
  K::run(a, sm);
}

template <int DK, int DV>
static hipError_t launch_dv_local(const void* args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((dv_local_kernel<DK, DV>), dim3(grid), dim3(256), 0, stream,
                     *static_cast<const ChunkArgs*>(args));
  return hipGetLastError();
}

LaunchFn find_dv_local(int dk, int dv) {
  if (dk == 128 && dv == 128) return &launch_dv_local<128, 128>;
  if (dk == 128 && dv == 64) return &launch_dv_local<128, 64>;
  if (dk == 64 && dv == 128) return &launch_dv_local<64, 128>;
  if (dk == 64 && dv == 64) return &launch_dv_local<64, 64>;
  return nullptr;
}

// ---------------------------------------------------------------- reverse scan
template <int DK>
struct ScanBwd {
  using S = St<bf16_t>;
  using frag = S::frag;
  static constexpr int BV = 64, NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int KS = DK / 32;
  static constexpr int DT = DK / 16;
  static constexpr int RB = DK * 2;       // bytes per K / Q / W row
  static constexpr int RBV = BV * 2;      // bytes per dO / dv_local row (this block)
  static constexpr int SKR = RB + 16;     // K rows (row fragments)
  static constexpr int SQT = RB + 32;     // Q, W rows (transpose reads)
  static constexpr int SDV = RBV + 32;    // dO, dv_local rows (transpose reads)
  static constexpr int CPR = RB / 16, CPV = RBV / 16;
  static constexpr int OFF_K = 0, OFF_Q = kChunk * SKR, OFF_W = OFF_Q + kChunk * SQT;
  static constexpr int OFF_DO = OFF_W + kChunk * SQT, OFF_DL = OFF_DO + kChunk * SDV;
  static constexpr int OFF_F = OFF_DL + kChunk * SDV;  // d_i = e^{gC - g_i}, f_t = scale e^{g_t}, then e^{gC}
  static constexpr int BUF = OFF_F + 2 * kChunk * 4 + 16;
  static constexpr int SMEM = BUF;
  static constexpr int R_PT = kChunk * CPR / NT;   // 16-byte K / Q / W vectors per thread
  static constexpr int V_PT = kChunk * CPV / NT;   // 16-byte dO / dv_local vectors per thread

  struct Stage {
    u32x4_t k[R_PT], q[R_PT], w[R_PT];
    u32x4_t d[V_PT], l[V_PT];
    float g;
  };

  struct Ctx {
    const ScanBwdArgs* a;
    int hd, col_blk, H, DV;
    int vo_r[R_PT], vo_v[V_PT];
  };

  __device__ static __forceinline__ void load(Stage& st, const Ctx& x, int64_t tok0, int nvalid) {
    const ScanBwdArgs& a = *x.a;
    const int64_t H = x.H;
    const bool any = nvalid > 0;  // chunks before the first read nothing
    const uint32_t rbytes = any ? static_cast<uint32_t>(((nvalid - 1) * H + 1) * DK * 2) : 0u;
    const uint32_t vbytes = any ? static_cast<uint32_t>(((nvalid - 1) * H * x.DV + BV) * 2) : 0u;
    const int64_t ro = (tok0 * H + x.hd) * DK, vo = (tok0 * H + x.hd) * x.DV + x.col_blk;
    const rsrc_t rk = make_rsrc(static_cast<const uint16_t*>(a.k) + ro, rbytes);
    const rsrc_t rq = make_rsrc(static_cast<const uint16_t*>(a.q) + ro, rbytes);
    const rsrc_t rw = make_rsrc(static_cast<const uint16_t*>(a.w) + ro, rbytes);
    const rsrc_t rd = make_rsrc(static_cast<const uint16_t*>(a.dO) + vo, vbytes);
    const rsrc_t rl = make_rsrc(static_cast<const uint16_t*>(a.dv_local) + vo, vbytes);
#pragma unroll
    for (int i = 0; i < R_PT; ++i) {
      st.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, x.vo_r[i], 0, 0);
      st.q[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, x.vo_r[i], 0, 0);
      st.w[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, x.vo_r[i], 0, 0);
    }
#pragma unroll
    for (int i = 0; i < V_PT; ++i) {
      st.d[i] = __builtin_amdgcn_raw_buffer_load_b128(rd, x.vo_v[i], 0, 0);
      st.l[i] = __builtin_amdgcn_raw_buffer_load_b128(rl, x.vo_v[i], 0, 0);
    }
    const rsrc_t rg = make_rsrc(a.g_cum + tok0 * H + x.hd, any ? static_cast<uint32_t>(((nvalid - 1) * H + 1) * 4) : 0u);
    st.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, static_cast<int>((threadIdx.x & 63) * H * 4), 0, 0));
  }

  __device__ static __forceinline__ void store(const Stage& st, const Ctx& x, char* buf, int nvalid) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < R_PT; ++i) {
      const int v = tid + i * NT, r = v / CPR, c = v % CPR;
      *reinterpret_cast<u32x4_t*>(buf + OFF_K + r * SKR + c * 16) = st.k[i];
      *reinterpret_cast<u32x4_t*>(buf + OFF_Q + r * SQT + c * 16) = st.q[i];
      *reinterpret_cast<u32x4_t*>(buf + OFF_W + r * SQT + c * 16) = st.w[i];
    }
#pragma unroll
    for (int i = 0; i < V_PT; ++i) {
      const int v = tid + i * NT, r = v / CPV, c = v % CPV;
      *reinterpret_cast<u32x4_t*>(buf + OFF_DO + r * SDV + c * 16) = st.d[i];
      *reinterpret_cast<u32x4_t*>(buf + OFF_DL + r * SDV + c * 16) = st.l[i];
    }
    if (tid < kChunk) {  // first wave: the chunk's decay factors
      const float g_last = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, st.g), nvalid - 1));
      float* f = reinterpret_cast<float*>(buf + OFF_F);
      const bool ok = tid < nvalid;
      f[tid] = ok ? exp_fast(g_last - st.g) : 0.f;                      // d_i
      f[kChunk + tid] = ok ? x.a->scale * exp_fast(st.g) : 0.f;        // f_t
      if (tid == 0) f[2 * kChunk] = exp_fast(g_last);
    }
  }

  // One chunk, dS carried in from the later chunks.
  __device__ static __forceinline__ void compute(f32x4_t (&Sacc)[DT], const char* buf, const Ctx& x, const Row& row,
                                                 int c) {
    const ScanBwdArgs& a = *x.a;
    const int lane = threadIdx.x & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int colw = 16 * wave;  // this wave's 16 columns of the block
    const int64_t H = x.H;
    const int DV = x.DV;
    const int64_t tok0 = static_cast<int64_t>(row.bos) + static_cast<int64_t>(c) * kChunk;
    const int nvalid = min(kChunk, row.len - c * kChunk);

    // dS as B operand; dh[c] = dS, stored from the registers (value row colw + c16, 4 keys per piece)
    frag Sb[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) Sb[s] = S::frag_from_f32(Sacc[2 * s], Sacc[2 * s + 1]);
    {
      uint16_t* hp = static_cast<uint16_t*>(a.dh) + ((static_cast<int64_t>(row.chunk_off) + c) * H + x.hd) * DV * DK +
                     static_cast<int64_t>(x.col_blk) * DK;
      const rsrc_t rh = make_rsrc(hp, a.dh != nullptr ? static_cast<uint32_t>(BV * DK * 2) : 0u);
      const int ho = ((colw + c16) * DK + 4 * g4) * 2;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const u32x4_t q = __builtin_bit_cast(u32x4_t, Sb[s].v);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{q.x, q.y}, rh, ho, 64 * s, 0);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{q.z, q.w}, rh, ho, 64 * s + 32, 0);
      }
    }
    // GEMM1: acc = K dS (tokens x this wave's columns)
    const char* kb = buf + OFF_K + c16 * SKR + 8 * g4;
    f32x4_t acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        S::mma(acc[mt], S::frag_from_quads(lds_b64(kb, 16 * mt * SKR + 64 * s), lds_b64(kb, 16 * mt * SKR + 64 * s + 32)),
               Sb[s]);
    // transposed operands of GEMM2 (contraction over tokens), read while GEMM1 runs
    const int tr = (4 * g4 + (c16 >> 2));
    const char* qb = buf + OFF_Q + tr * SQT + (c16 & 3) * 8;
    const char* wb = buf + OFF_W + tr * SQT + (c16 & 3) * 8;
    const char* dob = buf + OFF_DO + tr * SDV + (colw + 4 * (c16 & 3)) * 2;
    const char* dlb = buf + OFF_DL + tr * SDV + (colw + 4 * (c16 & 3)) * 2;
    const float* fv = reinterpret_cast<const float*>(buf + OFF_F);
    // dv_new = d_i * acc + dv_local (C layout: rows = tokens 16 mt + 4 g4 + r, column colw + c16)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f32x4_t d = *reinterpret_cast<const f32x4_t*>(fv + 16 * mt + 4 * g4);
      const u32x2_t l = lds_tr16(dlb, 16 * mt * SDV);
      const f32x4_t lf{__builtin_bit_cast(float, l.x << 16), __builtin_bit_cast(float, l.x & 0xffff0000u),
                       __builtin_bit_cast(float, l.y << 16), __builtin_bit_cast(float, l.y & 0xffff0000u)};
      acc[mt] = acc[mt] * d + lf;
    }
    {  // dv_new (rows = tokens, rows past the tail dropped by the range check)
      uint16_t* vp = static_cast<uint16_t*>(a.dv) + (tok0 * H + x.hd) * DV + x.col_blk;
      const rsrc_t rv =
          make_rsrc(vp, a.dv != nullptr ? static_cast<uint32_t>(((nvalid - 1) * H * DV + BV) * 2) : 0u);
      const int rs = static_cast<int>(H * DV * 2);
      const int voff = (4 * g4) * rs + (colw + c16) * 2;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const uint32_t pk = pack_bf16x2(acc[mt][r], acc[mt][r + 1]);
          const int so2 = (16 * mt + r) * rs;
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(pk), rv, voff, so2, 0);
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(pk >> 16), rv, voff, so2 + rs, 0);
        }
    }
    // B operands over tokens: -dv_new, and f_t dO_t
    frag Bv[2], Bd[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      Bv[s2] = S::frag_from_f32(-acc[2 * s2], -acc[2 * s2 + 1]);
      const f32x4_t f0 = *reinterpret_cast<const f32x4_t*>(fv + kChunk + 32 * s2 + 4 * g4);
      const f32x4_t f1 = *reinterpret_cast<const f32x4_t*>(fv + kChunk + 32 * s2 + 16 + 4 * g4);
      const u32x2_t d0 = lds_tr16(dob, 32 * s2 * SDV), d1 = lds_tr16(dob, (32 * s2 + 16) * SDV);
      const f32x4_t x0{__builtin_bit_cast(float, d0.x << 16) * f0[0], __builtin_bit_cast(float, d0.x & 0xffff0000u) * f0[1],
                       __builtin_bit_cast(float, d0.y << 16) * f0[2], __builtin_bit_cast(float, d0.y & 0xffff0000u) * f0[3]};
      const f32x4_t x1{__builtin_bit_cast(float, d1.x << 16) * f1[0], __builtin_bit_cast(float, d1.x & 0xffff0000u) * f1[1],
                       __builtin_bit_cast(float, d1.y << 16) * f1[2], __builtin_bit_cast(float, d1.y & 0xffff0000u) * f1[3]};
      Bd[s2] = S::frag_from_f32(x0, x1);
    }
    // GEMM2: dS = e^{gC} dS + Q^T (f dO) - W^T dv_new
    const float eg = fv[2 * kChunk];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) Sacc[dt] *= eg;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const frag aq = S::frag_from_quads(lds_tr16(qb, 32 * s2 * SQT + 32 * dt), lds_tr16(qb, (32 * s2 + 16) * SQT + 32 * dt));
        const frag aw = S::frag_from_quads(lds_tr16(wb, 32 * s2 * SQT + 32 * dt), lds_tr16(wb, (32 * s2 + 16) * SQT + 32 * dt));
        S::mma(Sacc[dt], aq, Bd[s2]);
        S::mma(Sacc[dt], aw, Bv[s2]);
      }
  }

  __device__ static void run(const ScanBwdArgs& a, char* smem) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int NJ = a.DV / BV;
    const int bx = blockIdx.x;
    const int xcd = bx & 7, slot = bx >> 3;
    const int pair = 8 * (slot / NJ) + xcd;
    const int jb = slot % NJ;
    if (pair >= a.n_rows * a.H) return;
    const Row row = a.rows[pair / a.H];
    Ctx x;
    x.a = &a;
    x.hd = pair % a.H;
    x.H = a.H;
    x.DV = a.DV;
    x.col_blk = jb * BV;
    const int64_t H = a.H;
#pragma unroll
    for (int i = 0; i < R_PT; ++i) {
      const int v = tid + i * NT;
      x.vo_r[i] = static_cast<int>((v / CPR) * H * DK * 2 + (v % CPR) * 16);
    }
#pragma unroll
    for (int i = 0; i < V_PT; ++i) {
      const int v = tid + i * NT;
      x.vo_v[i] = static_cast<int>((v / CPV) * H * x.DV * 2 + (v % CPV) * 16);
    }
    const int colw = 16 * wave;
    const int DV = x.DV;
    const int hd = x.hd;
    const int nchunks = (row.len + kChunk - 1) / kChunk;

    // dS after the last chunk: dhT (or zero)
    f32x4_t Sacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) Sacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (row.in_idx >= 0 && a.dhT != nullptr) {
      const float* base = a.dhT + (static_cast<int64_t>(row.in_idx) * H + hd) * DV * DK;
      const int j = x.col_blk + colw + c16;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int i0 = 16 * dt + 4 * g4;
        if (a.state_vk) {
          Sacc[dt] = *reinterpret_cast<const f32x4_t*>(base + static_cast<int64_t>(j) * DK + i0);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) Sacc[dt][r] = base[static_cast<int64_t>(i0 + r) * DV + j];
        }
      }
    }

    char* buf = smem;
    auto tok_of = [&](int c) { return static_cast<int64_t>(row.bos) + static_cast<int64_t>(c) * kChunk; };
    auto nv_of = [&](int c) { return c >= 0 ? min(kChunk, row.len - c * kChunk) : 0; };
    if (nchunks > 0) {
      Stage st;
      load(st, x, tok_of(nchunks - 1), nv_of(nchunks - 1));
      for (int c = nchunks - 1; c >= 0; --c) {
        __syncthreads();
        store(st, x, buf, nv_of(c));
        __syncthreads();
        load(st, x, tok_of(c - 1 >= 0 ? c - 1 : 0), nv_of(c - 1));
        compute(Sacc, buf, x, row, c);
      }
    }

    if (row.out_idx < 0 || a.dh0 == nullptr) return;
    float* base = a.dh0 + (static_cast<int64_t>(row.out_idx) * H + hd) * DV * DK;
    const int j = x.col_blk + colw + c16;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int i0 = 16 * dt + 4 * g4;
      if (a.state_vk) {
        *reinterpret_cast<f32x4_t*>(base + static_cast<int64_t>(j) * DK + i0) = Sacc[dt];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) base[static_cast<int64_t>(i0 + r) * DV + j] = Sacc[dt][r];
      }
    }
  }
};

template <int DK>
__global__ __launch_bounds__(256) void scan_bwd_kernel(const ScanBwdArgs a) {
  using K = ScanBwd<DK>;
  __shared__ __align__(16) char smem[K::SMEM];
  K::run(a, smem);
}

template <int DK>
static hipError_t launch_scan_bwd(const void* args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((scan_bwd_kernel<DK>), dim3(grid), dim3(256), 0, stream, *static_cast<const ScanBwdArgs*>(args));
  return hipGetLastError();
}

LaunchFn find_scan_bwd(int dk) {
  if (dk == 128) return &launch_scan_bwd<128>;
  if (dk == 64) return &launch_scan_bwd<64>;
  return nullptr;
}

}  // namespace gdr
