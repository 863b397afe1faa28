// The inter-chunk state scan of the gated delta rule on gfx950.
//
// One workgroup owns one unit (row = sequence or segment, head, block of BV
// value columns) and walks the row's 64-token chunks serially
// (kev pull request #259, opening section: one program per value block,
// serial over chunks).  Per chunk, with S the FP32 state [DK x BV]:
//
//     h[c]   = S                                  (pre-chunk state)
//     D      = U_c - W_c S                        (v_new, 64 x BV)
//     D'     = D * exp(gamma_last - gamma_t)      (rows past the tail -> 0)
//     S      = exp(gamma_last) S + K_c^T D'
//
// Mapping to CDNA4:
//   * S never leaves the wave: each of the NW waves owns BV/NW whole columns
//     of S (all DK rows) as MFMA accumulators.  With the k(g, e) operand map
//     of common.hpp, two stacked accumulator tiles ARE the B operand of the
//     next contraction, so S feeds W_c S and D' feeds K_c^T D' straight from
//     registers.
//   * W_c (row-major), K_c^T and U_c^T (transposed on the way into LDS) are
//     staged once per chunk per workgroup and shared by the waves; rows are
//     padded so the A-operand reads of 16 consecutive rows hit distinct banks.
//   * STAGES = 2 issues the next chunk's global loads before the current
//     chunk's matrix work, so the HBM latency overlaps the MFMA chain.
//   * Every column goes through the same instruction sequence whatever the
//     tile (BV, NW, STAGES): the tile only decides which wave owns a column
//     and when loads are issued, so all tiles give bit-identical results.
//
// MODE 1 runs the same recurrence for segment summaries (cuLA pull request
// #127, "Root cause and implementation"): the value blocks start from zero
// (local state), and DK extra columns start from the identity with U = 0, so
// after the segment they hold the segment's transition product M.
#include "kernels.hpp"

namespace gdr {

template <typename TI, int DK, int BV, int NW, int STAGES, int MODE>
struct ScanKernel {
  using S = St<TI>;
  using quad = typename S::quad;
  using frag = typename S::frag;
  static constexpr int NT = NW * 64;                 // threads
  static constexpr int NC = BV / (16 * NW);          // 16-column tiles per wave
  static constexpr int KS = DK / 32;                 // 32-wide k-steps over DK
  static constexpr int DT = DK / 16;                 // 16-row tiles of S
  static constexpr int EPV = 16 / sizeof(TI);        // elements per 16-byte vector
  static constexpr int LDW = DK + EPV;               // W row stride (elements), +16 B
  static constexpr int LDT = kChunk + 4;             // K^T / U^T row stride (elements)
  static constexpr int W_VECS = kChunk * DK / EPV;   // 16-byte vectors in W_c
  static constexpr int K_BLKS = (kChunk / 4) * (DK / 4);  // 4x4 blocks of K_c
  static constexpr int U_BLKS = (kChunk / 4) * (BV / 4);
  static constexpr int W_PT = (W_VECS + NT - 1) / NT;
  static constexpr int K_PT = (K_BLKS + NT - 1) / NT;
  static constexpr int U_PT = (U_BLKS + NT - 1) / NT;
  static_assert(BV % (16 * NW) == 0 && NC >= 1, "each wave owns whole 16-column tiles");
  static_assert(DK % 32 == 0, "DK must be a multiple of 32");

  struct Smem {
    TI w[kChunk * LDW];
    TI kt[DK * LDT];
    TI ut[BV * LDT];
    float g[kChunk];
  };

  struct Stage {
    u32x4_t wv[W_PT];
    quad kq[K_PT][4];
    quad uq[U_PT][4];
    float g;
  };

  __device__ static __forceinline__ void load(Stage& st, const ScanArgs& a, int64_t tok0, int nvalid,
                                              int hd, int col_blk, bool has_u) {
    const int tid = threadIdx.x;
    const TI* __restrict__ wp = static_cast<const TI*>(a.w);
    const TI* __restrict__ kp = static_cast<const TI*>(a.k);
    const TI* __restrict__ up = static_cast<const TI*>(a.u);
    const int64_t H = a.H;
#pragma unroll
    for (int i = 0; i < W_PT; ++i) {
      const int v = tid + i * NT;
      const int r = v / (DK / EPV), cv = v % (DK / EPV);
      u32x4_t x{0u, 0u, 0u, 0u};
      if ((W_VECS % NT == 0 || v < W_VECS) && r < nvalid)
        x = *reinterpret_cast<const u32x4_t*>(wp + ((tok0 + r) * H + hd) * DK + cv * EPV);
      st.wv[i] = x;
    }
#pragma unroll
    for (int i = 0; i < K_PT; ++i) {
      const int b = tid + i * NT;
      const int dq = b % (DK / 4), tq = b / (DK / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * tq + r;
        quad x = S::zero_quad();
        if ((K_BLKS % NT == 0 || b < K_BLKS) && t < nvalid) x = ld_quad<TI>(kp + ((tok0 + t) * H + hd) * DK + 4 * dq);
        st.kq[i][r] = x;
      }
    }
    if (has_u) {
      const int DV = a.DV;
#pragma unroll
      for (int i = 0; i < U_PT; ++i) {
        const int b = tid + i * NT;
        const int cq = b % (BV / 4), tq = b / (BV / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 4 * tq + r;
          quad x = S::zero_quad();
          if ((U_BLKS % NT == 0 || b < U_BLKS) && t < nvalid)
            x = ld_quad<TI>(up + ((tok0 + t) * H + hd) * DV + col_blk + 4 * cq);
          st.uq[i][r] = x;
        }
      }
    }
    st.g = 0.f;
    if (tid < kChunk && tid < nvalid) st.g = a.g_cum[(tok0 + tid) * H + hd];
  }

  __device__ static __forceinline__ void store(const Stage& st, Smem& sm, bool has_u) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < W_PT; ++i) {
      const int v = tid + i * NT;
      if (W_VECS % NT == 0 || v < W_VECS) {
        const int r = v / (DK / EPV), cv = v % (DK / EPV);
        *reinterpret_cast<u32x4_t*>(&sm.w[r * LDW + cv * EPV]) = st.wv[i];
      }
    }
#pragma unroll
    for (int i = 0; i < K_PT; ++i) {
      const int b = tid + i * NT;
      if (K_BLKS % NT == 0 || b < K_BLKS) {
        const int dq = b % (DK / 4), tq = b / (DK / 4);
        quad tr[4];
        S::transpose4(st.kq[i], tr);
#pragma unroll
        for (int j = 0; j < 4; ++j) st_quad<TI>(&sm.kt[(4 * dq + j) * LDT + 4 * tq], tr[j]);
      }
    }
    if (has_u) {
#pragma unroll
      for (int i = 0; i < U_PT; ++i) {
        const int b = tid + i * NT;
        if (U_BLKS % NT == 0 || b < U_BLKS) {
          const int cq = b % (BV / 4), tq = b / (BV / 4);
          quad tr[4];
          S::transpose4(st.uq[i], tr);
#pragma unroll
          for (int j = 0; j < 4; ++j) st_quad<TI>(&sm.ut[(4 * cq + j) * LDT + 4 * tq], tr[j]);
        }
      }
    }
    if (tid < kChunk) sm.g[tid] = st.g;
  }

  __device__ static void run(const ScanArgs& a, Smem& sm) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
    const int NJ = a.n_blk;
    const int bx = blockIdx.x;
    const int xcd = bx & 7, slot = bx >> 3;
    const int pair = 8 * (slot / NJ) + xcd;   // (row, head) pair; its blocks share an XCD
    const int jb = slot % NJ;
    if (pair >= a.n_rows * a.H) return;
    const int ri = pair / a.H, hd = pair % a.H;
    const Row row = a.rows[ri];
    const int64_t H = a.H;
    const int DV = a.DV;
    const int col_blk = jb * BV;                       // first column of the block
    const int colw = wave * (BV / NW);                 // wave's first column in the block
    const bool trans = (MODE == 1) && (col_blk >= DV); // transition columns (summaries)
    const bool has_u = !trans;
    const int nchunks = (row.len + kChunk - 1) / kChunk;

    // ---- initial state (C layout: Sacc[dt][ct][r] = S[16 dt + 4 g4 + r][col]) ----
    f32x4_t Sacc[DT][NC];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) Sacc[dt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (MODE == 0 && row.in_idx >= 0 && a.h_in != nullptr) {
      const float* base = a.h_in + (static_cast<int64_t>(row.in_idx) * H + hd) * DV * DK;
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        const int j = col_blk + colw + 16 * ct + c16;
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
    if (MODE == 1 && trans) {
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        const int jj = col_blk + colw + 16 * ct + c16 - DV;  // transition column
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) Sacc[dt][ct][r] = (16 * dt + 4 * g4 + r == jj) ? 1.f : 0.f;
      }
    }

    Stage st;
    if (STAGES == 2 && nchunks > 0)
      load(st, a, row.bos, min(kChunk, row.len), hd, col_blk, has_u);

    for (int c = 0; c < nchunks; ++c) {
      const int64_t tok0 = static_cast<int64_t>(row.bos) + static_cast<int64_t>(c) * kChunk;
      const int nvalid = min(kChunk, row.len - c * kChunk);
      if (STAGES == 1) load(st, a, tok0, nvalid, hd, col_blk, has_u);
      __syncthreads();  // previous chunk's LDS reads are done
      store(st, sm, has_u);
      __syncthreads();
      if (STAGES == 2 && c + 1 < nchunks)
        load(st, a, tok0 + kChunk, min(kChunk, row.len - (c + 1) * kChunk), hd, col_blk, has_u);

      // ---- S as B operand; emit h[c] ----
      frag Sb[KS][NC];
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) Sb[s][ct] = S::frag_from_f32(Sacc[2 * s][ct], Sacc[2 * s + 1][ct]);
      if (MODE == 0 && a.h != nullptr) {
        TI* hb = static_cast<TI*>(a.h) + ((static_cast<int64_t>(row.chunk_off) + c) * H + hd) * DV * DK;
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
          const int j = col_blk + colw + 16 * ct + c16;
          TI* hj = hb + static_cast<int64_t>(j) * DK;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            float f[4] = {Sacc[dt][ct][0], Sacc[dt][ct][1], Sacc[dt][ct][2], Sacc[dt][ct][3]};
            st_quad<TI>(hj + 16 * dt + 4 * g4, S::f32_to_quad(f));
          }
        }
      }

      // ---- D = U - W S ----
      f32x4_t Dm[4][NC];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
          if (has_u) {
            float f[4];
            S::quad_to_f32(ld_quad<TI>(&sm.ut[(colw + 16 * ct + c16) * LDT + 16 * mt + 4 * g4]), f);
            Dm[mt][ct] = f32x4_t{f[0], f[1], f[2], f[3]};
          } else {
            Dm[mt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
        }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const TI* wr = &sm.w[(16 * mt + c16) * LDW + 32 * s + 4 * g4];
          const frag aw = S::frag_from_quads_neg(ld_quad<TI>(wr), ld_quad<TI>(wr + 16));
#pragma unroll
          for (int ct = 0; ct < NC; ++ct) S::mma(Dm[mt][ct], aw, Sb[s][ct]);
        }
      }

      // ---- v_new, decay weights, masked tail ----
      const float g_last = sm.g[nvalid - 1];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4_t gm = *reinterpret_cast<const f32x4_t*>(&sm.g[16 * mt + 4 * g4]);
        float dsc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * mt + 4 * g4 + r;
          dsc[r] = (t < nvalid) ? expf(g_last - gm[r]) : 0.f;
        }
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) {
          if (MODE == 0 && a.v_new != nullptr) {
            TI* vp = static_cast<TI*>(a.v_new);
            const int j = col_blk + colw + 16 * ct + c16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = 16 * mt + 4 * g4 + r;
              if (t < nvalid) {
                const int64_t off = ((tok0 + t) * H + hd) * DV + j;
                if constexpr (sizeof(TI) == 2) {
                  reinterpret_cast<uint16_t*>(vp)[off] = f32_to_bf16(Dm[mt][ct][r]);
                } else {
                  reinterpret_cast<float*>(vp)[off] = Dm[mt][ct][r];
                }
              }
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) Dm[mt][ct][r] *= dsc[r];
        }
      }

      // ---- S = exp(g_last) S + K^T D' ----
      const float eg = expf(g_last);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) Sacc[dt][ct] *= eg;
      frag Db[2][NC];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) Db[s2][ct] = S::frag_from_f32(Dm[2 * s2][ct], Dm[2 * s2 + 1][ct]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const TI* kr = &sm.kt[(16 * dt + c16) * LDT + 32 * s2 + 4 * g4];
          const frag ak = S::frag_from_quads(ld_quad<TI>(kr), ld_quad<TI>(kr + 16));
#pragma unroll
          for (int ct = 0; ct < NC; ++ct) S::mma(Sacc[dt][ct], ak, Db[s2][ct]);
        }
      }
    }

    // ---- final state ----
    if (row.out_idx < 0) return;
    if (MODE == 0 || !trans) {
      if (a.h_out == nullptr) return;
      float* base = a.h_out + (static_cast<int64_t>(row.out_idx) * H + hd) * DV * DK;
      const bool vk = (MODE == 1) ? true : (a.out_vk != 0);
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        const int j = col_blk + colw + 16 * ct + c16;
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
        const int jj = col_blk + colw + 16 * ct + c16 - DV;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) base[static_cast<int64_t>(16 * dt + 4 * g4 + r) * DK + jj] = Sacc[dt][ct][r];
      }
    }
  }
};

template <typename TI, int DK, int BV, int NW, int STAGES, int MODE>
__global__ __launch_bounds__(NW * 64) void scan_kernel(const ScanArgs a) {
  using K = ScanKernel<TI, DK, BV, NW, STAGES, MODE>;
  __shared__ __align__(16) typename K::Smem sm;
  K::run(a, sm);
}

template <typename TI, int DK, int BV, int NW, int STAGES, int MODE>
static hipError_t launch_scan(const void* args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((scan_kernel<TI, DK, BV, NW, STAGES, MODE>), dim3(grid), dim3(NW * 64), 0, stream,
                     *static_cast<const ScanArgs*>(args));
  return hipGetLastError();
}

// Built tiles for float32 storage (bfloat16 storage uses scan2.hip):
// (dtype, DK, BV, waves, stages, mode).
#define GDR_SCAN_TILES(X, T, DTYPE, DK, MODE) \
  X(T, DTYPE, DK, 32, 2, 1, MODE)             \
  X(T, DTYPE, DK, 32, 2, 2, MODE)             \
  X(T, DTYPE, DK, 64, 4, 1, MODE)             \
  X(T, DTYPE, DK, 64, 4, 2, MODE)

#define GDR_SCAN_CASE(T, DTYPE, DK, BV, NW, ST, MODE)                                        \
  if (dtype == DTYPE && dk == DK && bv == BV && waves == NW && stages == ST && mode == MODE) \
    return &launch_scan<T, DK, BV, NW, ST, MODE>;

// bfloat16 storage takes the gfx950 kernel of scan2.hip up to DK = 128 and
// this generic kernel (plain and segmented passes) at DK = 256.
LaunchFn find_scan(int dtype, int dk, int bv, int waves, int stages, int mode) {
  if (dtype == 1 && dk <= 128) return find_scan2(dk, bv, waves, stages, mode, false);
  GDR_SCAN_TILES(GDR_SCAN_CASE, bf16_t, 1, 256, 0)
  GDR_SCAN_TILES(GDR_SCAN_CASE, float, 0, 128, 0)
  GDR_SCAN_TILES(GDR_SCAN_CASE, float, 0, 128, 1)
  GDR_SCAN_TILES(GDR_SCAN_CASE, float, 0, 64, 0)
  GDR_SCAN_TILES(GDR_SCAN_CASE, float, 0, 64, 1)
  return nullptr;
}

}  // namespace gdr
