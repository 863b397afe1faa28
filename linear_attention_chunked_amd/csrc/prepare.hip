// Chunk preparation: the WY factors the state scan consumes.
//
// One workgroup (4 waves) per (chunk, head).  With gamma the chunk-local
// inclusive cumulative sum of g, and n valid tokens:
//
//   A[t,i] = beta_t exp(gamma_t - gamma_i) (k_t . k_i)     (i < t)
//   T      = (I + A)^-1                                     FP32, blocked
//   w      = T diag(beta exp(gamma)) K,   u = T diag(beta) V
//
// (the unrolled delta rule inside one chunk: (I + A) Delta = diag(beta) V -
// diag(beta exp(gamma)) K S0, so Delta = u - w S0).
//
// Matrix work: the Gram matrix K K^T and the two products run on MFMA; the
// unit-lower-triangular inverse is done in FP32 on the VALU: four 16x16
// diagonal blocks by forward substitution (one wave each), then the
// off-diagonal blocks block-row by block-row,
//   T[bi][bj] = -T[bi][bi] * sum_{bj <= m < bi} A[bi][m] T[m][bj].
// For bfloat16 storage the FP32 factor T' = T diag(.) is split into
// hi + lo bfloat16 parts, so w and u carry one rounding (the final store).
#include "kernels.hpp"

namespace gdr {

template <typename TI, int DK, int DV>
struct PrepareKernel {
  using S = St<TI>;
  using quad = typename S::quad;
  using frag = typename S::frag;
  static constexpr int NT = 256;
  static constexpr int EPV = 16 / sizeof(TI);
  static constexpr int LDK = DK + EPV;     // row-major K (elements)
  static constexpr int LDT = kChunk + 4;   // transposed tiles (elements)
  static constexpr int LDA = kChunk + 4;   // FP32 64x64 matrices (floats)
  static constexpr int KS = DK / 32;

  struct Smem {
    union {
      TI k[kChunk * LDK];       // row-major K (Gram matrix)
      float t[kChunk * LDA];    // T = (I + A)^-1 (after the Gram matrix)
    } u0;
    float a[kChunk * LDA];      // A
    TI kt[DK * LDT];            // K^T
    TI vt[DV * LDT];            // V^T
    float x[3 * 16 * 17];       // off-diagonal block scratch
    float gam[kChunk];
    float beta[kChunk];
  };
  static_assert(sizeof(TI) * kChunk * LDK <= sizeof(float) * kChunk * LDA + 64 * 1024, "");

  __device__ static void run(const ChunkArgs& a, Smem& sm) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
    const int chunk = blockIdx.x / a.H;
    const int hd = blockIdx.x % a.H;
    if (chunk >= a.n_chunks) return;
    const Row row = row_of_chunk(a.rows, a.n_rows, chunk);
    const int cl = chunk - row.chunk_off;
    const int64_t tok0 = static_cast<int64_t>(row.bos) + static_cast<int64_t>(cl) * kChunk;
    const int nvalid = min(kChunk, row.len - cl * kChunk);
    const int64_t H = a.H;
    const TI* __restrict__ kp = static_cast<const TI*>(a.k);
    const TI* __restrict__ vp = static_cast<const TI*>(a.v);

    // ---- stage K (row-major), V^T, g, beta ----
    for (int v = tid; v < kChunk * DK / EPV; v += NT) {
      const int r = v / (DK / EPV), cv = v % (DK / EPV);
      u32x4_t x{0u, 0u, 0u, 0u};
      if (r < nvalid) x = *reinterpret_cast<const u32x4_t*>(kp + ((tok0 + r) * H + hd) * DK + cv * EPV);
      *reinterpret_cast<u32x4_t*>(&sm.u0.k[r * LDK + cv * EPV]) = x;
    }
    for (int b = tid; b < (kChunk / 4) * (DV / 4); b += NT) {
      const int cq = b % (DV / 4), tq = b / (DV / 4);
      quad in[4], tr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * tq + r;
        in[r] = (t < nvalid) ? ld_quad<TI>(vp + ((tok0 + t) * H + hd) * DV + 4 * cq) : S::zero_quad();
      }
      S::transpose4(in, tr);
#pragma unroll
      for (int j = 0; j < 4; ++j) st_quad<TI>(&sm.vt[(4 * cq + j) * LDT + 4 * tq], tr[j]);
    }
    if (wave == 0) {
      // inclusive prefix sum of g over the chunk (fixed shuffle order)
      float x = (lane < nvalid) ? a.g[(tok0 + lane) * H + hd] : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      sm.gam[lane] = x;
      sm.beta[lane] = (lane < nvalid) ? a.beta[(tok0 + lane) * H + hd] : 0.f;
      if (lane < nvalid) a.g_cum[(tok0 + lane) * H + hd] = x;
    }
    __syncthreads();

    // ---- K^T from the row-major copy (4x4 blocks) ----
    for (int b = tid; b < (kChunk / 4) * (DK / 4); b += NT) {
      const int dq = b % (DK / 4), tq = b / (DK / 4);
      quad in[4], tr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) in[r] = ld_quad<TI>(&sm.u0.k[(4 * tq + r) * LDK + 4 * dq]);
      S::transpose4(in, tr);
#pragma unroll
      for (int j = 0; j < 4; ++j) st_quad<TI>(&sm.kt[(4 * dq + j) * LDT + 4 * tq], tr[j]);
    }

    // ---- Gram matrix, row tile = wave; A = beta_t e^{gamma_t - gamma_i} G (i < t) ----
    {
      f32x4_t acc[4];
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) acc[tj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const TI* ar = &sm.u0.k[(16 * wave + c16) * LDK + 32 * s + 4 * g4];
        const frag fa = S::frag_from_quads(ld_quad<TI>(ar), ld_quad<TI>(ar + 16));
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
          if (tj <= wave) {
            const TI* br = &sm.u0.k[(16 * tj + c16) * LDK + 32 * s + 4 * g4];
            const frag fb = S::frag_from_quads(ld_quad<TI>(br), ld_quad<TI>(br + 16));
            S::mma(acc[tj], fa, fb);
          }
        }
      }
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        const int i = 16 * tj + c16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * wave + 4 * g4 + r;
          float val = 0.f;
          if (i < t) val = sm.beta[t] * expf(sm.gam[t] - sm.gam[i]) * acc[tj][r];
          sm.a[t * LDA + i] = val;
        }
      }
    }
    __syncthreads();  // A complete; the row-major K copy is dead from here on

    // ---- diagonal 16x16 blocks of T by forward substitution (wave = block) ----
    if (lane < 16) {
      const int b0 = 16 * wave, j = lane;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = (r == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) acc -= sm.a[(b0 + r) * LDA + b0 + i] * x[i];
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sm.u0.t[(b0 + r) * LDA + b0 + j] = x[r];
        // blocks right of the diagonal are zero
        for (int bj = wave + 1; bj < 4; ++bj) sm.u0.t[(b0 + r) * LDA + 16 * bj + j] = 0.f;
      }
    }
    __syncthreads();

    // ---- off-diagonal blocks, block row by block row ----
    for (int bi = 1; bi < 4; ++bi) {
      // X[bj] = sum_{m = bj}^{bi-1} A[bi][m] T[m][bj]
      for (int e = tid; e < bi * 256; e += NT) {
        const int bj = e >> 8, r = (e >> 4) & 15, c = e & 15;
        float acc = 0.f;
        for (int m = 16 * bj; m < 16 * bi; ++m)
          acc += sm.a[(16 * bi + r) * LDA + m] * sm.u0.t[m * LDA + 16 * bj + c];
        sm.x[bj * 272 + r * 17 + c] = acc;
      }
      __syncthreads();
      // T[bi][bj] = -T[bi][bi] X[bj]
      for (int e = tid; e < bi * 256; e += NT) {
        const int bj = e >> 8, r = (e >> 4) & 15, c = e & 15;
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) acc += sm.u0.t[(16 * bi + r) * LDA + 16 * bi + m] * sm.x[bj * 272 + m * 17 + c];
        sm.u0.t[(16 * bi + r) * LDA + 16 * bj + c] = -acc;
      }
      __syncthreads();
    }

    // ---- w^T = K^T T'^T and u^T = V^T T''^T; wave = token tile of the output ----
    // B operand (col t = 16 wave + c16, k = i): T[t][i] * beta_i e^{gamma_i} (w) or * beta_i (u).
    const int t = 16 * wave + c16;
    constexpr int NS = 2;  // 64 = 2 k-steps of 32
    frag bw_hi[NS], bw_lo[NS], bu_hi[NS], bu_lo[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int i0 = 32 * s + 4 * g4;
      const f32x4_t t0 = *reinterpret_cast<const f32x4_t*>(&sm.u0.t[t * LDA + i0]);
      const f32x4_t t1 = *reinterpret_cast<const f32x4_t*>(&sm.u0.t[t * LDA + i0 + 16]);
      f32x4_t w0, w1, u0, u1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float b0 = sm.beta[i0 + r], b1 = sm.beta[i0 + 16 + r];
        u0[r] = t0[r] * b0;
        u1[r] = t1[r] * b1;
        w0[r] = u0[r] * expf(sm.gam[i0 + r]);
        w1[r] = u1[r] * expf(sm.gam[i0 + 16 + r]);
      }
      bw_hi[s] = S::frag_from_f32(w0, w1);
      bu_hi[s] = S::frag_from_f32(u0, u1);
      if constexpr (sizeof(TI) == 2) {
        f32x4_t wl0, wl1, ul0, ul1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          wl0[r] = w0[r] - bf16_to_f32(f32_to_bf16(w0[r]));
          wl1[r] = w1[r] - bf16_to_f32(f32_to_bf16(w1[r]));
          ul0[r] = u0[r] - bf16_to_f32(f32_to_bf16(u0[r]));
          ul1[r] = u1[r] - bf16_to_f32(f32_to_bf16(u1[r]));
        }
        bw_lo[s] = S::frag_from_f32(wl0, wl1);
        bu_lo[s] = S::frag_from_f32(ul0, ul1);
      }
    }
    TI* __restrict__ wo = static_cast<TI*>(a.w);
    TI* __restrict__ uo = static_cast<TI*>(a.u);
    const int nsteps = (16 * wave + 15) / 32 + 1;  // T is lower triangular: i <= t
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt) {
      f32x4_t acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s < nsteps) {
          const TI* ar = &sm.kt[(16 * dt + c16) * LDT + 32 * s + 4 * g4];
          const frag fa = S::frag_from_quads(ld_quad<TI>(ar), ld_quad<TI>(ar + 16));
          S::mma(acc, fa, bw_hi[s]);
          if constexpr (sizeof(TI) == 2) S::mma(acc, fa, bw_lo[s]);
        }
      }
      if (t < nvalid) {
        float f[4] = {acc[0], acc[1], acc[2], acc[3]};
        st_quad<TI>(wo + ((tok0 + t) * H + hd) * DK + 16 * dt + 4 * g4, S::f32_to_quad(f));
      }
    }
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) {
      f32x4_t acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s < nsteps) {
          const TI* ar = &sm.vt[(16 * dt + c16) * LDT + 32 * s + 4 * g4];
          const frag fa = S::frag_from_quads(ld_quad<TI>(ar), ld_quad<TI>(ar + 16));
          S::mma(acc, fa, bu_hi[s]);
          if constexpr (sizeof(TI) == 2) S::mma(acc, fa, bu_lo[s]);
        }
      }
      if (t < nvalid) {
        float f[4] = {acc[0], acc[1], acc[2], acc[3]};
        st_quad<TI>(uo + ((tok0 + t) * H + hd) * DV + 16 * dt + 4 * g4, S::f32_to_quad(f));
      }
    }
  }
};

template <typename TI, int DK, int DV>
__global__ __launch_bounds__(256) void prepare_kernel(const ChunkArgs a) {
  using K = PrepareKernel<TI, DK, DV>;
  __shared__ __align__(16) typename K::Smem sm;
  K::run(a, sm);
}

template <typename TI, int DK, int DV>
static hipError_t launch_prepare(const void* args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((prepare_kernel<TI, DK, DV>), dim3(grid), dim3(256), 0, stream,
                     *static_cast<const ChunkArgs*>(args));
  return hipGetLastError();
}

LaunchFn find_prepare(int dtype, int dk, int dv) {
  // bfloat16 storage: the gfx950 kernel of prepare2.hip up to 128 x 128; this
  // generic kernel when DK or DV is 256
  if (dtype == 1 && dk <= 128 && dv <= 128) return find_prepare2(dk, dv);
#define GDR_PREP_CASE(T, DT, DK, DV) \
  if (dtype == DT && dk == DK && dv == DV) return &launch_prepare<T, DK, DV>;
  GDR_PREP_CASE(bf16_t, 1, 256, 256)
  GDR_PREP_CASE(bf16_t, 1, 256, 128)
  GDR_PREP_CASE(bf16_t, 1, 128, 256)
  GDR_PREP_CASE(bf16_t, 1, 128, 128)
  GDR_PREP_CASE(bf16_t, 1, 128, 64)
  GDR_PREP_CASE(bf16_t, 1, 64, 128)
  GDR_PREP_CASE(bf16_t, 1, 64, 64)
  GDR_PREP_CASE(float, 0, 128, 128)
  GDR_PREP_CASE(float, 0, 128, 64)
  GDR_PREP_CASE(float, 0, 64, 128)
  GDR_PREP_CASE(float, 0, 64, 64)
#undef GDR_PREP_CASE
  return nullptr;
}

}  // namespace gdr
