// The WY factors of one 64-token chunk of one head on four waves, shared by
// the chunk-parallel prepare (prepare2.hip) and the state scan with the
// prepare fused in (scan2.hip, PREP):
//
//   gamma  = chunk-local inclusive cumsum of g
//   A[t,i] = beta_t exp(gamma_t - gamma_i) (k_t . k_i)     (i < t)
//   T      = (I + A)^-1                                      FP32
//   w      = T diag(beta exp(gamma)) K,   u = T diag(beta) V
//
// The caller owns the LDS: the K tile (row-major bf16 rows, any padded
// stride; rows 8..15 of every 16 may sit kx bytes further on), the 64 x 64 FP32 scratch of A and T (lower block triangle, kTri
// floats, 16-byte aligned) and three 64-float vectors (gamma, beta,
// beta e^gamma).  The steps are the same instructions in the same order for
// both callers, so w and u come out as the same bits.
//
//   * The Gram matrix runs on bf16 MFMA in FP32.
//   * T by blocks of 16: the four diagonal blocks by forward substitution
//     (one wave each), then every off-diagonal block as FP32 MFMA products:
//       T[1][0] = -T[1][1] (A[1][0] T[0][0]),  T[3][2] likewise,
//       T[2:4][0:2] = -T[2:4][2:4] (A[2:4][0:2] T[0:2][0:2]).
//     In the 16x16x4 FP32 MFMA a product's accumulator (lane (g, c) holds rows
//     4g + r of column c) is directly the B operand of the next product when
//     the contraction index is ordered k = 4g + r, so chained products need
//     no LDS round trip.
//   * w and u from T' = T diag(.) split into bf16 hi + lo parts (one rounding:
//     the final store).
#pragma once

#include "gfx950.hpp"

namespace gdr {

// D (16x16, C layout) += X (16x16) Y (16x16) in FP32 with k = 4g + r:
// a[r] = X[c][4g + r] (row c of X), b[r] = Y[4g + r][c] (the C layout of Y).
__device__ __forceinline__ void wy_mm16(f32x4_t& d, const f32x4_t& a, const f32x4_t& b) {
#pragma unroll
  for (int r = 0; r < 4; ++r) d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], b[r], d, 0, 0, 0);
}

template <int DK>
struct WyCore {
  using S = St<bf16_t>;
  using frag = S::frag;
  static constexpr int KS = DK / 32;
  // A and T (64 x 64, FP32) keep only their blocks on or below the diagonal:
  // row t of block row b = t / 16 holds columns 0 .. 16 b + 15, with a row
  // stride of 16 b + 20 floats (pads keep the column and 16-byte row reads
  // free of bank conflicts).  Every block of T is written over the block of A
  // in the same place once nothing reads that A block any more.
  static constexpr int kTri = 2816;

  // first float of row t in the scratch
  __device__ static __forceinline__ int toff(int t) {
    const int b = t >> 4;
    return 128 * b * (b - 1) + 320 * b + (t & 15) * (16 * b + 20);
  }

  // First wave (lane = token): gamma by an inclusive scan of g (zero past
  // the chunk's nvalid tokens), beta and beta e^gamma into LDS; returns gamma.
  // The scan runs on DPP lane moves (no LDS round trip): shifts by 1, 2, 4, 8
  // within each row of 16 lanes, then the total of row 0 into row 1 and of
  // row 2 into row 3 (broadcast of lane 15 of a row to the next), then the
  // total of rows 0-1 into rows 2-3 (broadcast of lane 31).
  template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
  __device__ static __forceinline__ float dpp_add(float x) {
    const int y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, BOUND_ZERO);
    return x + __builtin_bit_cast(float, y);
  }
  __device__ static __forceinline__ float gamma_beta(float g, float b, int nvalid, float* gam, float* beta,
                                                     float* bg) {
    const int lane = threadIdx.x & 63;
    float x = (lane < nvalid) ? g : 0.f;
    x = dpp_add<0x111, 0xf, true>(x);   // row_shr:1
    x = dpp_add<0x112, 0xf, true>(x);   // row_shr:2
    x = dpp_add<0x114, 0xf, true>(x);   // row_shr:4
    x = dpp_add<0x118, 0xf, true>(x);   // row_shr:8
    x = dpp_add<0x142, 0xa, false>(x);  // row_bcast:15 into rows 1 and 3
    x = dpp_add<0x143, 0xc, false>(x);  // row_bcast:31 into rows 2 and 3
    const float bb = (lane < nvalid) ? b : 0.f;
    gam[lane] = x;
    beta[lane] = bb;
    bg[lane] = bb * exp_fast(x);
    return x;
  }

  // Gram matrix row tile WV (the calling wave); A = beta_t e^{gamma_t -
  // gamma_i} G (i < t) for its blocks on or below the diagonal.  The block
  // count is a compile-time constant per wave, so every LDS read of the tile
  // is issued ahead of the products (no branch between them).
  template <int WV>
  __device__ static __forceinline__ void gram_rows(const char* kt, int skb, int kx, float* t, const float* gam,
                                                   const float* beta) {
    const int lane = threadIdx.x & 63, g4 = lane >> 4, c16 = lane & 15;
    f32x4_t acc[WV + 1];
#pragma unroll
    for (int tj = 0; tj <= WV; ++tj) acc[tj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // both operands are K rows: the contiguous k map, 16 bytes per lane (skb a multiple of 16)
    const char* kr = kt + c16 * skb + kx * (c16 >> 3) + 16 * g4;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const frag fa = lds_frag16(kr, 16 * WV * skb + 64 * s);
#pragma unroll
      for (int tj = 0; tj <= WV; ++tj) S::mma(acc[tj], fa, lds_frag16(kr, 16 * tj * skb + 64 * s));
    }
    // Every LDS read is issued before any exponent: the (i < t) mask is a
    // select on values already in registers, not a branch around each read.
    // e^{gamma_t - gamma_i} may overflow where i > t; the select drops it.
    // Blocks above the diagonal are not stored.
    const int t0 = 16 * WV + 4 * g4;
    const f32x4_t gt = *reinterpret_cast<const f32x4_t*>(&gam[t0]);
    const f32x4_t bt = *reinterpret_cast<const f32x4_t*>(&beta[t0]);
    float gi[WV + 1];
#pragma unroll
    for (int tj = 0; tj <= WV; ++tj) gi[tj] = gam[16 * tj + c16];
#pragma unroll
    for (int tj = 0; tj <= WV; ++tj) {
      const int i = 16 * tj + c16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = t0 + r;
        const float full = bt[r] * exp_fast(gt[r] - gi[tj]) * acc[tj][r];
        const float val = (i < tt) ? full : 0.f;
        t[toff(tt) + i] = val;
      }
    }
  }

  // Gram matrix row tile `wave` (gram_rows), then the wave's diagonal block
  // T[b][b] = (I + A[b][b])^-1 (both in the wave's own rows of t: no
  // barrier).  K: row-major tile of stride skb (row shift kx).
  __device__ static __forceinline__ void gram_diag(const char* kt, int skb, int kx, float* t, const float* gam,
                                                   const float* beta) {
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    switch (wave) {
      case 0: gram_rows<0>(kt, skb, kx, t, gam, beta); break;
      case 1: gram_rows<1>(kt, skb, kx, t, gam, beta); break;
      case 2: gram_rows<2>(kt, skb, kx, t, gam, beta); break;
      default: gram_rows<3>(kt, skb, kx, t, gam, beta); break;
    }
    diag_solve(t);
  }

  // The calling wave's diagonal block T[b][b] = (I + A[b][b])^-1, b = wave,
  // from its own rows of A (written by gram_rows of the same wave).
  __device__ static __forceinline__ void diag_solve(float* t) {
    const int lane = threadIdx.x & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    // ---- diagonal blocks: T[b][b] = (I + A[b][b])^-1 by forward substitution, wave b ----
    // Lane (j, g) solves rows 4 g .. 4 g + 3 of column j, by blocks of four
    // rows: the lanes owning block q finish its rows, a shuffle hands the four
    // values to every lane of the same column, and the lanes of later blocks
    // subtract their terms.  Row r still subtracts its terms in the order
    // i = 0, 1, ...  The entries of A are 16-byte LDS reads of the wave's own
    // rows, off the dependent chain.  T[b][b] is written over A[b][b].
    {
      const int b0 = 16 * wave, j = c16, g = g4;
      float xr[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) xr[rr] = (4 * g + rr == j) ? 1.f : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4_t R[4];  // R[rr][ii] = A[b][b][4 g + rr][4 q + ii]
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          R[rr] = *reinterpret_cast<const f32x4_t*>(&t[toff(b0 + 4 * g + rr) + b0 + 4 * q]);
        if (g == q) {
#pragma unroll
          for (int rr = 1; rr < 4; ++rr)
#pragma unroll
            for (int ii = 0; ii < rr; ++ii) xr[rr] -= R[rr][ii] * xr[ii];
        }
        if (q < 3) {
          float xq[4];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) xq[ii] = __shfl(xr[ii], j + 16 * q, 64);
          if (g > q) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
#pragma unroll
              for (int ii = 0; ii < 4; ++ii) xr[rr] -= R[rr][ii] * xq[ii];
          }
        }
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) t[toff(b0 + 4 * g + rr) + b0 + j] = xr[rr];
    }
  }

  // The off-diagonal blocks of T, after a barrier that follows gram_diag.
  // Ends with a barrier: every block of T is in place.
  __device__ static __forceinline__ void off_diag(float* t) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // FP32 operand reads for wy_mm16: row-major rows (a) and C-layout columns (b)
    auto a_rows = [&](const float* m, int r0, int c0) {  // X[c16][4 g4 + r] of the block at (r0, c0)
      return *reinterpret_cast<const f32x4_t*>(m + toff(r0 + c16) + c0 + 4 * g4);
    };
    auto b_cols = [&](const float* m, int r0, int c0) {  // Y[4 g4 + r][c16]
      f32x4_t y;
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = m[toff(r0 + 4 * g4 + r) + c0 + c16];
      return y;
    };
    auto store_c = [&](float* m, int r0, int c0, const f32x4_t& d) {
#pragma unroll
      for (int r = 0; r < 4; ++r) m[toff(r0 + 4 * g4 + r) + c0 + c16] = d[r];
    };

    // ---- T[1][0] (wave 0) and T[3][2] (wave 1) ----
    if (wave < 2) {
      const int p = 32 * wave;  // block (p+16, p)
      f32x4_t y{0.f, 0.f, 0.f, 0.f}, x{0.f, 0.f, 0.f, 0.f};
      wy_mm16(y, a_rows(t, p + 16, p), b_cols(t, p, p));      // A[1][0] T[0][0]
      wy_mm16(x, a_rows(t, p + 16, p + 16), y);               // T[1][1] (.)
      store_c(t, p + 16, p, -x);
    }
    __syncthreads();

    // ---- T[2+i][j] = -(T_hi[i][0] Y[0][j] + T_hi[i][1] Y[1][j]),  Y = A[2:4][0:2] T[0:2][j] ----
    {
      const int i = wave >> 1, j = wave & 1;
      f32x4_t y0{0.f, 0.f, 0.f, 0.f}, y1{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (k >= j) {  // T[0][1] is zero
          const f32x4_t tb = b_cols(t, 16 * k, 16 * j);
          wy_mm16(y0, a_rows(t, 32, 16 * k), tb);
          wy_mm16(y1, a_rows(t, 48, 16 * k), tb);
        }
      }
      __syncthreads();  // every wave has read A[2:4][0:2] before any T block replaces it
      f32x4_t x{0.f, 0.f, 0.f, 0.f};
      wy_mm16(x, a_rows(t, 32 + 16 * i, 32), y0);                   // T_hi[i][0] (T[2][2] or T[3][2])
      if (i == 1) wy_mm16(x, a_rows(t, 48, 48), y1);                // T_hi[1][1] = T[3][3]
      store_c(t, 32 + 16 * i, 16 * j, -x);
    }
    __syncthreads();
  }

  // This lane's operand fragments of row 16 wave + c16 of T diag(coef), split
  // into bf16 hi + lo; column blocks past the diagonal (not stored) are zero.
  __device__ static __forceinline__ void row_frags(const float* t, const float* coef, frag (&hi)[2], frag (&lo)[2]) {
    row_frags_of(__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)), t, coef, hi, lo);
  }

  // The same for row 16 rb + c16 (rb: a 16-row block, uniform over the wave).
  // No multiply-add contraction here: lo = x - bf16(x) of the rounded product
  // x = T coef, whichever wave and kernel form it (the compiler would fuse
  // the product into the subtraction in some inlined copies and not in
  // others, and w / u would differ in their last bits between callers).
  __device__ static __forceinline__ void row_frags_of(int rb, const float* t, const float* coef, frag (&hi)[2],
                                                      frag (&lo)[2]) {
#pragma clang fp contract(off)
    const int wave = rb;
    const int lane = threadIdx.x & 63, g4 = lane >> 4, c16 = lane & 15;
    const int tt = 16 * wave + c16;
    const int nsteps = (16 * wave + 15) / 32 + 1;  // T is lower triangular
    const float* tr = &t[toff(tt)];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s >= nsteps) continue;
      const int i0 = 32 * s + 4 * g4;
      const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(&tr[i0]) * *reinterpret_cast<const f32x4_t*>(&coef[i0]);
      const f32x4_t x1 = (2 * s + 1 <= wave)
                             ? *reinterpret_cast<const f32x4_t*>(&tr[i0 + 16]) *
                                   *reinterpret_cast<const f32x4_t*>(&coef[i0 + 16])
                             : f32x4_t{0.f, 0.f, 0.f, 0.f};
      hi[s] = S::frag_from_f32(x0, x1);
      f32x4_t l0, l1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        l0[r] = x0[r] - bf16_to_f32(f32_to_bf16(x0[r]));
        l1[r] = x1[r] - bf16_to_f32(f32_to_bf16(x1[r]));
      }
      lo[s] = S::frag_from_f32(l0, l1);
    }
  }

  // Rows 16 wave .. 16 wave + 15 of (T diag(coef)) X for a row-major bf16 tile
  // X (64 rows, stride `stride`, rows 8..15 of every 16 kx bytes further on,
  // D columns): for every 16-column tile dt,
  // out(dt, acc) with acc[r] = result[16 wave + c16][16 dt + 4 g4 + r] in FP32.
  // A operand X^T[d][i] by transpose reads of the row-major tile.  NS = the
  // 32-token steps below the diagonal (1 for the first two waves, 2 for the
  // others), a compile-time constant, so the reads of later tiles can be
  // issued ahead of the products of earlier ones.
  template <int NS, int D, class Out>
  __device__ static __forceinline__ void product_ns(const char* tile, int stride, int kx, const frag (&hi)[2],
                                                    const frag (&lo)[2], Out& out) {
    product_tiles<NS, 0, D / 16>(tile, stride, kx, hi, lo, out);
  }

  // The same for the 16-column tiles T0 <= dt < T1 only (rows: those of the
  // fragments).  Every output element is the same products in the same order
  // whichever wave forms it.
  template <int NS, int T0, int T1, class Out>
  __device__ static __forceinline__ void product_tiles(const char* tile, int stride, int kx, const frag (&hi)[2],
                                                       const frag (&lo)[2], Out& out) {
    const int lane = threadIdx.x & 63, g4 = lane >> 4, c16 = lane & 15;
    const int tr_row = 4 * g4 + (c16 >> 2);
    const int tr_col = 8 * (c16 & 3) + kx * (g4 >> 1);  // (row tr_row has bit 3 = g4 >> 1)
#pragma unroll
    for (int dt = T0; dt < T1; ++dt) {
      f32x4_t acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const char* base = tile + (32 * s + tr_row) * stride + 32 * dt + tr_col;
        const frag fa = S::frag_from_quads(lds_tr16(base, 0), lds_tr16(base, 16 * stride));
        S::mma(acc, fa, hi[s]);
        S::mma(acc, fa, lo[s]);
      }
      out(dt, acc);
    }
  }

  template <int D, class Out>
  __device__ static __forceinline__ void product(const char* tile, int stride, int kx, const frag (&hi)[2],
                                                 const frag (&lo)[2], Out out) {
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    if (wave >= 2)
      product_ns<2, D>(tile, stride, kx, hi, lo, out);
    else
      product_ns<1, D>(tile, stride, kx, hi, lo, out);
  }
};

}  // namespace gdr
