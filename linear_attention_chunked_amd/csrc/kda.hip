// Per-key-channel decay (the FlashKDA-style gate of cuLA pull request #127,
// "Summary"): chunk preparation and chunk output on gfx950, bfloat16
// storage.  The state scan is scan2.hip with its per-channel decay switch.
//
// Per chunk with Gam = the chunk-local cumulative sum of the per-channel log
// decays (Gam_t in R^DK), derived from the token recurrence
// S_t = (I - b_t k_t k_t^T) diag(e^{g_t}) S_{t-1} + b_t k_t v_t^T:
//
//   A[t,i] = b_t sum_d k_td k_id e^{Gam_td - Gam_id}     (i < t)
//   T = (I + A)^-1;  w = T diag(b) (K * e^{Gam});  u = T diag(b) V
//   kg = K * e^{Gam_last - Gam};  decay = e^{Gam_last}
//   (scan)   v_new = u - w S;  S <- diag(decay) S + kg^T v_new
//   (output) o_t = scale ((q_t * e^{Gam_t})^T S + sum_{i<=t} P[t,i] v_new_i),
//            P[t,i] = sum_d q_td k_id e^{Gam_td - Gam_id}
//
// The products with a per-pair, per-channel decay are formed per 16-token
// block of rows I against the columns of every block J <= I, each factor
// referenced at the block's first token r = 16 I:
//   x_td e^{Gam_td - Gam_rd}  (t >= r: at most 1)  times  y_id e^{Gam_rd - Gam_id},
// which is at most 1 for i < r; for i >= r (the diagonal block) it is at most
// e^{-(Gam over 15 tokens)}, finite while every channel's log decay stays
// above -5 per token (the documented input range).  The products run on
// FP32 MFMA (v_mfma_f32_16x16x4_f32): lane (c, g) supplies, for step
// j = 4 q + m, the channel d = 16 q + 4 g + m of row c, so each lane reads
// four consecutive channels at a time.
#include "gfx950.hpp"
#include "kernels.hpp"

namespace gdr {

namespace {

__device__ __forceinline__ void mm16f(f32x4_t& d, const f32x4_t& a, const f32x4_t& b) {
#pragma unroll
  for (int r = 0; r < 4; ++r) d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], b[r], d, 0, 0, 0);
}

// bf16 hi + lo split of an FP32 value (hi = RNE bf16, lo = bf16 of the rest)
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

}  // namespace

// Shared by prepare and output: the decayed products of one 16-row block.
//   xs[j]: this lane's A-side values (row 16 I + c, channel d(j)), already
//          multiplied by e^{Gam_td - Gam_rd};
//   ys: bf16 rows (stride SY bytes), gam: FP32 Gam rows (stride GS floats).
// Returns D[4 g + r][c] = sum_d xs_td ys_id e^{Gam_rd - Gam_id} for i = 16 J + c.
template <int DK, int SY, int GS>
__device__ __forceinline__ f32x4_t kda_block_product(const float (&xs)[DK / 4], const char* ys, const float* gam,
                                                     int I, int J, int g4, int c16) {
  const float* gr = gam + (16 * I) * GS;            // reference row r = 16 I (broadcast)
  const float* gi = gam + (16 * J + c16) * GS;      // this lane's column row i
  const char* yi = ys + (16 * J + c16) * SY;
  f32x4_t d{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < DK / 16; ++q) {
    const int d0 = 16 * q + 4 * g4;
    const f32x4_t grv = *reinterpret_cast<const f32x4_t*>(gr + d0);
    const f32x4_t giv = *reinterpret_cast<const f32x4_t*>(gi + d0);
    const u32x2_t yq = *reinterpret_cast<const u32x2_t*>(yi + 2 * d0);
    f32x4_t yb, xa;
    yb[0] = __builtin_bit_cast(float, yq.x << 16) * exp_fast(grv[0] - giv[0]);
    yb[1] = __builtin_bit_cast(float, yq.x & 0xffff0000u) * exp_fast(grv[1] - giv[1]);
    yb[2] = __builtin_bit_cast(float, yq.y << 16) * exp_fast(grv[2] - giv[2]);
    yb[3] = __builtin_bit_cast(float, yq.y & 0xffff0000u) * exp_fast(grv[3] - giv[3]);
#pragma unroll
    for (int m = 0; m < 4; ++m) xa[m] = xs[4 * q + m];
    mm16f(d, xa, yb);
  }
  return d;
}

// This lane's A-side values of row t = 16 I + c16: x_td e^{Gam_td - Gam_rd}.
template <int DK, int SX, int GS>
__device__ __forceinline__ void kda_row_side(float (&xs)[DK / 4], const char* xrows, const float* gam, int I, int g4,
                                             int c16) {
  const float* gr = gam + (16 * I) * GS;
  const float* gt = gam + (16 * I + c16) * GS;
  const char* xt = xrows + (16 * I + c16) * SX;
#pragma unroll
  for (int q = 0; q < DK / 16; ++q) {
    const int d0 = 16 * q + 4 * g4;
    const f32x4_t grv = *reinterpret_cast<const f32x4_t*>(gr + d0);
    const f32x4_t gtv = *reinterpret_cast<const f32x4_t*>(gt + d0);
    const u32x2_t xq = *reinterpret_cast<const u32x2_t*>(xt + 2 * d0);
    xs[4 * q + 0] = __builtin_bit_cast(float, xq.x << 16) * exp_fast(gtv[0] - grv[0]);
    xs[4 * q + 1] = __builtin_bit_cast(float, xq.x & 0xffff0000u) * exp_fast(gtv[1] - grv[1]);
    xs[4 * q + 2] = __builtin_bit_cast(float, xq.y << 16) * exp_fast(gtv[2] - grv[2]);
    xs[4 * q + 3] = __builtin_bit_cast(float, xq.y & 0xffff0000u) * exp_fast(gtv[3] - grv[3]);
  }
}

// ------------------------------------------------------------------ prepare
template <int DK, int DV>
struct KdaPrepare {
  using S = St<bf16_t>;
  using frag = S::frag;
  static constexpr int NT = 512;            // 8 waves
  static constexpr int SKB = DK * 2 + 16;   // bf16 rows (bytes)
  static constexpr int SVB = DV * 2 + 16;
  static constexpr int GS = DK + 4;         // FP32 Gam rows (floats), padded
  static constexpr int kTri = 2816;         // floats of the lower block triangle of A / T

  // Regions reused once their first contents are dead, so that two 8-wave
  // workgroups share a CU (about 66 KB at 128 x 128): K then V (V waits in
  // registers until the decayed products no longer read K); Gam then the
  // bf16 hi / lo parts of K e^{Gam}; A then T.  A and T keep only their
  // blocks on or below the diagonal: row t of block row b = t / 16 holds
  // columns 0 .. 16 b + 15 with a row stride of 16 b + 20 floats.
  static constexpr int RKV = (SKB > SVB ? SKB : SVB) * kChunk;
  static constexpr int RG = (GS * 4 > 2 * SKB ? GS * 4 : 2 * SKB) * kChunk;
  struct Smem {
    union {
      char k[RKV];
      char v[RKV];
    };
    union {
      float gam[RG / 4];
      char ke[RG];              // ke_hi rows [0, 64), ke_lo rows [64, 128), stride SKB
    };
    float t[kTri];              // A, then T
    float beta[kChunk];
    float part[3][DK];          // per-channel sums of the first three 16-token quarters
  };
  // first float of row t in Smem::t
  __device__ static __forceinline__ int toff(int t) {
    const int b = t >> 4;
    return 128 * b * (b - 1) + 320 * b + (t & 15) * (16 * b + 20);
  }

  __device__ static void run(const KdaArgs& a, Smem& sm) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int item = blockIdx.x;
    const int chunk = item / a.H;
    const int hd = item % a.H;
    if (chunk >= a.n_chunks) return;
    const Row row = row_of_chunk(a.rows, a.n_rows, chunk);
    const int cl = chunk - row.chunk_off;
    const int64_t tok0 = static_cast<int64_t>(row.bos) + static_cast<int64_t>(cl) * kChunk;
    const int nvalid = min(kChunk, row.len - cl * kChunk);
    const int64_t H = a.H;

    // ---- K (bf16), g (FP32), beta into LDS, V into registers; rows past the tail read as zero ----
    constexpr int VPT = kChunk * (DV / 8) / NT;
    u32x4_t vreg[VPT];
    {
      const uint16_t* kp = static_cast<const uint16_t*>(a.k) + (tok0 * H + hd) * DK;
      const uint16_t* vp = static_cast<const uint16_t*>(a.v) + (tok0 * H + hd) * DV;
      const float* gp = a.g + (tok0 * H + hd) * DK;
      const rsrc_t rk = make_rsrc(kp, static_cast<uint32_t>(((nvalid - 1) * H + 1) * DK * 2));
      const rsrc_t rv = make_rsrc(vp, static_cast<uint32_t>(((nvalid - 1) * H + 1) * DV * 2));
      const rsrc_t rg = make_rsrc(gp, static_cast<uint32_t>(((nvalid - 1) * H + 1) * DK * 4));
      constexpr int CK = DK / 8, CV = DV / 8, CG = DK / 4;
#pragma unroll
      for (int i = 0; i < kChunk * CK / NT; ++i) {
        const int vv = tid + i * NT, r = vv / CK, c = vv % CK;
        *reinterpret_cast<u32x4_t*>(sm.k + r * SKB + c * 16) =
            __builtin_amdgcn_raw_buffer_load_b128(rk, static_cast<int>(r * H * DK * 2 + c * 16), 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kChunk * CV / NT; ++i) {
        const int vv = tid + i * NT, r = vv / CV, c = vv % CV;
        vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, static_cast<int>(r * H * DV * 2 + c * 16), 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kChunk * CG / NT; ++i) {
        const int vv = tid + i * NT, r = vv / CG, c = vv % CG;
        *reinterpret_cast<u32x4_t*>(sm.gam + r * GS + c * 4) =
            __builtin_amdgcn_raw_buffer_load_b128(rg, static_cast<int>(r * H * DK * 4 + c * 16), 0, 0);
      }
      if (tid < kChunk) {
        const float* bp = a.beta + tok0 * H + hd;
        const float b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
            make_rsrc(bp, static_cast<uint32_t>(((nvalid - 1) * H + 1) * 4)), static_cast<int>(tid * H * 4), 0, 0));
        sm.beta[tid] = b;
      }
    }
    __syncthreads();

    // ---- Gam: inclusive cumulative sum over the chunk's tokens, per channel
    //      (rows past the tail add zero, so they repeat the last value):
    //      thread (quarter, channel) sums its 16 tokens, then adds the sums of
    //      the quarters before it ----
    {
      constexpr int QL = kChunk / 4;
      const int gd = tid % DK, gq = tid / DK;
      float gv[QL];
      if (gq < 4) {
#pragma unroll
        for (int t = 0; t < QL; ++t) gv[t] = sm.gam[(QL * gq + t) * GS + gd];
        float x = 0.f;
#pragma unroll
        for (int t = 0; t < QL; ++t) {
          x += gv[t];
          gv[t] = x;
        }
        if (gq < 3) sm.part[gq][gd] = x;
      }
      __syncthreads();
      if (gq < 4) {
        float off = 0.f;
#pragma unroll
        for (int p = 0; p < 3; ++p)
          if (p < gq) off += sm.part[p][gd];
        float* go = a.g_cum + (tok0 * H + hd) * DK;
        const rsrc_t rgo = make_rsrc(go, static_cast<uint32_t>(((nvalid - 1) * H + 1) * DK * 4));
#pragma unroll
        for (int t = 0; t < QL; ++t) {
          const float x = off + gv[t];
          const int row = QL * gq + t;
          sm.gam[row * GS + gd] = x;
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), rgo,
                                                static_cast<int>((row * H * DK + gd) * 4), 0, 0);
        }
        if (gq == 3) a.decay[((static_cast<int64_t>(a.chunk_base) + chunk) * H + hd) * DK + gd] = exp_fast(off + gv[QL - 1]);
      }
    }
    __syncthreads();

    // ---- A rows of block I = wave % 4: b_t sum_d k_td k_id e^{Gam_td - Gam_id}, i < t;
    //      the column blocks J <= I are split between waves I and I + 4 ----
    {
      const int I = wave & 3, nj = I + 1;
      const int j0 = (wave >> 2) ? (nj + 1) / 2 : 0, j1 = (wave >> 2) ? nj : (nj + 1) / 2;
      if (j0 < j1) {
        float xs[DK / 4];
        kda_row_side<DK, SKB, GS>(xs, sm.k, sm.gam, I, g4, c16);
        const int t0 = 16 * I + 4 * g4;
        const f32x4_t bt = *reinterpret_cast<const f32x4_t*>(&sm.beta[t0]);
        for (int J = j0; J < j1; ++J) {
          const f32x4_t d = kda_block_product<DK, SKB, GS>(xs, sm.k, sm.gam, I, J, g4, c16);
          const int i = 16 * J + c16;
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.t[toff(t0 + r) + i] = (i < t0 + r) ? bt[r] * d[r] : 0.f;
        }
      }
    }
    __syncthreads();

    // ---- K * e^{Gam} (hi / lo parts, registers) and kg = K * e^{Gam_last - Gam} (global) ----
    constexpr int KPT = kChunk * (DK / 8) / NT;
    u32x4_t khi[KPT], klo[KPT];
    {
      uint16_t* kgp = static_cast<uint16_t*>(a.kg) + (tok0 * H + hd) * DK;
      const rsrc_t rkg = make_rsrc(kgp, static_cast<uint32_t>(((nvalid - 1) * H + 1) * DK * 2));
      constexpr int CK = DK / 8;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int vv = tid + i * NT, r = vv / CK, c = vv % CK;
        const u32x4_t kq = *reinterpret_cast<const u32x4_t*>(sm.k + r * SKB + c * 16);
        const float* gt = sm.gam + r * GS + 8 * c;
        const float* gl = sm.gam + (kChunk - 1) * GS + 8 * c;
        uint32_t hw[4], lw[4], gw[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t wd = kq[p];
          const float k0 = __builtin_bit_cast(float, wd << 16), k1 = __builtin_bit_cast(float, wd & 0xffff0000u);
          uint16_t h0, l0, h1, l1;
          split_bf16(k0 * exp_fast(gt[2 * p]), h0, l0);
          split_bf16(k1 * exp_fast(gt[2 * p + 1]), h1, l1);
          hw[p] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
          lw[p] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
          gw[p] = pack_bf16x2(k0 * exp_fast(gl[2 * p] - gt[2 * p]), k1 * exp_fast(gl[2 * p + 1] - gt[2 * p + 1]));
        }
        khi[i] = u32x4_t{hw[0], hw[1], hw[2], hw[3]};
        klo[i] = u32x4_t{lw[0], lw[1], lw[2], lw[3]};
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{gw[0], gw[1], gw[2], gw[3]}, rkg,
                                               static_cast<int>(r * H * DK * 2 + c * 16), 0, 0);
      }
    }
    __syncthreads();  // K and Gam are dead: V over K, the parts of K e^{Gam} over Gam
    {
      constexpr int CK = DK / 8, CV = DV / 8;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int vv = tid + i * NT, r = vv / CK, c = vv % CK;
        *reinterpret_cast<u32x4_t*>(sm.ke + r * SKB + c * 16) = khi[i];
        *reinterpret_cast<u32x4_t*>(sm.ke + (kChunk + r) * SKB + c * 16) = klo[i];
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int vv = tid + i * NT, r = vv / CV, c = vv % CV;
        *reinterpret_cast<u32x4_t*>(sm.v + r * SVB + c * 16) = vreg[i];
      }
    }

    // ---- T = (I + A)^-1 by 16-blocks: diagonal blocks by forward substitution
    //      (wave b < 4; lane (j, g) solves rows 4 g .. 4 g + 3 of column j by
    //      blocks of four rows, each finished block handed to the later lanes
    //      of its column by ds_bpermute, so row r still subtracts its terms in
    //      the order i = 0, 1, ...), off-diagonal blocks as FP32 products
    //      (A and T share one matrix) ----
    if (wave < 4) {
      const int b0 = 16 * wave, j = c16, g = g4;
      float xr[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) xr[rr] = (4 * g + rr == j) ? 1.f : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4_t R[4];  // R[rr][ii] = A[b][b][4 g + rr][4 q + ii]
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          R[rr] = *reinterpret_cast<const f32x4_t*>(&sm.t[toff(b0 + 4 * g + rr) + b0 + 4 * q]);
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
      for (int rr = 0; rr < 4; ++rr) sm.t[toff(b0 + 4 * g + rr) + b0 + j] = xr[rr];
    }
    __syncthreads();
    auto a_rows = [&](const float* m, int r0, int c0) {
      return *reinterpret_cast<const f32x4_t*>(m + toff(r0 + c16) + c0 + 4 * g4);
    };
    auto b_cols = [&](const float* m, int r0, int c0) {
      f32x4_t y;
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = m[toff(r0 + 4 * g4 + r) + c0 + c16];
      return y;
    };
    auto store_c = [&](float* m, int r0, int c0, const f32x4_t& d) {
#pragma unroll
      for (int r = 0; r < 4; ++r) m[toff(r0 + 4 * g4 + r) + c0 + c16] = d[r];
    };
    if (wave < 2) {
      const int p = 32 * wave;
      f32x4_t y{0.f, 0.f, 0.f, 0.f}, x{0.f, 0.f, 0.f, 0.f};
      mm16f(y, a_rows(sm.t, p + 16, p), b_cols(sm.t, p, p));
      mm16f(x, a_rows(sm.t, p + 16, p + 16), y);
      store_c(sm.t, p + 16, p, -x);
    }
    __syncthreads();
    {
      const int i = (wave >> 1) & 1, j = wave & 1;  // waves 0 .. 3
      f32x4_t y0{0.f, 0.f, 0.f, 0.f}, y1{0.f, 0.f, 0.f, 0.f};
      if (wave < 4) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          if (k >= j) {
            const f32x4_t tb = b_cols(sm.t, 16 * k, 16 * j);
            mm16f(y0, a_rows(sm.t, 32, 16 * k), tb);
            mm16f(y1, a_rows(sm.t, 48, 16 * k), tb);
          }
        }
      }
      __syncthreads();  // every wave has read A[2:4][0:2] before any T block replaces it
      if (wave < 4) {
        f32x4_t x{0.f, 0.f, 0.f, 0.f};
        mm16f(x, a_rows(sm.t, 32 + 16 * i, 32), y0);
        if (i == 1) mm16f(x, a_rows(sm.t, 48, 48), y1);
        store_c(sm.t, 32 + 16 * i, 16 * j, -x);
      }
    }
    __syncthreads();

    // ---- w^T = (K e^Gam)^T (T diag(b))^T, u^T = V^T (T diag(b))^T; wave = (token tile,
    //      half of the columns) ----
    const int tt = wave & 3, half = wave >> 2;
    const int t = 16 * tt + c16;
    const int nsteps = (16 * tt + 15) / 32 + 1;  // T is lower triangular
    frag bb_hi[2], bb_lo[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s >= nsteps) continue;
      const int i0 = 32 * s + 4 * g4;
      const float* tr = &sm.t[toff(t)];
      const f32x4_t t0 = *reinterpret_cast<const f32x4_t*>(&tr[i0]);
      const f32x4_t t1 = (2 * s + 1 <= tt) ? *reinterpret_cast<const f32x4_t*>(&tr[i0 + 16])
                                           : f32x4_t{0.f, 0.f, 0.f, 0.f};  // blocks past the diagonal
      const f32x4_t be0 = *reinterpret_cast<const f32x4_t*>(&sm.beta[i0]);
      const f32x4_t be1 = *reinterpret_cast<const f32x4_t*>(&sm.beta[i0 + 16]);
      const f32x4_t u0 = t0 * be0, u1 = t1 * be1;
      bb_hi[s] = S::frag_from_f32(u0, u1);
      f32x4_t l0, l1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        l0[r] = u0[r] - bf16_to_f32(f32_to_bf16(u0[r]));
        l1[r] = u1[r] - bf16_to_f32(f32_to_bf16(u1[r]));
      }
      bb_lo[s] = S::frag_from_f32(l0, l1);
    }
    const int tr_row = 4 * g4 + (c16 >> 2);
    const int tr_col = 8 * (c16 & 3);
    uint16_t* wo = static_cast<uint16_t*>(a.w) + (tok0 * H + hd) * DK;
    uint16_t* uo = static_cast<uint16_t*>(a.u) + (tok0 * H + hd) * DV;
    const rsrc_t rwo = make_rsrc(wo, static_cast<uint32_t>(((nvalid - 1) * H + 1) * DK * 2));
    const rsrc_t ruo = make_rsrc(uo, static_cast<uint32_t>(((nvalid - 1) * H + 1) * DV * 2));
#pragma unroll
    for (int e = 0; e < DK / 32; ++e) {
      const int dt = half * (DK / 32) + e;
      f32x4_t acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (s < nsteps) {
          const int off = (32 * s + tr_row) * SKB + 32 * dt + tr_col;
          const frag fh = S::frag_from_quads(lds_tr16(sm.ke, off), lds_tr16(sm.ke, off + 16 * SKB));
          const frag fl = S::frag_from_quads(lds_tr16(sm.ke, kChunk * SKB + off), lds_tr16(sm.ke, (kChunk + 16) * SKB + off));
          S::mma(acc, fh, bb_hi[s]);
          S::mma(acc, fh, bb_lo[s]);
          S::mma(acc, fl, bb_hi[s]);
        }
      }
      __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])}, rwo,
                                            static_cast<int>(t * H * DK * 2 + (16 * dt + 4 * g4) * 2), 0, 0);
    }
#pragma unroll
    for (int e = 0; e < DV / 32; ++e) {
      const int dt = half * (DV / 32) + e;
      f32x4_t acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (s < nsteps) {
          const int off = (32 * s + tr_row) * SVB + 32 * dt + tr_col;
          const frag fa = S::frag_from_quads(lds_tr16(sm.v, off), lds_tr16(sm.v, off + 16 * SVB));
          S::mma(acc, fa, bb_hi[s]);
          S::mma(acc, fa, bb_lo[s]);
        }
      }
      __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])}, ruo,
                                            static_cast<int>(t * H * DV * 2 + (16 * dt + 4 * g4) * 2), 0, 0);
    }
  }
};

// ------------------------------------------------------------------ output
// One workgroup (4 waves) per (chunk, head) over all value columns (P is
// formed once per chunk); wave I owns the rows of token block I.  Two phases
// share one LDS region so that two workgroups fit on a CU: first Q, K and Gam
// give each wave its rows of P and its A operand Q e^{Gam} (bf16 hi and lo
// parts), both kept in registers; then the pre-chunk state and v_new (read
// into registers at the start) and P take the region for the two products.
template <int DK, int DV>
struct KdaOutput {
  using S = St<bf16_t>;
  using frag = S::frag;
  static constexpr int NT = 256;
  static constexpr int NCT = DV / 16;
  static constexpr int SQ = DK * 2 + 16;
  static constexpr int SV = DV * 2 + 32;
  static constexpr int GS = DK + 4;
  static constexpr int LP = 64 + 4;
  static constexpr int KS = DK / 32;

  struct PhaseA {
    char q[kChunk * SQ];
    char k[kChunk * SQ];
    float gam[kChunk * GS];
  };
  struct PhaseB {
    char h[DV * SQ];
    char v[kChunk * SV];
    float p[kChunk * LP];
  };
  union Smem {
    PhaseA A;
    PhaseB B;
  };

  static constexpr int CQ = DK / 8, CV = DV / 8, CG = DK / 4;
  static constexpr int HPT = DV * CQ / NT, VPT = kChunk * CV / NT;

  __device__ static void run(const KdaArgs& a, Smem& sm) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int item = blockIdx.x;
    const int chunk = item / a.H;
    const int hd = item % a.H;
    if (chunk >= a.n_chunks) return;
    const Row row = row_of_chunk(a.rows, a.n_rows, chunk);
    const int cl = chunk - row.chunk_off;
    const int64_t tok0 = static_cast<int64_t>(row.bos) + static_cast<int64_t>(cl) * kChunk;
    const int nvalid = min(kChunk, row.len - cl * kChunk);
    const int64_t H = a.H;

    // ---- Q, K, Gam into LDS; S_c and v_new into registers (rows past the tail read as zero) ----
    u32x4_t hreg[HPT], vreg[VPT];
    {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (tok0 * H + hd) * DK;
      const uint16_t* kp = static_cast<const uint16_t*>(a.k) + (tok0 * H + hd) * DK;
      const uint16_t* vp = static_cast<const uint16_t*>(a.v) + (tok0 * H + hd) * DV;
      const uint16_t* hp = static_cast<const uint16_t*>(a.h) + ((static_cast<int64_t>(a.chunk_base) + chunk) * H + hd) * DV * DK;
      const float* gp = a.g + (tok0 * H + hd) * DK;
      const uint32_t qk_bytes = static_cast<uint32_t>(((nvalid - 1) * H + 1) * DK * 2);
      const rsrc_t rq = make_rsrc(qp, qk_bytes);
      const rsrc_t rk = make_rsrc(kp, qk_bytes);
      const rsrc_t rv = make_rsrc(vp, static_cast<uint32_t>(((nvalid - 1) * H + 1) * DV * 2));
      const rsrc_t rh = make_rsrc(hp, static_cast<uint32_t>(DV * DK * 2));
      const rsrc_t rg = make_rsrc(gp, static_cast<uint32_t>(((nvalid - 1) * H + 1) * DK * 4));
#pragma unroll
      for (int i = 0; i < HPT; ++i) {
        const int vv = tid + i * NT, r = vv / CQ, c = vv % CQ;
        hreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rh, static_cast<int>(r * DK * 2 + c * 16), 0, 0);
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int vv = tid + i * NT, r = vv / CV, c = vv % CV;
        vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, static_cast<int>(r * H * DV * 2 + c * 16), 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kChunk * CQ / NT; ++i) {
        const int vv = tid + i * NT, r = vv / CQ, c = vv % CQ;
        const int go = static_cast<int>(r * H * DK * 2 + c * 16);
        *reinterpret_cast<u32x4_t*>(sm.A.q + r * SQ + c * 16) = __builtin_amdgcn_raw_buffer_load_b128(rq, go, 0, 0);
        *reinterpret_cast<u32x4_t*>(sm.A.k + r * SQ + c * 16) = __builtin_amdgcn_raw_buffer_load_b128(rk, go, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kChunk * CG / NT; ++i) {
        const int vv = tid + i * NT, r = vv / CG, c = vv % CG;
        *reinterpret_cast<u32x4_t*>(sm.A.gam + r * GS + c * 4) =
            __builtin_amdgcn_raw_buffer_load_b128(rg, static_cast<int>(r * H * DK * 4 + c * 16), 0, 0);
      }
    }
    __syncthreads();

    // ---- P rows of block `wave` (registers): sum_d q_td k_id e^{Gam_td - Gam_id}, i <= t ----
    f32x4_t pr[4];
    {
      float xs[DK / 4];
      kda_row_side<DK, SQ, GS>(xs, sm.A.q, sm.A.gam, wave, g4, c16);
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        pr[J] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (J <= wave) {
          const f32x4_t d = kda_block_product<DK, SQ, GS>(xs, sm.A.k, sm.A.gam, wave, J, g4, c16);
#pragma unroll
          for (int r = 0; r < 4; ++r) pr[J][r] = (16 * J + c16 <= 16 * wave + 4 * g4 + r) ? d[r] : 0.f;
        }
      }
    }
    // ---- this lane's A-operand fragments of Q e^{Gam} (row 16 wave + c16) ----
    frag qh[KS], ql[KS];
    {
      const char* qrow = sm.A.q + (16 * wave + c16) * SQ;
      const float* grow = sm.A.gam + (16 * wave + c16) * GS;
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) {
        f32x4_t x[2], lo[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int d0 = 32 * s2 + 16 * half + 4 * g4;
          const u32x2_t qq = *reinterpret_cast<const u32x2_t*>(qrow + 2 * d0);
          const f32x4_t gv = *reinterpret_cast<const f32x4_t*>(grow + d0);
          x[half] = f32x4_t{__builtin_bit_cast(float, qq.x << 16) * exp_fast(gv[0]),
                            __builtin_bit_cast(float, qq.x & 0xffff0000u) * exp_fast(gv[1]),
                            __builtin_bit_cast(float, qq.y << 16) * exp_fast(gv[2]),
                            __builtin_bit_cast(float, qq.y & 0xffff0000u) * exp_fast(gv[3])};
#pragma unroll
          for (int r = 0; r < 4; ++r) lo[half][r] = x[half][r] - bf16_to_f32(f32_to_bf16(x[half][r]));
        }
        qh[s2] = S::frag_from_f32(x[0], x[1]);
        ql[s2] = S::frag_from_f32(lo[0], lo[1]);
      }
    }
    __syncthreads();  // Q, K, Gam are dead

    // ---- phase B: S_c, v_new and P into the region ----
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
      const int vv = tid + i * NT, r = vv / CQ, c = vv % CQ;
      *reinterpret_cast<u32x4_t*>(sm.B.h + r * SQ + c * 16) = hreg[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int vv = tid + i * NT, r = vv / CV, c = vv % CV;
      *reinterpret_cast<u32x4_t*>(sm.B.v + r * SV + c * 16) = vreg[i];
    }
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.B.p[(16 * wave + 4 * g4 + r) * LP + 16 * J + c16] = pr[J][r];
    __syncthreads();

    // ---- O^T = S_c^T (Q e^Gam)^T + v_new^T P^T for the tokens of tile `wave`: each
    //      lane ends with four consecutive value columns of its token (8-byte stores) ----
    const char* rowh = sm.B.h + c16 * SQ + (g4 >> 1) * 16 + (g4 & 1) * 8;
    auto rfrag = [&](const char* base, int tile, int s) {
      return S::frag_from_quads(*reinterpret_cast<const u32x2_t*>(base + 16 * tile * SQ + 64 * s),
                                *reinterpret_cast<const u32x2_t*>(base + 16 * tile * SQ + 64 * s + 32));
    };
    f32x4_t acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const frag hb = rfrag(rowh, ct, s);
        S::mma(acc[ct], hb, qh[s]);
        S::mma(acc[ct], hb, ql[s]);
      }
    const char* vb_ = sm.B.v + (4 * g4 + (c16 >> 2)) * SV + 8 * (c16 & 3);
    const int t = 16 * wave + c16;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (32 * s <= 16 * wave + 15) {
        const f32x4_t p0 = *reinterpret_cast<const f32x4_t*>(&sm.B.p[t * LP + 32 * s + 4 * g4]);
        const f32x4_t p1 = *reinterpret_cast<const f32x4_t*>(&sm.B.p[t * LP + 32 * s + 16 + 4 * g4]);
        f32x4_t l0, l1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          l0[r] = p0[r] - bf16_to_f32(f32_to_bf16(p0[r]));
          l1[r] = p1[r] - bf16_to_f32(f32_to_bf16(p1[r]));
        }
        const frag ph = S::frag_from_f32(p0, p1);
        const frag pl = S::frag_from_f32(l0, l1);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const frag vf = S::frag_from_quads(lds_tr16(vb_, 32 * s * SV + 32 * ct), lds_tr16(vb_, (32 * s + 16) * SV + 32 * ct));
          S::mma(acc[ct], vf, ph);
          S::mma(acc[ct], vf, pl);
        }
      }
    }

    uint16_t* op = static_cast<uint16_t*>(a.o) + (tok0 * H + hd) * DV;
    const rsrc_t ro = make_rsrc(op, static_cast<uint32_t>(((nvalid - 1) * H + 1) * DV * 2));
    const int voff = t * static_cast<int>(H * DV * 2) + 8 * g4;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(a.scale * acc[ct][0], a.scale * acc[ct][1]),
                                                    pack_bf16x2(a.scale * acc[ct][2], a.scale * acc[ct][3])},
                                            ro, voff, 32 * ct, 0);
  }
};

template <int DK, int DV>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void kda_prepare_kernel(const KdaArgs a) {
  using K = KdaPrepare<DK, DV>;
  __shared__ __align__(16) typename K::Smem sm;
  K::run(a, sm);
}

template <int DK, int DV>
__global__ __launch_bounds__(256) void kda_output_kernel(const KdaArgs a) {
  using K = KdaOutput<DK, DV>;
  __shared__ __align__(16) typename K::Smem sm;
  K::run(a, sm);
}

template <int DK, int DV>
static hipError_t launch_kda_prepare(const void* args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((kda_prepare_kernel<DK, DV>), dim3(grid), dim3(KdaPrepare<DK, DV>::NT), 0, stream,
                     *static_cast<const KdaArgs*>(args));
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_kda_output(const void* args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((kda_output_kernel<DK, DV>), dim3(grid), dim3(256), 0, stream, *static_cast<const KdaArgs*>(args));
  return hipGetLastError();
}

LaunchFn find_kda_prepare(int dk, int dv) {
  if (dk == 128 && dv == 128) return &launch_kda_prepare<128, 128>;
  if (dk == 128 && dv == 64) return &launch_kda_prepare<128, 64>;
  if (dk == 64 && dv == 128) return &launch_kda_prepare<64, 128>;
  if (dk == 64 && dv == 64) return &launch_kda_prepare<64, 64>;
  return nullptr;
}

LaunchFn find_kda_output(int dk, int dv) {
  if (dk == 128 && dv == 128) return &launch_kda_output<128, 128>;
  if (dk == 128 && dv == 64) return &launch_kda_output<128, 64>;
  if (dk == 64 && dv == 128) return &launch_kda_output<64, 128>;
  if (dk == 64 && dv == 64) return &launch_kda_output<64, 64>;
  return nullptr;
}

}  // namespace gdr
