// Chunk preparation for bfloat16 storage on gfx950 (float32 storage keeps
// prepare.hip).  Same factors:
//
//   gamma  = chunk-local inclusive cumsum of g
//   A[t,i] = beta_t exp(gamma_t - gamma_i) (k_t . k_i)     (i < t)
//   T      = (I + A)^-1                                      FP32
//   w      = T diag(beta exp(gamma)) K,   u = T diag(beta) V
//
// One workgroup (4 waves) per (chunk, head).  Layout of the work:
//   * K and V land in LDS row-major (tail rows read as zero through the buffer
//     range check); the products that contract over tokens read them as MFMA
//     operands with ds_read_b64_tr_b16.
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
//   * V is loaded (into registers) once the diagonal blocks are done and
//     takes the place of K in LDS once the w product has read K.  A and T
//     keep only their blocks on or below the diagonal; the footprint (29.4 KB
//     at 128 x 128) and at most 96 VGPRs let five workgroups share a CU.
#include "gfx950.hpp"
#include "kernels.hpp"

namespace gdr {

namespace {

// D (16x16, C layout) += X (16x16) Y (16x16) in FP32 with k = 4g + r:
// a[r] = X[c][4g + r] (row c of X), b[r] = Y[4g + r][c] (the C layout of Y).
__device__ __forceinline__ void mm16(f32x4_t& d, const f32x4_t& a, const f32x4_t& b) {
#pragma unroll
  for (int r = 0; r < 4; ++r) d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], b[r], d, 0, 0, 0);
}

}  // namespace

template <int DK, int DV>
struct Prepare2 {
  using S = St<bf16_t>;
  using frag = S::frag;
  static constexpr int NT = 256;
  static constexpr int SKB = DK * 2 + 16;   // padded row strides (bytes)
  static constexpr int SVB = DV * 2 + 16;
  static constexpr int SKV = SKB > SVB ? SKB : SVB;
  static constexpr int KS = DK / 32;
  static constexpr int kTri = 2816;         // floats of the lower block triangle (rows below)

  // A and T (64 x 64, FP32) keep only their blocks on or below the diagonal:
  // row t of block row b = t / 16 holds columns 0 .. 16 b + 15, with a row
  // stride of 16 b + 20 floats (pads keep the column and 16-byte row reads
  // free of bank conflicts).  Every block of T is written over the block of A
  // in the same place once nothing reads that A block any more (T[b][b] after
  // its own substitution, T[1][0] and T[3][2] from the wave that read their A
  // blocks, the last four blocks after a barrier).  V takes the place of K
  // once the w product has read K.  29.4 KB at 128 x 128: five workgroups
  // share a CU.
  struct Smem {
    char kv[kChunk * SKV];
    float t[kTri];
    float gam[kChunk];
    float beta[kChunk];
    float bg[kChunk];  // beta exp(gamma)
  };
  // first float of row t in Smem::t
  __device__ static __forceinline__ int toff(int t) {
    const int b = t >> 4;
    return 128 * b * (b - 1) + 320 * b + (t & 15) * (16 * b + 20);
  }

  __device__ static int find_row(const ChunkArgs& a, int chunk) {
    int lo = 0, hi = a.n_rows - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.rows[mid].chunk_off <= chunk) lo = mid; else hi = mid - 1;
    }
    return lo;
  }

  // K rows (and g, beta for the first wave) pass through registers on their
  // way to LDS.
  static constexpr int KV_PT = kChunk * (DK / 8) / NT;  // 16-byte K vectors per thread
  static constexpr int VV_PT = kChunk * (DV / 8) / NT;
  struct Pref {
    u32x4_t k[KV_PT];
    float g, b;
  };

  struct Item {
    int hd;
    int64_t tok0;
    int nvalid;
  };

  __device__ static Item item_of(const ChunkArgs& a, int item) {
    const int chunk = item / a.H;
    const Row row = a.rows[find_row(a, chunk)];
    const int cl = chunk - row.chunk_off;
    return Item{item % a.H, static_cast<int64_t>(row.bos) + static_cast<int64_t>(cl) * kChunk,
                min(kChunk, row.len - cl * kChunk)};
  }

  __device__ static void load(Pref& pf, const ChunkArgs& a, const Item& it) {
    const int tid = threadIdx.x;
    const int64_t H = a.H;
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + (it.tok0 * H + it.hd) * DK;
    const rsrc_t rk = make_rsrc(kp, static_cast<uint32_t>(((it.nvalid - 1) * H + 1) * DK * 2));
    constexpr int CK = DK / 8;  // 16-byte chunks per row
#pragma unroll
    for (int i = 0; i < KV_PT; ++i) {
      const int vv = tid + i * NT, r = vv / CK, c = vv % CK;
      pf.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, static_cast<int>(r * H * DK * 2 + c * 16), 0, 0);
    }
    const float* gp = a.g + it.tok0 * H + it.hd;
    const float* bp = a.beta + it.tok0 * H + it.hd;
    const uint32_t gb = static_cast<uint32_t>(((it.nvalid - 1) * H + 1) * 4);
    const int go = static_cast<int>((tid & 63) * H * 4);
    pf.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(gp, gb), go, 0, 0));
    pf.b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(bp, gb), go, 0, 0));
  }

  // One workgroup per item (item = chunk * H + head).
  __device__ static void run(const ChunkArgs& a, Smem& sm) {
    const int nitems = a.n_chunks * a.H;
    const int item = blockIdx.x;
    if (item >= nitems) return;
    const Item it = item_of(a, item);
    Pref pf;
    load(pf, a, it);
    one(a, sm, pf, it);
  }

  __device__ static __forceinline__ void one(const ChunkArgs& a, Smem& sm, Pref& pf, const Item& it) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hd = it.hd;
    const int64_t tok0 = it.tok0;
    const int nvalid = it.nvalid;
    const int64_t H = a.H;

    // ---- K rows (zero past the tail), gamma and beta, from the loads issued at entry ----
    constexpr int CV = DV / 8;
    {
      constexpr int CK = DK / 8;
#pragma unroll
      for (int i = 0; i < KV_PT; ++i) {
        const int vv = tid + i * NT, r = vv / CK, c = vv % CK;
        *reinterpret_cast<u32x4_t*>(sm.kv + r * SKB + c * 16) = pf.k[i];
      }
      if (wave == 0) {
        float x = (lane < nvalid) ? pf.g : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(x, off, 64);
          if (lane >= off) x += y;
        }
        const float b = (lane < nvalid) ? pf.b : 0.f;
        sm.gam[lane] = x;
        sm.beta[lane] = b;
        sm.bg[lane] = b * exp_fast(x);
        if (lane < nvalid) a.g_cum[(tok0 + lane) * H + hd] = x;
      }
    }
    __syncthreads();

    // ---- Gram matrix row tile `wave`; A = beta_t e^{gamma_t - gamma_i} G (i < t) ----
    {
      f32x4_t acc[4];
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) acc[tj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const char* kr = sm.kv + c16 * SKB + (g4 >> 1) * 16 + (g4 & 1) * 8;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const frag fa = S::frag_from_quads(*reinterpret_cast<const u32x2_t*>(kr + 16 * wave * SKB + 64 * s),
                                           *reinterpret_cast<const u32x2_t*>(kr + 16 * wave * SKB + 64 * s + 32));
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
          if (tj <= wave) {
            const frag fb = S::frag_from_quads(*reinterpret_cast<const u32x2_t*>(kr + 16 * tj * SKB + 64 * s),
                                               *reinterpret_cast<const u32x2_t*>(kr + 16 * tj * SKB + 64 * s + 32));
            S::mma(acc[tj], fa, fb);
          }
        }
      }
      // Every LDS read is issued before any exponent: the (i < t) mask is a
      // select on values already in registers, not a branch around each
      // read.  e^{gamma_t - gamma_i} may overflow where i > t; the select
      // drops it.  Blocks above the diagonal (tj > wave) are not stored.
      const int t0 = 16 * wave + 4 * g4;
      const f32x4_t gt = *reinterpret_cast<const f32x4_t*>(&sm.gam[t0]);
      const f32x4_t bt = *reinterpret_cast<const f32x4_t*>(&sm.beta[t0]);
      float gi[4];
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) gi[tj] = sm.gam[16 * tj + c16];
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        const int i = 16 * tj + c16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + r;
          if (tj <= wave) {
            const float full = bt[r] * exp_fast(gt[r] - gi[tj]) * acc[tj][r];
            const float val = (i < t) ? full : 0.f;
            sm.t[toff(t) + i] = val;
          }
        }
      }
    }

    // ---- diagonal blocks: T[b][b] = (I + A[b][b])^-1 by forward substitution, wave b ----
    // Lane (j, g) solves rows 4 g .. 4 g + 3 of column j, by blocks of four
    // rows: the lanes owning block q finish its rows, ds_bpermute hands the
    // four values to every lane of the same column, and the lanes of later
    // blocks subtract their terms.  Row r still subtracts its terms in the
    // order i = 0, 1, ...  The entries of A are 16-byte LDS reads of the
    // wave's own rows, off the dependent chain.  T[b][b] is written over
    // A[b][b] (both in the wave's own rows: no barrier).
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
    // V rows for the last product (zero past the tail): in flight during the off-diagonal blocks and w
    u32x4_t vcur[VV_PT];
    {
      const uint16_t* vp = static_cast<const uint16_t*>(a.v) + (tok0 * H + hd) * DV;
      const rsrc_t rv = make_rsrc(vp, static_cast<uint32_t>(((nvalid - 1) * H + 1) * DV * 2));
#pragma unroll
      for (int i = 0; i < VV_PT; ++i) {
        const int vv = tid + i * NT, r = vv / CV, c = vv % CV;
        vcur[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, static_cast<int>(r * H * DV * 2 + c * 16), 0, 0);
      }
    }
    __syncthreads();

    // FP32 operand reads for mm16: row-major rows (a) and C-layout columns (b)
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
      mm16(y, a_rows(sm.t, p + 16, p), b_cols(sm.t, p, p));      // A[1][0] T[0][0]
      mm16(x, a_rows(sm.t, p + 16, p + 16), y);                  // T[1][1] (.)
      store_c(sm.t, p + 16, p, -x);
    }
    __syncthreads();

    // ---- T[2+i][j] = -(T_hi[i][0] Y[0][j] + T_hi[i][1] Y[1][j]),  Y = A[2:4][0:2] T[0:2][j] ----
    {
      const int i = wave >> 1, j = wave & 1;
      f32x4_t y0{0.f, 0.f, 0.f, 0.f}, y1{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (k >= j) {  // T[0][1] is zero
          const f32x4_t tb = b_cols(sm.t, 16 * k, 16 * j);
          mm16(y0, a_rows(sm.t, 32, 16 * k), tb);
          mm16(y1, a_rows(sm.t, 48, 16 * k), tb);
        }
      }
      __syncthreads();  // every wave has read A[2:4][0:2] before any T block replaces it
      f32x4_t x{0.f, 0.f, 0.f, 0.f};
      mm16(x, a_rows(sm.t, 32 + 16 * i, 32), y0);                   // T_hi[i][0] (T[2][2] or T[3][2])
      if (i == 1) mm16(x, a_rows(sm.t, 48, 48), y1);                // T_hi[1][1] = T[3][3]
      store_c(sm.t, 32 + 16 * i, 16 * j, -x);
    }
    __syncthreads();

    // ---- w^T = K^T T'^T and u^T = V^T T''^T; wave = token tile of the output ----
    const int t = 16 * wave + c16;
    const int nsteps = (16 * wave + 15) / 32 + 1;  // T is lower triangular
    // this lane's operand fragments of row t of T diag(coef), split into bf16
    // hi + lo; column blocks past the diagonal (not stored) are zero
    auto row_frags = [&](const float* coef, frag (&hi)[2], frag (&lo)[2]) {
      const float* tr = &sm.t[toff(t)];
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
    };
    // A operand K^T[d][i] / V^T[d][i] via transpose reads of the row-major tiles
    const int tr_row = 4 * g4 + (c16 >> 2);
    const int tr_col = 8 * (c16 & 3);
    auto product = [&](const char* tile, int stride, int D, const frag (&hi)[2], const frag (&lo)[2], void* out) {
      uint16_t* op = static_cast<uint16_t*>(out) + (tok0 * H + hd) * D;
      const rsrc_t ro = make_rsrc(op, static_cast<uint32_t>(((nvalid - 1) * H + 1) * D * 2));
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        f32x4_t acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (s < nsteps) {
            const char* base = tile + (32 * s + tr_row) * stride + 32 * dt + tr_col;
            const frag fa = S::frag_from_quads(lds_tr16(base, 0), lds_tr16(base, 16 * stride));
            S::mma(acc, fa, hi[s]);
            S::mma(acc, fa, lo[s]);
          }
        }
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])}, ro,
                                              static_cast<int>(t * H * D * 2 + (16 * dt + 4 * g4) * 2), 0, 0);
      }
    };
    {
      frag hi[2], lo[2];
      row_frags(sm.bg, hi, lo);  // T diag(beta e^gamma)
      product(sm.kv, SKB, DK, hi, lo, a.w);
    }
    __syncthreads();  // every wave is done with K: V replaces it
#pragma unroll
    for (int i = 0; i < VV_PT; ++i) {
      const int vv = tid + i * NT, r = vv / CV, c = vv % CV;
      *reinterpret_cast<u32x4_t*>(sm.kv + r * SVB + c * 16) = vcur[i];
    }
    __syncthreads();
    {
      frag hi[2], lo[2];
      row_frags(sm.beta, hi, lo);  // T diag(beta)
      product(sm.kv, SVB, DV, hi, lo, a.u);
    }
  }
};

template <int DK, int DV>
__global__ __launch_bounds__(256) void prepare2_kernel(const ChunkArgs a) {
  using K = Prepare2<DK, DV>;
  __shared__ __align__(16) typename K::Smem sm;
  K::run(a, sm);
}

template <int DK, int DV>
static hipError_t launch_prepare2(const void* args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((prepare2_kernel<DK, DV>), dim3(grid), dim3(256), 0, stream, *static_cast<const ChunkArgs*>(args));
  return hipGetLastError();
}

LaunchFn find_prepare2(int dk, int dv) {
  if (dk == 128 && dv == 128) return &launch_prepare2<128, 128>;
  if (dk == 128 && dv == 64) return &launch_prepare2<128, 64>;
  if (dk == 64 && dv == 128) return &launch_prepare2<64, 128>;
  if (dk == 64 && dv == 64) return &launch_prepare2<64, 64>;
  return nullptr;
}

}  // namespace gdr
