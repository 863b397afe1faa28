// ABC slot-state construction on gfx950 (flash-linear-attention fork issue
// #23, "[Perf][B300] Parallelize ABC chunk state construction with affine
// summaries": "Problem" and "Proposed Dataflow").
//
// Normaliser: z_t = log(e^{z_{t-1}} + e^{s_t}) per slot.  Two levels:
//   abc_chunk_lse   one wave per (b, chunk, h), lane = slot: the chunk-local
//                   running log-sum-exp (written to z when requested) and the
//                   chunk total;
//   abc_carry       one wave per (b, h): z at chunk ends,
//                   zc[c] = logaddexp(zc[c-1], lse[c]), serial over chunks;
//   abc_fix_z       (only when z is requested) z_t = logaddexp(zc[c-1], local_t).
//
// States: every 64-token chunk applies the exact diagonal affine map
//   S <- S * r_c + c_c,   r_c = exp(zc[c-1] - zc[c]),  E_t = exp(s_t - zc[c]),
//   Hk [K x M]:  c_c = K_c^T E   (r over columns)
//   Hv [M x V]:  c_c = E^T V_c   (r over rows)
// One workgroup owns a 64x64 tile of Hk or Hv of one (b, h) and walks the
// chunks in order: the chunk contribution is formed on MFMA in FP32
// accumulators and added to the FP32 state in registers, so the "FP32
// summary" of the page never leaves the chip; the state before each chunk is
// written once, in the storage dtype.
#include <math.h>

#include "kernels.hpp"

namespace gdr {

__device__ __forceinline__ float logaddexp_f(float a, float b) {
  const float m = fmaxf(a, b);
  if (m == -INFINITY) return -INFINITY;
  return m + log1pf(expf(-fabsf(a - b)));
}

// ---------------------------------------------------------------- normaliser
__global__ __launch_bounds__(64) void abc_chunk_lse(const AbcArgs a) {
  const int m = threadIdx.x;  // slot (M == 64)
  const int bx = blockIdx.x;
  const int h = bx % a.H;
  const int c = (bx / a.H) % a.NC;
  const int b = bx / (a.H * a.NC);
  const uint16_t* s = static_cast<const uint16_t*>(a.s);
  const int t0 = c * kChunk;
  const int n = min(kChunk, a.T - t0);
  float L = -INFINITY;
  for (int t = 0; t < n; ++t) {
    const int64_t off = ((static_cast<int64_t>(b) * a.T + t0 + t) * a.H + h) * a.M + m;
    L = logaddexp_f(L, bf16_to_f32(s[off]));
    if (a.z != nullptr) a.z[off] = L;
  }
  a.zc[((static_cast<int64_t>(b) * a.NC + c) * a.H + h) * a.M + m] = L;
}

__global__ __launch_bounds__(64) void abc_carry(const AbcArgs a) {
  const int m = threadIdx.x;
  const int h = blockIdx.x % a.H;
  const int b = blockIdx.x / a.H;
  float z = -INFINITY;
  for (int c = 0; c < a.NC; ++c) {
    const int64_t off = ((static_cast<int64_t>(b) * a.NC + c) * a.H + h) * a.M + m;
    z = logaddexp_f(z, a.zc[off]);
    a.zc[off] = z;
  }
}

__global__ __launch_bounds__(256) void abc_fix_z(const AbcArgs a) {
  // one workgroup per (b, chunk >= 1, h): 64 tokens x 64 slots
  const int bx = blockIdx.x;
  const int h = bx % a.H;
  const int c = 1 + (bx / a.H) % (a.NC - 1);
  const int b = bx / (a.H * (a.NC - 1));
  const int t0 = c * kChunk;
  const int n = min(kChunk, a.T - t0);
  for (int e = threadIdx.x; e < kChunk * 64; e += 256) {
    const int t = e / 64, m = e % 64;
    if (t < n) {
      const float zp = a.zc[((static_cast<int64_t>(b) * a.NC + c - 1) * a.H + h) * a.M + m];
      const int64_t off = ((static_cast<int64_t>(b) * a.T + t0 + t) * a.H + h) * a.M + m;
      a.z[off] = logaddexp_f(zp, a.z[off]);
    }
  }
}

// ---------------------------------------------------------------- states
struct AbcStates {
  using S = St<bf16_t>;
  using quad = S::quad;
  using frag = S::frag;
  static constexpr int LDT = kChunk + 4;  // transposed tiles, bf16 elements

  struct Smem {
    uint16_t xt[64 * LDT];   // X^T: 64 state rows/cols (k or v) x 64 tokens
    uint16_t et[64 * LDT];   // E^T: 64 slots x 64 tokens
    float r[64];
  };

  __device__ static void run(const AbcArgs& a, Smem& sm) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
    const int nk = a.K / 64, nv = a.V / 64;
    const int tiles = nk + nv;
    const int bx = blockIdx.x;
    const int tile = bx % tiles;
    const int h = (bx / tiles) % a.H;
    const int b = bx / (tiles * a.H);
    const bool is_k = tile < nk;
    const int x0 = is_k ? 64 * tile : 64 * (tile - nk);  // first k row / v column of the tile
    const int X = is_k ? a.K : a.V;
    const uint16_t* xp = static_cast<const uint16_t*>(is_k ? a.k : a.v);
    const uint16_t* sp = static_cast<const uint16_t*>(a.s);
    const int64_t H = a.H, M = a.M;

    f32x4_t acc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int c = 0; c < a.NC; ++c) {
      const int t0 = c * kChunk;
      const int n = min(kChunk, a.T - t0);
      const int64_t zrow = ((static_cast<int64_t>(b) * a.NC + c) * H + h) * M;
      __syncthreads();
      // X^T and E^T (4x4 register transposes), r
      {
        const int blk = tid;  // 16 token quads x 16 column quads = 256 blocks
        const int cq = blk % 16, tq = blk / 16;
        quad in[4], tr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 4 * tq + r;
          in[r] = (t < n) ? ld_quad<bf16_t>(reinterpret_cast<const bf16_t*>(
                                xp + ((static_cast<int64_t>(b) * a.T + t0 + t) * H + h) * X + x0 + 4 * cq))
                          : S::zero_quad();
        }
        S::transpose4(in, tr);
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<quad*>(&sm.xt[(4 * cq + j) * LDT + 4 * tq]) = tr[j];
        const f32x4_t zl = *reinterpret_cast<const f32x4_t*>(a.zc + zrow + 4 * cq);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 4 * tq + r;
          float e[4] = {0.f, 0.f, 0.f, 0.f};
          if (t < n) {
            const quad sq = ld_quad<bf16_t>(reinterpret_cast<const bf16_t*>(
                sp + ((static_cast<int64_t>(b) * a.T + t0 + t) * H + h) * M + 4 * cq));
            float sv[4];
            S::quad_to_f32(sq, sv);
#pragma unroll
            for (int j = 0; j < 4; ++j) e[j] = expf(sv[j] - zl[j]);
          }
          in[r] = S::f32_to_quad(e);
        }
        S::transpose4(in, tr);
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<quad*>(&sm.et[(4 * cq + j) * LDT + 4 * tq]) = tr[j];
        if (tid < 64) {
          const float zc = a.zc[zrow + tid];
          const float zp = (c == 0) ? -INFINITY : a.zc[zrow - H * M + tid];
          sm.r[tid] = (c == 0) ? 0.f : expf(zp - zc);
        }
      }
      __syncthreads();

      // pre-chunk state (storage dtype)
      uint16_t* hp = static_cast<uint16_t*>(is_k ? a.hk : a.hv);
      const int64_t hbase = (static_cast<int64_t>(b) * a.NC + c) * H + h;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * wave + 4 * g4 + r, col = 16 * ct + c16;
          int64_t off;
          if (is_k) off = (hbase * a.K + x0 + row) * M + col;           // Hk[k][m]
          else off = (hbase * M + row) * a.V + x0 + col;                 // Hv[m][v]
          hp[off] = f32_to_bf16(acc[ct][r]);
        }
      }

      // S <- S * r + contribution
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float rr = is_k ? sm.r[16 * ct + c16] : sm.r[16 * wave + 4 * g4 + r];
          acc[ct][r] *= rr;
        }
      }
      // Hk: A = X^T rows (k), B = E^T rows (m).  Hv: A = E^T rows (m), B = X^T rows (v).
      const uint16_t* arows = is_k ? sm.xt : sm.et;
      const uint16_t* brows = is_k ? sm.et : sm.xt;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint16_t* ar = &arows[(16 * wave + c16) * LDT + 32 * s + 4 * g4];
        const frag fa = S::frag_from_quads(*reinterpret_cast<const quad*>(ar), *reinterpret_cast<const quad*>(ar + 16));
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const uint16_t* br = &brows[(16 * ct + c16) * LDT + 32 * s + 4 * g4];
          S::mma(acc[ct], fa, S::frag_from_quads(*reinterpret_cast<const quad*>(br), *reinterpret_cast<const quad*>(br + 16)));
        }
      }
    }

    float* fp = is_k ? a.hk_final : a.hv_final;
    if (fp == nullptr) return;
    const int64_t fbase = static_cast<int64_t>(b) * H + h;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * wave + 4 * g4 + r, col = 16 * ct + c16;
        if (is_k) fp[(fbase * a.K + x0 + row) * M + col] = acc[ct][r];
        else fp[(fbase * M + row) * a.V + x0 + col] = acc[ct][r];
      }
    }
  }
};

__global__ __launch_bounds__(256) void abc_states(const AbcArgs a) {
  __shared__ __align__(16) AbcStates::Smem sm;
  AbcStates::run(a, sm);
}

hipError_t launch_abc_z(const AbcArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(abc_chunk_lse, dim3(a.B * a.NC * a.H), dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(abc_carry, dim3(a.B * a.H), dim3(64), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.z == nullptr || a.NC < 2) return e;
  hipLaunchKernelGGL(abc_fix_z, dim3(a.B * (a.NC - 1) * a.H), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_abc_scan(const AbcArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(abc_states, dim3(a.B * a.H * (a.K / 64 + a.V / 64)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdr
