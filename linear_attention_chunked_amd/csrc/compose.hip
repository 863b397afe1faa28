// Segment composition in FP32 (cuLA pull request #127, "Root cause and
// implementation": the transition is kept canonically in FP32 and segments
// are composed one after another):
//
//   S_init(0) = h0 (or 0),   S_init(s+1) = M_s S_init(s) + S_loc(s)
//
// One workgroup per (sequence, head, 16 value columns) with one wave per 16
// rows of the state (DK/16 waves).  Wave w keeps its rows of the running
// state in FP32 accumulator registers and produces its rows of the next one
// with FP32 MFMA (v_mfma_f32_16x16x4_f32, one independent accumulator per
// 32-wide k-step so the products overlap): the A operand is its 16 rows of M_s,
// read straight from global memory, the B operand the whole current state,
// shared through LDS (double-buffered, one barrier per segment).
//
// The chain is latency-bound (a few dozen workgroups, one product per
// segment), so the operands of segment s+2 are requested while segment s
// computes: three register sets rotate through an unrolled loop, and each
// set's loads are issued ahead of the state stores so that waiting for them
// never waits for a store.  The workgroups of one (sequence, head) share an
// XCD (blockIdx modulo 8), so M_s and S_loc(s) come from HBM once per XCD and
// from that XCD's L2 for the other column blocks.
#include "kernels.hpp"

namespace gdr {

template <int DK>
struct ComposeKernel {
  using S = St<float>;
  using frag = S::frag;
  static constexpr int BVC = 16;
  static constexpr int NW = DK / 16;
  static constexpr int KS = DK / 32;
  static constexpr int LDS_ = DK + 4;

  struct Smem {
    float s[2][BVC * LDS_];
  };

  struct Ops {
    frag m[KS];  // this lane's part of the wave's 16 rows of M_s
    f32x4_t l;   // this lane's four rows of S_loc(s) in its column
  };

  struct Ctx {
    const ComposeArgs* a;
    int64_t n, hd, H;
    int col, row0, wave, g4, c16;
  };

  __device__ static __forceinline__ void load(Ops& o, const Ctx& x, int s) {
    const ComposeArgs& a = *x.a;
    const int64_t seg = x.n * a.P + s;
    const float* mr = a.seg_trans + (seg * x.H + x.hd) * DK * DK + static_cast<int64_t>(16 * x.wave + x.c16) * DK;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(mr + 32 * ks + 4 * x.g4);
      const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(mr + 32 * ks + 16 + 4 * x.g4);
      o.m[ks] = S::frag_from_f32(x0, x1);
    }
    o.l = *reinterpret_cast<const f32x4_t*>(a.seg_state + (seg * x.H + x.hd) * a.DV * DK +
                                            static_cast<int64_t>(x.col) * DK + x.row0);
  }

  // Segment s: operands in `cur_ops`, requests segment s+2 into `next2`.
  __device__ static __forceinline__ void step(f32x4_t& cur, const Ops& ops, Ops& next2, const Ctx& x, int s,
                                              Smem& sm) {
    const ComposeArgs& a = *x.a;
    // unconditional (the last segment is re-read near the end), so every step
    // issues the same loads and the compiler's wait counts stay two steps deep
    load(next2, x, min(s + 2, a.P - 1));
    const int64_t seg = x.n * a.P + s;
    *reinterpret_cast<f32x4_t*>(a.seg_init + (seg * x.H + x.hd) * a.DV * DK + static_cast<int64_t>(x.col) * DK +
                                x.row0) = cur;
    const float* sb = &sm.s[s & 1][x.c16 * LDS_ + 4 * x.g4];
    frag bs[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      bs[ks] = S::frag_from_f32(*reinterpret_cast<const f32x4_t*>(sb + 32 * ks),
                                *reinterpret_cast<const f32x4_t*>(sb + 32 * ks + 16));
    f32x4_t part[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) part[ks] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        part[ks] = __builtin_amdgcn_mfma_f32_16x16x4f32(ops.m[ks].v[e], bs[ks].v[e], part[ks], 0, 0, 0);
    f32x4_t acc = ops.l;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc += part[ks];
    cur = acc;
    *reinterpret_cast<f32x4_t*>(&sm.s[(s + 1) & 1][x.c16 * LDS_ + x.row0]) = cur;
    __syncthreads();
  }

  __device__ static void run(const ComposeArgs& a, Smem& sm) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int NVB = a.DV / BVC;
    const int bx = blockIdx.x;
    const int xcd = bx & 7, slot = bx >> 3;
    const int pair = 8 * (slot / NVB) + xcd;
    const int vb = slot % NVB;
    if (pair >= a.N * a.H) return;
    Ctx x;
    x.a = &a;
    x.n = pair / a.H;
    x.hd = pair % a.H;
    x.H = a.H;
    x.g4 = lane >> 4;
    x.c16 = lane & 15;
    x.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    x.col = vb * BVC + x.c16;           // this lane's value column
    x.row0 = 16 * x.wave + 4 * x.g4;    // this lane's four state rows
    const int DV = a.DV;
    const int P = a.P;

    // S_init(0) rows of this wave (C layout)
    f32x4_t cur{0.f, 0.f, 0.f, 0.f};
    if (a.h0 != nullptr) {
      const float* hb = a.h0 + (x.n * x.H + x.hd) * DV * DK;
      if (a.state_vk) {
        cur = *reinterpret_cast<const f32x4_t*>(hb + static_cast<int64_t>(x.col) * DK + x.row0);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) cur[r] = hb[static_cast<int64_t>(x.row0 + r) * DV + x.col];
      }
    }
    *reinterpret_cast<f32x4_t*>(&sm.s[0][x.c16 * LDS_ + x.row0]) = cur;
    Ops A, B, C;
    if (P > 0) {
      load(A, x, 0);
      load(B, x, min(1, P - 1));
    }
    __syncthreads();
    for (int s = 0; s < P; s += 3) {
      step(cur, A, C, x, s, sm);
      if (s + 1 >= P) break;
      step(cur, B, A, x, s + 1, sm);
      if (s + 2 >= P) break;
      step(cur, C, B, x, s + 2, sm);
    }
    if (a.hT != nullptr) {
      float* hb = a.hT + (x.n * x.H + x.hd) * DV * DK;
      if (a.state_vk) {
        *reinterpret_cast<f32x4_t*>(hb + static_cast<int64_t>(x.col) * DK + x.row0) = cur;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) hb[static_cast<int64_t>(x.row0 + r) * DV + x.col] = cur[r];
      }
    }
  }
};

template <int DK>
__global__ __launch_bounds__(DK * 4) void compose_kernel(const ComposeArgs a) {
  using K = ComposeKernel<DK>;
  __shared__ __align__(16) typename K::Smem sm;
  K::run(a, sm);
}

template <int DK>
static hipError_t launch_compose(const void* args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((compose_kernel<DK>), dim3(grid), dim3(DK * 4), 0, stream,
                     *static_cast<const ComposeArgs*>(args));
  return hipGetLastError();
}

LaunchFn find_compose(int dk) {
  if (dk == 128) return &launch_compose<128>;
  if (dk == 64) return &launch_compose<64>;
  return nullptr;
}

}  // namespace gdr
