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
// read straight from HBM, the B operand the whole current state, shared
// through LDS (double-buffered, one barrier per segment).  The next segment's
// rows of M and of S_loc are fetched while the current product runs, and
// S_init(s) is written straight from the accumulators.
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

  __device__ static void load_m(frag (&am)[KS], const float* mb, int wave, int g4, int c16) {
    const float* mr = mb + static_cast<int64_t>(16 * wave + c16) * DK;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(mr + 32 * ks + 4 * g4);
      const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(mr + 32 * ks + 16 + 4 * g4);
      am[ks] = S::frag_from_f32(x0, x1);
    }
  }

  __device__ static void run(const ComposeArgs& a, Smem& sm) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int NVB = a.DV / BVC;
    const int vb = blockIdx.x % NVB;
    const int rest = blockIdx.x / NVB;
    const int hd = rest % a.H;
    const int n = rest / a.H;
    if (n >= a.N) return;
    const int64_t H = a.H;
    const int DV = a.DV;
    const int col = vb * BVC + c16;           // this lane's value column
    const int row0 = 16 * wave + 4 * g4;      // this lane's four state rows
    const int P = a.P;

    // S_init(0) rows of this wave (C layout)
    f32x4_t cur{0.f, 0.f, 0.f, 0.f};
    if (a.h0 != nullptr) {
      const float* hb = a.h0 + (static_cast<int64_t>(n) * H + hd) * DV * DK;
      if (a.state_vk) {
        cur = *reinterpret_cast<const f32x4_t*>(hb + static_cast<int64_t>(col) * DK + row0);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) cur[r] = hb[static_cast<int64_t>(row0 + r) * DV + col];
      }
    }
    *reinterpret_cast<f32x4_t*>(&sm.s[0][c16 * LDS_ + row0]) = cur;
    frag am[KS];
    f32x4_t sl{0.f, 0.f, 0.f, 0.f};
    if (P > 0) {
      const int64_t seg = static_cast<int64_t>(n) * P;
      load_m(am, a.seg_trans + (seg * H + hd) * DK * DK, wave, g4, c16);
      sl = *reinterpret_cast<const f32x4_t*>(a.seg_state + (seg * H + hd) * DV * DK + static_cast<int64_t>(col) * DK + row0);
    }
    __syncthreads();

    for (int s = 0; s < P; ++s) {
      const int64_t seg = static_cast<int64_t>(n) * P + s;
      // emit S_init(s)
      *reinterpret_cast<f32x4_t*>(a.seg_init + (seg * H + hd) * DV * DK + static_cast<int64_t>(col) * DK + row0) = cur;
      // B operand: the whole S_init(s) from LDS
      const float* sb = &sm.s[s & 1][c16 * LDS_ + 4 * g4];
      frag bs[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        bs[ks] = S::frag_from_f32(*reinterpret_cast<const f32x4_t*>(sb + 32 * ks),
                                  *reinterpret_cast<const f32x4_t*>(sb + 32 * ks + 16));
      // next segment's operands in flight during the product
      frag an[KS];
      f32x4_t sn{0.f, 0.f, 0.f, 0.f};
      const bool more = (s + 1 < P);
      if (more) {
        load_m(an, a.seg_trans + ((seg + 1) * H + hd) * DK * DK, wave, g4, c16);
        sn = *reinterpret_cast<const f32x4_t*>(a.seg_state + ((seg + 1) * H + hd) * DV * DK +
                                               static_cast<int64_t>(col) * DK + row0);
      }
      // independent accumulators per 32-wide k-step break the MFMA dependency chain
      f32x4_t part[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) part[ks] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          part[ks] = __builtin_amdgcn_mfma_f32_16x16x4f32(am[ks].v[e], bs[ks].v[e], part[ks], 0, 0, 0);
      f32x4_t acc = sl;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc += part[ks];
      cur = acc;
      *reinterpret_cast<f32x4_t*>(&sm.s[(s + 1) & 1][c16 * LDS_ + row0]) = cur;
      if (more) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) am[ks] = an[ks];
        sl = sn;
      }
      __syncthreads();
    }
    if (a.hT != nullptr) {
      float* hb = a.hT + (static_cast<int64_t>(n) * H + hd) * DV * DK;
      if (a.state_vk) {
        *reinterpret_cast<f32x4_t*>(hb + static_cast<int64_t>(col) * DK + row0) = cur;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) hb[static_cast<int64_t>(row0 + r) * DV + col] = cur[r];
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
