// Segment composition in FP32 (cuLA pull request #127, "Root cause and
// implementation": the transition is kept canonically in FP32 and segments
// are composed one after another):
//
//   S_init(0) = h0 (or 0),   S_init(s+1) = M_s S_init(s) + S_loc(s)
//
// One workgroup (4 waves) per (sequence, head, 16 value columns).  The
// running state S [DK x 16] lives in LDS (value-major, FP32) so every wave can
// read all of it as the B operand; wave w produces output rows
// [w DK/4, (w+1) DK/4) with FP32 MFMA (v_mfma_f32_16x16x4_f32), reading its
// rows of M_s straight from HBM as the A operand.  The next segment's rows of
// M are fetched into registers while the current product runs.
#include "kernels.hpp"

namespace gdr {

template <int DK>
struct ComposeKernel {
  using S = St<float>;
  using frag = S::frag;
  static constexpr int BVC = 16;
  static constexpr int DTW = DK / 64;   // 16-row tiles per wave
  static constexpr int KS = DK / 32;
  static constexpr int LDS_ = DK + 4;

  struct Smem {
    float s[2][BVC * LDS_];
  };

  __device__ static void load_m(frag (&am)[DTW][KS], const float* mb, int wave, int g4, int c16) {
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt) {
      const float* mr = mb + static_cast<int64_t>(16 * (wave * DTW + dt) + c16) * DK;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(mr + 32 * ks + 4 * g4);
        const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(mr + 32 * ks + 16 + 4 * g4);
        am[dt][ks] = S::frag_from_f32(x0, x1);
      }
    }
  }

  __device__ static void run(const ComposeArgs& a, Smem& sm) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
    const int NVB = a.DV / BVC;
    const int vb = blockIdx.x % NVB;
    const int rest = blockIdx.x / NVB;
    const int hd = rest % a.H;
    const int n = rest / a.H;
    if (n >= a.N) return;
    const int64_t H = a.H;
    const int DV = a.DV;
    const int col0 = vb * BVC;
    const int P = a.P;

    // S_init(0)
    for (int e = tid; e < BVC * DK; e += 256) {
      const int j = e / DK, i = e % DK;
      float x = 0.f;
      if (a.h0 != nullptr) {
        const float* hb = a.h0 + (static_cast<int64_t>(n) * H + hd) * DV * DK;
        x = a.state_vk ? hb[static_cast<int64_t>(col0 + j) * DK + i] : hb[static_cast<int64_t>(i) * DV + col0 + j];
      }
      sm.s[0][j * LDS_ + i] = x;
    }
    frag am[DTW][KS];
    if (P > 0) load_m(am, a.seg_trans + (static_cast<int64_t>(n) * P * H + hd) * DK * DK, wave, g4, c16);
    __syncthreads();

    for (int s = 0; s < P; ++s) {
      const int cur = s & 1;
      const int64_t seg = static_cast<int64_t>(n) * P + s;
      // emit S_init(s)
      float* ib = a.seg_init + (seg * H + hd) * DV * DK;
      for (int e = tid; e < BVC * DK / 4; e += 256) {
        const int j = e / (DK / 4), i4 = e % (DK / 4);
        *reinterpret_cast<f32x4_t*>(ib + static_cast<int64_t>(col0 + j) * DK + 4 * i4) =
            *reinterpret_cast<const f32x4_t*>(&sm.s[cur][j * LDS_ + 4 * i4]);
      }
      // acc = S_loc(s) rows of this wave
      const float* lb = a.seg_state + (seg * H + hd) * DV * DK + static_cast<int64_t>(col0 + c16) * DK;
      f32x4_t acc[DTW];
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt)
        acc[dt] = *reinterpret_cast<const f32x4_t*>(lb + 16 * (wave * DTW + dt) + 4 * g4);
      // B operand: S_init(s) from LDS
      frag bs[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const float* sr = &sm.s[cur][c16 * LDS_ + 32 * ks + 4 * g4];
        bs[ks] = S::frag_from_f32(*reinterpret_cast<const f32x4_t*>(sr),
                                  *reinterpret_cast<const f32x4_t*>(sr + 16));
      }
      frag an[DTW][KS];
      const bool more = (s + 1 < P);
      if (more) load_m(an, a.seg_trans + ((seg + 1) * H + hd) * DK * DK, wave, g4, c16);
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) S::mma(acc[dt], am[dt][ks], bs[ks]);
      // S_init(s+1) rows of this wave -> the other buffer
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt)
        *reinterpret_cast<f32x4_t*>(&sm.s[cur ^ 1][c16 * LDS_ + 16 * (wave * DTW + dt) + 4 * g4]) = acc[dt];
      if (more) {
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) am[dt][ks] = an[dt][ks];
      }
      __syncthreads();
    }
    if (a.hT != nullptr) {
      float* hb = a.hT + (static_cast<int64_t>(n) * H + hd) * DV * DK;
      const int fin = P & 1;
      for (int e = tid; e < BVC * DK; e += 256) {
        const int j = e / DK, i = e % DK;
        const float x = sm.s[fin][j * LDS_ + i];
        if (a.state_vk) hb[static_cast<int64_t>(col0 + j) * DK + i] = x;
        else hb[static_cast<int64_t>(i) * DV + col0 + j] = x;
      }
    }
  }
};

template <int DK>
__global__ __launch_bounds__(256) void compose_kernel(const ComposeArgs a) {
  using K = ComposeKernel<DK>;
  __shared__ __align__(16) typename K::Smem sm;
  K::run(a, sm);
}

template <int DK>
static hipError_t launch_compose(const void* args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((compose_kernel<DK>), dim3(grid), dim3(256), 0, stream,
                     *static_cast<const ComposeArgs*>(args));
  return hipGetLastError();
}

LaunchFn find_compose(int dk) {
  if (dk == 128) return &launch_compose<128>;
  if (dk == 64) return &launch_compose<64>;
  return nullptr;
}

}  // namespace gdr
