// Chunk output: o for every token of a chunk, from the pre-chunk state.
//
// For token t of chunk c (gamma = chunk-local cumulative g):
//   o_t = scale * ( e^{gamma_t} q_t^T S_c  +  sum_{i <= t} e^{gamma_t - gamma_i} (q_t . k_i) v_new_i )
// which unrolls S_t^T q_t of the token recurrence over the chunk.
//
// One workgroup (4 waves) per (chunk, head, 64 value columns); wave w owns the
// output rows of token tile w.  P^T = K Q^T is computed in accumulator
// layout, so (with the k(g, e) operand map) the causal block P is already
// the A operand of P v_new; v_new and h are staged in LDS in the layouts
// their B operands read contiguously.
#include "kernels.hpp"

namespace gdr {

template <typename TI, int DK, int DV>
struct OutputKernel {
  using S = St<TI>;
  using quad = typename S::quad;
  using frag = typename S::frag;
  static constexpr int NT = 256;
  static constexpr int BVO = 64;              // value columns per workgroup
  static constexpr int NCT = BVO / 16;
  static constexpr int EPV = 16 / sizeof(TI);
  static constexpr int LDQ = DK + EPV;        // row-major Q, K, h rows
  static constexpr int LDT = kChunk + 4;      // v_new^T
  static constexpr int KS = DK / 32;

  struct Smem {
    TI q[kChunk * LDQ];
    TI k[kChunk * LDQ];
    TI h[BVO * LDQ];      // h^T rows: value column j, DK contiguous
    TI vt[BVO * LDT];     // v_new^T
    float gam[kChunk];
  };

  __device__ static void run(const ChunkArgs& a, Smem& sm) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
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
    const TI* __restrict__ qp = static_cast<const TI*>(a.q);
    const TI* __restrict__ kp = static_cast<const TI*>(a.k);
    const TI* __restrict__ vp = static_cast<const TI*>(a.v);
    const TI* __restrict__ hp = static_cast<const TI*>(a.h) +
                                ((static_cast<int64_t>(a.chunk_base) + chunk) * H + hd) * DV * DK;

    for (int v = tid; v < kChunk * DK / EPV; v += NT) {
      const int r = v / (DK / EPV), cv = v % (DK / EPV);
      u32x4_t xq{0u, 0u, 0u, 0u}, xk{0u, 0u, 0u, 0u};
      if (r < nvalid) {
        xq = *reinterpret_cast<const u32x4_t*>(qp + ((tok0 + r) * H + hd) * DK + cv * EPV);
        xk = *reinterpret_cast<const u32x4_t*>(kp + ((tok0 + r) * H + hd) * DK + cv * EPV);
      }
      *reinterpret_cast<u32x4_t*>(&sm.q[r * LDQ + cv * EPV]) = xq;
      *reinterpret_cast<u32x4_t*>(&sm.k[r * LDQ + cv * EPV]) = xk;
    }
    for (int v = tid; v < BVO * DK / EPV; v += NT) {
      const int j = v / (DK / EPV), cv = v % (DK / EPV);
      *reinterpret_cast<u32x4_t*>(&sm.h[j * LDQ + cv * EPV]) =
          *reinterpret_cast<const u32x4_t*>(hp + static_cast<int64_t>(col0 + j) * DK + cv * EPV);
    }
    for (int b = tid; b < (kChunk / 4) * (BVO / 4); b += NT) {
      const int cq = b % (BVO / 4), tq = b / (BVO / 4);
      quad in[4], tr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * tq + r;
        in[r] = (t < nvalid) ? ld_quad<TI>(vp + ((tok0 + t) * H + hd) * DV + col0 + 4 * cq) : S::zero_quad();
      }
      S::transpose4(in, tr);
#pragma unroll
      for (int j = 0; j < 4; ++j) st_quad<TI>(&sm.vt[(4 * cq + j) * LDT + 4 * tq], tr[j]);
    }
    if (tid < kChunk) sm.gam[tid] = (tid < nvalid) ? a.g[(tok0 + tid) * H + hd] : 0.f;
    __syncthreads();

    // ---- P^T[i][t] = k_i . q_t for t in tile `wave`, i tiles 0..wave ----
    const int t = 16 * wave + c16;  // this lane's token as a column of P^T / row of P
    f32x4_t pt[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) pt[it] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const TI* br = &sm.q[t * LDQ + 32 * s + 4 * g4];
      const frag fb = S::frag_from_quads(ld_quad<TI>(br), ld_quad<TI>(br + 16));
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        if (it <= wave) {
          const TI* ar = &sm.k[(16 * it + c16) * LDQ + 32 * s + 4 * g4];
          const frag fa = S::frag_from_quads(ld_quad<TI>(ar), ld_quad<TI>(ar + 16));
          S::mma(pt[it], fa, fb);
        }
      }
    }
    const float gt = sm.gam[t];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * it + 4 * g4 + r;
        pt[it][r] = (i <= t && t < nvalid) ? pt[it][r] * expf(gt - sm.gam[i]) : 0.f;
      }
    }

    // ---- O = diag(e^gamma) Q S_c  +  P v_new ----
    f32x4_t acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const TI* ar = &sm.q[(16 * wave + c16) * LDQ + 32 * s + 4 * g4];
      const frag fa = S::frag_from_quads(ld_quad<TI>(ar), ld_quad<TI>(ar + 16));
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const TI* br = &sm.h[(16 * ct + c16) * LDQ + 32 * s + 4 * g4];
        S::mma(acc[ct], fa, S::frag_from_quads(ld_quad<TI>(br), ld_quad<TI>(br + 16)));
      }
    }
    float eg[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) eg[r] = expf(sm.gam[16 * wave + 4 * g4 + r]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[ct][r] *= eg[r];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (32 * s <= 16 * wave + 15) {
        const frag fa = S::frag_from_f32(pt[2 * s], pt[2 * s + 1]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const TI* br = &sm.vt[(16 * ct + c16) * LDT + 32 * s + 4 * g4];
          S::mma(acc[ct], fa, S::frag_from_quads(ld_quad<TI>(br), ld_quad<TI>(br + 16)));
        }
      }
    }

    // ---- store ----
    TI* __restrict__ op = static_cast<TI*>(a.o);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int j = col0 + 16 * ct + c16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = 16 * wave + 4 * g4 + r;
        if (tt < nvalid) {
          const int64_t off = ((tok0 + tt) * H + hd) * DV + j;
          const float val = a.scale * acc[ct][r];
          if constexpr (sizeof(TI) == 2) {
            reinterpret_cast<uint16_t*>(op)[off] = f32_to_bf16(val);
          } else {
            reinterpret_cast<float*>(op)[off] = val;
          }
        }
      }
    }
  }
};

template <typename TI, int DK, int DV>
__global__ __launch_bounds__(256) void output_kernel(const ChunkArgs a) {
  using K = OutputKernel<TI, DK, DV>;
  __shared__ __align__(16) typename K::Smem sm;
  K::run(a, sm);
}

template <typename TI, int DK, int DV>
static hipError_t launch_output(const void* args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((output_kernel<TI, DK, DV>), dim3(grid), dim3(256), 0, stream,
                     *static_cast<const ChunkArgs*>(args));
  return hipGetLastError();
}

LaunchFn find_output(int dtype, int dk, int dv) {
  // bfloat16 storage: the gfx950 kernel of output2.hip up to 128 x 128; this
  // generic kernel when DK or DV is 256
  if (dtype == 1 && dk <= 128 && dv <= 128) return find_output2(dk, dv);
#define GDR_OUT_CASE(T, DT, DK, DV) \
  if (dtype == DT && dk == DK && dv == DV) return &launch_output<T, DK, DV>;
  GDR_OUT_CASE(bf16_t, 1, 256, 256)
  GDR_OUT_CASE(bf16_t, 1, 256, 128)
  GDR_OUT_CASE(bf16_t, 1, 128, 256)
  GDR_OUT_CASE(bf16_t, 1, 128, 128)
  GDR_OUT_CASE(bf16_t, 1, 128, 64)
  GDR_OUT_CASE(bf16_t, 1, 64, 128)
  GDR_OUT_CASE(bf16_t, 1, 64, 64)
  GDR_OUT_CASE(float, 0, 128, 128)
  GDR_OUT_CASE(float, 0, 128, 64)
  GDR_OUT_CASE(float, 0, 64, 128)
  GDR_OUT_CASE(float, 0, 64, 64)
#undef GDR_OUT_CASE
  return nullptr;
}

}  // namespace gdr
