// Chunk output for bfloat16 storage on gfx950 (float32 storage keeps
// output.hip).  For token t of a chunk (gamma = chunk-local cumulative g):
//
//   o_t = scale * ( e^{gamma_t} q_t^T S_c + sum_{i <= t} e^{gamma_t - gamma_i} (q_t . k_i) v_new_i )
//
// One workgroup (4 waves) per (chunk, head) for all DV value columns; wave w
// owns the rows of token tile w.  Two LDS phases share one region (53 KB at
// 128 x 128, so three workgroups fit a CU):
//   A  Q, K and gamma land in LDS row-major through range-checked buffer loads
//      (tail rows read as zero) while the pre-chunk state and the v_new tile
//      travel in registers; P^T = K Q^T is formed in accumulator layout, which
//      (with the k(g, e) map of common.hpp) is already the A operand of
//      P v_new, and the wave's Q fragments stay in registers;
//   B  the state and v_new tiles replace Q and K; O = e^{gamma} (Q S_c) +
//      P v_new, with v_new's operand (contraction over tokens) from
//      ds_read_b64_tr_b16.
// Q and K are read from HBM once per (chunk, head) and P^T is formed once,
// not once per block of value columns.
#include "gfx950.hpp"
#include "kernels.hpp"

namespace gdr {

template <int DK, int DV>
struct Output2 {
  using S = St<bf16_t>;
  using frag = S::frag;
  static constexpr int NT = 256;
  static constexpr int NCT = DV / 16;
  static constexpr int SQ = DK * 2 + 16;   // Q, K, h rows (bytes): 16 consecutive rows hit distinct banks
  static constexpr int SV = DV * 2 + 32;   // v_new rows (transpose reads)
  static constexpr int KS = DK / 32;

  struct PhaseA {
    char q[kChunk * SQ];
    char k[kChunk * SQ];
    float gam[kChunk];
  };
  struct PhaseB {
    char h[DV * SQ];
    char v[kChunk * SV];
  };
  union Smem {
    PhaseA A;
    PhaseB B;
  };

  static constexpr int CQ = DK / 8, CV = DV / 8;  // 16-byte vectors per row
  static constexpr int QPT = kChunk * CQ / NT, HPT = DV * CQ / NT, VPT = kChunk * CV / NT;

  __device__ static void run(const ChunkArgs& a, Smem& sm) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int item = blockIdx.x;  // chunk * H + head
    const int chunk = item / a.H;
    const int hd = item % a.H;
    if (chunk >= a.n_chunks) return;
    const Row row = row_of_chunk(a.rows, a.n_rows, chunk);
    const int cl = chunk - row.chunk_off;
    const int64_t tok0 = static_cast<int64_t>(row.bos) + static_cast<int64_t>(cl) * kChunk;
    const int nvalid = min(kChunk, row.len - cl * kChunk);
    const int64_t H = a.H;

    // ---- Q, K, gamma into LDS; S_c and v_new into registers ----
    u32x4_t hreg[HPT], vreg[VPT];
    {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (tok0 * H + hd) * DK;
      const uint16_t* kp = static_cast<const uint16_t*>(a.k) + (tok0 * H + hd) * DK;
      const uint16_t* vp = static_cast<const uint16_t*>(a.v) + (tok0 * H + hd) * DV;
      const uint16_t* hp =
          static_cast<const uint16_t*>(a.h) + ((static_cast<int64_t>(a.chunk_base) + chunk) * H + hd) * DV * DK;
      const uint32_t qk_bytes = static_cast<uint32_t>(((nvalid - 1) * H + 1) * DK * 2);
      const rsrc_t rq = make_rsrc(qp, qk_bytes);
      const rsrc_t rk = make_rsrc(kp, qk_bytes);
      const rsrc_t rv = make_rsrc(vp, static_cast<uint32_t>(((nvalid - 1) * H + 1) * DV * 2));
      const rsrc_t rh = make_rsrc(hp, static_cast<uint32_t>(DV * DK * 2));
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
      for (int i = 0; i < QPT; ++i) {
        const int vv = tid + i * NT, r = vv / CQ, c = vv % CQ;
        const int go = static_cast<int>(r * H * DK * 2 + c * 16);
        *reinterpret_cast<u32x4_t*>(sm.A.q + r * SQ + c * 16) = __builtin_amdgcn_raw_buffer_load_b128(rq, go, 0, 0);
        *reinterpret_cast<u32x4_t*>(sm.A.k + r * SQ + c * 16) = __builtin_amdgcn_raw_buffer_load_b128(rk, go, 0, 0);
      }
      if (tid < kChunk) {
        const float* gp = a.g + tok0 * H + hd;
        const float g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
            make_rsrc(gp, static_cast<uint32_t>(((nvalid - 1) * H + 1) * 4)), static_cast<int>(tid * H * 4), 0, 0));
        sm.A.gam[tid] = (tid < nvalid) ? g : 0.f;
      }
    }
    __syncthreads();

    // row fragments in the contiguous k map (16 bytes per lane)
    const char* rowq = sm.A.q + c16 * SQ + 16 * g4;  // + 16 tile SQ + 64 s
    const char* rowk = sm.A.k + c16 * SQ + 16 * g4;
    auto rfrag = [&](const char* base, int tile, int s) { return lds_frag16(base, 16 * tile * SQ + 64 * s); };

    // ---- P^T[i][t] = k_i . q_t for t in tile `wave`, i tiles 0..wave; Q fragments kept ----
    frag fq[KS];
    f32x4_t pt[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) pt[it] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      fq[s] = rfrag(rowq, wave, s);
#pragma unroll
      for (int it = 0; it < 4; ++it)
        if (it <= wave) S::mma(pt[it], rfrag(rowk, it, s), fq[s]);
    }
    const int t = 16 * wave + c16;
    const float gt = sm.A.gam[t];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const f32x4_t gi = *reinterpret_cast<const f32x4_t*>(&sm.A.gam[16 * it + 4 * g4]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * it + 4 * g4 + r;
        pt[it][r] = (i <= t && t < nvalid) ? pt[it][r] * exp_fast(gt - gi[r]) : 0.f;
      }
    }
    const f32x4_t gr = *reinterpret_cast<const f32x4_t*>(&sm.A.gam[16 * wave + 4 * g4]);
    f32x4_t eg;
#pragma unroll
    for (int r = 0; r < 4; ++r) eg[r] = exp_fast(gr[r]);
    __syncthreads();  // Q, K, gamma are dead

    // ---- phase B: S_c and v_new into the region ----
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
    __syncthreads();

    // ---- O = e^{gamma} (Q S_c) + P v_new, rows of token tile `wave` ----
    const char* rowh = sm.B.h + c16 * SQ + 16 * g4;
    f32x4_t acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) S::mma(acc[ct], fq[s], rfrag(rowh, ct, s));
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] *= eg;
    const char* vb_ = sm.B.v + (4 * g4 + (c16 >> 2)) * SV + 8 * (c16 & 3);  // + 32 s SV (+16 SV) + 32 ct
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (32 * s <= 16 * wave + 15) {
        const frag fa = S::frag_from_f32(pt[2 * s], pt[2 * s + 1]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          S::mma(acc[ct], fa, S::frag_from_quads(lds_tr16(vb_, 32 * s * SV + 32 * ct),
                                                  lds_tr16(vb_, (32 * s + 16) * SV + 32 * ct)));
      }
    }

    // ---- store o (rows past the tail dropped by the range check) ----
    uint16_t* op = static_cast<uint16_t*>(a.o) + (tok0 * H + hd) * DV;
    const rsrc_t ro = make_rsrc(op, static_cast<uint32_t>(((nvalid - 1) * H + 1) * DV * 2));
    const int rs = static_cast<int>(H * DV * 2);
    const int voff = (16 * wave + 4 * g4) * rs + c16 * 2;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const uint32_t pk = pack_bf16x2(a.scale * acc[ct][r], a.scale * acc[ct][r + 1]);
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(pk), ro, voff, r * rs + 32 * ct, 0);
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(pk >> 16), ro, voff, (r + 1) * rs + 32 * ct, 0);
      }
  }
};

template <int DK, int DV>
__global__ __launch_bounds__(256) void output2_kernel(const ChunkArgs a) {
  using K = Output2<DK, DV>;
  __shared__ __align__(16) typename K::Smem sm;
  K::run(a, sm);
}

template <int DK, int DV>
static hipError_t launch_output2(const void* args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((output2_kernel<DK, DV>), dim3(grid), dim3(256), 0, stream, *static_cast<const ChunkArgs*>(args));
  return hipGetLastError();
}

LaunchFn find_output2(int dk, int dv) {
  if (dk == 128 && dv == 128) return &launch_output2<128, 128>;
  if (dk == 128 && dv == 64) return &launch_output2<128, 64>;
  if (dk == 64 && dv == 128) return &launch_output2<64, 128>;
  if (dk == 64 && dv == 64) return &launch_output2<64, 64>;
  return nullptr;
}

}  // namespace gdr
