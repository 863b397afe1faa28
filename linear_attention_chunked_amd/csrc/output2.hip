// Chunk output for bfloat16 storage on gfx950 (float32 storage keeps
// output.hip).  For token t of a chunk (gamma = chunk-local cumulative g):
//
//   o_t = scale * ( e^{gamma_t} q_t^T S_c + sum_{i <= t} e^{gamma_t - gamma_i} (q_t . k_i) v_new_i )
//
// One workgroup (4 waves) per (chunk, head, 64 value columns); wave w owns the
// rows of token tile w.  Q, K, v_new and the pre-chunk state land in LDS
// row-major through range-checked buffer loads (tail rows read as zero).
// P^T = K Q^T is formed in accumulator layout, which (with the k(g, e) map of
// common.hpp) is already the A operand of P v_new; v_new's operand, whose
// contraction runs over tokens, comes from ds_read_b64_tr_b16.
#include "gfx950.hpp"
#include "kernels.hpp"

namespace gdr {

template <int DK, int DV>
struct Output2 {
  using S = St<bf16_t>;
  using frag = S::frag;
  static constexpr int NT = 256;
  static constexpr int BVO = 64;
  static constexpr int NCT = BVO / 16;
  static constexpr int SQ = DK * 2 + 16;   // Q, K, h rows (bytes): 16 consecutive rows hit distinct banks
  static constexpr int SV = BVO * 2 + 32;  // v_new rows (transpose reads)
  static constexpr int KS = DK / 32;

  struct Smem {
    char q[kChunk * SQ];
    char k[kChunk * SQ];
    char h[BVO * SQ];
    char v[kChunk * SV];
    float gam[kChunk];
  };

  __device__ static int find_row(const ChunkArgs& a, int chunk) {
    int lo = 0, hi = a.n_rows - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.rows[mid].chunk_off <= chunk) lo = mid; else hi = mid - 1;
    }
    return lo;
  }

  // The next item's tiles travel in registers while the current one computes.
  static constexpr int CQ = DK / 8, CV = BVO / 8;        // 16-byte vectors per row
  static constexpr int Q_PT = kChunk * CQ / NT;          // per thread: q, k and h rows
  static constexpr int V_PT = kChunk * CV / NT;
  struct Pref {
    u32x4_t q[Q_PT], k[Q_PT], h[Q_PT], v[V_PT];
    float g;
  };

  struct Item {
    int hd, col0, chunk;
    int64_t tok0;
    int nvalid;
  };

  __device__ static Item item_of(const ChunkArgs& a, int item) {
    constexpr int NVB = DV / BVO;
    const int vb = item % NVB;
    const int rest = item / NVB;
    const int chunk = rest / a.H;
    const Row row = a.rows[find_row(a, chunk)];
    const int cl = chunk - row.chunk_off;
    return Item{rest % a.H, vb * BVO, chunk, static_cast<int64_t>(row.bos) + static_cast<int64_t>(cl) * kChunk,
                min(kChunk, row.len - cl * kChunk)};
  }

  // Items past the end get empty buffer ranges (the loads still issue and read nothing).
  __device__ static void load(Pref& pf, const ChunkArgs& a, int item, int nitems) {
    const int tid = threadIdx.x;
    const bool live = item < nitems;
    const Item it = item_of(a, live ? item : 0);
    const int64_t H = a.H;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (it.tok0 * H + it.hd) * DK;
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + (it.tok0 * H + it.hd) * DK;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + (it.tok0 * H + it.hd) * DV + it.col0;
    const uint16_t* hp = static_cast<const uint16_t*>(a.h) +
                         ((static_cast<int64_t>(a.chunk_base) + it.chunk) * H + it.hd) * DV * DK +
                         static_cast<int64_t>(it.col0) * DK;
    const uint32_t qk_bytes = live ? static_cast<uint32_t>(((it.nvalid - 1) * H + 1) * DK * 2) : 0u;
    const rsrc_t rq = make_rsrc(qp, qk_bytes);
    const rsrc_t rk = make_rsrc(kp, qk_bytes);
    const rsrc_t rv = make_rsrc(vp, live ? static_cast<uint32_t>(((it.nvalid - 1) * H * DV + BVO) * 2) : 0u);
    const rsrc_t rh = make_rsrc(hp, live ? static_cast<uint32_t>(BVO * DK * 2) : 0u);
#pragma unroll
    for (int i = 0; i < Q_PT; ++i) {
      const int vv = tid + i * NT, r = vv / CQ, c = vv % CQ;
      const int go = static_cast<int>(r * H * DK * 2 + c * 16);
      pf.q[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, go, 0, 0);
      pf.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, go, 0, 0);
      pf.h[i] = __builtin_amdgcn_raw_buffer_load_b128(rh, static_cast<int>(r * DK * 2 + c * 16), 0, 0);
    }
#pragma unroll
    for (int i = 0; i < V_PT; ++i) {
      const int vv = tid + i * NT, r = vv / CV, c = vv % CV;
      pf.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, static_cast<int>(r * H * DV * 2 + c * 16), 0, 0);
    }
    const float* gp = a.g + it.tok0 * H + it.hd;
    pf.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
        make_rsrc(gp, live ? static_cast<uint32_t>(((it.nvalid - 1) * H + 1) * 4) : 0u),
        static_cast<int>((tid & 63) * H * 4), 0, 0));
  }

  // Persistent: workgroup b takes items b, b + gridDim.x, ... (item = (chunk * H + head) * (DV / 64) + block).
  __device__ static void run(const ChunkArgs& a, Smem& sm) {
    const int nitems = a.n_chunks * a.H * (DV / BVO);
    int item = blockIdx.x;
    if (item >= nitems) return;
    Pref pf;
    load(pf, a, item, nitems);
    for (; item < nitems; item += gridDim.x) {
      one(a, sm, pf, item, nitems);
      __syncthreads();  // LDS is reused by the next item
    }
  }

  __device__ static __forceinline__ void one(const ChunkArgs& a, Smem& sm, Pref& pf, int item, int nitems) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Item it = item_of(a, item);
    const int hd = it.hd;
    const int64_t tok0 = it.tok0;
    const int nvalid = it.nvalid;
    const int64_t H = a.H;
    const int col0 = it.col0;
#pragma unroll
    for (int i = 0; i < Q_PT; ++i) {
      const int vv = tid + i * NT, r = vv / CQ, c = vv % CQ;
      *reinterpret_cast<u32x4_t*>(sm.q + r * SQ + c * 16) = pf.q[i];
      *reinterpret_cast<u32x4_t*>(sm.k + r * SQ + c * 16) = pf.k[i];
      *reinterpret_cast<u32x4_t*>(sm.h + r * SQ + c * 16) = pf.h[i];
    }
#pragma unroll
    for (int i = 0; i < V_PT; ++i) {
      const int vv = tid + i * NT, r = vv / CV, c = vv % CV;
      *reinterpret_cast<u32x4_t*>(sm.v + r * SV + c * 16) = pf.v[i];
    }
    if (tid < kChunk) sm.gam[tid] = (tid < nvalid) ? pf.g : 0.f;
    load(pf, a, item + gridDim.x, nitems);
    __syncthreads();

    const char* rowq = sm.q + c16 * SQ + (g4 >> 1) * 16 + (g4 & 1) * 8;  // + 16 tile SQ + 64 s (+32)
    const char* rowk = sm.k + c16 * SQ + (g4 >> 1) * 16 + (g4 & 1) * 8;
    const char* rowh = sm.h + c16 * SQ + (g4 >> 1) * 16 + (g4 & 1) * 8;
    auto rfrag = [&](const char* base, int tile, int s) {
      return S::frag_from_quads(*reinterpret_cast<const u32x2_t*>(base + 16 * tile * SQ + 64 * s),
                                *reinterpret_cast<const u32x2_t*>(base + 16 * tile * SQ + 64 * s + 32));
    };

    // ---- P^T[i][t] = k_i . q_t for t in tile `wave`, i tiles 0..wave; O = Q S_c ----
    f32x4_t pt[4], acc[NCT];
#pragma unroll
    for (int it = 0; it < 4; ++it) pt[it] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const frag fq = rfrag(rowq, wave, s);
#pragma unroll
      for (int it = 0; it < 4; ++it)
        if (it <= wave) S::mma(pt[it], rfrag(rowk, it, s), fq);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) S::mma(acc[ct], fq, rfrag(rowh, ct, s));
    }
    const int t = 16 * wave + c16;
    const float gt = sm.gam[t];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const f32x4_t gi = *reinterpret_cast<const f32x4_t*>(&sm.gam[16 * it + 4 * g4]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * it + 4 * g4 + r;
        pt[it][r] = (i <= t && t < nvalid) ? pt[it][r] * exp_fast(gt - gi[r]) : 0.f;
      }
    }
    const f32x4_t gr = *reinterpret_cast<const f32x4_t*>(&sm.gam[16 * wave + 4 * g4]);
    f32x4_t eg;
#pragma unroll
    for (int r = 0; r < 4; ++r) eg[r] = exp_fast(gr[r]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] *= eg;

    // ---- O += P v_new (B operand from transpose reads of the row-major v_new tile) ----
    const char* vb_ = sm.v + (4 * g4 + (c16 >> 2)) * SV + 8 * (c16 & 3);  // + 32 s SV (+16 SV) + 32 ct
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (32 * s <= 16 * wave + 15) {
        const frag fa = S::frag_from_f32(pt[2 * s], pt[2 * s + 1]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          S::mma(acc[ct], fa, S::frag_from_quads(lds_tr16(vb_, 32 * s * SV + 32 * ct), lds_tr16(vb_, (32 * s + 16) * SV + 32 * ct)));
      }
    }

    // ---- store o (rows past the tail dropped by the range check) ----
    uint16_t* op = static_cast<uint16_t*>(a.o) + (tok0 * H + hd) * DV + col0;
    const rsrc_t ro = make_rsrc(op, static_cast<uint32_t>(((nvalid - 1) * H * DV + BVO) * 2));
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
