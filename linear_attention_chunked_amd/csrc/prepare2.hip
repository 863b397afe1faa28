// Chunk preparation for bfloat16 storage on gfx950 (float32 storage keeps
// prepare.hip): the WY factors of wy_core.hpp,
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
//   * Gram matrix, T by 16-row blocks and the hi + lo products: wy_core.hpp.
//   * Every load of the item (K, V, g, beta) issues at entry, after one round
//     of loads that finds the item's row (row_of_chunk); V waits in registers
//     and takes the place of K in LDS once the w product has read K.  A and T
//     keep only their blocks on or below the diagonal; the footprint (29.4 KB
//     at 128 x 128) and at most 96 VGPRs let five workgroups share a CU.
#include <type_traits>

#include "gfx950.hpp"
#include "kernels.hpp"
#include "wy_core.hpp"

namespace gdr {

template <int DK, int DV>
struct Prepare2 {
  using S = St<bf16_t>;
  using frag = S::frag;
  static constexpr int NT = 256;
  // Padded row strides (bytes).  K is read by rows (Gram) and transposed
  // (w); rows 8..15 of every 16 sit KX bytes further on, so that both read
  // patterns are free of LDS bank conflicts (64 banks of 4 bytes); V is only
  // read transposed.
  static constexpr int SKB = DK * 2 + 32;
  static constexpr int SVB = DV * 2 + 32;
  static constexpr int KX = 16;
  static constexpr int SKV = SKB > SVB ? SKB : SVB;
  static constexpr int KS = DK / 32;
  using W = WyCore<DK>;
  static constexpr int kTri = W::kTri;      // floats of the lower block triangle

  // A and T share one FP32 scratch (wy_core.hpp); V takes the place of K
  // once the w product has read K.  29.4 KB at 128 x 128: five workgroups
  // share a CU.
  struct Smem {
    char kv[kChunk * SKV];
    float t[kTri];
    float gam[kChunk];
    float beta[kChunk];
    float bg[kChunk];  // beta exp(gamma)
  };

  // K and V rows, g and beta are loaded at entry, all in one round: K, g and
  // beta pass through registers to LDS at once, V waits in registers until
  // the w product has read K.
  static constexpr int KV_PT = kChunk * (DK / 8) / NT;  // 16-byte K vectors per thread
  static constexpr int VV_PT = kChunk * (DV / 8) / NT;
  struct Pref {
    u32x4_t k[KV_PT];
    u32x4_t v[VV_PT];
    float g, b;
  };

  struct Item {
    int hd;
    int64_t tok0;
    int nvalid;
  };

  __device__ static Item item_of(const ChunkArgs& a, int item) {
    const int chunk = item / a.H;
    const Row row = row_of_chunk(a.rows, a.n_rows, chunk);
    const int cl = chunk - row.chunk_off;
    return Item{item % a.H, static_cast<int64_t>(row.bos) + static_cast<int64_t>(cl) * kChunk,
                min(kChunk, row.len - cl * kChunk)};
  }

  __device__ static void load(Pref& pf, const ChunkArgs& a, const Item& it) {
    const int tid = threadIdx.x;
    const int64_t H = a.H;
    const uint32_t rows = static_cast<uint32_t>((it.nvalid - 1) * H + 1);
    // every wave loads g and beta (only the first uses them): loads taken
    // under that wave's branch would issue after K has arrived
    const float* gp = a.g + it.tok0 * H + it.hd;
    const float* bp = a.beta + it.tok0 * H + it.hd;
    const int go = static_cast<int>((tid & 63) * H * 4);
    pf.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(gp, rows * 4), go, 0, 0));
    pf.b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(bp, rows * 4), go, 0, 0));
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + (it.tok0 * H + it.hd) * DK;
    const rsrc_t rk = make_rsrc(kp, rows * DK * 2);
    constexpr int CK = DK / 8;  // 16-byte chunks per row
#pragma unroll
    for (int i = 0; i < KV_PT; ++i) {
      const int vv = tid + i * NT, r = vv / CK, c = vv % CK;
      pf.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, static_cast<int>(r * H * DK * 2 + c * 16), 0, 0);
    }
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + (it.tok0 * H + it.hd) * DV;
    const rsrc_t rv = make_rsrc(vp, rows * DV * 2);
    constexpr int CV = DV / 8;
#pragma unroll
    for (int i = 0; i < VV_PT; ++i) {
      const int vv = tid + i * NT, r = vv / CV, c = vv % CV;
      pf.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, static_cast<int>(r * H * DV * 2 + c * 16), 0, 0);
    }
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
        *reinterpret_cast<u32x4_t*>(sm.kv + r * SKB + KX * ((r >> 3) & 1) + c * 16) = pf.k[i];
      }
      asm volatile("" ::"v"(pf.g), "v"(pf.b));  // g and beta arrive with K, not after it
      if (wave == 0) {
        const float x = W::gamma_beta(pf.g, pf.b, nvalid, sm.gam, sm.beta, sm.bg);
        if (lane < nvalid) a.g_cum[(tok0 + lane) * H + hd] = x;
      }
    }
    __syncthreads();

    // ---- Gram matrix and the diagonal blocks of T ----
    W::gram_diag(sm.kv, SKB, KX, sm.t, sm.gam, sm.beta);
    __syncthreads();
    W::off_diag(sm.t);

    // ---- w^T = K^T T'^T and u^T = V^T T''^T by 16-token row blocks rb ----
    // Row blocks 2 and 3 contract over twice the tokens of blocks 0 and 1 (T
    // is lower triangular), so waves 2 and 3 form all but the last D / 64
    // column tiles of their own block and waves 0 and 1 form those tiles
    // after their own blocks: twelve tile-steps per wave at D = 128 instead
    // of 8, 8, 16, 16.  Each element is the same products either way.
    auto store_to = [&](void* out, int D, int rb) {
      uint16_t* op = static_cast<uint16_t*>(out) + (tok0 * H + hd) * D;
      const rsrc_t ro = make_rsrc(op, static_cast<uint32_t>(((nvalid - 1) * H + 1) * D * 2));
      const int base = static_cast<int>((16 * rb + c16) * H * D * 2 + 4 * g4 * 2);
      return [=](int dt, const f32x4_t& acc) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])}, ro,
                                              base + 32 * dt, 0, 0);
      };
    };
    auto product = [&](const float* coef, const char* tile, int stride, int kx, void* out, auto dcols) {
      constexpr int D = decltype(dcols)::value;
      constexpr int NT16 = D / 16, XT = D / 64;  // column tiles; tiles moved to waves 0 and 1
      frag hi[2], lo[2];
      W::row_frags(sm.t, coef, hi, lo);
      if (wave >= 2) {
        auto o = store_to(out, D, wave);
        W::template product_tiles<2, 0, NT16 - XT>(tile, stride, kx, hi, lo, o);
      } else {
        auto o = store_to(out, D, wave);
        W::template product_tiles<1, 0, NT16>(tile, stride, kx, hi, lo, o);
        W::row_frags_of(wave + 2, sm.t, coef, hi, lo);
        auto o2 = store_to(out, D, wave + 2);
        W::template product_tiles<2, NT16 - XT, NT16>(tile, stride, kx, hi, lo, o2);
      }
    };
    product(sm.bg, sm.kv, SKB, KX, a.w, std::integral_constant<int, DK>{});  // T diag(beta e^gamma) K
    __syncthreads();  // every wave is done with K: V replaces it
#pragma unroll
    for (int i = 0; i < VV_PT; ++i) {
      const int vv = tid + i * NT, r = vv / CV, c = vv % CV;
      *reinterpret_cast<u32x4_t*>(sm.kv + r * SVB + c * 16) = pf.v[i];
    }
    __syncthreads();
    product(sm.beta, sm.kv, SVB, 0, a.u, std::integral_constant<int, DV>{});  // T diag(beta) V
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
