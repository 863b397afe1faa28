// Segment composition in FP32 (cuLA pull request #127, "Root cause and
// implementation": the transition is kept canonically in FP32 and segments
// are composed one after another):
//
//   S_init(0) = h0 (or 0),   S_init(s+1) = M_s S_init(s) + S_loc(s)
//
// One workgroup per (sequence, head, 16 value columns) with one wave per 16
// rows of the state (DK/16 waves).  Wave w keeps its rows of the running
// state in FP32 accumulator registers and produces its rows of the next one
// with FP32 MFMA (v_mfma_f32_16x16x4_f32, 2 DK/32 independent accumulator
// chains of four products, summed by a pairwise tree): the A operand is its
// 16 rows of M_s, the B operand the whole current state, shared through LDS
// (double-buffered, one barrier per segment).
//
// What bounds the chain is moving M_s (DK x DK FP32 per segment) into every
// workgroup.  An A fragment gives each of 16 lanes a different row, so
// reading it straight from global memory touches 16 rows per instruction;
// instead each wave reads its 16 rows as one contiguous block (every load
// instruction covers whole consecutive 16-byte pieces), stages them in its
// own LDS region with rows padded by 16 bytes (the fragment reads of 16 rows
// at one column then fall in distinct banks), and reads the fragments from
// there.  The wave's region is private, so staging needs no barrier.
// Pipeline per segment s: the loads of M_{s+2} are issued, the fragments of
// M_s are read from LDS buffer s & 1, the products run, M_{s+1} (loaded one
// segment earlier) is staged into buffer (s+1) & 1, and the state is
// exchanged.  All global accesses go through buffer resources built per
// segment in scalar registers with per-lane offsets fixed for the whole
// chain.  With 16 segments (the split of the long-sequence workloads) the
// chain is straight-line code, so every wait count is exact; other counts
// run the same steps in a loop.  The workgroups of one (sequence, head)
// share an XCD (blockIdx modulo 8), so M_s and S_loc(s) come from HBM once
// per XCD and from that XCD's L2 for the other column blocks.
#include "gfx950.hpp"
#include "kernels.hpp"

namespace gdr {

template <int DK, int PFIX>
struct ComposeKernel {
  using S = St<float>;
  using frag = S::frag;
  static constexpr int BVC = 16;
  static constexpr int NW = DK / 16;
  static constexpr int KS = DK / 32;
  static constexpr int LDS_ = DK + 4;          // state exchange: one value column per row
  static constexpr int LDM = DK + 4;           // staged M rows (floats), padded by 16 bytes
  static constexpr int MPW = 16 * DK / 4 / 64; // 16-byte pieces of the wave's 16 rows per lane
  static constexpr int QPR = DK / 4;           // 16-byte pieces per row

  struct Smem {
    float s[2][BVC * LDS_];
    float m[2][NW][16 * LDM];
  };

  struct Ops {
    u32x4_t m[MPW];  // this lane's pieces of the wave's 16 rows of M_s (piece i*64 + lane)
    f32x4_t l;       // this lane's four rows of S_loc(s) in its column
  };

  struct Ctx {
    const ComposeArgs* a;
    int64_t n, hd, H;
    int col, row0, wave, g4, c16, lane;
    int vo_s;   // byte offset of this lane's four state rows within a segment-head block
  };

  __device__ static __forceinline__ void load(Ops& o, const Ctx& x, int s) {
    const ComposeArgs& a = *x.a;
    const int64_t seg = x.n * a.P + s;
    // the wave's 16 rows: one contiguous 16 * DK * 4-byte block
    const rsrc_t rm = make_rsrc(a.seg_trans + ((seg * x.H + x.hd) * DK + 16 * x.wave) * DK, 16 * DK * 4);
#pragma unroll
    for (int i = 0; i < MPW; ++i) o.m[i] = __builtin_amdgcn_raw_buffer_load_b128(rm, 16 * x.lane, 1024 * i, 0);
    const rsrc_t rs = make_rsrc(a.seg_state + (seg * x.H + x.hd) * a.DV * DK, static_cast<uint32_t>(a.DV * DK * 4));
    o.l = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, x.vo_s, 0, 0));
  }

  // M pieces -> the wave's LDS region (row-major, padded rows)
  __device__ static __forceinline__ void stage(const Ops& o, const Ctx& x, Smem& sm, int buf) {
    float* mb = sm.m[buf][x.wave];
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
      const int p = 64 * i + x.lane;
      *reinterpret_cast<u32x4_t*>(mb + (p / QPR) * LDM + 4 * (p % QPR)) = o.m[i];
    }
  }

  // Segment s: M_s fragments from LDS buffer s & 1, S_loc(s) from `ops`;
  // requests segment s+2 into `next2`, stages segment s+1 from `next1`.
  __device__ static __forceinline__ void step(f32x4_t& cur, const Ops& ops, const Ops& next1, Ops& next2,
                                              const Ctx& x, int s, Smem& sm) {
    const ComposeArgs& a = *x.a;
    // unconditional (the last segment is re-read near the end), so every step
    // issues the same loads and the compiler's wait counts stay two steps deep
    load(next2, x, min(s + 2, a.P - 1));
    const int64_t seg = x.n * a.P + s;
    const rsrc_t ri = make_rsrc(a.seg_init + (seg * x.H + x.hd) * a.DV * DK, static_cast<uint32_t>(a.DV * DK * 4));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, cur), ri, x.vo_s, 0, 0);
    const float* sb = &sm.s[s & 1][x.c16 * LDS_ + 4 * x.g4];
    const float* mb = &sm.m[s & 1][x.wave][x.c16 * LDM + 4 * x.g4];
    frag bs[KS], am[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      am[ks] = S::frag_from_f32(*reinterpret_cast<const f32x4_t*>(mb + 32 * ks),
                                *reinterpret_cast<const f32x4_t*>(mb + 32 * ks + 16));
      bs[ks] = S::frag_from_f32(*reinterpret_cast<const f32x4_t*>(sb + 32 * ks),
                                *reinterpret_cast<const f32x4_t*>(sb + 32 * ks + 16));
    }
    f32x4_t part[2 * KS];
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) part[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          part[2 * ks + h] =
              __builtin_amdgcn_mfma_f32_16x16x4f32(am[ks].v[4 * h + e], bs[ks].v[4 * h + e], part[2 * ks + h], 0, 0, 0);
#pragma unroll
    for (int w = 1; w < 2 * KS; w *= 2)  // pairwise tree over the chains
#pragma unroll
      for (int i = 0; i < 2 * KS; i += 2 * w) part[i] += part[i + w];
    cur = ops.l + part[0];
    if (s + 1 < (PFIX > 0 ? PFIX : a.P)) stage(next1, x, sm, (s + 1) & 1);
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
    x.lane = lane;
    x.g4 = lane >> 4;
    x.c16 = lane & 15;
    x.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    x.col = vb * BVC + x.c16;           // this lane's value column
    x.row0 = 16 * x.wave + 4 * x.g4;    // this lane's four state rows
    x.vo_s = (x.col * DK + x.row0) * 4;
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
    if (P > 0) {
      if constexpr (PFIX > 0) {
        Ops o[3];
        load(o[0], x, 0);
        load(o[1], x, min(1, PFIX - 1));
        stage(o[0], x, sm, 0);
        __syncthreads();
#pragma unroll
        for (int s = 0; s < PFIX; ++s) step(cur, o[s % 3], o[(s + 1) % 3], o[(s + 2) % 3], x, s, sm);
      } else {
        Ops A, B, C;
        load(A, x, 0);
        load(B, x, min(1, P - 1));
        stage(A, x, sm, 0);
        __syncthreads();
        for (int s = 0; s < P; s += 3) {
          step(cur, A, B, C, x, s, sm);
          if (s + 1 >= P) break;
          step(cur, B, C, A, x, s + 1, sm);
          if (s + 2 >= P) break;
          step(cur, C, A, B, x, s + 2, sm);
        }
      }
    } else {
      __syncthreads();
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

template <int DK, int PFIX>
__global__ __launch_bounds__(DK * 4) void compose_kernel(const ComposeArgs a) {
  using K = ComposeKernel<DK, PFIX>;
  __shared__ __align__(16) typename K::Smem sm;
  K::run(a, sm);
}

template <int DK, int PFIX>
static hipError_t launch_compose(const void* args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((compose_kernel<DK, PFIX>), dim3(grid), dim3(DK * 4), 0, stream,
                     *static_cast<const ComposeArgs*>(args));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Pairwise combination of half-segment summaries (the same composition rule
// applied to the two halves of one segment, all segments in parallel):
//   S = M_b S_a + S_b,   M = M_b M_a
// The split into halves runs for bfloat16 storage only, and there the
// products run as three bf16 matrix-core products per FP32 product:
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi) (16 bits of the 24-bit
// mantissa), and M_b X ~ lo(M_b) hi(X) + hi(M_b) lo(X) + hi(M_b) hi(X)
// (the lo x lo term, below 2^-16 of the product, dropped), accumulated in
// FP32 on v_mfma_f32_16x16x32_bf16: about 1e-5 relative to each product,
// far below the bfloat16 rounding of every stored state.  One workgroup per
// (segment, head, 64 of the DV + DK output columns), one wave per 16 rows.
// The 64 columns of [S_a | M_a] are split once and staged in LDS as bf16
// hi and lo tiles, S_a value-major as stored (one column per padded row), M_a
// row-major as stored (one matrix row per padded row, read through
// ds_read_b64_tr_b16); each wave splits its 16 rows of M_b in registers and
// runs the four 16-column tiles.  Lane group g of a fragment holds the
// contraction indices 32 s + 4 g + e and 32 s + 16 + 4 g + e (e < 4) in both
// operands.
template <int DK>
struct Combine {
  using S = St<bf16_t>;
  using frag = S::frag;
  static constexpr int NW = DK / 16;
  static constexpr int KS = DK / 32;
  static constexpr int CW = 64;          // output columns per workgroup
  static constexpr int LDC = DK * 2 + 16;  // state tile: one column per row (bytes), padded
  static constexpr int LDR = CW * 2 + 32;  // transition tile: one matrix row per row (bytes), padded
  static constexpr int TB = (CW * LDC > DK * LDR ? CW * LDC : DK * LDR);  // bytes of one tile
  static constexpr int SMEM = 2 * TB;      // hi, lo

  __device__ static __forceinline__ void split(float x, uint16_t& h, uint16_t& l) {
    h = f32_to_bf16(x);
    l = f32_to_bf16(x - bf16_to_f32(h));
  }

  __device__ static void run(const CombineArgs& a, char* sm) {
    const int NB = (a.DV + DK) / CW;
    const int bx = blockIdx.x;
    const int xcd = bx & 7, slot = bx >> 3;
    const int pair = 8 * (slot / NB) + xcd;  // the column blocks of one (segment, head) share an XCD
    const int cb = slot % NB;
    if (pair >= a.n_seg * a.H) return;
    const int64_t seg = pair / a.H, hd = pair % a.H, H = a.H;
    const int tid = threadIdx.x, lane = tid & 63, c16 = lane & 15, g4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int DV = a.DV;
    const bool state = CW * cb < DV;
    const int col0 = state ? CW * cb : CW * cb - DV;  // first column of the block within S or M
    char* thi = sm;
    char* tlo = sm + TB;
    // stage the 64 columns of [S_a | M_a] as bf16 hi / lo (16-byte loads, coalesced)
    if (state) {
      const float* src = a.half_state + ((2 * seg) * H + hd) * DV * DK + static_cast<int64_t>(col0) * DK;
      for (int v = tid; v < CW * DK / 4; v += NW * 64) {
        const int c = v / (DK / 4), k4 = v % (DK / 4);
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(src + 4 * v);
        uint16_t h[4], l[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split(x[i], h[i], l[i]);
        *reinterpret_cast<u32x2_t*>(thi + c * LDC + 8 * k4) =
            u32x2_t{h[0] | (static_cast<uint32_t>(h[1]) << 16), h[2] | (static_cast<uint32_t>(h[3]) << 16)};
        *reinterpret_cast<u32x2_t*>(tlo + c * LDC + 8 * k4) =
            u32x2_t{l[0] | (static_cast<uint32_t>(l[1]) << 16), l[2] | (static_cast<uint32_t>(l[3]) << 16)};
      }
    } else {
      const float* src = a.half_trans + ((2 * seg) * H + hd) * DK * DK + col0;
      for (int v = tid; v < DK * CW / 4; v += NW * 64) {
        const int r = v / (CW / 4), c4 = v % (CW / 4);
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(src + static_cast<int64_t>(r) * DK + 4 * c4);
        uint16_t h[4], l[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split(x[i], h[i], l[i]);
        *reinterpret_cast<u32x2_t*>(thi + r * LDR + 8 * c4) =
            u32x2_t{h[0] | (static_cast<uint32_t>(h[1]) << 16), h[2] | (static_cast<uint32_t>(h[3]) << 16)};
        *reinterpret_cast<u32x2_t*>(tlo + r * LDR + 8 * c4) =
            u32x2_t{l[0] | (static_cast<uint32_t>(l[1]) << 16), l[2] | (static_cast<uint32_t>(l[3]) << 16)};
      }
    }
    // this wave's 16 rows of M_b (A operand), split in registers
    const float* arow = a.half_trans + ((2 * seg + 1) * H + hd) * DK * DK +
                        static_cast<int64_t>(16 * wave + c16) * DK + 4 * g4;
    frag ah[KS], al[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(arow + 32 * s);
      const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(arow + 32 * s + 16);
      ah[s] = S::frag_from_f32(x0, x1);
      f32x4_t l0, l1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        l0[r] = x0[r] - bf16_to_f32(f32_to_bf16(x0[r]));
        l1[r] = x1[r] - bf16_to_f32(f32_to_bf16(x1[r]));
      }
      al[s] = S::frag_from_f32(l0, l1);
    }
    __syncthreads();
    const int row0 = 16 * wave + 4 * g4;  // this lane's four output rows
    // B fragments of column tile ct, contraction step s
    auto bfrag = [&](const char* t, int ct, int s) {
      if (state) {
        const char* cp = t + (16 * ct + c16) * LDC + 2 * (32 * s + 4 * g4);
        return S::frag_from_quads(lds_b64(cp, 0), lds_b64(cp, 32));
      }
      const char* tb = t + (4 * g4 + (c16 >> 2)) * LDR + 8 * (c16 & 3) + 32 * ct;
      return S::frag_from_quads(lds_tr16(tb, 32 * s * LDR), lds_tr16(tb, (32 * s + 16) * LDR));
    };
#pragma unroll 1
    for (int ct = 0; ct < CW / 16; ++ct) {
      const int c = 16 * ct + c16;  // column within the block
      f32x4_t acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const frag bh = bfrag(thi, ct, s), bl = bfrag(tlo, ct, s);
        S::mma(acc, al[s], bh);
        S::mma(acc, ah[s], bl);
        S::mma(acc, ah[s], bh);
      }
      if (state) {
        const int64_t off = (seg * H + hd) * DV * DK + static_cast<int64_t>(col0 + c) * DK + row0;
        const f32x4_t sb = *reinterpret_cast<const f32x4_t*>(a.half_state + ((2 * seg + 1) * H + hd) * DV * DK +
                                                             static_cast<int64_t>(col0 + c) * DK + row0);
        *reinterpret_cast<f32x4_t*>(a.seg_state + off) = acc + sb;
      } else {
        float* mo = a.seg_trans + (seg * H + hd) * DK * DK + static_cast<int64_t>(row0) * DK + col0 + c;
#pragma unroll
        for (int j = 0; j < 4; ++j) mo[static_cast<int64_t>(j) * DK] = acc[j];
      }
    }
  }
};

template <int DK>
__global__ __launch_bounds__(DK * 4) void combine_kernel(const CombineArgs a) {
  __shared__ __align__(16) char sm[Combine<DK>::SMEM];
  Combine<DK>::run(a, sm);
}

template <int DK>
static hipError_t launch_combine(const void* args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((combine_kernel<DK>), dim3(grid), dim3(DK * 4), 0, stream,
                     *static_cast<const CombineArgs*>(args));
  return hipGetLastError();
}

LaunchFn find_combine(int dk) { return dk == 128 ? &launch_combine<128> : nullptr; }

// 16 segments (the split the long-sequence workloads use) get the
// straight-line chain; other counts take the loop.
LaunchFn find_compose(int dk, int P) {
  if (dk == 128) return P == 16 ? &launch_compose<128, 16> : &launch_compose<128, 0>;
  if (dk == 64) return P == 16 ? &launch_compose<64, 16> : &launch_compose<64, 0>;
  return nullptr;
}

}  // namespace gdr
