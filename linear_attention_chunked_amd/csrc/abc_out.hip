// ABC read per 64-token chunk on gfx950: slot scores, softmax over the slots,
// value read (flash-linear-attention fork issue #23, "Problem": chunk_abc,
// whose forward reads the slot states the state walk builds; its default
// geometry H=4, K=256, M=64, V=512).
//
// After token t's update the states are read as
//   score_t = scale Hk_t^T q_t,   p_t = softmax over the M slots,   o_t = Hv_t^T p_t.
// Inside chunk c (tokens t0..t0+n-1, zp = zc[c-1] the normaliser before the
// chunk, zl = zc[c] at its last token, E_i = e^{s_i - zl} <= 1):
//   Hk_t = Hk[c] X1_t + sum_{i<=t} k_i (x) E_i X2_t     (per slot column)
//   X1_t = e^{zp - z_t} <= 1,  X2_t = e^{zl - z_t} >= 1
// so with A = Q K^T masked to i <= t:
//   score = scale (X1 .* (Q Hk[c]) + X2 .* (A E))
//   o     = (p .* X1) Hv[c] + mask((p .* X2) E^T) V
// One workgroup (8 waves) per (b, chunk, h).  Waves 0-3 form the scores of
// 16 tokens each (Q Hk[c] with Hk[c] through ds_read_b64_tr_b16, A^T as C
// tiles that become the operand of A E directly), take the softmax across
// the 16 lanes that hold a row, and leave P1 = p X1 and P2 = p X2 in LDS.
// All 8 waves then form o^T (value rows, token columns) for V/8 columns each,
// so every lane holds four adjacent outputs of one token: one 8-byte store.
// The value-side tiles (Hv[c], V) are requested with the score-side ones
// and held in registers until the score phase frees the LDS.
#include "gfx950.hpp"
#include "kernels.hpp"

namespace gdr {

template <int K, int V>
struct AbcOut {
  using S = St<bf16_t>;
  using frag = S::frag;
  static constexpr int NT = 512;
  static constexpr int M = 64;            // slots of the tiles (a.M = 32 is padding above it)
  static constexpr int SQ = K * 2 + 16;   // Q, K rows (row fragments)
  static constexpr int SHK = M * 2 + 32;  // Hk rows (transpose reads)
  static constexpr int SVV = V * 2 + 32;  // Hv, V rows (transpose reads)
  static constexpr int SP = M * 2 + 16;   // E, P1, P2 rows
  static constexpr int RA = 2 * kChunk * SQ + K * SHK;
  static constexpr int RB = 2 * kChunk * SVV;
  static constexpr int R = RA > RB ? RA : RB;
  static constexpr int OFF_Q = 0, OFF_K = kChunk * SQ, OFF_HK = 2 * kChunk * SQ;
  static constexpr int OFF_HV = 0, OFF_V = kChunk * SVV;
  static constexpr int OFF_E = R, OFF_P1 = R + kChunk * SP, OFF_P2 = R + 2 * kChunk * SP;
  static constexpr int SMEM = R + 3 * kChunk * SP;
  static_assert(SMEM <= 163840, "LDS");
  static constexpr int LQ = K / 64;   // 16-byte pieces per thread of Q (also K, Hk)
  static constexpr int LV = V / 64;   // ... of Hv (also V)
  static constexpr int NVT = V / 128; // 16-wide value tiles per wave in the read

  __device__ static __forceinline__ frag rfrag(const char* base, int stride, int tile, int s) {
    return S::frag_from_quads(lds_b64(base, 16 * tile * stride + 64 * s), lds_b64(base, 16 * tile * stride + 64 * s + 32));
  }
  __device__ static __forceinline__ frag tfrag(const char* base, int stride, int s, int tile) {
    return S::frag_from_quads(lds_tr16(base, 32 * s * stride + 32 * tile), lds_tr16(base, (32 * s + 16) * stride + 32 * tile));
  }

  __device__ static void run(const AbcOutArgs& a, char* sm) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bx = blockIdx.x;
    const int h = bx % a.H;
    const int c = (bx / a.H) % a.NC;
    const int b = bx / (a.H * a.NC);
    const int n = min(kChunk, a.T - c * kChunk);
    const int64_t H = a.H;
    const int64_t tok0 = static_cast<int64_t>(b) * a.T + static_cast<int64_t>(c) * kChunk;
    const int64_t plane = (static_cast<int64_t>(b) * a.NC + c) * H + h;
    const int MS = a.M;  // stored slots (32 or 64): slots past MS are padding, score -inf, p = 0

    const rsrc_t rq = make_rsrc(static_cast<const uint16_t*>(a.q) + (tok0 * H + h) * K,
                                static_cast<uint32_t>(((n - 1) * H * K + K) * 2));
    const rsrc_t rk = make_rsrc(static_cast<const uint16_t*>(a.k) + (tok0 * H + h) * K,
                                static_cast<uint32_t>(((n - 1) * H * K + K) * 2));
    const rsrc_t rhk = make_rsrc(static_cast<const uint16_t*>(a.hk) + plane * K * MS, K * MS * 2);
    const rsrc_t rs = make_rsrc(static_cast<const uint16_t*>(a.s) + (tok0 * H + h) * MS,
                                static_cast<uint32_t>(((n - 1) * H * MS + MS) * 2));
    const rsrc_t rz = make_rsrc(a.z + (tok0 * H + h) * MS, static_cast<uint32_t>(((n - 1) * H * MS + MS) * 4));
    const rsrc_t rzp = make_rsrc(a.z + (c > 0 ? ((tok0 - 1) * H + h) * MS : 0), c > 0 ? MS * 4 : 0u);
    const rsrc_t rhv = make_rsrc(static_cast<const uint16_t*>(a.hv) + plane * MS * V, MS * V * 2);
    const rsrc_t rv = make_rsrc(static_cast<const uint16_t*>(a.v) + (tok0 * H + h) * V,
                                static_cast<uint32_t>(((n - 1) * H * V + V) * 2));

    // ---- requests: score side, the score rows' normalisers, value side
    u32x4_t lq[LQ], lk[LQ], lh[LQ];
#pragma unroll
    for (int i = 0; i < LQ; ++i) {
      const int v = tid + i * NT, r = v / (K / 8), cc = v % (K / 8);
      const int go = static_cast<int>(r * H * K * 2 + cc * 16);
      lq[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, go, 0, 0);
      lk[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, go, 0, 0);
      // Hk row v >> 3, 16-byte piece v & 7 (pieces past the stored slots read as zero)
      lh[i] = 8 * (v & 7) < MS ? __builtin_amdgcn_raw_buffer_load_b128(
                                     rhk, static_cast<int>((v >> 3) * MS * 2 + (v & 7) * 16), 0, 0)
                               : u32x4_t{0u, 0u, 0u, 0u};
    }
    const int srow = tid >> 3, scv = tid & 7;
    const bool sl = 8 * scv < MS;  // this thread's eight slots are stored ones
    const u32x4_t ls = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>((srow * H * MS + 8 * scv) * 2), 0, 0);
    const int zlo = static_cast<int>(((n - 1) * H * MS) * 4);
    const f32x4_t zl0 = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rz, zlo + 32 * scv, 0, 0));
    const f32x4_t zl1 = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rz, zlo + 32 * scv + 16, 0, 0));
    // score rows of waves 0-3: z[t][m] for t = 16 wave + 4 g4 + r, m = 16 mt + c16
    const int tb = wave & 3;
    float zt[4][4], zpv[4], zlv[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int m = 16 * mt + c16;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        zt[mt][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  rz, static_cast<int>(((16 * tb + 4 * g4 + r) * H * MS + m) * 4), 0, 0));
      zpv[mt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rzp, 4 * m, 0, 0));
      zlv[mt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rz, zlo + 4 * m, 0, 0));
    }
    u32x4_t lhv[LV], lv[LV];
#pragma unroll
    for (int i = 0; i < LV; ++i) {
      const int v = tid + i * NT, r = v / (V / 8), cc = v % (V / 8);
      lhv[i] = __builtin_amdgcn_raw_buffer_load_b128(rhv, static_cast<int>(v * 16), 0, 0);
      lv[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, static_cast<int>(r * H * V * 2 + cc * 16), 0, 0);
    }

    // ---- score-side tiles to LDS; E = e^{s - zl} (zero past the chunk's end)
#pragma unroll
    for (int i = 0; i < LQ; ++i) {
      const int v = tid + i * NT, r = v / (K / 8), cc = v % (K / 8);
      *reinterpret_cast<u32x4_t*>(sm + OFF_Q + r * SQ + cc * 16) = lq[i];
      *reinterpret_cast<u32x4_t*>(sm + OFF_K + r * SQ + cc * 16) = lk[i];
      *reinterpret_cast<u32x4_t*>(sm + OFF_HK + (v >> 3) * SHK + (v & 7) * 16) = lh[i];
    }
    {
      const float zz[8] = {zl0[0], zl0[1], zl0[2], zl0[3], zl1[0], zl1[1], zl1[2], zl1[3]};
      const uint32_t w[4] = {ls.x, ls.y, ls.z, ls.w};
      uint32_t pk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pk[j] = (srow < n && sl) ? pack_bf16x2(exp_fast(__builtin_bit_cast(float, w[j] << 16) - zz[2 * j]),
                                       exp_fast(__builtin_bit_cast(float, w[j] & 0xffff0000u) - zz[2 * j + 1]))
                         : 0u;
      *reinterpret_cast<u32x4_t*>(sm + OFF_E + srow * SP + 16 * scv) = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
    }
    __syncthreads();

    // ---- scores and softmax: wave tb < 4 owns tokens 16 tb .. 16 tb + 15
    if (wave < 4) {
      const char* qrow = sm + OFF_Q + c16 * SQ + 8 * g4;
      const char* krow = sm + OFF_K + c16 * SQ + 8 * g4;
      const char* hkb = sm + OFF_HK + (4 * g4 + (c16 >> 2)) * SHK + 8 * (c16 & 3);
      const char* eb = sm + OFF_E + (4 * g4 + (c16 >> 2)) * SP + 8 * (c16 & 3);
      f32x4_t s1[4], s2[4], at[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) s1[j] = s2[j] = at[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < K / 32; ++s) {
        const frag fq = rfrag(qrow, SQ, tb, s);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) S::mma(s1[mt], fq, tfrag(hkb, SHK, s, mt));
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
          if (ib <= tb) S::mma(at[ib], rfrag(krow, SQ, ib, s), fq);  // C[i][t] = k_i . q_t
      }
      const int t = 16 * tb + c16;
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * ib + 4 * g4 + r > t) at[ib][r] = 0.f;
#pragma unroll
      for (int s2i = 0; s2i < 2; ++s2i) {
        if (2 * s2i <= tb) {
          const frag fa = S::frag_from_f32(at[2 * s2i], at[2 * s2i + 1]);  // rows t, contraction i
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) S::mma(s2[mt], fa, tfrag(eb, SP, s2i, mt));
        }
      }
      // scores (C layout: rows t = 16 tb + 4 g4 + r, column m = 16 mt + c16)
      float x1[4][4], x2[4][4], sc[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float zp = c > 0 ? zpv[mt] : -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x1[mt][r] = exp_fast(zp - zt[mt][r]);
          x2[mt][r] = exp_fast(zlv[mt] - zt[mt][r]);
          sc[mt][r] = 16 * mt + c16 < MS ? a.scale * (x1[mt][r] * s1[mt][r] + x2[mt][r] * s2[mt][r]) : -INFINITY;
        }
      }
      uint16_t* pp = static_cast<uint16_t*>(a.p);
      const rsrc_t rp = make_rsrc(pp + (pp != nullptr ? (tok0 * H + h) * MS : 0),
                                  pp != nullptr ? static_cast<uint32_t>(((n - 1) * H * MS + MS) * 2) : 0u);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tr = 16 * tb + 4 * g4 + r;
        float mx = fmaxf(fmaxf(sc[0][r], sc[1][r]), fmaxf(sc[2][r], sc[3][r]));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        float e[4], sum = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          e[mt] = exp_fast(sc[mt][r] - mx);
          sum += e[mt];
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o);
        const float inv = 1.f / sum;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int m = 16 * mt + c16;
          // rows past the end read zeros and may hold non-finite scores; padding slots hold none
          const bool live = tr < n && m < MS;
          const float p = live ? e[mt] * inv : 0.f;
          *reinterpret_cast<__bf16*>(sm + OFF_P1 + tr * SP + 2 * m) = static_cast<__bf16>(live ? p * x1[mt][r] : 0.f);
          *reinterpret_cast<__bf16*>(sm + OFF_P2 + tr * SP + 2 * m) = static_cast<__bf16>(live ? p * x2[mt][r] : 0.f);
          if (m < MS) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(p), rp, static_cast<int>((tr * H * MS + m) * 2), 0, 0);
        }
      }
    }
    __syncthreads();

    // ---- value side: o^T = Hv[c]^T P1^T + V^T mask(E P2^T)
#pragma unroll
    for (int i = 0; i < LV; ++i) {
      const int v = tid + i * NT, r = v / (V / 8), cc = v % (V / 8);
      *reinterpret_cast<u32x4_t*>(sm + OFF_HV + r * SVV + cc * 16) = lhv[i];
      *reinterpret_cast<u32x4_t*>(sm + OFF_V + r * SVV + cc * 16) = lv[i];
    }
    __syncthreads();
    f32x4_t acc[NVT][4];
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) acc[vt][t4] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const char* hvb = sm + OFF_HV + (4 * g4 + (c16 >> 2)) * SVV + 8 * (c16 & 3);
    const char* vb = sm + OFF_V + (4 * g4 + (c16 >> 2)) * SVV + 8 * (c16 & 3);
    const char* p1r = sm + OFF_P1 + c16 * SP + 8 * g4;
    const char* p2r = sm + OFF_P2 + c16 * SP + 8 * g4;
    const char* er = sm + OFF_E + c16 * SP + 8 * g4;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      frag fp[4];
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) fp[t4] = rfrag(p1r, SP, t4, s);
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const frag fh = tfrag(hvb, SVV, s, wave * NVT + vt);
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) S::mma(acc[vt][t4], fh, fp[t4]);
      }
    }
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      f32x4_t bt[4];
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) bt[ib] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const frag fp2 = rfrag(p2r, SP, t4, s);
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
          if (ib <= t4) S::mma(bt[ib], rfrag(er, SP, ib, s), fp2);  // C[i][t] = E_i . P2_t
      }
      const int t = 16 * t4 + c16;
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * ib + 4 * g4 + r > t) bt[ib][r] = 0.f;
#pragma unroll
      for (int s2i = 0; s2i < 2; ++s2i) {
        if (2 * s2i <= t4) {
          const frag fb = S::frag_from_f32(bt[2 * s2i], bt[2 * s2i + 1]);  // columns t, contraction i
#pragma unroll
          for (int vt = 0; vt < NVT; ++vt) S::mma(acc[vt][t4], tfrag(vb, SVV, s2i, wave * NVT + vt), fb);
        }
      }
    }
    // o[t][v .. v+3] for v = 16 (wave NVT + vt) + 4 g4, t = 16 t4 + c16
    const rsrc_t ro = make_rsrc(static_cast<uint16_t*>(a.o) + (tok0 * H + h) * V,
                                static_cast<uint32_t>(((n - 1) * H * V + V) * 2));
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const int t = 16 * t4 + c16;
        const int v0 = 16 * (wave * NVT + vt) + 4 * g4;
        const u32x2_t pk{pack_bf16x2(acc[vt][t4][0], acc[vt][t4][1]), pack_bf16x2(acc[vt][t4][2], acc[vt][t4][3])};
        __builtin_amdgcn_raw_buffer_store_b64(pk, ro, static_cast<int>((t * H * V + v0) * 2), 0, 0);
      }
  }
};

template <int K, int V>
__global__ __launch_bounds__(512) void abc_out_kernel(const AbcOutArgs a) {
  __shared__ __align__(16) char sm[AbcOut<K, V>::SMEM];
  AbcOut<K, V>::run(a, sm);
}

template <int K, int V>
static hipError_t launch_abc_out_t(const AbcOutArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((abc_out_kernel<K, V>), dim3(a.B * a.NC * a.H), dim3(512), 0, stream, a);
  return hipGetLastError();
}

bool abc_out_supported(int K, int V) {
  return (K == 64 && V == 128) || (K == 128 && V == 128) || (K == 128 && V == 256) || (K == 256 && V == 256) ||
         (K == 256 && V == 512);
}

hipError_t launch_abc_out(const AbcOutArgs& a, hipStream_t stream) {
  if (a.NC == 0) return hipSuccess;
  if (a.K == 64 && a.V == 128) return launch_abc_out_t<64, 128>(a, stream);
  if (a.K == 128 && a.V == 128) return launch_abc_out_t<128, 128>(a, stream);
  if (a.K == 128 && a.V == 256) return launch_abc_out_t<128, 256>(a, stream);
  if (a.K == 256 && a.V == 256) return launch_abc_out_t<256, 256>(a, stream);
  if (a.K == 256 && a.V == 512) return launch_abc_out_t<256, 512>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdr
