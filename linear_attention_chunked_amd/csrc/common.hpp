// Device-side building blocks shared by the gfx950 kernels.
//
// Matrix-core fragments
// ---------------------
// Every contraction in this library is written in terms of one "virtual"
// 16x16x32 MFMA step: D[16x16] += A[16x32] * B[32x16] with FP32 accumulation.
//   * bfloat16 storage: one v_mfma_f32_16x16x32_bf16.
//   * float32 storage: eight v_mfma_f32_16x16x4_f32, one per operand element.
// Lane l of a wave (g = l / 16, c = l % 16) supplies
//   A row c, B column c, and 8 operand elements e = 0..7 that stand for the
//   contraction index  k(g, e) = 4 g + (e & 3) + 16 (e >> 2)  of the 32-wide step.
// Because A and B use the same k(g, e) the product is the full contraction no
// matter how the hardware orders the slots.  The 16x16 accumulator ("C
// layout") gives lane l the four values D[4 g + r][c], r = 0..3.
//
// The k(g, e) map is chosen so that two vertically adjacent C-layout tiles
// (rows 0..15 and 16..31 of a 32-row block) are exactly one B-operand fragment
// of the next contraction:  C-tile 0 values r -> elements r, C-tile 1 values
// r -> elements 4 + r.  That is what lets the scan keep its FP32 state in
// accumulator registers and feed it straight back as a matrix-core operand,
// with no LDS round trip.
//
// A product whose two operands are both read from memory (not from an
// accumulator) may use the contiguous map k(g, e) = 8 g + e instead: each
// lane then reads 16 contiguous bytes of a row, one ds_read_b128, where the
// map above needs two 8-byte pieces 32 bytes apart (one ds_read2_b64, which
// gfx950 serves at half the rate).  Kernels whose results must agree bit for
// bit (the chunk output and the state scan with the output fused) use the
// same map for the same product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bfloat16 storage element (raw bits).
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (the hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two RNE bfloat16 in one dword (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// ---------------------------------------------------------------------------
// Storage traits: a "quad" is 4 consecutive storage elements (8 B for bf16,
// 16 B for fp32); a "frag" is one MFMA operand of a virtual 16x16x32 step.
template <typename TI>
struct St;

template <>
struct St<bf16_t> {
  using quad = u32x2_t;
  struct frag {
    bf16x8_t v;
  };
  static constexpr int bytes = 2;
  __device__ static __forceinline__ void quad_to_f32(quad q, float* f) {
    f[0] = __builtin_bit_cast(float, q.x << 16);
    f[1] = __builtin_bit_cast(float, q.x & 0xffff0000u);
    f[2] = __builtin_bit_cast(float, q.y << 16);
    f[3] = __builtin_bit_cast(float, q.y & 0xffff0000u);
  }
  __device__ static __forceinline__ quad f32_to_quad(const float* f) {
    quad q;
    q.x = pack_bf16x2(f[0], f[1]);
    q.y = pack_bf16x2(f[2], f[3]);
    return q;
  }
  __device__ static __forceinline__ quad zero_quad() { return quad{0u, 0u}; }
  // elements 0..3 from q0, 4..7 from q1
  __device__ static __forceinline__ frag frag_from_quads(quad q0, quad q1) {
    u32x4_t u{q0.x, q0.y, q1.x, q1.y};
    return frag{__builtin_bit_cast(bf16x8_t, u)};
  }
  __device__ static __forceinline__ frag frag_from_quads_neg(quad q0, quad q1) {
    const uint32_t s = 0x80008000u;
    u32x4_t u{q0.x ^ s, q0.y ^ s, q1.x ^ s, q1.y ^ s};
    return frag{__builtin_bit_cast(bf16x8_t, u)};
  }
  // elements 0..3 from x0, 4..7 from x1 (rounded to bf16)
  __device__ static __forceinline__ frag frag_from_f32(f32x4_t x0, f32x4_t x1) {
    u32x4_t u{pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]), pack_bf16x2(x1[0], x1[1]),
              pack_bf16x2(x1[2], x1[3])};
    return frag{__builtin_bit_cast(bf16x8_t, u)};
  }
  __device__ static __forceinline__ void mma(f32x4_t& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
  }
  // 4x4 transpose of quads: out[j] element i = in[i] element j
  __device__ static __forceinline__ void transpose4(const quad* in, quad* out) {
    out[0].x = (in[0].x & 0xffffu) | (in[1].x << 16);
    out[0].y = (in[2].x & 0xffffu) | (in[3].x << 16);
    out[1].x = (in[0].x >> 16) | (in[1].x & 0xffff0000u);
    out[1].y = (in[2].x >> 16) | (in[3].x & 0xffff0000u);
    out[2].x = (in[0].y & 0xffffu) | (in[1].y << 16);
    out[2].y = (in[2].y & 0xffffu) | (in[3].y << 16);
    out[3].x = (in[0].y >> 16) | (in[1].y & 0xffff0000u);
    out[3].y = (in[2].y >> 16) | (in[3].y & 0xffff0000u);
  }
};

template <>
struct St<float> {
  using quad = f32x4_t;
  struct frag {
    float v[8];
  };
  static constexpr int bytes = 4;
  __device__ static __forceinline__ void quad_to_f32(quad q, float* f) {
    f[0] = q[0];
    f[1] = q[1];
    f[2] = q[2];
    f[3] = q[3];
  }
  __device__ static __forceinline__ quad f32_to_quad(const float* f) {
    return quad{f[0], f[1], f[2], f[3]};
  }
  __device__ static __forceinline__ quad zero_quad() { return quad{0.f, 0.f, 0.f, 0.f}; }
  __device__ static __forceinline__ frag frag_from_quads(quad q0, quad q1) {
    return frag{{q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]}};
  }
  __device__ static __forceinline__ frag frag_from_quads_neg(quad q0, quad q1) {
    return frag{{-q0[0], -q0[1], -q0[2], -q0[3], -q1[0], -q1[1], -q1[2], -q1[3]}};
  }
  __device__ static __forceinline__ frag frag_from_f32(f32x4_t x0, f32x4_t x1) {
    return frag{{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]}};
  }
  __device__ static __forceinline__ void mma(f32x4_t& acc, const frag& a, const frag& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
  }
  __device__ static __forceinline__ void transpose4(const quad* in, quad* out) {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = quad{in[0][j], in[1][j], in[2][j], in[3][j]};
  }
};

// Global / LDS quad access (16-byte aligned for fp32, 8-byte for bf16).
template <typename TI>
__device__ __forceinline__ typename St<TI>::quad ld_quad(const TI* p) {
  return *reinterpret_cast<const typename St<TI>::quad*>(p);
}
template <typename TI>
__device__ __forceinline__ void st_quad(TI* p, typename St<TI>::quad q) {
  *reinterpret_cast<typename St<TI>::quad*>(p) = q;
}

// Fast e^x via the hardware 2^x (v_exp_f32).
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// A row of a per-launch plan: one sequence (or one segment of a sequence).
struct Row {
  int32_t bos;        // first token (flattened over the [B, T] rows)
  int32_t len;        // tokens
  int32_t chunk_off;  // first row of h for this row's chunks
  int32_t in_idx;     // initial-state index (h0 / seg_init), -1 = zeros
  int32_t out_idx;    // final-state index (hT / seg_state), -1 = none
};

constexpr int kChunk = 64;
constexpr int kMaxRows = 112;  // rows carried by value in one launch's arguments

// The row of a launch's plan that holds chunk `chunk` (chunks relative to the
// launch; rows sorted by chunk_off, the first at 0): the last row whose first
// chunk is at or before it.  One round of vector loads from the argument
// block instead of a chain of dependent scalar loads: lane l reads rows l and
// l + 64, a ballot counts the rows that start at or before the chunk, and the
// fields come from the lane that read that row.  Call with the whole wave
// active; the result is uniform.
static_assert(kMaxRows <= 128, "row lookup reads two rows per lane");
__device__ __forceinline__ Row row_of_chunk(const Row* rows, int n_rows, int chunk) {
  const int lane = static_cast<int>(threadIdx.x & 63);
  const int last = max(n_rows - 1, 0);  // every lane reads inside the list, also for an empty one
  const Row x0 = rows[min(lane, last)];
  const Row x1 = rows[min(lane + 64, last)];
  const uint64_t m0 = __ballot(lane < n_rows && x0.chunk_off <= chunk);
  const uint64_t m1 = __ballot(lane + 64 < n_rows && x1.chunk_off <= chunk);
  const int idx = __builtin_amdgcn_readfirstlane(__popcll(m0) + __popcll(m1) - 1);
  const Row& x = idx < 64 ? x0 : x1;
  const int l = idx & 63;
  return Row{__builtin_amdgcn_readlane(x.bos, l), __builtin_amdgcn_readlane(x.len, l),
             __builtin_amdgcn_readlane(x.chunk_off, l), __builtin_amdgcn_readlane(x.in_idx, l),
             __builtin_amdgcn_readlane(x.out_idx, l)};
}

}  // namespace gdr
