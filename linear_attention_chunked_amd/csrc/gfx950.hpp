// Small gfx950 device helpers shared by the bfloat16 kernels.
#pragma once

#include "common.hpp"

namespace gdr {

using rsrc_t = __amdgpu_buffer_rsrc_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// Raw buffer resource over [base, base + bytes): loads past the end return
// zero and stores past the end are dropped by the hardware range check.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, static_cast<int>(bytes), 0x00020000);
}

// Cache policy of a buffer store whose data no later access of the same
// kernel reads (the staged per-chunk states and v_new rows of the scans, the
// ABC states; all written as whole 16-byte pieces of full lines):
// non-temporal, so the streamed output does not push
// the inputs that the column blocks of one (sequence, head) share out of the
// XCD's L2.  Measured: the 64K x 8-head segmented pass 179 -> 172 us, the
// 32-head packed scan 229 -> 222 us, ABC's slot-state walk (forward call
// 202 -> 159 us, reverse 188 -> 163 us).
// Stores of partial 128-byte lines (the fused output's 8-byte pieces, the
// reverse walk's dh and dv pieces straight from its accumulators) stay on
// the default policy: non-temporal there, L2 no longer merges them before
// they go to HBM (88 -> 97 MB written per question_rows launch of the fused
// pass; 97 -> 74 MB and 40.5 -> 37.0 us for the reverse walk).  The same
// policy bit on a load marks a stream that one workgroup reads once (the
// scan's U columns on long chains).
constexpr int kStreamStore = 2;

// e^x on the hardware base-2 exponential.
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j names 8 bytes
// (four bf16 of a row-major 4 x 16 block) and lane i receives column i of
// that block, i.e. four consecutive rows of one column.
__device__ __forceinline__ u32x2_t lds_tr16(const char* base, int byte_off) {
  const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + byte_off));
  return __builtin_bit_cast(u32x2_t, v);
}

__device__ __forceinline__ u32x2_t lds_b64(const char* base, int byte_off) {
  return *reinterpret_cast<const u32x2_t*>(base + byte_off);
}

// A bf16 row fragment in the contiguous k map (common.hpp): the lane's 16
// bytes at base + byte_off, one ds_read_b128 (16-byte aligned).
__device__ __forceinline__ St<bf16_t>::frag lds_frag16(const char* base, int byte_off) {
  const u32x4_t q = *reinterpret_cast<const u32x4_t*>(base + byte_off);
  return St<bf16_t>::frag_from_quads(u32x2_t{q.x, q.y}, u32x2_t{q.z, q.w});
}

}  // namespace gdr
