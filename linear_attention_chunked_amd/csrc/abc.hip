// ABC slot-state construction on gfx950 (flash-linear-attention fork issue
// #23, "[Perf][B300] Parallelize ABC chunk state construction with affine
// summaries": "Problem" and "Proposed Dataflow").
//
// Normaliser: z_t = log(e^{z_{t-1}} + e^{s_t}) per slot.  Three levels:
//   abc_chunk_lse   one workgroup per (b, chunk, h): four waves take 16 tokens
//                   each (lane = slot, every score load issued ahead of the
//                   chain), combine through LDS, and write the chunk's total
//                   lse[c] (and, when requested, the chunk-local running
//                   values into z);
//   abc_carry       one wave per (b, h, 4 slots): zc[c] = logaddexp(zc[c-1],
//                   lse[c]) over 64 stretches of the chunk range in parallel;
//   abc_weights     one workgroup per (b, chunk, h): the chunk's weights
//                   E_t = exp(s_t - zc[c]) in the storage dtype, once for all
//                   the state tiles that use them, and (when z is requested)
//                   z_t = logaddexp(zc[c-1], local_t).
// log-add-exp runs on the hardware base-2 exponential and logarithm: the
// correction term log(1 + e^{-|a-b|}) lies in [0, ln 2], so its absolute
// error (a few 1e-8) stays below the rounding of the FP32 sum it is added to.
//
// States: every 64-token chunk applies the exact diagonal affine map
//   S <- S * r_c + c_c,   r_c = exp(zc[c-1] - zc[c]),  E_t = exp(s_t - zc[c]),
//   Hk [K x M]:  c_c = K_c^T E   (r over columns)
//   Hv [M x V]:  c_c = E^T V_c   (r over rows)
// One workgroup owns a 64x64 tile of Hk or Hv of one (b, h) and walks the
// chunks in order.  c_c does not depend on the state, so the walk is a
// stream, not a latency chain: the global loads of the next D chunks are in
// flight (a ring of register stages), each chunk is staged once in LDS
// row-major exactly as loaded, and the MFMA operands, which contract over
// tokens, come from the row-major tiles through ds_read_b64_tr_b16 (E
// arrives precomputed, so a chunk costs the state tile no exponentials).  The
// contribution is accumulated in FP32 on top of the scaled state, so the
// page's FP32 summary never leaves the chip; the state before each chunk is
// written once, in the storage dtype.  The tile is held transposed (rows =
// the contiguous dimension of the stored state), so each lane's four
// accumulator rows are four adjacent elements in memory: one 8-byte store.
#include <math.h>
#include <stdlib.h>

#include <algorithm>

#include "gfx950.hpp"
#include "kernels.hpp"

namespace gdr {

__device__ __forceinline__ float logaddexp_f(float a, float b) {
  const float m = fmaxf(a, b);
  const float d = exp_fast(-fabsf(a - b));  // in [0, 1]; NaN only when both are -inf
  const float l = m + 0.69314718055994531f * __builtin_amdgcn_logf(1.f + d);
  return m == -INFINITY ? -INFINITY : l;
}

// ---------------------------------------------------------------- normaliser
__global__ __launch_bounds__(256) void abc_chunk_lse(const AbcArgs a) {
  __shared__ float tot[4][64];
  const int m = threadIdx.x & 63;  // slot (lanes past M (32) carry -inf and write nothing)
  const bool live_m = m < a.M;
  const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // 16-token group (one per wave)
  const int bx = blockIdx.x;
  const int h = bx % a.H;
  const int c = (bx / a.H) % a.NC;
  const int b = bx / (a.H * a.NC);
  const int t0 = c * kChunk + 16 * grp;
  const int n = __builtin_amdgcn_readfirstlane(max(0, min(16, a.T - t0)));  // (uniform: a scalar resource)
  const int64_t rs = static_cast<int64_t>(a.H) * a.M;  // elements between tokens
  // the group's 16 scores of slot m, all loads ahead of the chain (tokens
  // past the end read as zero through the range check and are skipped)
  const uint16_t* sp = static_cast<const uint16_t*>(a.s) + ((static_cast<int64_t>(b) * a.T + t0) * a.H + h) * a.M;
  const rsrc_t rsr = make_rsrc(sp, n > 0 ? static_cast<uint32_t>(((n - 1) * rs + a.M) * 2) : 0u);
  uint16_t v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    v[i] = __builtin_amdgcn_raw_buffer_load_b16(rsr, static_cast<int>((i * rs + m) * 2), 0, 0);
  // the group's total as max + log(sum of exp(x - max)): independent exponentials
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (i < n) mx = fmaxf(mx, bf16_to_f32(v[i]));
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (i < n) sum += exp_fast(bf16_to_f32(v[i]) - mx);
  const float L = (n > 0 && live_m) ? mx + 0.69314718055994531f * __builtin_amdgcn_logf(sum) : -INFINITY;
  tot[grp][m] = L;
  __syncthreads();
  float off = -INFINITY;
  for (int g = 0; g < grp; ++g) off = logaddexp_f(off, tot[g][m]);
  if (a.z != nullptr && live_m) {  // the chunk-local running values (a chain, only when z is requested)
    float run = off;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i < n) {
        run = logaddexp_f(run, bf16_to_f32(v[i]));
        a.z[((static_cast<int64_t>(b) * a.T + t0 + i) * a.H + h) * a.M + m] = run;
      }
  }
  if (grp == 3 && live_m) a.lse[((static_cast<int64_t>(b) * a.NC + c) * a.H + h) * a.M + m] = logaddexp_f(off, L);
}

// DPP lane move of x with -inf where the move has no source (or the row is
// masked off): the identity of logaddexp.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_ninf(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, -INFINITY),
                                                               __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, false));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ f32x4_t lae4_dpp(f32x4_t x) {
  f32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = logaddexp_f(dpp_ninf<CTRL, ROW_MASK>(x[j]), x[j]);
  return r;
}

__global__ __launch_bounds__(64) void abc_carry(const AbcArgs a) {
  // zc[c] = logaddexp(zc[c-1], lse[c]) per slot (M = 32 or 64).  One wave per
  // (b, h, quad of slots 4p .. 4p + 3; 16-byte loads and stores); lane s
  // takes stretch s, one of 64 contiguous stretches of the chunk range.
  // Pass 1 forms each stretch's total as max + log(sum of exp(x - max)); an
  // inclusive scan of the stretch totals across the wave on DPP lane moves
  // (shifts by 1, 2, 4, 8 within rows of 16 lanes, then the row broadcasts of
  // lanes 15 and 31; no LDS, no barrier) and a shift by one lane give each
  // stretch the total of the ones before it; pass 2 re-runs the stretch's
  // chain from there and writes zc.  Stretches of up to 8 chunks stay in
  // registers (up to 512 chunks per call); longer ones read their totals
  // again in pass 2.
  const int st = threadIdx.x & 63;
  const int nq = a.M / 4;  // quads of slots per (b, h)
  const int p = blockIdx.x % nq;
  const int h = (blockIdx.x / nq) % a.H;
  const int b = (blockIdx.x / nq) / a.H;
  const int per = (a.NC + 63) / 64;
  const int c0 = min(a.NC, st * per), c1 = min(a.NC, c0 + per);
  const int64_t step = static_cast<int64_t>(a.H) * a.M;
  const int64_t row0 = (static_cast<int64_t>(b) * a.NC * a.H + h) * a.M + 4 * p;
  auto lse_at = [&](int c) { return *reinterpret_cast<const f32x4_t*>(a.lse + row0 + c * step); };
  auto lae4 = [](f32x4_t x, f32x4_t y) {
    f32x4_t r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = logaddexp_f(x[j], y[j]);
    return r;
  };
  constexpr int R = 8;
  const int nr = min(R, c1 - c0);
  f32x4_t l[R];
  {
    // one resource for the (b, h) slice (uniform, so no per-lane descriptors);
    // chunks past this stretch are masked below, past the slice read as zero
    const float* bh = a.lse + (static_cast<int64_t>(b) * a.NC * a.H + h) * a.M;
    const rsrc_t rl = make_rsrc(bh, static_cast<uint32_t>(((a.NC - 1) * step + a.M) * 4));
#pragma unroll
    for (int i = 0; i < R; ++i)
      l[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                             rl, static_cast<int>(((c0 + i) * step + 4 * p) * 4), 0, 0));
  }
  const f32x4_t ninf{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  f32x4_t mx = ninf;
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (i < nr)
#pragma unroll
      for (int j = 0; j < 4; ++j) mx[j] = fmaxf(mx[j], l[i][j]);
  for (int c = c0 + R; c < c1; ++c) {
    const f32x4_t v = lse_at(c);
#pragma unroll
    for (int j = 0; j < 4; ++j) mx[j] = fmaxf(mx[j], v[j]);
  }
  f32x4_t sm{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (i < nr)
#pragma unroll
      for (int j = 0; j < 4; ++j) sm[j] += exp_fast(l[i][j] - mx[j]);
  for (int c = c0 + R; c < c1; ++c) {
    const f32x4_t v = lse_at(c);
#pragma unroll
    for (int j = 0; j < 4; ++j) sm[j] += exp_fast(v[j] - mx[j]);
  }
  f32x4_t t;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    t[j] = mx[j] == -INFINITY ? -INFINITY : mx[j] + 0.69314718055994531f * __builtin_amdgcn_logf(sm[j]);
  t = lae4_dpp<0x111, 0xf>(t);  // row_shr:1
  t = lae4_dpp<0x112, 0xf>(t);  // row_shr:2
  t = lae4_dpp<0x114, 0xf>(t);  // row_shr:4
  t = lae4_dpp<0x118, 0xf>(t);  // row_shr:8
  t = lae4_dpp<0x142, 0xa>(t);  // row_bcast:15 into rows 1 and 3
  t = lae4_dpp<0x143, 0xc>(t);  // row_bcast:31 into rows 2 and 3
  f32x4_t z;
#pragma unroll
  for (int j = 0; j < 4; ++j) z[j] = dpp_ninf<0x138, 0xf>(t[j]);  // wave_shr:1: the stretches before this one
  float* zc = a.zc + row0;
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (i < nr) {
      z = lae4(z, l[i]);
      *reinterpret_cast<f32x4_t*>(zc + (c0 + i) * step) = z;
    }
  for (int c = c0 + R; c < c1; ++c) {
    z = lae4(z, lse_at(c));
    *reinterpret_cast<f32x4_t*>(zc + c * step) = z;
  }
}

__global__ __launch_bounds__(256) void abc_weights(const AbcArgs a) {
  // 64 tokens x 64 slots: thread = (row, 8 slots), rows row and row + 32
  const int bx = blockIdx.x;
  const int h = bx % a.H;
  const int c = (bx / a.H) % a.NC;
  const int b = bx / (a.H * a.NC);
  const int tid = threadIdx.x;
  const int row = tid >> 3, cv = tid & 7;
  if (8 * cv >= a.M) return;  // M = 32: half the threads
  const int n = min(kChunk, a.T - c * kChunk);
  const int64_t H = a.H, M = a.M;
  const float* zp = a.zc + ((static_cast<int64_t>(b) * a.NC + c) * H + h) * M + 8 * cv;
  const f32x4_t z0 = *reinterpret_cast<const f32x4_t*>(zp);
  const f32x4_t z1 = *reinterpret_cast<const f32x4_t*>(zp + 4);
  const float zz[8] = {z0[0], z0[1], z0[2], z0[3], z1[0], z1[1], z1[2], z1[3]};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = row + 32 * i;
    if (r >= n) continue;
    const int64_t off = ((static_cast<int64_t>(b) * a.T + static_cast<int64_t>(c) * kChunk + r) * H + h) * M + 8 * cv;
    const u32x4_t q = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.s) + off);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    uint32_t pk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      pk[j] = pack_bf16x2(exp_fast(__builtin_bit_cast(float, w[j] << 16) - zz[2 * j]),
                          exp_fast(__builtin_bit_cast(float, w[j] & 0xffff0000u) - zz[2 * j + 1]));
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.e) + off) = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
    if (a.z != nullptr && c > 0) {
      const float* zq = zp - H * M;  // zc[c - 1]
      const f32x4_t p0 = *reinterpret_cast<const f32x4_t*>(zq);
      const f32x4_t p1 = *reinterpret_cast<const f32x4_t*>(zq + 4);
      f32x4_t* zl = reinterpret_cast<f32x4_t*>(a.z + off);
      f32x4_t l0 = zl[0], l1 = zl[1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        l0[j] = logaddexp_f(p0[j], l0[j]);
        l1[j] = logaddexp_f(p1[j], l1[j]);
      }
      zl[0] = l0;
      zl[1] = l1;
    }
  }
}

// Reverse weights, one workgroup per (b, chunk, h), thread = (token row, 8
// slots): with zp = zc[c-1] (the forward's normaliser at the previous chunk's
// last token; -inf for the first chunk, whose weights are then zero)
//   Yk_t = scale dscore_t e^{zp - z_t},   Yv_t = p_t e^{zp - z_t}     (<= |.|)
// in the storage dtype, and zc[c] = z at the chunk's last token.
__global__ __launch_bounds__(256) void abc_bwd_weights(const AbcArgs a) {
  const int bx = blockIdx.x;
  const int h = bx % a.H;
  const int c = (bx / a.H) % a.NC;
  const int b = bx / (a.H * a.NC);
  const int tid = threadIdx.x;
  const int row = tid >> 3, cv = tid & 7;
  const int n = min(kChunk, a.T - c * kChunk);
  const int64_t H = a.H, M = a.M;
  const int64_t tok0 = static_cast<int64_t>(b) * a.T + static_cast<int64_t>(c) * kChunk;
  if (tid < a.M / 4) {  // zc[c]: the M slots, four per thread
    const f32x4_t zl = *reinterpret_cast<const f32x4_t*>(a.z + ((tok0 + n - 1) * H + h) * M + 4 * tid);
    *reinterpret_cast<f32x4_t*>(a.zc + ((static_cast<int64_t>(b) * a.NC + c) * H + h) * M + 4 * tid) = zl;
  }
  if (8 * cv >= a.M) return;  // M = 32: half the threads
  float zp[8];
  if (c > 0) {
    const float* q = a.z + ((tok0 - 1) * H + h) * M + 8 * cv;
    const f32x4_t p0 = *reinterpret_cast<const f32x4_t*>(q);
    const f32x4_t p1 = *reinterpret_cast<const f32x4_t*>(q + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      zp[j] = p0[j];
      zp[4 + j] = p1[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) zp[j] = -INFINITY;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = row + 32 * i;
    if (r >= n) continue;
    const int64_t off = ((tok0 + r) * H + h) * M + 8 * cv;
    const f32x4_t z0 = *reinterpret_cast<const f32x4_t*>(a.z + off);
    const f32x4_t z1 = *reinterpret_cast<const f32x4_t*>(a.z + off + 4);
    const float zt[8] = {z0[0], z0[1], z0[2], z0[3], z1[0], z1[1], z1[2], z1[3]};
    const u32x4_t dq = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.s) + off);
    const u32x4_t pq = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.pw) + off);
    const uint32_t dw[4] = {dq.x, dq.y, dq.z, dq.w};
    const uint32_t pw[4] = {pq.x, pq.y, pq.z, pq.w};
    uint32_t yk[4], yv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x0 = exp_fast(zp[2 * j] - zt[2 * j]);
      const float x1 = exp_fast(zp[2 * j + 1] - zt[2 * j + 1]);
      yk[j] = pack_bf16x2(a.scale * __builtin_bit_cast(float, dw[j] << 16) * x0,
                          a.scale * __builtin_bit_cast(float, dw[j] & 0xffff0000u) * x1);
      yv[j] = pack_bf16x2(__builtin_bit_cast(float, pw[j] << 16) * x0,
                          __builtin_bit_cast(float, pw[j] & 0xffff0000u) * x1);
    }
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.e) + off) = u32x4_t{yk[0], yk[1], yk[2], yk[3]};
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.e2) + off) = u32x4_t{yv[0], yv[1], yv[2], yv[3]};
  }
}

// ---------------------------------------------------------------- states
// IS_K: the tile is XW rows (k) of Hk, held as Hk^T [slot][k]; otherwise XW
// columns (v) of Hv, held as Hv^T [v][slot].  XW (64, 32 or 16) sets how many
// workgroups share one (b, h): the chunk walk is a fixed-latency loop, so
// narrower tiles put more of the chip to work when B * H is small.
// The chunk loop runs over a multiple of D chunks; chunks past the end read
// and write empty buffer ranges and act as the identity (E = 0, r = 1), so
// every iteration issues the same memory operations and the compiler's wait
// counts keep D chunks in flight.
//
// Segments (the map is diagonal-affine, so segments compose exactly): the
// chunks of a sequence are split into P runs.  MODE 1 walks run j < P-1 from
// a zero state without storing anything and leaves its end state L_j (FP32,
// normalised at the run's last chunk).  MODE 0 walks run j from
//   S_start(j) = sum_{i<j} L_i * exp(zc[end_i] - zc[start_j - 1])   (per slot)
// storing the pre-chunk states; with P = 1 it is the plain serial walk.
//
// REV: the reverse (dH) walk.  Logical step j handles chunk NC-1-j; per step
//   store dH[c]; dH <- dH * r_c + c'_c,  r_c = exp(zc[c-1] - zc[c]),
//   key side c'_c = Q_c^T Yk, value side c'_c = Yv^T dO_c
// with Yk = scale dscore e^{zc[c-1]-z}, Yv = p e^{zc[c-1]-z} from
// abc_bwd_weights: the forward step with the chunk order reversed and other
// operands, so the same code runs it.  The walk starts from the final
// states' gradient; run j of MODE 0 starts from
//   G_end e^{zc[p_j] - zc[NC-1]} + sum_{i<j} L_i e^{zc[p_j] - zc[a_i - 1]}
// (p_j: run j's first chunk, a_i: run i's last, both in chunk order).
template <bool IS_K, int XW, int MODE, bool REV>
struct AbcStates {
  using S = St<bf16_t>;
  using frag = S::frag;
  // HS: the walk stores the pre-chunk states (through the LDS staging
  // buffers).  The run-end pass (MODE 1) stores nothing: without the staging
  // buffers and with 4 chunks in flight (132 VGPRs, 41 KB of LDS at XW = 64)
  // three of its workgroups share a CU, so its 7 x 96 units at B = 2, H = 4,
  // K = 256, V = 512 run in one round instead of two (whole forward call
  // 156 -> 148 us, reverse 161 -> 155 us).  The walk itself moves the states
  // out at about the copy rate with two workgroups per CU (three, with one
  // staging buffer and 4 chunks in flight, measured the same).
  static constexpr bool HS = (MODE == 0);
  static constexpr int D = HS ? 8 : 4;    // chunks in flight
  static constexpr int NR = XW / 16;      // 16-wide blocks of the x dimension = MFMA tiles per wave
  static constexpr int STE = 128 + 32;    // LDS row stride (bytes) of the 64-slot E tile
  static constexpr int STX = XW * 2 + (XW == 64 ? 32 : 16);  // ... and of the x tile
  static constexpr int XB = XW / 2;       // x bytes per thread per chunk (64 rows x XW bf16 / 256 threads)

  // pre-chunk state staged in its memory layout: Hk rows (k) of 64 slots, or
  // Hv rows (slots) of XW columns; written out the next chunk in whole rows
  static constexpr int STH = IS_K ? 64 * 2 + 16 : XW * 2 + 16;
  static constexpr int HSZ = (XW * (64 * 2 + 16) > 64 * (XW * 2 + 16)) ? XW * (64 * 2 + 16) : 64 * (XW * 2 + 16);

  struct Smem {
    char x[2][kChunk * STX];  // k or v tile of the chunk, row-major [token][column]
    char e[2][kChunk * STE];  // E, row-major [token][slot]
    char hs[HS ? 2 : 1][HS ? HSZ : 16];  // staged pre-chunk state, by chunk parity
    float r[3][64];           // r_c by chunk modulo 3
  };

  struct Stage {
    u32x4_t x[XB >= 16 ? XB / 16 : 1];
    u32x4_t e[2];
    float z;                  // zc of the chunk for slot tid % 64
  };

  struct Ctx {
    const AbcArgs* a;
    int b, h, x0, X;
    int c_lo, c_hi;           // this workgroup's chunks
    int vo_x[XB >= 16 ? XB / 16 : 1], vo_e[2];  // per-thread byte offsets inside a chunk
    int lo_x[XB >= 16 ? XB / 16 : 1];           // ... and in the LDS x tile
    int vo_h[NR];             // per-lane byte offsets of the state tile (finals)
    int lo_h[NR];             // ... and in the staging buffer
    int vo_o[XB >= 16 ? XB / 16 : 1], lo_o[XB >= 16 ? XB / 16 : 1];  // write-out: global / staging
  };

  // chunk of logical step c
  __device__ static __forceinline__ int chunk_of(const AbcArgs& a, int c) { return REV ? a.NC - 1 - c : c; }

  __device__ static __forceinline__ void load(Stage& st, const Ctx& x, int c) {
    const AbcArgs& a = *x.a;
    const int64_t H = a.H;
    const int pc = chunk_of(a, c);
    const bool exists = pc >= 0 && pc < a.NC;
    const bool any = exists && c < x.c_hi;
    const int pcc = exists ? pc : 0;
    const int n = min(kChunk, a.T - pcc * kChunk);
    const int64_t tok0 = static_cast<int64_t>(x.b) * a.T + static_cast<int64_t>(pcc) * kChunk;
    const uint16_t* xp = static_cast<const uint16_t*>(IS_K ? a.k : a.v) + (tok0 * H + x.h) * x.X + x.x0;
    const uint16_t* ep = static_cast<const uint16_t*>(IS_K ? a.e : a.e2) + (tok0 * H + x.h) * a.M;
    const float* lp = a.zc + ((static_cast<int64_t>(x.b) * a.NC + pcc) * H + x.h) * a.M;
    const rsrc_t rx = make_rsrc(xp, any ? static_cast<uint32_t>(((n - 1) * H * x.X + XW) * 2) : 0u);
    const rsrc_t re = make_rsrc(ep, any ? static_cast<uint32_t>(((n - 1) * H * a.M + a.M) * 2) : 0u);
    // the reverse ratio of a run's last step needs zc of the chunk after the run
    // (slots past M read as zero: r = 1 there)
    const rsrc_t rl = make_rsrc(lp, (REV ? exists : any) ? static_cast<uint32_t>(4 * a.M) : 0u);
    if constexpr (XB >= 16) {
#pragma unroll
      for (int i = 0; i < XB / 16; ++i) st.x[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, x.vo_x[i], 0, 0);
    } else {
      const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rx, x.vo_x[0], 0, 0);
      st.x[0] = u32x4_t{v.x, v.y, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) st.e[i] = __builtin_amdgcn_raw_buffer_load_b128(re, x.vo_e[i], 0, 0);
    st.z = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, 4 * (threadIdx.x & 63), 0, 0));
  }

  // Chunk c, first half: stage -> LDS as loaded (rows past the chunk's end
  // read as zero); the first wave publishes r of chunk c+1 (zc of c+1 in `nxt`).
  __device__ static __forceinline__ void stage_in(const Stage& st, const Stage& nxt, const Ctx& x, int c, Smem& sm) {
    const AbcArgs& a = *x.a;
    const int tid = threadIdx.x;
    char* xb = sm.x[c & 1];
    char* eb = sm.e[c & 1];
    if constexpr (XB >= 16) {
#pragma unroll
      for (int i = 0; i < XB / 16; ++i) *reinterpret_cast<u32x4_t*>(xb + x.lo_x[i]) = st.x[i];
    } else {
      *reinterpret_cast<u32x2_t*>(xb + x.lo_x[0]) = u32x2_t{st.x[0].x, st.x[0].y};
    }
    const int row = tid >> 3, cv = tid & 7;
    const bool slots = 8 * cv < a.M;  // M = 32: the upper 32 slots of the tile stay zero
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4_t*>(eb + (row + 32 * i) * STE + 16 * cv) = slots ? st.e[i] : u32x4_t{0u, 0u, 0u, 0u};
    if (REV) {  // this step's ratio, r_pc = exp(zc[pc-1] - zc[pc]); nothing precedes chunk 0
      if (tid < 64) sm.r[c % 3][tid] = (c < x.c_hi) ? (chunk_of(a, c) > 0 ? exp_fast(nxt.z - st.z) : 0.f) : 1.f;
    } else {
      if (tid < 64) sm.r[(c + 1) % 3][tid] = (c + 1 < x.c_hi) ? exp_fast(st.z - nxt.z) : 1.f;  // past the end: r = 1
    }
  }

  // The staged state of chunk c (written before the last barrier) goes out in
  // whole rows: the Hk slab is contiguous, Hv rows are XW columns long.
  // Chunks outside [0, NC) write an empty range.
  __device__ static __forceinline__ void write_out(const Ctx& x, int c, const Smem& sm) {
    const AbcArgs& a = *x.a;
    const int64_t H = a.H, M = a.M;
    const bool live = MODE == 0 && c >= x.c_lo && c < x.c_hi;
    const int64_t cc = live ? chunk_of(a, c) : 0;
    const int64_t plane = static_cast<int64_t>(x.b * a.NC + cc) * H + x.h;
    uint16_t* hp = static_cast<uint16_t*>(IS_K ? a.hk : a.hv) +
                   (IS_K ? (plane * a.K + x.x0) * M : plane * M * a.V + x.x0);
    const uint32_t slab = IS_K ? static_cast<uint32_t>(XW * M * 2) : static_cast<uint32_t>(((M - 1) * a.V + XW) * 2);
    const rsrc_t rh = make_rsrc(hp, live ? slab : 0u);
    const char* hs = sm.hs[c & 1];
    if constexpr (XB >= 16) {
#pragma unroll
      for (int i = 0; i < XB / 16; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4_t*>(hs + x.lo_o[i]), rh, x.vo_o[i], 0,
                                               kStreamStore);
    } else {
      __builtin_amdgcn_raw_buffer_store_b64(*reinterpret_cast<const u32x2_t*>(hs + x.lo_o[0]), rh, x.vo_o[0], 0, 0);
    }
  }

  // Chunk c, second half: stage the pre-chunk state, scale, add K^T E or E^T V.
  __device__ static __forceinline__ void accumulate(f32x4_t (&acc)[NR], const Ctx& x, int c, Smem& sm) {
    const AbcArgs& a = *x.a;
    const int lane = threadIdx.x & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t H = a.H, M = a.M;
    if constexpr (HS) {
#pragma unroll
      for (int j = 0; j < NR; ++j)
        *reinterpret_cast<u32x2_t*>(sm.hs[c & 1] + x.lo_h[j]) =
            u32x2_t{pack_bf16x2(acc[j][0], acc[j][1]), pack_bf16x2(acc[j][2], acc[j][3])};
    }
    const float* rr = sm.r[c % 3];
    // Hk^T: wave w owns slot block w, tiles j = k blocks.  Hv^T: wave w owns
    // v block w % NR, tiles j = slot blocks (w / NR) * NR + j.
    const int rt = IS_K ? wave : wave % NR;
    const int ct0 = IS_K ? 0 : (wave / NR) * NR;
    if (IS_K) {  // Hk^T rows are slots
      const f32x4_t r4 = *reinterpret_cast<const f32x4_t*>(rr + 16 * wave + 4 * g4);
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j] *= r4;
    } else {     // Hv^T columns are slots
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j] *= rr[16 * (ct0 + j) + c16];
    }
    // A rows: Hk^T -> slots (E), Hv^T -> v (x); B columns: Hk^T -> k (x), Hv^T -> slots (E)
    const char* xt = sm.x[c & 1];
    const char* et = sm.e[c & 1];
    const int lbx = (4 * g4 + (c16 >> 2)) * STX + (c16 & 3) * 8;
    const int lbe = (4 * g4 + (c16 >> 2)) * STE + (c16 & 3) * 8;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const frag fa = IS_K ? S::frag_from_quads(lds_tr16(et, lbe + 32 * s * STE + 32 * rt),
                                                lds_tr16(et, lbe + (32 * s + 16) * STE + 32 * rt))
                           : S::frag_from_quads(lds_tr16(xt, lbx + 32 * s * STX + 32 * rt),
                                                lds_tr16(xt, lbx + (32 * s + 16) * STX + 32 * rt));
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const frag fb = IS_K ? S::frag_from_quads(lds_tr16(xt, lbx + 32 * s * STX + 32 * j),
                                                  lds_tr16(xt, lbx + (32 * s + 16) * STX + 32 * j))
                             : S::frag_from_quads(lds_tr16(et, lbe + 32 * s * STE + 32 * (ct0 + j)),
                                                  lds_tr16(et, lbe + (32 * s + 16) * STE + 32 * (ct0 + j)));
        S::mma(acc[j], fa, fb);
      }
    }
  }

  // Per-slot factors of this lane's accumulator elements: Hk^T rows are slots
  // (4 per lane), Hv^T columns are slots (one per tile).
  // Slots past M (32) are padding: nothing is read for them.
  __device__ static __forceinline__ void slot_scale(f32x4_t (&acc)[NR], const float* z_from, const float* z_to,
                                                    const f32x4_t (&add)[NR], int M) {
    const int lane = threadIdx.x & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int rt = IS_K ? wave : wave % NR;
    const int ct0 = IS_K ? 0 : (wave / NR) * NR;
    if (IS_K) {
      if (16 * rt >= M) return;
      f32x4_t f;
#pragma unroll
      for (int r = 0; r < 4; ++r) f[r] = exp_fast(z_from[16 * rt + 4 * g4 + r] - z_to[16 * rt + 4 * g4 + r]);
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j] += add[j] * f;
    } else {
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const int m = 16 * (ct0 + j) + c16;
        if (m < M) acc[j] += add[j] * exp_fast(z_from[m] - z_to[m]);
      }
    }
  }

  // Whether this lane's accumulator tile j holds real slots (M = 32 pads the
  // slot dimension to 64): Hk^T rows are slots, Hv^T columns are slots.
  __device__ static __forceinline__ bool slot_live(int j, int M) {
    const int lane = threadIdx.x & 63, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int rt = IS_K ? wave : wave % NR;
    const int ct0 = IS_K ? 0 : (wave / NR) * NR;
    return IS_K ? 16 * rt < M : 16 * (ct0 + j) + c16 < M;
  }

  __device__ static void run(const AbcArgs& a, Smem& sm, int b, int h, int x0, int seg, int unit) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    Ctx x;
    x.a = &a;
    x.b = b;
    x.h = h;
    x.x0 = x0;
    x.X = IS_K ? a.K : a.V;
    // chunks of run `seg`: NC split evenly, the first NC mod P runs one longer
    {
      const int base = a.NC / a.P, extra = a.NC % a.P;
      x.c_lo = seg * base + min(seg, extra);
      x.c_hi = x.c_lo + base + (seg < extra ? 1 : 0);
    }
    if constexpr (XB >= 16) {
#pragma unroll
      for (int i = 0; i < XB / 16; ++i) {
        const int v = tid + 256 * i;
        const int row = v / (XW / 8), cv = v % (XW / 8);
        x.vo_x[i] = (row * a.H * x.X + 8 * cv) * 2;
        x.lo_x[i] = row * STX + 16 * cv;
      }
    } else {
      const int row = tid >> 2, cv = tid & 3;
      x.vo_x[0] = (row * a.H * x.X + 4 * cv) * 2;
      x.lo_x[0] = row * STX + 8 * cv;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = (tid >> 3) + 32 * i;
      x.vo_e[i] = (row * a.H * a.M + 8 * (tid & 7)) * 2;
    }
    const int rt = IS_K ? wave : wave % NR;
    const int ct0 = IS_K ? 0 : (wave / NR) * NR;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      // element (row, col) of the transposed tile held by this lane: rows 4 g4 + r, column c16
      x.vo_h[j] = IS_K ? ((16 * j + c16) * a.M + 16 * rt + 4 * g4) * 2
                       : ((16 * (ct0 + j) + c16) * a.V + 16 * rt + 4 * g4) * 2;
      x.lo_h[j] = IS_K ? (16 * j + c16) * STH + (16 * rt + 4 * g4) * 2
                       : (16 * (ct0 + j) + c16) * STH + (16 * rt + 4 * g4) * 2;
    }
    {
      // write-out: thread tid moves bytes [tid XB, tid XB + XB) of the slab's rows
      constexpr int RB = IS_K ? 64 * 2 : XW * 2;  // bytes per staged row
      constexpr int NV = XB >= 16 ? XB / 16 : 1;
      constexpr int VB = XB >= 16 ? 16 : 8;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int byte = (tid + 256 * i) * VB;
        const int row = byte / RB, off = byte % RB;
        x.lo_o[i] = row * STH + off;
        x.vo_o[i] = IS_K ? row * a.M * 2 + off : row * a.V * 2 + off;
        // M = 32: the staged Hk rows hold 64 slots; the upper half is never
        // stored (an offset past every slab, dropped by the range check).
        // Hv rows past M already fall past the slab.
        if (IS_K && off >= a.M * 2) x.vo_o[i] = 0x40000000;
      }
    }
    f32x4_t acc[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // this lane's slice of a run-end state in the workspace (C-layout order)
    auto lsum_at = [&](int run) {
      return a.lsum + ((static_cast<int64_t>(b * a.H + h) * (a.P - 1) + run) * (a.K + a.V) * 64 +
                       static_cast<int64_t>(unit) * (XW * 64) + tid * 4 * NR);
    };
    if (MODE == 0 && !REV && seg > 0) {
      // S_start(seg) from the earlier runs' end states
      const float* zrow = a.zc + (static_cast<int64_t>(b) * a.NC * a.H + h) * a.M;  // + c * H * M
      const int64_t zs = static_cast<int64_t>(a.H) * a.M;
      const float* z_start = zrow + (x.c_lo - 1) * zs;
      const int base = a.NC / a.P, extra = a.NC % a.P;
      for (int i = 0; i < seg; ++i) {
        const int end_i = (i + 1) * base + min(i + 1, extra) - 1;  // last chunk of run i
        f32x4_t l[NR];
        const float* lp = lsum_at(i);
#pragma unroll
        for (int j = 0; j < NR; ++j) l[j] = *reinterpret_cast<const f32x4_t*>(lp + 4 * j);
        slot_scale(acc, zrow + end_i * zs, z_start, l, a.M);
      }
    }
    if (MODE == 0 && REV && x.c_lo < x.c_hi) {
      // the final states' gradient and the later runs' end states, carried to
      // this run's first chunk p = NC-1-c_lo
      const float* zrow = a.zc + (static_cast<int64_t>(b) * a.NC * a.H + h) * a.M;
      const int64_t zs = static_cast<int64_t>(a.H) * a.M;
      const float* z_from = zrow + (a.NC - 1 - x.c_lo) * zs;
      const float* ge = IS_K ? a.gk_end : a.gv_end;
      if (ge != nullptr) {
        const int64_t fb = static_cast<int64_t>(b) * a.H + h;
        const float* gb = ge + (IS_K ? (fb * a.K + x0) * a.M : fb * a.M * a.V + x0);
        f32x4_t l[NR];
#pragma unroll
        for (int j = 0; j < NR; ++j)
          l[j] = slot_live(j, a.M) ? *reinterpret_cast<const f32x4_t*>(gb + x.vo_h[j] / 2) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        slot_scale(acc, z_from, zrow + (a.NC - 1) * zs, l, a.M);
      }
      const int base = a.NC / a.P, extra = a.NC % a.P;
      for (int i = 0; i < seg; ++i) {
        const int hi_i = (i + 1) * base + min(i + 1, extra);  // run i's steps end here
        f32x4_t l[NR];
        const float* lp = lsum_at(i);
#pragma unroll
        for (int j = 0; j < NR; ++j) l[j] = *reinterpret_cast<const f32x4_t*>(lp + 4 * j);
        slot_scale(acc, z_from, zrow + (a.NC - hi_i - 1) * zs, l, a.M);  // a_i - 1 = NC - hi_i - 1
      }
    }

    const int nc = x.c_hi - x.c_lo;
    if (nc > 0) {
      Stage st[D];
#pragma unroll
      for (int i = 0; i < D; ++i) load(st[i], x, x.c_lo + i);
      if (!REV && tid < 64) {
        // r of the run's first chunk (0 at the sequence start: nothing before it; 1 on padding slots)
        const float* zr = a.zc + ((static_cast<int64_t>(b) * a.NC + x.c_lo) * a.H + h) * a.M + tid;
        sm.r[x.c_lo % 3][tid] =
            tid >= a.M ? 1.f : x.c_lo == 0 ? 0.f : exp_fast(zr[-static_cast<int64_t>(a.H) * a.M] - zr[0]);
      }
      __syncthreads();
      const int ncp = (nc + D - 1) / D * D;
      for (int c0 = x.c_lo; c0 < x.c_lo + ncp; c0 += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
          const int c = c0 + i;
          stage_in(st[i], st[(i + 1) % D], x, c, sm);
          load(st[i], x, c + D);
          __syncthreads();
          if constexpr (HS) write_out(x, c - 1, sm);
          accumulate(acc, x, c, sm);
        }
      }
      if constexpr (HS) {
        __syncthreads();
        write_out(x, x.c_lo + ncp - 1, sm);
      }
    }

    if (MODE == 1) {
      float* lp = const_cast<float*>(lsum_at(seg));
#pragma unroll
      for (int j = 0; j < NR; ++j) *reinterpret_cast<f32x4_t*>(lp + 4 * j) = acc[j];
      return;
    }
    float* fp = IS_K ? a.hk_final : a.hv_final;
    if (REV || fp == nullptr || x.c_hi != a.NC) return;
    const int64_t fb = static_cast<int64_t>(b) * a.H + h;
    float* base = fp + (IS_K ? (fb * a.K + x0) * a.M : fb * a.M * a.V + x0);
#pragma unroll
    for (int j = 0; j < NR; ++j)
      if (slot_live(j, a.M)) *reinterpret_cast<f32x4_t*>(base + x.vo_h[j] / 2) = acc[j];
  }
};

template <int XW, int MODE, bool REV>
__global__ __launch_bounds__(256) void abc_states(const AbcArgs a) {
  using SK = AbcStates<true, XW, MODE, REV>;
  using SV = AbcStates<false, XW, MODE, REV>;
  static_assert(sizeof(typename SK::Smem) == sizeof(typename SV::Smem), "one LDS layout");
  __shared__ __align__(16) typename SK::Smem sm;
  const int nk = a.K / XW, tiles = nk + a.V / XW;
  const int nseg = MODE == 1 ? a.P - 1 : a.P;
  // the units of one (b, h) share blockIdx modulo 8 (one XCD, so E comes from its L2)
  const int bx = blockIdx.x;
  const int xcd = bx & 7, slot = bx >> 3;
  const int pair = 8 * (slot / (tiles * nseg)) + xcd;
  const int u = slot % (tiles * nseg);
  const int tile = u % tiles, seg = u / tiles;
  if (pair >= a.B * a.H) return;
  if (tile < nk) {
    SK::run(a, sm, pair / a.H, pair % a.H, XW * tile, seg, tile);
  } else {
    SV::run(a, *reinterpret_cast<typename SV::Smem*>(&sm), pair / a.H, pair % a.H, XW * (tile - nk), seg, tile);
  }
}

// Runs per sequence: enough that the (b, h, 64-column tile, run) units of
// the state walk reach about three workgroups per CU, each run at least 8
// chunks, at most 8 runs.  Independent of the tile width, so every width
// gives the same arithmetic.  GDR_ABC_SEGMENTS forces a count.  Measured on
// B=2, H=4, K=256, V=512 (MI355X, whole call): 64-wide tiles with 1 / 2 / 4 /
// 8 runs 230 / 230 / 211 / 195 us; 32-wide 217 / 237 / 233 / 213 us.
int abc_segments(int B, int H, int K, int V, int NC) {
  int p = 0;
  if (const char* env = getenv("GDR_ABC_SEGMENTS")) p = atoi(env);
  if (p <= 0) {
    const int64_t units64 = static_cast<int64_t>(B) * H * ((K + V) / 64);
    p = static_cast<int>((768 + units64 - 1) / units64);
  }
  p = std::min(p, 8);
  p = std::min(p, NC / 8);
  return std::max(p, 1);
}

// Tile width: the widest whose walk units (with the runs) give at least one
// workgroup per CU, else the widest with half as many; GDR_ABC_XW forces one
// (16, 32 or 64).
int abc_tile_width(const AbcArgs& a) {
  if (const char* env = getenv("GDR_ABC_XW")) {
    const int w = atoi(env);
    if (w == 16 || w == 32 || w == 64) return w;
  }
  const int64_t pairs = static_cast<int64_t>(a.B) * a.H;
  for (int w = 64; w > 16; w /= 2)
    if (pairs * ((a.K + a.V) / w) * a.P >= 256) return w;
  for (int w = 64; w > 16; w /= 2)
    if (pairs * ((a.K + a.V) / w) * a.P >= 128) return w;
  return 16;
}

hipError_t launch_abc(const AbcArgs& a, hipStream_t stream) {
  if (a.NC > 0) {
    hipLaunchKernelGGL(abc_chunk_lse, dim3(a.B * a.NC * a.H), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.NC > 0) {
    hipLaunchKernelGGL(abc_carry, dim3(a.B * a.H * (a.M / 4)), dim3(64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.NC > 0) {
    hipLaunchKernelGGL(abc_weights, dim3(a.B * a.NC * a.H), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int xw = abc_tile_width(a);
  const int tiles_w = (a.K + a.V) / xw;
  const int pairs8 = (a.B * a.H + 7) / 8;
  if (a.P > 1) {  // end states of every run but the last
    const dim3 g1(8 * tiles_w * (a.P - 1) * pairs8);
    if (xw == 64) hipLaunchKernelGGL((abc_states<64, 1, false>), g1, dim3(256), 0, stream, a);
    else if (xw == 32) hipLaunchKernelGGL((abc_states<32, 1, false>), g1, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((abc_states<16, 1, false>), g1, dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid(8 * tiles_w * a.P * pairs8);
  if (xw == 64) hipLaunchKernelGGL((abc_states<64, 0, false>), grid, dim3(256), 0, stream, a);
  else if (xw == 32) hipLaunchKernelGGL((abc_states<32, 0, false>), grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((abc_states<16, 0, false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_abc_bwd(const AbcArgs& a, hipStream_t stream) {
  if (a.NC == 0) return hipSuccess;
  hipLaunchKernelGGL(abc_bwd_weights, dim3(a.B * a.NC * a.H), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int xw = abc_tile_width(a);
  const int tiles_w = (a.K + a.V) / xw;
  const int pairs8 = (a.B * a.H + 7) / 8;
  if (a.P > 1) {  // end states of every run but the last (in reverse chunk order)
    const dim3 g1(8 * tiles_w * (a.P - 1) * pairs8);
    if (xw == 64) hipLaunchKernelGGL((abc_states<64, 1, true>), g1, dim3(256), 0, stream, a);
    else if (xw == 32) hipLaunchKernelGGL((abc_states<32, 1, true>), g1, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((abc_states<16, 1, true>), g1, dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid(8 * tiles_w * a.P * pairs8);
  if (xw == 64) hipLaunchKernelGGL((abc_states<64, 0, true>), grid, dim3(256), 0, stream, a);
  else if (xw == 32) hipLaunchKernelGGL((abc_states<32, 0, true>), grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((abc_states<16, 0, true>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdr
