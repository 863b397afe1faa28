// Launch-argument structs and launcher declarations shared by the host API
// and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace gdr {

// Serial chunk scan (plain scan, segmented final pass, segment summaries).
struct ScanArgs {
  const void* k;
  const void* w;
  const void* u;
  const float* g_cum;
  const float* h_in;   // h0 or seg_init (nullable)
  void* h;             // pre-chunk states (nullable)
  void* v_new;         // (nullable)
  float* h_out;        // hT or seg_state (nullable)
  float* trans_out;    // seg_trans (summaries only)
  const float* decay;  // per-key-channel decay: [NT, H, DK] channel decays of every chunk (else null)
  const void* q;       // fused chunk output (scan2 with FO): queries, output o, scale
  void* o;
  float scale;
  // prepare fused in (scan2 with PREP): v, g, beta in place of w, u, g_cum;
  // g_cum_out (nullable) receives the chunk-local cumsum of g
  const void* v;
  const float* g;
  const float* beta;
  float* g_cum_out;
  int32_t H;
  int32_t DV;
  int32_t in_vk;       // layout of h_in: 1 = [.., DV, DK], 0 = [.., DK, DV]
  int32_t out_vk;      // layout of h_out
  int32_t n_rows;
  int32_t n_blk;       // column blocks per (row, head)
  Row rows[kMaxRows];
};

// Chunk-parallel kernels (prepare, output): rows in natural order, each
// workgroup finds its row by the row's first chunk.
struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;       // v (prepare) or v_new (output)
  const float* g;      // g (prepare) or g_cum (output)
  const float* beta;
  const void* h;       // output: pre-chunk states
  float* g_cum;        // prepare output
  void* w;             // prepare output
  void* u;             // prepare output
  void* o;             // output output
  float scale;
  int32_t H;
  int32_t n_rows;
  int32_t n_chunks;    // chunks covered by this launch
  int32_t chunk_base;  // h row of this launch's first chunk
  Row rows[kMaxRows];  // chunk_off relative to chunk_base
};

// Reverse state scan (rows as in ScanArgs; in_idx = dhT row, out_idx = dh0 row).
struct ScanBwdArgs {
  const void* q;
  const void* k;
  const void* w;
  const float* g_cum;
  const void* dO;
  const void* dv_local;
  const float* dhT;    // nullable
  void* dh;            // [NT, H, DV, DK] storage dtype (nullable)
  void* dv;            // write-vector gradient [B, T, H, DV] (nullable)
  float* dh0;          // nullable
  float scale;
  int32_t H;
  int32_t DV;
  int32_t state_vk;    // layout of dhT / dh0
  int32_t n_rows;
  Row rows[kMaxRows];
};

struct ComposeArgs {
  const float* seg_state;
  const float* seg_trans;
  const float* h0;
  float* seg_init;
  float* hT;
  int32_t H;
  int32_t DV;
  int32_t P;
  int32_t N;
  int32_t state_vk;
};

// Pairwise combination of half-segment summaries: for every segment s,
// (S, M) = (M_b S_a + S_b, M_b M_a) with a = half 2s, b = half 2s + 1.
struct CombineArgs {
  const float* half_state;  // [2 n_seg, H, DV, DK]
  const float* half_trans;  // [2 n_seg, H, DK, DK]
  float* seg_state;         // [n_seg, H, DV, DK]
  float* seg_trans;         // [n_seg, H, DK, DK]
  int32_t H;
  int32_t DV;
  int32_t n_seg;
};

// Forward (slot-state construction) and reverse (dH recurrence) share the
// state walk.  Reverse: k = q, v = dO, s = dscore, pw = p; z is the
// forward's normaliser (input); e / e2 hold the key- / value-side weights;
// hk / hv receive dhk / dhv; gk_end / gv_end are the final states' gradients.
struct AbcArgs {
  const void* k;
  const void* v;
  const void* s;
  const void* pw;      // reverse: slot weights of the value read
  float* z;            // forward: nullable full normaliser (output); reverse: input
  float* lse;          // workspace: [B, NC, H, M] log-sum-exp of each chunk
  float* zc;           // workspace: [B, NC, H, M] normaliser at chunk ends
  void* e;             // workspace: [B, T, H, M] key-side weights, storage dtype
  void* e2;            // workspace: value-side weights (the forward: == e)
  float* lsum;         // workspace: [B*H, P-1, K+V, M] end states of the runs (P > 1)
  void* hk;
  void* hv;
  float* hk_final;
  float* hv_final;
  const float* gk_end;  // reverse: nullable [B, H, K, M]
  const float* gv_end;  // reverse: nullable [B, H, M, V]
  float scale;          // reverse: score scale
  int32_t B;
  int32_t T;
  int32_t H, K, M, V;
  int32_t NC;
  int32_t P;           // runs per sequence of the state walk
};

// Per-key-channel decay: chunk preparation and chunk output (one workgroup
// per (chunk, head) each; rows as in ChunkArgs).
struct KdaArgs {
  const void* q;
  const void* k;
  const void* v;       // v (prepare) or v_new (output)
  const float* g;      // prepare: per-channel log decays [B,T,H,DK]; output: g_cum
  const float* beta;
  const void* h;       // output: pre-chunk states
  float* g_cum;        // prepare outputs ...
  void* w;
  void* u;
  void* kg;
  float* decay;        // [NT, H, DK]
  void* o;             // output output
  float scale;
  int32_t H;
  int32_t n_rows;
  int32_t n_chunks;
  int32_t chunk_base;
  Row rows[kMaxRows];
};

using LaunchFn = hipError_t (*)(const void* args, int grid, hipStream_t stream);

// Lookup of an instantiated kernel; nullptr when the combination is not built.
LaunchFn find_scan(int dtype, int dk, int bv, int waves, int stages, int mode);
LaunchFn find_scan2(int dk, int bv, int waves, int stages, int mode, bool kd);
LaunchFn find_scan2_fused(int dk, int bv, int waves, int stages);  // plain pass + chunk output (bf16)
// The same plain pass (optionally with per-channel decay or the fused output)
// in its dense form, three workgroups per CU; null where there is none.
LaunchFn find_scan2_dense(int dk, int bv, int waves, int stages, int mode, bool kd, bool fo);
// The plain pass with the chunk prepare and the chunk output fused (bf16,
// DK = 128, 64-column blocks, four waves, the dense form).
LaunchFn find_scan2_prep(int dk);
LaunchFn find_prepare(int dtype, int dk, int dv);
LaunchFn find_prepare2(int dk, int dv);
LaunchFn find_kda_prepare(int dk, int dv);
LaunchFn find_kda_output(int dk, int dv);
LaunchFn find_output(int dtype, int dk, int dv);
LaunchFn find_output2(int dk, int dv);
LaunchFn find_compose(int dk, int P);
LaunchFn find_combine(int dk);
LaunchFn find_dv_local(int dk, int dv);
LaunchFn find_scan_bwd(int dk);
hipError_t launch_abc(const AbcArgs& a, hipStream_t s);
hipError_t launch_abc_bwd(const AbcArgs& a, hipStream_t s);

// ABC read per chunk: scores, softmax over the slots, value read.
struct AbcOutArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* s;
  const float* z;      // the forward's normaliser [B, T, H, M]
  const void* hk;      // [B, NC, H, K, M]
  const void* hv;      // [B, NC, H, M, V]
  void* o;             // [B, T, H, V]
  void* p;             // nullable [B, T, H, M]
  float scale;
  int32_t B, T, H, K, V, NC;
  int32_t M;           // slots: 64, or 32 (padded to 64 inside the kernel)
};
bool abc_out_supported(int K, int V);
hipError_t launch_abc_out(const AbcOutArgs& a, hipStream_t s);
int abc_segments(int B, int H, int K, int V, int NC);

}  // namespace gdr
