// C-ABI entry points (include/gdr.h): argument checks, planning, dispatch.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "../../include/gdr.h"
#include "kernels.hpp"
#include "plan.hpp"

namespace {

thread_local std::string g_err;

gdr_status fail(gdr_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

gdr_status need(const void* p, const char* name) {
  if (p == nullptr) return fail(GDR_ERR_INVALID_ARG, std::string(name) + " must not be NULL");
  if (!aligned16(p)) return fail(GDR_ERR_INVALID_ARG, std::string(name) + " must be 16-byte aligned");
  return GDR_OK;
}

gdr_status opt(const void* p, const char* name) {
  if (p != nullptr && !aligned16(p)) return fail(GDR_ERR_INVALID_ARG, std::string(name) + " must be 16-byte aligned");
  return GDR_OK;
}

#define GDR_TRY(x)                   \
  do {                               \
    gdr_status _s = (x);             \
    if (_s != GDR_OK) return _s;     \
  } while (0)

gdr_status parse(const gdr_problem* p, gdr::Problem& out) {
  if (p == nullptr) return fail(GDR_ERR_INVALID_ARG, "problem must not be NULL");
  std::string err;
  if (!gdr::parse_problem(p->B, p->T, p->H, p->DK, p->DV, p->N, p->cu_seqlens_host, p->dtype, p->state_layout,
                          p->state_indices_host, p->pool_size, out, err))
    return fail(GDR_ERR_INVALID_ARG, err);
  return GDR_OK;
}

gdr_status tile_for(const gdr::Problem& pr, const gdr_tile* tile, int mode, int64_t rows, gdr::Tile& t) {
  std::string err;
  int32_t req[3];
  const int32_t* r = nullptr;
  if (tile != nullptr) {
    req[0] = tile->bv;
    req[1] = tile->waves;
    req[2] = tile->stages;
    r = req;
  }
  if (!gdr::choose_tile(pr, r, mode, rows, t, err)) return fail(GDR_ERR_UNSUPPORTED, err);
  return GDR_OK;
}

// bfloat16 up to 128 x 128 runs the gfx950 kernels of prepare2.hip /
// output2.hip (each one workgroup per (chunk, head)); DK or DV = 256
// and float32 run the generic kernels (per (chunk, head); output per 64 value
// columns).
constexpr int kCUs = 256;  // compute units of one MI355X

bool fast_bf16(const gdr::Problem& pr) { return pr.dtype == GDR_BF16 && pr.DK <= 128 && pr.DV <= 128; }

gdr_status hip_fail(hipError_t e, const char* what) {
  return fail(GDR_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// The chunk output fused into the plain pass (queries, output, scale).
struct FusedOut {
  const void* q;
  void* o;
  float scale;
};

// The plain pass has the chunk output fused for bfloat16 with DK 64 or 128
// and the scalar gate on the one-buffer four-wave tiles.
bool fusable(const gdr::Problem& pr, const gdr::Tile& t) {
  return pr.dtype == GDR_BF16 && pr.DV <= 128 && gdr::find_scan2_fused(pr.DK, t.bv, t.waves, t.stages) != nullptr;
}

gdr_status run_scan(const gdr::Problem& pr, const gdr::Tile& t, int mode, int P, const void* k, const void* w,
                    const void* u, const float* g_cum, const float* h_in, int in_vk, void* h, void* v_new,
                    float* h_out, int out_vk, float* trans_out, hipStream_t stream, const float* decay = nullptr,
                    int split = 1, const FusedOut* fo = nullptr) {
  const int kmode = (mode == 1) ? gdr::summary_kernel_mode(pr) : 0;
  gdr::LaunchFn fn = fo != nullptr      ? gdr::find_scan2_fused(pr.DK, t.bv, t.waves, t.stages)
                     : decay != nullptr ? gdr::find_scan2(pr.DK, t.bv, t.waves, t.stages, kmode, true)
                                        : gdr::find_scan(pr.dtype, pr.DK, t.bv, t.waves, t.stages, kmode);
  if (fn == nullptr) return fail(GDR_ERR_UNSUPPORTED, "no scan kernel for this dtype/DK/tile");
  const bool has_in = (h_in != nullptr);
  const bool has_out = (h_out != nullptr);
  std::vector<gdr::Launch> plan = gdr::plan_scan(pr, t, mode, P, has_in, has_out, split);
  gdr::ScanArgs a;
  memset(&a, 0, sizeof(a));
  a.k = k;
  a.w = w;
  a.u = u;
  a.g_cum = g_cum;
  a.h_in = h_in;
  a.h = h;
  a.v_new = v_new;
  a.h_out = h_out;
  a.trans_out = trans_out;
  a.decay = decay;
  if (fo != nullptr) {
    a.q = fo->q;
    a.o = fo->o;
    a.scale = fo->scale;
  }
  a.H = pr.H;
  a.DV = pr.DV;
  a.in_vk = in_vk;
  a.out_vk = out_vk;
  a.n_blk = gdr::scan_blocks(pr, t, mode);
  // A launch with more workgroups than two per CU runs the dense form where
  // one exists (the same results bit for bit); GDR_SCAN_DENSE=0 / 1 forces
  // the full / dense form.
  gdr::LaunchFn dense = (pr.dtype == GDR_BF16 && kmode == 0)
                            ? gdr::find_scan2_dense(pr.DK, t.bv, t.waves, t.stages, 0, decay != nullptr, fo != nullptr)
                            : nullptr;
  int force = -1;
  if (const char* env = getenv("GDR_SCAN_DENSE")) force = atoi(env) != 0 ? 1 : 0;
  for (const gdr::Launch& l : plan) {
    if (l.grid == 0) continue;
    a.n_rows = static_cast<int32_t>(l.rows.size());
    memcpy(a.rows, l.rows.data(), l.rows.size() * sizeof(gdr::Row));
    const bool use_dense = dense != nullptr && (force >= 0 ? force == 1 : l.grid > 2 * kCUs);
    hipError_t e = (use_dense ? dense : fn)(&a, l.grid, stream);
    if (e != hipSuccess) return hip_fail(e, "scan launch");
  }
  return GDR_OK;
}

}  // namespace

namespace gdr_internal {
void set_last_error(const std::string& m) { g_err = m; }
}  // namespace gdr_internal

extern "C" {

const char* gdr_status_string(gdr_status s) {
  switch (s) {
    case GDR_OK: return "GDR_OK";
    case GDR_ERR_INVALID_ARG: return "GDR_ERR_INVALID_ARG";
    case GDR_ERR_UNSUPPORTED: return "GDR_ERR_UNSUPPORTED";
    case GDR_ERR_HIP: return "GDR_ERR_HIP";
  }
  return "unknown gdr_status";
}

const char* gdr_last_error(void) { return g_err.c_str(); }

int64_t gdr_num_chunks(const gdr_problem* p) {
  gdr::Problem pr;
  if (parse(p, pr) != GDR_OK) return -1;
  return pr.n_chunks;
}

gdr_status gdr_chunk_prepare(const gdr_problem* p, const void* k, const void* v, const float* g,
                             const float* beta, float* g_cum, void* w, void* u, void* stream) {
  g_err.clear();
  gdr::Problem pr;
  GDR_TRY(parse(p, pr));
  GDR_TRY(need(k, "k"));
  GDR_TRY(need(v, "v"));
  GDR_TRY(need(g, "g"));
  GDR_TRY(need(beta, "beta"));
  GDR_TRY(need(g_cum, "g_cum"));
  GDR_TRY(need(w, "w"));
  GDR_TRY(need(u, "u"));
  gdr::LaunchFn fn = gdr::find_prepare(pr.dtype, pr.DK, pr.DV);
  if (fn == nullptr) return fail(GDR_ERR_UNSUPPORTED, "no prepare kernel for this dtype/DK/DV");
  gdr::ChunkArgs a;
  memset(&a, 0, sizeof(a));
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.g_cum = g_cum;
  a.w = w;
  a.u = u;
  a.H = pr.H;
  for (const gdr::Launch& l : gdr::plan_chunks(pr, 1)) {
    a.n_rows = static_cast<int32_t>(l.rows.size());
    a.n_chunks = l.n_chunks;
    a.chunk_base = l.chunk_base;
    memcpy(a.rows, l.rows.data(), l.rows.size() * sizeof(gdr::Row));
    hipError_t e = fn(&a, l.grid, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "prepare launch");
  }
  return GDR_OK;
}

gdr_status gdr_state_scan(const gdr_problem* p, const gdr_tile* tile, const gdr_segments* seg, const void* k,
                          const void* w, const void* u, const float* g_cum, const float* h0, void* h, void* v_new,
                          float* hT, void* stream) {
  g_err.clear();
  gdr::Problem pr;
  GDR_TRY(parse(p, pr));
  GDR_TRY(need(k, "k"));
  GDR_TRY(need(w, "w"));
  GDR_TRY(need(u, "u"));
  GDR_TRY(need(g_cum, "g_cum"));
  GDR_TRY(opt(h0, "h0"));
  GDR_TRY(opt(h, "h"));
  GDR_TRY(opt(v_new, "v_new"));
  GDR_TRY(opt(hT, "hT"));
  int mode = 0, P = 1;
  const float* h_in = h0;
  int in_vk = pr.state_vk;
  if (seg != nullptr) {
    if (!pr.pool_idx.empty()) return fail(GDR_ERR_UNSUPPORTED, "indexed states are supported by the serial scan only");
    if (seg->n_segments < 1) return fail(GDR_ERR_INVALID_ARG, "n_segments must be >= 1");
    GDR_TRY(need(seg->seg_init, "seg_init"));
    mode = 2;
    P = seg->n_segments;
    h_in = seg->seg_init;
    in_vk = 1;
  }
  gdr::Tile t;
  GDR_TRY(tile_for(pr, tile, 0, static_cast<int64_t>(pr.N) * P, t));
  return run_scan(pr, t, mode, P, k, w, u, g_cum, h_in, in_vk, h, v_new, hT, pr.state_vk, nullptr,
                  static_cast<hipStream_t>(stream));
}

gdr_status gdr_state_scan_output(const gdr_problem* p, const gdr_tile* tile, const gdr_segments* seg, const void* q,
                                 const void* k, const void* w, const void* u, const float* g_cum, const float* h0,
                                 float scale, void* h, void* v_new, float* hT, void* o, void* stream) {
  g_err.clear();
  gdr::Problem pr;
  GDR_TRY(parse(p, pr));
  GDR_TRY(need(q, "q"));
  GDR_TRY(need(k, "k"));
  GDR_TRY(need(w, "w"));
  GDR_TRY(need(u, "u"));
  GDR_TRY(need(g_cum, "g_cum"));
  GDR_TRY(need(o, "o"));
  GDR_TRY(opt(h0, "h0"));
  GDR_TRY(opt(h, "h"));
  GDR_TRY(opt(v_new, "v_new"));
  GDR_TRY(opt(hT, "hT"));
  int mode = 0, P = 1;
  const float* h_in = h0;
  int in_vk = pr.state_vk;
  if (seg != nullptr) {
    if (!pr.pool_idx.empty()) return fail(GDR_ERR_UNSUPPORTED, "indexed states are supported by the serial scan only");
    if (seg->n_segments < 1) return fail(GDR_ERR_INVALID_ARG, "n_segments must be >= 1");
    GDR_TRY(need(seg->seg_init, "seg_init"));
    mode = 2;
    P = seg->n_segments;
    h_in = seg->seg_init;
    in_vk = 1;
  }
  gdr::Tile t;
  GDR_TRY(tile_for(pr, tile, 0, static_cast<int64_t>(pr.N) * P, t));
  if (tile == nullptr && !fusable(pr, t)) {
    // the planner's tile has no fused form: the one-buffer four-wave tile of 64 columns
    const gdr::Tile t64{64, 4, 2};
    if (fusable(pr, t64)) t = t64;
  }
  if (fusable(pr, t)) {
    const FusedOut fo{q, o, scale};
    return run_scan(pr, t, mode, P, k, w, u, g_cum, h_in, in_vk, h, v_new, hT, pr.state_vk, nullptr,
                    static_cast<hipStream_t>(stream), nullptr, 1, &fo);
  }
  // no fused kernel: the plain pass, then the chunk output from h and v_new
  if (h == nullptr || v_new == nullptr)
    return fail(GDR_ERR_UNSUPPORTED, "this dtype / DK / tile has no fused output: h and v_new must be given");
  GDR_TRY(run_scan(pr, t, mode, P, k, w, u, g_cum, h_in, in_vk, h, v_new, hT, pr.state_vk, nullptr,
                   static_cast<hipStream_t>(stream)));
  return gdr_chunk_output(p, q, k, v_new, h, g_cum, scale, o, stream);
}

gdr_status gdr_chunk_forward(const gdr_problem* p, const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const float* h0, float scale, float* g_cum, void* h, void* v_new,
                             float* hT, void* o, void* stream) {
  g_err.clear();
  gdr::Problem pr;
  GDR_TRY(parse(p, pr));
  GDR_TRY(need(q, "q"));
  GDR_TRY(need(k, "k"));
  GDR_TRY(need(v, "v"));
  GDR_TRY(need(g, "g"));
  GDR_TRY(need(beta, "beta"));
  GDR_TRY(need(o, "o"));
  GDR_TRY(opt(h0, "h0"));
  GDR_TRY(opt(g_cum, "g_cum"));
  GDR_TRY(opt(h, "h"));
  GDR_TRY(opt(v_new, "v_new"));
  GDR_TRY(opt(hT, "hT"));
  if (pr.dtype != GDR_BF16 || pr.DK != 128 || pr.DV % 64 != 0)
    return fail(GDR_ERR_UNSUPPORTED, "the fused forward step is built for bfloat16, DK = 128, DV a multiple of 64");
  gdr::LaunchFn fn = gdr::find_scan2_prep(pr.DK);
  if (fn == nullptr) return fail(GDR_ERR_UNSUPPORTED, "no fused forward kernel for this DK");
  const gdr::Tile t{64, 4, 2};
  gdr::ScanArgs a;
  memset(&a, 0, sizeof(a));
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.g_cum_out = g_cum;
  a.q = q;
  a.o = o;
  a.scale = scale;
  a.h_in = h0;
  a.h = h;
  a.v_new = v_new;
  a.h_out = hT;
  a.H = pr.H;
  a.DV = pr.DV;
  a.in_vk = pr.state_vk;
  a.out_vk = pr.state_vk;
  a.n_blk = gdr::scan_blocks(pr, t, 0);
  for (const gdr::Launch& l : gdr::plan_scan(pr, t, 0, 1, h0 != nullptr, hT != nullptr)) {
    if (l.grid == 0) continue;
    a.n_rows = static_cast<int32_t>(l.rows.size());
    memcpy(a.rows, l.rows.data(), l.rows.size() * sizeof(gdr::Row));
    hipError_t e = fn(&a, l.grid, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "forward launch");
  }
  return GDR_OK;
}

gdr_status gdr_chunk_output(const gdr_problem* p, const void* q, const void* k, const void* v_new, const void* h,
                            const float* g_cum, float scale, void* o, void* stream) {
  g_err.clear();
  gdr::Problem pr;
  GDR_TRY(parse(p, pr));
  GDR_TRY(need(q, "q"));
  GDR_TRY(need(k, "k"));
  GDR_TRY(need(v_new, "v_new"));
  GDR_TRY(need(h, "h"));
  GDR_TRY(need(g_cum, "g_cum"));
  GDR_TRY(need(o, "o"));
  gdr::LaunchFn fn = gdr::find_output(pr.dtype, pr.DK, pr.DV);
  if (fn == nullptr) return fail(GDR_ERR_UNSUPPORTED, "no output kernel for this dtype/DK/DV");
  gdr::ChunkArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v_new;
  a.g = g_cum;
  a.h = h;
  a.o = o;
  a.scale = scale;
  a.H = pr.H;
  // bfloat16 up to 128 x 128: one workgroup per (chunk, head) for all value columns; else per 64 columns
  for (const gdr::Launch& l : gdr::plan_chunks(pr, fast_bf16(pr) ? 1 : pr.DV / 64)) {
    a.n_rows = static_cast<int32_t>(l.rows.size());
    a.n_chunks = l.n_chunks;
    a.chunk_base = l.chunk_base;
    memcpy(a.rows, l.rows.data(), l.rows.size() * sizeof(gdr::Row));
    hipError_t e = fn(&a, l.grid, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "output launch");
  }
  return GDR_OK;
}

gdr_status gdr_chunk_dv_local(const gdr_problem* p, const void* q, const void* k, const float* g_cum,
                              const void* dO, float scale, void* dv_local, void* stream) {
  g_err.clear();
  gdr::Problem pr;
  GDR_TRY(parse(p, pr));
  GDR_TRY(need(q, "q"));
  GDR_TRY(need(k, "k"));
  GDR_TRY(need(g_cum, "g_cum"));
  GDR_TRY(need(dO, "dO"));
  GDR_TRY(need(dv_local, "dv_local"));
  if (pr.dtype != GDR_BF16) return fail(GDR_ERR_UNSUPPORTED, "the reverse pass is built for bfloat16 storage");
  gdr::LaunchFn fn = gdr::find_dv_local(pr.DK, pr.DV);
  if (fn == nullptr) return fail(GDR_ERR_UNSUPPORTED, "no dv_local kernel for this DK/DV");
  gdr::ChunkArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = dO;
  a.g = g_cum;
  a.o = dv_local;
  a.scale = scale;
  a.H = pr.H;
  for (const gdr::Launch& l : gdr::plan_chunks(pr, 1)) {
    a.n_rows = static_cast<int32_t>(l.rows.size());
    a.n_chunks = l.n_chunks;
    a.chunk_base = l.chunk_base;
    memcpy(a.rows, l.rows.data(), l.rows.size() * sizeof(gdr::Row));
    hipError_t e = fn(&a, l.grid, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "dv_local launch");
  }
  return GDR_OK;
}

gdr_status gdr_state_scan_bwd(const gdr_problem* p, const void* q, const void* k, const void* w, const float* g_cum,
                              const void* dO, const void* dv_local, const float* dhT, float scale, void* dh,
                              void* dv_new_grad, float* dh0, void* stream) {
  g_err.clear();
  gdr::Problem pr;
  GDR_TRY(parse(p, pr));
  if (!pr.pool_idx.empty()) return fail(GDR_ERR_UNSUPPORTED, "indexed states are supported by the forward scan only");
  GDR_TRY(need(q, "q"));
  GDR_TRY(need(k, "k"));
  GDR_TRY(need(w, "w"));
  GDR_TRY(need(g_cum, "g_cum"));
  GDR_TRY(need(dO, "dO"));
  GDR_TRY(need(dv_local, "dv_local"));
  GDR_TRY(opt(dhT, "dhT"));
  GDR_TRY(opt(dh, "dh"));
  GDR_TRY(opt(dv_new_grad, "dv_new_grad"));
  GDR_TRY(opt(dh0, "dh0"));
  if (pr.dtype != GDR_BF16) return fail(GDR_ERR_UNSUPPORTED, "the reverse pass is built for bfloat16 storage");
  gdr::LaunchFn fn = gdr::find_scan_bwd(pr.DK);
  if (fn == nullptr) return fail(GDR_ERR_UNSUPPORTED, "no reverse scan kernel for this DK");
  if (pr.DV % 64 != 0) return fail(GDR_ERR_UNSUPPORTED, "the reverse scan takes 64-column blocks");
  gdr::ScanBwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.w = w;
  a.g_cum = g_cum;
  a.dO = dO;
  a.dv_local = dv_local;
  a.dhT = dhT;
  a.dh = dh;
  a.dv = dv_new_grad;
  a.dh0 = dh0;
  a.scale = scale;
  a.H = pr.H;
  a.DV = pr.DV;
  a.state_vk = pr.state_vk;
  gdr::Tile t;
  t.bv = 64;
  t.waves = 4;
  t.stages = 2;
  for (const gdr::Launch& l : gdr::plan_scan(pr, t, 0, 1, dhT != nullptr, dh0 != nullptr)) {
    a.n_rows = static_cast<int32_t>(l.rows.size());
    memcpy(a.rows, l.rows.data(), l.rows.size() * sizeof(gdr::Row));
    hipError_t e = fn(&a, l.grid, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "reverse scan launch");
  }
  return GDR_OK;
}

size_t gdr_segment_summaries_workspace_size(const gdr_problem* p, int32_t n_segments) {
  g_err.clear();
  gdr::Problem pr;
  if (parse(p, pr) != GDR_OK) return 0;  // (gdr_last_error says why)
  if (n_segments < 1) {
    fail(GDR_ERR_INVALID_ARG, "n_segments must be >= 1");
    return 0;
  }
  if (gdr::summary_split(pr, n_segments) != 2) return 0;
  // the half-segment summaries: 2 N P (S_loc, M) pairs in FP32
  return static_cast<size_t>(2) * pr.N * n_segments * pr.H * pr.DK * (pr.DV + pr.DK) * sizeof(float);
}

gdr_status gdr_segment_summaries_ws(const gdr_problem* p, const gdr_tile* tile, int32_t n_segments, const void* k,
                                    const void* w, const void* u, const float* g_cum, float* seg_state,
                                    float* seg_trans, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  gdr::Problem pr;
  GDR_TRY(parse(p, pr));
  if (!pr.pool_idx.empty()) return fail(GDR_ERR_UNSUPPORTED, "indexed states are supported by the serial scan only");
  if (n_segments < 1) return fail(GDR_ERR_INVALID_ARG, "n_segments must be >= 1");
  GDR_TRY(need(k, "k"));
  GDR_TRY(need(w, "w"));
  GDR_TRY(need(u, "u"));
  GDR_TRY(need(g_cum, "g_cum"));
  GDR_TRY(need(seg_state, "seg_state"));
  GDR_TRY(need(seg_trans, "seg_trans"));
  GDR_TRY(opt(workspace, "workspace"));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int split = workspace != nullptr ? gdr::summary_split(pr, n_segments) : 1;
  const size_t need_bytes = gdr_segment_summaries_workspace_size(p, n_segments);
  if (split == 2 && workspace_bytes < need_bytes)
    return fail(GDR_ERR_INVALID_ARG, "workspace_bytes " + std::to_string(workspace_bytes) + " < the " +
                                         std::to_string(need_bytes) + " bytes this problem needs");
  gdr::Tile t;
  GDR_TRY(tile_for(pr, tile, 1, static_cast<int64_t>(pr.N) * n_segments * split, t));
  if (split == 1)
    return run_scan(pr, t, 1, n_segments, k, w, u, g_cum, nullptr, 0, nullptr, nullptr, seg_state, 1, seg_trans, st);
  gdr::LaunchFn fn = gdr::find_combine(pr.DK);
  if (fn == nullptr) return fail(GDR_ERR_UNSUPPORTED, "no summary combine kernel for this DK");
  float* half_state = static_cast<float*>(workspace);
  float* half_trans = half_state + static_cast<size_t>(2) * pr.N * n_segments * pr.H * pr.DV * pr.DK;
  GDR_TRY(run_scan(pr, t, 1, n_segments, k, w, u, g_cum, nullptr, 0, nullptr, nullptr, half_state, 1, half_trans, st,
                   nullptr, 2));
  if (pr.N == 0) return GDR_OK;
  gdr::CombineArgs a;
  memset(&a, 0, sizeof(a));
  a.half_state = half_state;
  a.half_trans = half_trans;
  a.seg_state = seg_state;
  a.seg_trans = seg_trans;
  a.H = pr.H;
  a.DV = pr.DV;
  a.n_seg = pr.N * n_segments;
  const int64_t pairs = static_cast<int64_t>(pr.N) * n_segments * pr.H;
  // 64-column blocks (DV and DK are multiples of 64 here: the split needs DK = DV = 128)
  const int grid = static_cast<int>(8 * ((pr.DV + pr.DK) / 64) * ((pairs + 7) / 8));
  hipError_t e = fn(&a, grid, st);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return GDR_OK;
}

gdr_status gdr_segment_summaries(const gdr_problem* p, const gdr_tile* tile, int32_t n_segments, const void* k,
                                 const void* w, const void* u, const float* g_cum, float* seg_state,
                                 float* seg_trans, void* stream) {
  return gdr_segment_summaries_ws(p, tile, n_segments, k, w, u, g_cum, seg_state, seg_trans, nullptr, 0, stream);
}

gdr_status gdr_segment_compose(const gdr_problem* p, int32_t n_segments, const float* seg_state,
                               const float* seg_trans, const float* h0, float* seg_init, float* hT, void* stream) {
  g_err.clear();
  gdr::Problem pr;
  GDR_TRY(parse(p, pr));
  if (!pr.pool_idx.empty()) return fail(GDR_ERR_UNSUPPORTED, "indexed states are supported by the serial scan only");
  if (n_segments < 1) return fail(GDR_ERR_INVALID_ARG, "n_segments must be >= 1");
  GDR_TRY(need(seg_state, "seg_state"));
  GDR_TRY(need(seg_trans, "seg_trans"));
  GDR_TRY(need(seg_init, "seg_init"));
  GDR_TRY(opt(h0, "h0"));
  GDR_TRY(opt(hT, "hT"));
  gdr::LaunchFn fn = gdr::find_compose(pr.DK, n_segments);
  if (fn == nullptr) return fail(GDR_ERR_UNSUPPORTED, "no compose kernel for this DK");
  if (pr.N == 0) return GDR_OK;
  gdr::ComposeArgs a;
  memset(&a, 0, sizeof(a));
  a.seg_state = seg_state;
  a.seg_trans = seg_trans;
  a.h0 = h0;
  a.seg_init = seg_init;
  a.hT = hT;
  a.H = pr.H;
  a.DV = pr.DV;
  a.P = n_segments;
  a.N = pr.N;
  a.state_vk = pr.state_vk;
  // XCD-major order: the column blocks of one (sequence, head) share blockIdx modulo 8
  const int grid = 8 * (pr.DV / 16) * ((pr.N * pr.H + 7) / 8);
  hipError_t e = fn(&a, grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "compose launch");
  return GDR_OK;
}

int32_t gdr_plan_segments(const gdr_problem* p) {
  g_err.clear();
  gdr::Problem pr;
  if (parse(p, pr) != GDR_OK) return -1;
  return gdr::auto_segments(pr);
}

namespace {
// Byte offsets of the auto scan's workspace parts (each 256-byte aligned):
// seg_state, seg_trans, seg_init, then the summaries' own workspace.
struct AutoWs {
  size_t state, trans, init, summ, total;
};

AutoWs auto_layout(const gdr::Problem& pr, int P, size_t summ_bytes) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t n = static_cast<size_t>(pr.N) * P * pr.H;
  AutoWs w;
  w.state = 0;
  w.trans = up(w.state + n * pr.DV * pr.DK * sizeof(float));
  w.init = up(w.trans + n * pr.DK * pr.DK * sizeof(float));
  w.summ = up(w.init + n * pr.DV * pr.DK * sizeof(float));
  w.total = w.summ + summ_bytes;
  return w;
}
}  // namespace

size_t gdr_state_scan_auto_workspace_size(const gdr_problem* p) {
  g_err.clear();
  gdr::Problem pr;
  if (parse(p, pr) != GDR_OK) return 0;
  const int P = gdr::auto_segments(pr);
  if (P == 0) return 0;
  return auto_layout(pr, P, gdr_segment_summaries_workspace_size(p, P)).total;
}

gdr_status gdr_state_scan_auto(const gdr_problem* p, const void* q, const void* k, const void* w, const void* u,
                               const float* g_cum, const float* h0, float scale, void* h, void* v_new, float* hT,
                               void* o, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  gdr::Problem pr;
  GDR_TRY(parse(p, pr));
  if ((q == nullptr) != (o == nullptr)) return fail(GDR_ERR_INVALID_ARG, "q and o are given together or not at all");
  const int P = gdr::auto_segments(pr);
  if (P == 0) {
    if (o != nullptr)
      return gdr_state_scan_output(p, nullptr, nullptr, q, k, w, u, g_cum, h0, scale, h, v_new, hT, o, stream);
    return gdr_state_scan(p, nullptr, nullptr, k, w, u, g_cum, h0, h, v_new, hT, stream);
  }
  // every check of the three calls below, before the first launch
  GDR_TRY(need(k, "k"));
  GDR_TRY(need(w, "w"));
  GDR_TRY(need(u, "u"));
  GDR_TRY(need(g_cum, "g_cum"));
  GDR_TRY(opt(q, "q"));
  GDR_TRY(opt(o, "o"));
  GDR_TRY(opt(h0, "h0"));
  GDR_TRY(opt(h, "h"));
  GDR_TRY(opt(v_new, "v_new"));
  GDR_TRY(opt(hT, "hT"));
  GDR_TRY(need(workspace, "workspace"));
  const size_t summ_bytes = gdr_segment_summaries_workspace_size(p, P);
  const AutoWs lay = auto_layout(pr, P, summ_bytes);
  if (workspace_bytes < lay.total)
    return fail(GDR_ERR_INVALID_ARG, "workspace_bytes " + std::to_string(workspace_bytes) + " < the " +
                                         std::to_string(lay.total) + " bytes this problem needs");
  if (o != nullptr) {
    gdr::Tile t;
    GDR_TRY(tile_for(pr, nullptr, 0, static_cast<int64_t>(pr.N) * P, t));
    if (!fusable(pr, t)) t = gdr::Tile{64, 4, 2};  // the fallback gdr_state_scan_output takes
    if (!fusable(pr, t) && (h == nullptr || v_new == nullptr))
      return fail(GDR_ERR_UNSUPPORTED, "the output is not fused for this problem: h and v_new must be given");
  }
  char* ws = static_cast<char*>(workspace);
  float* seg_state = reinterpret_cast<float*>(ws + lay.state);
  float* seg_trans = reinterpret_cast<float*>(ws + lay.trans);
  float* seg_init = reinterpret_cast<float*>(ws + lay.init);
  GDR_TRY(gdr_segment_summaries_ws(p, nullptr, P, k, w, u, g_cum, seg_state, seg_trans,
                                   summ_bytes ? ws + lay.summ : nullptr, summ_bytes, stream));
  GDR_TRY(gdr_segment_compose(p, P, seg_state, seg_trans, h0, seg_init, nullptr, stream));
  const gdr_segments seg{P, seg_init};
  if (o != nullptr)
    return gdr_state_scan_output(p, nullptr, &seg, q, k, w, u, g_cum, nullptr, scale, h, v_new, hT, o, stream);
  return gdr_state_scan(p, nullptr, &seg, k, w, u, g_cum, nullptr, h, v_new, hT, stream);
}

gdr_status gdr_plan_query(const gdr_problem* p, const gdr_tile* tile, int32_t n_segments, int64_t out[6]) {
  g_err.clear();
  if (out == nullptr) return fail(GDR_ERR_INVALID_ARG, "out must not be NULL");
  gdr::Problem pr;
  GDR_TRY(parse(p, pr));
  const int mode = n_segments > 0 ? 1 : 0;
  const int split = mode == 1 ? gdr::summary_split(pr, n_segments) : 1;  // as gdr_segment_summaries_ws runs it
  gdr::Tile t;
  GDR_TRY(tile_for(pr, tile, mode, static_cast<int64_t>(pr.N) * (n_segments > 0 ? n_segments : 1) * split, t));
  std::vector<gdr::Launch> plan = gdr::plan_scan(pr, t, mode, n_segments > 0 ? n_segments : 1, true, true, split);
  int64_t wg = 0, maxrows = 0;
  for (auto& l : plan) {
    wg += l.grid;
    maxrows = std::max<int64_t>(maxrows, static_cast<int64_t>(l.rows.size()));
  }
  out[0] = t.bv;
  out[1] = t.waves;
  out[2] = t.stages;
  out[3] = wg;
  out[4] = static_cast<int64_t>(plan.size());
  out[5] = maxrows;
  return GDR_OK;
}

/* ----------------------------------------------------------- per-channel decay */

gdr_status kda_chunk_prepare(const gdr_problem* p, const void* k, const void* v, const float* g, const float* beta,
                             float* g_cum, void* w, void* u, void* kg, float* decay, void* stream) {
  g_err.clear();
  gdr::Problem pr;
  GDR_TRY(parse(p, pr));
  GDR_TRY(need(k, "k"));
  GDR_TRY(need(v, "v"));
  GDR_TRY(need(g, "g"));
  GDR_TRY(need(beta, "beta"));
  GDR_TRY(need(g_cum, "g_cum"));
  GDR_TRY(need(w, "w"));
  GDR_TRY(need(u, "u"));
  GDR_TRY(need(kg, "kg"));
  GDR_TRY(need(decay, "decay"));
  if (pr.dtype != GDR_BF16) return fail(GDR_ERR_UNSUPPORTED, "the per-channel decay path is built for bfloat16 storage");
  gdr::LaunchFn fn = gdr::find_kda_prepare(pr.DK, pr.DV);
  if (fn == nullptr) return fail(GDR_ERR_UNSUPPORTED, "no per-channel prepare kernel for this DK/DV");
  gdr::KdaArgs a;
  memset(&a, 0, sizeof(a));
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.g_cum = g_cum;
  a.w = w;
  a.u = u;
  a.kg = kg;
  a.decay = decay;
  a.H = pr.H;
  for (const gdr::Launch& l : gdr::plan_chunks(pr, 1)) {
    a.n_rows = static_cast<int32_t>(l.rows.size());
    a.n_chunks = l.n_chunks;
    a.chunk_base = l.chunk_base;
    memcpy(a.rows, l.rows.data(), l.rows.size() * sizeof(gdr::Row));
    hipError_t e = fn(&a, l.grid, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "per-channel prepare launch");
  }
  return GDR_OK;
}

gdr_status kda_state_scan(const gdr_problem* p, const gdr_tile* tile, const gdr_segments* seg, const void* kg,
                          const void* w, const void* u, const float* decay, const float* h0, void* h, void* v_new,
                          float* hT, void* stream) {
  g_err.clear();
  gdr::Problem pr;
  GDR_TRY(parse(p, pr));
  GDR_TRY(need(kg, "kg"));
  GDR_TRY(need(w, "w"));
  GDR_TRY(need(u, "u"));
  GDR_TRY(need(decay, "decay"));
  GDR_TRY(opt(h0, "h0"));
  GDR_TRY(opt(h, "h"));
  GDR_TRY(opt(v_new, "v_new"));
  GDR_TRY(opt(hT, "hT"));
  if (pr.dtype != GDR_BF16) return fail(GDR_ERR_UNSUPPORTED, "the per-channel decay path is built for bfloat16 storage");
  int mode = 0, P = 1;
  const float* h_in = h0;
  int in_vk = pr.state_vk;
  if (seg != nullptr) {
    if (!pr.pool_idx.empty()) return fail(GDR_ERR_UNSUPPORTED, "indexed states are supported by the serial scan only");
    if (seg->n_segments < 1) return fail(GDR_ERR_INVALID_ARG, "n_segments must be >= 1");
    GDR_TRY(need(seg->seg_init, "seg_init"));
    mode = 2;
    P = seg->n_segments;
    h_in = seg->seg_init;
    in_vk = 1;
  }
  gdr::Tile t;
  GDR_TRY(tile_for(pr, tile, 0, static_cast<int64_t>(pr.N) * P, t));
  return run_scan(pr, t, mode, P, kg, w, u, nullptr, h_in, in_vk, h, v_new, hT, pr.state_vk, nullptr,
                  static_cast<hipStream_t>(stream), decay);
}

gdr_status kda_segment_summaries(const gdr_problem* p, const gdr_tile* tile, int32_t n_segments, const void* kg,
                                 const void* w, const void* u, const float* decay, float* seg_state, float* seg_trans,
                                 void* stream) {
  g_err.clear();
  gdr::Problem pr;
  GDR_TRY(parse(p, pr));
  if (!pr.pool_idx.empty()) return fail(GDR_ERR_UNSUPPORTED, "indexed states are supported by the serial scan only");
  if (n_segments < 1) return fail(GDR_ERR_INVALID_ARG, "n_segments must be >= 1");
  GDR_TRY(need(kg, "kg"));
  GDR_TRY(need(w, "w"));
  GDR_TRY(need(u, "u"));
  GDR_TRY(need(decay, "decay"));
  GDR_TRY(need(seg_state, "seg_state"));
  GDR_TRY(need(seg_trans, "seg_trans"));
  if (pr.dtype != GDR_BF16) return fail(GDR_ERR_UNSUPPORTED, "the per-channel decay path is built for bfloat16 storage");
  gdr::Tile t;
  GDR_TRY(tile_for(pr, tile, 1, static_cast<int64_t>(pr.N) * n_segments, t));
  return run_scan(pr, t, 1, n_segments, kg, w, u, nullptr, nullptr, 0, nullptr, nullptr, seg_state, 1, seg_trans,
                  static_cast<hipStream_t>(stream), decay);
}

gdr_status kda_chunk_output(const gdr_problem* p, const void* q, const void* k, const void* v_new, const void* h,
                            const float* g_cum, float scale, void* o, void* stream) {
  g_err.clear();
  gdr::Problem pr;
  GDR_TRY(parse(p, pr));
  GDR_TRY(need(q, "q"));
  GDR_TRY(need(k, "k"));
  GDR_TRY(need(v_new, "v_new"));
  GDR_TRY(need(h, "h"));
  GDR_TRY(need(g_cum, "g_cum"));
  GDR_TRY(need(o, "o"));
  if (pr.dtype != GDR_BF16) return fail(GDR_ERR_UNSUPPORTED, "the per-channel decay path is built for bfloat16 storage");
  gdr::LaunchFn fn = gdr::find_kda_output(pr.DK, pr.DV);
  if (fn == nullptr) return fail(GDR_ERR_UNSUPPORTED, "no per-channel output kernel for this DK/DV");
  gdr::KdaArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v_new;
  a.g = g_cum;
  a.h = h;
  a.o = o;
  a.scale = scale;
  a.H = pr.H;
  for (const gdr::Launch& l : gdr::plan_chunks(pr, 1)) {  // one workgroup per (chunk, head)
    a.n_rows = static_cast<int32_t>(l.rows.size());
    a.n_chunks = l.n_chunks;
    a.chunk_base = l.chunk_base;
    memcpy(a.rows, l.rows.data(), l.rows.size() * sizeof(gdr::Row));
    hipError_t e = fn(&a, l.grid, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "per-channel output launch");
  }
  return GDR_OK;
}

}  // extern "C"
