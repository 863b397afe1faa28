// ABC slot-state construction entry points (include/gdr.h).
#include <hip/hip_runtime.h>
#include <string.h>

#include <string>

#include "../../include/gdr.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_abc_err;

bool abc_valid(const abc_problem* p, std::string& err) {
  if (p == nullptr) {
    err = "problem must not be NULL";
    return false;
  }
  if (p->B < 1 || p->T < 0 || p->H < 1) {
    err = "B >= 1, T >= 0 and H >= 1 are required";
    return false;
  }
  if (p->T > (int64_t(1) << 30)) {
    err = "T too large";
    return false;
  }
  if (p->M != 64 && p->M != 32) {
    err = "M (slots) must be 32 or 64";
    return false;
  }
  if (p->K < 64 || p->K % 64 != 0 || p->V < 64 || p->V % 64 != 0 || p->K > 4096 || p->V > 4096) {
    err = "K and V must be multiples of 64 (64..4096)";
    return false;
  }
  if (p->dtype != GDR_BF16) {
    err = "abc_affine_scan supports bfloat16 storage";
    return false;
  }
  return true;
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

}  // namespace

// Shares the thread-local message with the gated-delta entry points.
extern "C" const char* gdr_last_error(void);
namespace gdr_internal {
void set_last_error(const std::string& m);
}

extern "C" {

size_t abc_workspace_size(const abc_problem* p) {
  std::string err;
  if (!abc_valid(p, err)) return 0;
  const int64_t nc = (p->T + 63) / 64;
  // chunk log-sum-exps and chunk-end normalisers (FP32), the weights E
  // (storage dtype), then the end states of the state walk's runs (FP32,
  // always 64 slots: M = 32 is padded)
  const int P = gdr::abc_segments(p->B, p->H, p->K, p->V, static_cast<int>(nc));
  return 2 * static_cast<size_t>(p->B) * nc * p->H * p->M * sizeof(float) +
         static_cast<size_t>(p->B) * p->T * p->H * p->M * 2 + 16 +
         static_cast<size_t>(p->B) * p->H * (P - 1) * (p->K + p->V) * 64 * sizeof(float);
}

gdr_status abc_affine_scan(const abc_problem* p, const void* k, const void* v, const void* s, float* z, void* hk,
                           void* hv, float* hk_final, float* hv_final, void* workspace, size_t workspace_bytes,
                           void* stream) {
  std::string err;
  if (!abc_valid(p, err)) {
    gdr_internal::set_last_error(err);
    return GDR_ERR_INVALID_ARG;
  }
  const void* req[] = {k, v, s, hk, hv, workspace};
  const char* names[] = {"k", "v", "s", "hk", "hv", "workspace"};
  for (int i = 0; i < 6; ++i) {
    if (req[i] == nullptr || !aligned16(req[i])) {
      gdr_internal::set_last_error(std::string(names[i]) + " must be non-NULL and 16-byte aligned");
      return GDR_ERR_INVALID_ARG;
    }
  }
  const void* opt[] = {z, hk_final, hv_final};
  for (const void* q : opt) {
    if (q != nullptr && !aligned16(q)) {
      gdr_internal::set_last_error("optional outputs must be 16-byte aligned");
      return GDR_ERR_INVALID_ARG;
    }
  }
  if (workspace_bytes < abc_workspace_size(p)) {
    gdr_internal::set_last_error("workspace smaller than abc_workspace_size()");
    return GDR_ERR_INVALID_ARG;
  }
  gdr::AbcArgs a;
  memset(&a, 0, sizeof(a));
  a.k = k;
  a.v = v;
  a.s = s;
  a.z = z;
  a.lse = static_cast<float*>(workspace);
  a.hk = hk;
  a.hv = hv;
  a.hk_final = hk_final;
  a.hv_final = hv_final;
  a.B = p->B;
  a.T = static_cast<int32_t>(p->T);
  a.H = p->H;
  a.K = p->K;
  a.M = p->M;
  a.V = p->V;
  a.NC = static_cast<int32_t>((p->T + 63) / 64);
  a.zc = a.lse + static_cast<int64_t>(a.B) * a.NC * a.H * a.M;
  a.e = a.zc + static_cast<int64_t>(a.B) * a.NC * a.H * a.M;
  a.e2 = a.e;
  a.P = gdr::abc_segments(a.B, a.H, a.K, a.V, a.NC);
  {
    // after E (B*T*H*M bf16), rounded up to 16 bytes
    const uintptr_t e_end = reinterpret_cast<uintptr_t>(a.e) + static_cast<uintptr_t>(a.B) * a.T * a.H * a.M * 2;
    a.lsum = reinterpret_cast<float*>((e_end + 15) & ~static_cast<uintptr_t>(15));
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = gdr::launch_abc(a, st);
  if (e != hipSuccess) {
    gdr_internal::set_last_error(std::string("abc launch: ") + hipGetErrorString(e));
    return GDR_ERR_HIP;
  }
  return GDR_OK;
}

gdr_status abc_chunk_output(const abc_problem* p, const void* q, const void* k, const void* v, const void* s,
                            const float* z, const void* hk, const void* hv, float scale, void* o, void* p_out,
                            void* stream) {
  std::string err;
  if (!abc_valid(p, err)) {
    gdr_internal::set_last_error(err);
    return GDR_ERR_INVALID_ARG;
  }
  if (!gdr::abc_out_supported(p->K, p->V)) {
    gdr_internal::set_last_error("abc_chunk_output is built for (K, V) in {(64,128), (128,128), (128,256), (256,256), (256,512)}");
    return GDR_ERR_UNSUPPORTED;
  }
  const void* req[] = {q, k, v, s, z, hk, hv, o};
  const char* names[] = {"q", "k", "v", "s", "z", "hk", "hv", "o"};
  for (int i = 0; i < 8; ++i) {
    if (req[i] == nullptr || !aligned16(req[i])) {
      gdr_internal::set_last_error(std::string(names[i]) + " must be non-NULL and 16-byte aligned");
      return GDR_ERR_INVALID_ARG;
    }
  }
  if (p_out != nullptr && !aligned16(p_out)) {
    gdr_internal::set_last_error("p must be 16-byte aligned");
    return GDR_ERR_INVALID_ARG;
  }
  gdr::AbcOutArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.s = s;
  a.z = z;
  a.hk = hk;
  a.hv = hv;
  a.o = o;
  a.p = p_out;
  a.scale = scale;
  a.B = p->B;
  a.T = static_cast<int32_t>(p->T);
  a.H = p->H;
  a.K = p->K;
  a.V = p->V;
  a.NC = static_cast<int32_t>((p->T + 63) / 64);
  a.M = p->M;
  hipError_t e = gdr::launch_abc_out(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    gdr_internal::set_last_error(std::string("abc read launch: ") + hipGetErrorString(e));
    return GDR_ERR_HIP;
  }
  return GDR_OK;
}

size_t abc_bwd_workspace_size(const abc_problem* p) {
  std::string err;
  if (!abc_valid(p, err)) return 0;
  const int64_t nc = (p->T + 63) / 64;
  // chunk-end normalisers (FP32), the two weight tensors (storage dtype),
  // then the end states of the reverse walk's runs (FP32, always 64 slots)
  const int P = gdr::abc_segments(p->B, p->H, p->K, p->V, static_cast<int>(nc));
  return static_cast<size_t>(p->B) * nc * p->H * p->M * sizeof(float) +
         2 * static_cast<size_t>(p->B) * p->T * p->H * p->M * 2 + 16 +
         static_cast<size_t>(p->B) * p->H * (P - 1) * (p->K + p->V) * 64 * sizeof(float);
}

gdr_status abc_affine_scan_bwd(const abc_problem* p, const void* q, const void* dscore, const void* pw,
                               const void* dO, const float* z, const float* dhk_final, const float* dhv_final,
                               float scale, void* dhk, void* dhv, void* workspace, size_t workspace_bytes,
                               void* stream) {
  std::string err;
  if (!abc_valid(p, err)) {
    gdr_internal::set_last_error(err);
    return GDR_ERR_INVALID_ARG;
  }
  const void* req[] = {q, dscore, pw, dO, z, dhk, dhv, workspace};
  const char* names[] = {"q", "dscore", "p", "dO", "z", "dhk", "dhv", "workspace"};
  for (int i = 0; i < 8; ++i) {
    if (req[i] == nullptr || !aligned16(req[i])) {
      gdr_internal::set_last_error(std::string(names[i]) + " must be non-NULL and 16-byte aligned");
      return GDR_ERR_INVALID_ARG;
    }
  }
  if ((dhk_final != nullptr && !aligned16(dhk_final)) || (dhv_final != nullptr && !aligned16(dhv_final))) {
    gdr_internal::set_last_error("final-state gradients must be 16-byte aligned");
    return GDR_ERR_INVALID_ARG;
  }
  if (workspace_bytes < abc_bwd_workspace_size(p)) {
    gdr_internal::set_last_error("workspace smaller than abc_bwd_workspace_size()");
    return GDR_ERR_INVALID_ARG;
  }
  gdr::AbcArgs a;
  memset(&a, 0, sizeof(a));
  a.k = q;
  a.v = dO;
  a.s = dscore;
  a.pw = pw;
  a.z = const_cast<float*>(z);
  a.hk = dhk;
  a.hv = dhv;
  a.gk_end = dhk_final;
  a.gv_end = dhv_final;
  a.scale = scale;
  a.B = p->B;
  a.T = static_cast<int32_t>(p->T);
  a.H = p->H;
  a.K = p->K;
  a.M = p->M;
  a.V = p->V;
  a.NC = static_cast<int32_t>((p->T + 63) / 64);
  a.zc = static_cast<float*>(workspace);
  const int64_t nzc = static_cast<int64_t>(a.B) * a.NC * a.H * a.M;
  const int64_t nw = static_cast<int64_t>(a.B) * a.T * a.H * a.M;
  a.e = a.zc + nzc;
  a.e2 = static_cast<uint16_t*>(a.e) + nw;
  {
    const uintptr_t e2_end = reinterpret_cast<uintptr_t>(static_cast<uint16_t*>(a.e2) + nw);
    a.lsum = reinterpret_cast<float*>((e2_end + 15) & ~static_cast<uintptr_t>(15));
  }
  a.P = gdr::abc_segments(a.B, a.H, a.K, a.V, a.NC);
  hipError_t e = gdr::launch_abc_bwd(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    gdr_internal::set_last_error(std::string("abc reverse launch: ") + hipGetErrorString(e));
    return GDR_ERR_HIP;
  }
  return GDR_OK;
}

}  // extern "C"
