// Segment summaries for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): gdr_segment_summaries_ws with its half-segment workspace taken
// from a file-scope device array instead of a caller buffer.
//
// The array lives in the library's code object, one copy per GPU, for as long
// as the process runs.  Host code never passes the array's name to a kernel
// (on the host that name is only a stand-in): on the first call on a device,
// with that device current, hipGetSymbolAddress gives the array's address on
// that device, which is kept per device and used from then on.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "../../include/gdr.h"

namespace gdr_internal {
void set_last_error(const std::string& m);
}

namespace gdr_noalloc {

constexpr size_t kScratchBytes = size_t(48) << 20;  // GDR_NOALLOC_SCRATCH_BYTES in gdr.h

__device__ __align__(256) char scratch[kScratchBytes];

}  // namespace gdr_noalloc

namespace {

using gdr_noalloc::kScratchBytes;
constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device (looked up once
// per device).
gdr_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    gdr_internal::set_last_error(std::string("hipGetDevice: ") + hipGetErrorString(e));
    return GDR_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    gdr_internal::set_last_error("device index " + std::to_string(dev) + " out of range for the scratch table");
    return GDR_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(gdr_noalloc::scratch));
    if (e != hipSuccess || p == nullptr) {
      gdr_internal::set_last_error(std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
      return GDR_ERR_HIP;
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return GDR_OK;
}

}  // namespace

extern "C" {

gdr_status gdr_segment_summaries_noalloc(const gdr_problem* p, const gdr_tile* tile, int32_t n_segments,
                                         const void* k, const void* w, const void* u, const float* g_cum,
                                         float* seg_state, float* seg_trans, void* stream) {
  const size_t need_bytes = gdr_segment_summaries_workspace_size(p, n_segments);
  if (need_bytes == 0) {
    if (gdr_last_error()[0] != '\0') return GDR_ERR_INVALID_ARG;  // invalid problem or segment count
    // the direct form: no workspace
    return gdr_segment_summaries_ws(p, tile, n_segments, k, w, u, g_cum, seg_state, seg_trans, nullptr, 0, stream);
  }
  if (need_bytes > kScratchBytes) {
    gdr_internal::set_last_error("this problem needs " + std::to_string(need_bytes) +
                                 " bytes of summary workspace; the library's static scratch holds " +
                                 std::to_string(kScratchBytes) + " (use gdr_segment_summaries_ws)");
    return GDR_ERR_INVALID_ARG;
  }
  void* ws = nullptr;
  const gdr_status s = scratch_ptr(&ws);
  if (s != GDR_OK) return s;
  return gdr_segment_summaries_ws(p, tile, n_segments, k, w, u, g_cum, seg_state, seg_trans, ws, need_bytes, stream);
}

}  // extern "C"
