// ABC slot-state construction entry points (include/gdr.h).
#include <hip/hip_runtime.h>

#include <string>

#include "../../include/gdr.h"

extern "C" {

size_t abc_workspace_size(const abc_problem* p) {
  (void)p;
  return 0;
}

gdr_status abc_affine_scan(const abc_problem* p, const void* k, const void* v, const void* s, float* z, void* hk,
                           void* hv, float* hk_final, float* hv_final, void* workspace, size_t workspace_bytes,
                           void* stream) {
  (void)p; (void)k; (void)v; (void)s; (void)z; (void)hk; (void)hv; (void)hk_final; (void)hv_final;
  (void)workspace; (void)workspace_bytes; (void)stream;
  return GDR_ERR_UNSUPPORTED;
}

}  // extern "C"
