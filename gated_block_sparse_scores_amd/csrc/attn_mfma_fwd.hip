// bf16 MFMA forward for gated block-sparse attention (gfx950).
#include "common.h"
#include "internal.h"

namespace sas {

bool mfma_fwd_supported(const Dims& dm) {
  (void)dm;
  return false;
}

hipError_t launch_fwd_mfma(const Dims& dm, const void* q, const void* k, const void* v,
                           const int32_t* idx, const float* logg, void* o, float* lse,
                           hipStream_t st) {
  (void)dm; (void)q; (void)k; (void)v; (void)idx; (void)logg; (void)o; (void)lse; (void)st;
  return hipErrorInvalidValue;
}

}  // namespace sas
