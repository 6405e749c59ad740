// bf16 MFMA backward for gated block-sparse attention (gfx950).
#include "common.h"
#include "internal.h"

namespace sas {

bool mfma_bwd_supported(const Dims& dm) {
  (void)dm;
  return false;
}

hipError_t launch_bwd_mfma(const Dims& dm, const void* q, const void* k, const void* v,
                           const void* dout, const float* lse, const int32_t* idx,
                           const float* logg, void* dq, void* dk, void* dv,
                           const BwdWorkspace& ws, int* nchunk_out, hipStream_t st) {
  (void)dm; (void)q; (void)k; (void)v; (void)dout; (void)lse; (void)idx; (void)logg;
  (void)dq; (void)dk; (void)dv; (void)ws; (void)nchunk_out; (void)st;
  return hipErrorInvalidValue;
}

}  // namespace sas
