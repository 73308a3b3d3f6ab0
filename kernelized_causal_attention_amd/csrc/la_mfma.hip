// bf16 MFMA kernels (placeholder until the MFMA path lands).
#include "la_internal.h"

namespace la {
int mfma_supported(int, int64_t, int64_t, int) { return 0; }
hipError_t launch_forward_mfma(int, const SegGeom&, const void*, const void*, const void*, void*, float*,
                               const float*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_seg_state_mfma(const SegGeom&, const void*, const void*, float*, int64_t, float*, int64_t,
                                 hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_dq_mfma(int, const SegGeom&, const void*, const void*, const void*, const void*,
                              const void*, const float*, const float*, void*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_bwd_dkdv_mfma(int, const SegGeom&, const void*, const void*, const void*, const void*,
                                const void*, const float*, const float*, void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace la
