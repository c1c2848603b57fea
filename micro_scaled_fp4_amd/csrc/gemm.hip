// Block-scaled FP4 GEMM (placeholder until the MFMA kernels land).
#include "fp4_internal.h"

namespace fp4impl {
hipError_t launch_gemm(bool, const uint8_t*, const uint8_t*, const float*, const uint8_t*,
                       const uint8_t*, const float*, float, int64_t, int64_t, int64_t, void*, bool,
                       hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace fp4impl
