// NVFP4-style path (placeholder until the kernels land).
#include "bsfp8_internal.h"

namespace bsfp8 {

size_t fp4_quant_workspace_bytes(int64_t, int64_t) { return 0; }
size_t fp4_gemm_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_fp4_quant(const uint16_t*, int64_t, int64_t, int, uint8_t*, uint8_t*, float*,
                            void*, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_fp4_gemm(const uint8_t*, const uint8_t*, const float*, const uint8_t*,
                           const uint8_t*, const float*, uint16_t*, int64_t, int64_t, int64_t,
                           void*, size_t, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace bsfp8
