// Placeholder launchers for entry points whose kernels are not built yet.
#include "common.hpp"

namespace amp {

hipError_t launch_gemm(int, int, int64_t, int64_t, int64_t, const void*, int, int64_t,
                       const float*, const void*, int, int64_t, const float*, void*, int,
                       int64_t, const amp_block_scales*, const amp_block_scales*, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_nvfp4_quantize(const void*, int, int64_t, int64_t, int64_t, int, int, int,
                                 uint64_t, int, uint64_t, uint8_t*, uint8_t*, float*,
                                 hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace amp
