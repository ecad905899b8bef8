// Placeholder launchers for entry points whose kernels are not built yet.
#include "common.hpp"

namespace amp {

hipError_t launch_nvfp4_quantize(const void*, int, int64_t, int64_t, int64_t, int, int, int,
                                 uint64_t, int, uint64_t, uint8_t*, uint8_t*, float*,
                                 hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace amp
