// Reference copy for the HBM roofline of the element-wise kernels.
//
// The optimizer pass reads as many bytes as it writes (28 B/param: 14 read,
// 14 written), so its practical ceiling on a given part is the rate of a plain
// device copy with the same access shape: 16-byte loads and stores, every
// thread with several loads in flight, a grid-stride loop over a launch of
// 64 work-groups per CU.  This kernel is that copy; the bench times it in the
// same run as the optimizer so that both figures come from one box.
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace amp {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst,
                                                                   int64_t nvec) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
  const int64_t nthr = static_cast<int64_t>(gridDim.x) * kCopyThreads;
  int64_t i = tid;
  for (; i + (kCopyUnroll - 1) * nthr < nvec; i += kCopyUnroll * nthr) {
    u32x4 w[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) w[u] = src[i + u * nthr];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) dst[i + u * nthr] = w[u];
  }
  for (; i < nvec; i += nthr) dst[i] = src[i];
}

__global__ void stream_copy_tail(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                 int64_t from, int64_t bytes) {
  const int64_t i = from + static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < bytes) dst[i] = src[i];
}

}  // namespace

hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t nvec = bytes / 16;
  if (nvec > 0) {
    int64_t blocks = (nvec + kCopyThreads - 1) / kCopyThreads;
    if (blocks > 256 * 64) blocks = 256 * 64;
    stream_copy_kernel<<<dim3(static_cast<unsigned>(blocks)), kCopyThreads, 0, s>>>(
        static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), nvec);
  }
  const int64_t done = nvec * 16;
  if (done < bytes)
    stream_copy_tail<<<1, 64, 0, s>>>(static_cast<const uint8_t*>(src),
                                      static_cast<uint8_t*>(dst), done, bytes);
  return hipGetLastError();
}

}  // namespace amp
