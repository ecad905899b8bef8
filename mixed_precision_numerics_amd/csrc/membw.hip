// Reference copy for the HBM roofline of the element-wise kernels.
//
// The optimizer pass reads as many bytes as it writes (28 B/param: 14 read,
// 14 written), so its practical ceiling on a given part is the rate of a plain
// device copy.  This kernel is the fastest copy measured here: each
// work-group copies one contiguous 256 KiB range, every thread with four
// 16-byte non-temporal loads in flight before its stores (5.54 TB/s for 4 GiB
// on MI355X, against 5.06 for a grid-stride copy and 4.5 for hipMemcpy).  The
// bench times it in the same run as the optimizer so that both figures come
// from one box.
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace amp {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int64_t kCopyChunk = 16384;        // 16-byte vectors per work-group (256 KiB)

__global__ __launch_bounds__(kCopyThreads) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst,
                                                                   int64_t nvec) {
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * kCopyChunk;
  const int64_t b1 = b0 + kCopyChunk < nvec ? b0 + kCopyChunk : nvec;
  int64_t i = b0 + threadIdx.x;
  for (; i + (kCopyUnroll - 1) * kCopyThreads < b1; i += kCopyUnroll * kCopyThreads) {
    u32x4 w[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) w[u] = __builtin_nontemporal_load(src + i + u * kCopyThreads);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(w[u], dst + i + u * kCopyThreads);
  }
  for (; i < b1; i += kCopyThreads) dst[i] = src[i];
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
    const int64_t blocks = (nvec + kCopyChunk - 1) / kCopyChunk;
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
