// One FP8 matrix-core instruction per wave on caller-provided operand bytes.
//
// This is the measurement behind the choice of the exact FP8 route (page
// hwlabs, section "GEMM 누적 정밀도 문제": FP8 matrix units may keep limited
// precision in their partial sums): it lets a test feed each FP8 instruction
// shape of gfx950 the same kind of operands and compare its outputs with exact
// sums.  It is not a step of the training path.
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace amp {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// SHAPE 0: 32x32x16 FP8, 1: 16x16x32 FP8, 2: block-scaled 32x32x64 f8f6f4,
// 3: block-scaled 16x16x128 f8f6f4 (neutral scales).  FA: A is E4M3 (0) or
// E5M2 (1); B is E4M3.
template <int SHAPE, int FA>
__global__ __launch_bounds__(256) void fp8_probe_kernel(const uint8_t* __restrict__ A,
                                                        const uint8_t* __restrict__ B,
                                                        float* __restrict__ C, int64_t tiles) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= tiles) return;
  constexpr int kBytes = SHAPE <= 1 ? 8 : 32;
  constexpr int kOut = SHAPE == 0 || SHAPE == 2 ? 16 : 4;
  const uint8_t* a = A + (t * 64 + lane) * kBytes;
  const uint8_t* b = B + (t * 64 + lane) * kBytes;
  float* c = C + (t * 64 + lane) * kOut;
  if constexpr (SHAPE <= 1) {
    const long av = *reinterpret_cast<const long*>(a);
    const long bv = *reinterpret_cast<const long*>(b);
    if constexpr (SHAPE == 0) {
      f32x16 acc = {};
      if constexpr (FA == 0) acc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(av, bv, acc, 0, 0, 0);
      else acc = __builtin_amdgcn_mfma_f32_32x32x16_bf8_fp8(av, bv, acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) c[r] = acc[r];
    } else {
      f32x4v acc = {};
      if constexpr (FA == 0) acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(av, bv, acc, 0, 0, 0);
      else acc = __builtin_amdgcn_mfma_f32_16x16x32_bf8_fp8(av, bv, acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) c[r] = acc[r];
    }
  } else {
    const i32x8 av = *reinterpret_cast<const i32x8*>(a);
    const i32x8 bv = *reinterpret_cast<const i32x8*>(b);
    if constexpr (SHAPE == 2) {
      f32x16 acc = {};
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, FA, 0, 0, 127, 0, 127);
#pragma unroll
      for (int r = 0; r < 16; ++r) c[r] = acc[r];
    } else {
      f32x4v acc = {};
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, FA, 0, 0, 127, 0, 127);
#pragma unroll
      for (int r = 0; r < 4; ++r) c[r] = acc[r];
    }
  }
}

template <int SHAPE>
void launch_shape(int fa, const uint8_t* a, const uint8_t* b, float* c, int64_t tiles, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((tiles + 3) / 4));
  if (fa == AMP_E4M3) fp8_probe_kernel<SHAPE, 0><<<grid, 256, 0, s>>>(a, b, c, tiles);
  else fp8_probe_kernel<SHAPE, 1><<<grid, 256, 0, s>>>(a, b, c, tiles);
}

}  // namespace

hipError_t launch_fp8_mfma_probe(int shape, int at, const void* a, const void* b, float* c,
                                 int64_t tiles, hipStream_t s) {
  const uint8_t* pa = static_cast<const uint8_t*>(a);
  const uint8_t* pb = static_cast<const uint8_t*>(b);
  switch (shape) {
    case 0: launch_shape<0>(at, pa, pb, c, tiles, s); break;
    case 1: launch_shape<1>(at, pa, pb, c, tiles, s); break;
    case 2: launch_shape<2>(at, pa, pb, c, tiles, s); break;
    default: launch_shape<3>(at, pa, pb, c, tiles, s); break;
  }
  return hipGetLastError();
}

}  // namespace amp
