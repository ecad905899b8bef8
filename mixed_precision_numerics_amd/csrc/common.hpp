// Shared host/device helpers of the HIP library (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "amp.h"

namespace amp {

constexpr int kWave = 64;

// Native clang vectors (usable with the non-temporal load/store builtins).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Max-reduce an unsigned value over a block of `kThreads` threads; the result
// is valid in thread 0.  `lds` must hold kThreads / 64 words.
template <int kThreads>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* lds) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, kWave));
    v = v > o ? v : o;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  if (kThreads > kWave) {
    if (lane == 0) lds[wid] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
      for (int w = 1; w < kThreads / kWave; ++w) v = v > lds[w] ? v : lds[w];
    }
  }
  return v;
}

// Canonicalise a maximum of |x| bit patterns: any NaN -> 0x7FC00000.
__device__ __forceinline__ uint32_t canon_amax(uint32_t m) {
  return m > 0x7f800000u ? 0x7fc00000u : m;
}

// *d_amax = max(*d_amax, m) on FP32 bit patterns (m canonicalized).  The
// stored value only grows, so a read of at least m proves the atomic
// unneeded: work-groups whose maximum is already covered skip it, and the
// atomics of thousands of work-groups no longer queue on one address (on a
// 235 M-element cast they had cost 60-85 us of 200).
__device__ __forceinline__ void amax_update(void* d_amax, uint32_t m) {
  const uint32_t c = canon_amax(m);
  unsigned int* p = static_cast<unsigned int*>(d_amax);
  if (c > __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(p, c);
}

// Element sizes of the ABI dtypes (E2M1X2: one byte holds two elements).
inline int dtype_bytes(int dt) {
  switch (dt) {
    case AMP_F32: return 4;
    case AMP_F16: case AMP_BF16: return 2;
    case AMP_E4M3: case AMP_E5M2: case AMP_E2M1X2: return 1;
    default: return 0;
  }
}

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Launchers implemented in the kernel translation units.  They return the
// hipError_t of the launch.
hipError_t launch_cast(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                       void* y, int yt, int64_t ldy, void* y_t, int64_t ldy_t,
                       const float* d_scale, float* d_amax, unsigned long long* d_sat,
                       hipStream_t s);
hipError_t launch_cast_current(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                               void* y, int yt, int64_t ldy, void* y_t, int64_t ldy_t,
                               float fp8_max, float margin, amp_fp8_meta* meta, hipStream_t s);
hipError_t launch_quantize_blockwise(const void* x, int xt, int64_t rows, int64_t cols,
                                     int64_t ldx, int yt, int block, uint8_t* q, int64_t ldq,
                                     float* s, int64_t lds, uint8_t* qt, int64_t ldqt, float* st,
                                     int64_t ldst, hipStream_t hs);
hipError_t launch_found_inf_from_amax(const float* amax, int32_t n, int yt, const float* d_scale,
                                      amp_scaler_state* st, hipStream_t s);
hipError_t launch_check_overflow(const void* g, int gt, int64_t n, amp_scaler_state* st,
                                 hipStream_t s);
hipError_t launch_optimizer_apply(float* master, float* m, float* v, const void* g, int gt,
                                  void* w16, int wt, int64_t n, const amp_adamw_hparams& hp,
                                  amp_scaler_state* st, const float* mult, hipStream_t s);
hipError_t launch_grad_accumulate(float* acc, const void* g, int gt, int64_t n, int first,
                                  hipStream_t s);
hipError_t launch_grad_norm_init(amp_grad_norm_state* ns, hipStream_t s);
hipError_t launch_grad_norm_noalloc(const void* g, int gt, int64_t n, amp_scaler_state* st,
                                    double* sumsq, hipStream_t s);
hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);
hipError_t launch_fp8_mfma_probe(int shape, int at, const void* a, const void* b, float* c,
                                 int64_t tiles, hipStream_t s);
hipError_t launch_grad_norm(const void* g, int gt, int64_t n, amp_scaler_state* st,
                            amp_grad_norm_state* ns, hipStream_t s);
hipError_t launch_clip_coefficient(const amp_grad_norm_state* ns, float max_norm,
                                   const amp_scaler_state* st, float* out, hipStream_t s);
hipError_t launch_optimizer_commit(amp_scaler_state* st, const amp_adamw_hparams& hp,
                                   hipStream_t s);
hipError_t launch_scaler_init(amp_scaler_state* st, float init_scale, hipStream_t s);
hipError_t launch_scaler_update(amp_scaler_state* st, const amp_scaler_params& p,
                                hipStream_t s);
hipError_t launch_meta_init(amp_fp8_meta* metas, float* hist, int32_t n, int32_t len,
                            hipStream_t s);
hipError_t launch_delayed_update(amp_fp8_meta* metas, float* hist, int32_t n,
                                 const amp_delayed_recipe& r, hipStream_t s);
hipError_t launch_gemm(int opA, int opB, int64_t M, int64_t N, int64_t K, const void* A,
                       int at, int64_t lda, const float* alphaA, const void* B, int bt,
                       int64_t ldb, const float* alphaB, void* C, int ct, int64_t ldc,
                       const amp_block_scales* bsA, const amp_block_scales* bsB,
                       int flags, hipStream_t s);
hipError_t launch_gemm_blockwise(int64_t M, int64_t N, int64_t K, const void* A, int at,
                                 int64_t lda, const float* sA, int64_t ldsA, int a_block,
                                 const void* B, int bt, int64_t ldb, const float* sB,
                                 int64_t ldsB, int b_block, void* C, int ct, int64_t ldc,
                                 hipStream_t s);
hipError_t launch_nvfp4_quantize(const void* x, int xt, int64_t rows, int64_t cols,
                                 int64_t ldx, int transpose, int block2d, int rht,
                                 uint64_t rht_seed, int rnd, uint64_t sr_seed, uint8_t* q,
                                 uint8_t* scales, float* d_tensor, hipStream_t s);

hipError_t launch_mx_quantize(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                              int transpose, int yt, uint8_t* q, uint8_t* scales, hipStream_t s);
hipError_t launch_bias_gelu(const float* acc, int64_t rows, int64_t cols, const void* b16,
                            void* z16, void* a16, hipStream_t s);
hipError_t launch_softmax_xent(const void* logits16, const int32_t* labels, int64_t rows,
                               int64_t cols, const amp_scaler_state* st, float* loss,
                               void* dlog16, hipStream_t s);
hipError_t launch_gelu_backward(const void* dA16, const void* z16, int64_t n, void* dz16,
                                hipStream_t s);
hipError_t launch_colsum(const void* x16, int64_t rows, int64_t cols, void* out16, hipStream_t s);

}  // namespace amp
