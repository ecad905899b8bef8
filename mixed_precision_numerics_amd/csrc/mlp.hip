// Element-wise and small reduction kernels of the FP16 AMP training step of a
// two-layer MLP (gfx950): bias + GELU, FP32 softmax cross-entropy with the
// loss-scaled FP16 logit gradient, GELU backward, bias-gradient column sums.
//
// Page "혼합 정밀도 학습" (itwiki), section "FP16 학습 루프" (Linear(512,2048) ->
// GELU -> Linear(2048,10), cross-entropy in FP32 under autocast, backward from
// S * loss) and section "PyTorch 자동 혼합 정밀도(torch.amp)" (linear layers in
// FP16; softmax and cross-entropy in FP32); page "Mixed Precision
// Training/es" (marovi), "Operaciones que permanecen en FP32".
//
// Conventions (FP16 working copies and gradients, FP32 arithmetic):
//   z   = round16(fl32(acc + b16))              bias added to the FP32 accumulator
//   a   = round16(gelu(z)),  gelu(z) = z/2 (1 + erf(z / sqrt 2))
//   loss = mean_r (logsumexp(l_r) - l_r[y_r])   in FP32
//   dl  = round16(S * (softmax(l_r) - onehot(y_r)) / rows)
//   dz  = round16(fl32(dA * fl32(gelu'(z))))
//   db  = round16(fl32(sum_r g[r][c]))          sequential FP32 sum per column
#include "common.hpp"
#include "formats.hpp"

namespace amp {
namespace {

__device__ __forceinline__ float h2f(uint16_t h) { return f16_to_f32(h); }

__device__ __forceinline__ float gelu(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

__device__ __forceinline__ float gelu_grad(float z) {
  const float cdf = 0.5f * (1.0f + erff(z * 0.70710678118654752f));
  const float pdf = expf(-0.5f * z * z) * 0.39894228040143268f;
  return cdf + z * pdf;
}

__global__ void bias_gelu_kernel(const float* __restrict__ acc, int64_t rows, int64_t cols,
                                 const uint16_t* __restrict__ b16, uint16_t* __restrict__ z16,
                                 uint16_t* __restrict__ a16) {
  const int64_t n = rows * cols;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const float z = acc[i] + (b16 ? h2f(b16[i % cols]) : 0.0f);
    const uint32_t zc = f32_to_f16(z);
    z16[i] = static_cast<uint16_t>(zc);
    if (a16) a16[i] = static_cast<uint16_t>(f32_to_f16(gelu(h2f(static_cast<uint16_t>(zc)))));
  }
}

// One block; thread-per-row loop; deterministic loss reduction.
__global__ __launch_bounds__(256) void softmax_xent_kernel(
    const uint16_t* __restrict__ logits, const int32_t* __restrict__ labels, int64_t rows,
    int64_t cols, const amp_scaler_state* __restrict__ st, float* __restrict__ loss,
    uint16_t* __restrict__ dlog) {
  __shared__ float part[256];
  const float S = st ? st->scale : 1.0f;
  const float inv_rows = 1.0f / static_cast<float>(rows);
  float acc = 0.0f;
  for (int64_t r = threadIdx.x; r < rows; r += 256) {
    const uint16_t* l = logits + r * cols;
    float m = -INFINITY;
    for (int64_t c = 0; c < cols; ++c) m = fmaxf(m, h2f(l[c]));
    float s = 0.0f;
    for (int64_t c = 0; c < cols; ++c) s += expf(h2f(l[c]) - m);
    const float lse = m + logf(s);
    const int32_t y = labels[r];
    if (y < 0 || y >= cols) {
      // a label outside 0..cols-1 has no loss term: the row adds NaN to the
      // loss and contributes a zero gradient (nothing out of range is read)
      acc += __builtin_nanf("");
      if (dlog)
        for (int64_t c = 0; c < cols; ++c) dlog[r * cols + c] = 0;
      continue;
    }
    acc += lse - h2f(l[y]);
    if (dlog) {
      const float inv_s = 1.0f / s;
      for (int64_t c = 0; c < cols; ++c) {
        const float p = expf(h2f(l[c]) - m) * inv_s;
        const float d = (p - (c == y ? 1.0f : 0.0f)) * S * inv_rows;
        dlog[r * cols + c] = static_cast<uint16_t>(f32_to_f16(d));
      }
    }
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.0f;
    for (int i = 0; i < 256; ++i) tot += part[i];
    if (loss) *loss = tot * inv_rows;
  }
}

__global__ void gelu_backward_kernel(const uint16_t* __restrict__ dA, const uint16_t* __restrict__ z,
                                     int64_t n, uint16_t* __restrict__ dz) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const float g = gelu_grad(h2f(z[i]));
    dz[i] = static_cast<uint16_t>(f32_to_f16(h2f(dA[i]) * g));
  }
}

__global__ void colsum_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                              uint16_t* __restrict__ out) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (c >= cols) return;
  float s = 0.0f;
  for (int64_t r = 0; r < rows; ++r) s += h2f(x[r * cols + c]);
  out[c] = static_cast<uint16_t>(f32_to_f16(s));
}

unsigned grid_of(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b > 4096) b = 4096;
  return static_cast<unsigned>(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_bias_gelu(const float* acc, int64_t rows, int64_t cols, const void* b16,
                            void* z16, void* a16, hipStream_t s) {
  bias_gelu_kernel<<<grid_of(rows * cols), 256, 0, s>>>(
      acc, rows, cols, static_cast<const uint16_t*>(b16), static_cast<uint16_t*>(z16),
      static_cast<uint16_t*>(a16));
  return hipGetLastError();
}

hipError_t launch_softmax_xent(const void* logits16, const int32_t* labels, int64_t rows,
                               int64_t cols, const amp_scaler_state* st, float* loss,
                               void* dlog16, hipStream_t s) {
  softmax_xent_kernel<<<1, 256, 0, s>>>(static_cast<const uint16_t*>(logits16), labels, rows, cols,
                                        st, loss, static_cast<uint16_t*>(dlog16));
  return hipGetLastError();
}

hipError_t launch_gelu_backward(const void* dA16, const void* z16, int64_t n, void* dz16,
                                hipStream_t s) {
  gelu_backward_kernel<<<grid_of(n), 256, 0, s>>>(static_cast<const uint16_t*>(dA16),
                                                  static_cast<const uint16_t*>(z16), n,
                                                  static_cast<uint16_t*>(dz16));
  return hipGetLastError();
}

hipError_t launch_colsum(const void* x16, int64_t rows, int64_t cols, void* out16, hipStream_t s) {
  colsum_kernel<<<static_cast<unsigned>((cols + 255) / 256), 256, 0, s>>>(
      static_cast<const uint16_t*>(x16), rows, cols, static_cast<uint16_t*>(out16));
  return hipGetLastError();
}

}  // namespace amp
