// C ABI front of the HIP library: argument validation, device check and
// dispatch to the kernel launchers.  Nothing is enqueued unless every
// argument is valid; no call synchronises the host or allocates memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "amp.h"
#include "common.hpp"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other
std::mutex g_device_mu;

int check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    g_last_hip_error = static_cast<int>(e);
    return AMP_ENODEVICE;
  }
  int st = g_device_ok[dev].load(std::memory_order_acquire);
  if (st == 0) {
    std::lock_guard<std::mutex> lk(g_device_mu);
    st = g_device_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
      hipDeviceProp_t prop;
      e = hipGetDeviceProperties(&prop, dev);
      if (e != hipSuccess) {
        g_last_hip_error = static_cast<int>(e);
        return AMP_ENODEVICE;
      }
      st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
      g_device_ok[dev].store(st, std::memory_order_release);
    }
  }
  return st == 1 ? AMP_OK : AMP_ENODEVICE;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return AMP_OK;
  g_last_hip_error = static_cast<int>(e);
  return AMP_EHIP;
}

bool is_cast_in(int t) { return t == AMP_F32 || t == AMP_F16 || t == AMP_BF16; }
bool is_cast_out(int t) { return t == AMP_F16 || t == AMP_BF16 || t == AMP_E4M3 || t == AMP_E5M2; }
bool is_grad(int t) { return t == AMP_F32 || t == AMP_F16 || t == AMP_BF16; }
bool is_fp8(int t) { return t == AMP_E4M3 || t == AMP_E5M2; }

// Device state and scalar pointers must be naturally aligned (they are read
// as wide words and updated by atomics); a misaligned one is an argument
// error, not a memory fault.  NULL passes (optional arguments).
bool al(const void* p, uintptr_t a) { return p == nullptr || amp::aligned(p, a); }

}  // namespace

extern "C" {

int amp_abi_version(void) { return AMP_ABI_VERSION; }

const char* amp_status_string(int status) {
  switch (status) {
    case AMP_OK: return "ok";
    case AMP_EINVAL: return "invalid argument";
    case AMP_EUNSUPPORTED: return "unsupported dtype or layout";
    case AMP_EHIP: return "HIP runtime error";
    case AMP_ENODEVICE: return "no gfx950 device is current";
    default: return "unknown status";
  }
}

int amp_last_hip_error(void) { return g_last_hip_error; }

int amp_cast(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx, void* y, int yt,
             int64_t ldy, void* y_t, int64_t ldy_t, const float* d_scale, float* d_amax,
             void* stream) {
  return amp_cast_ex(x, xt, rows, cols, ldx, y, yt, ldy, y_t, ldy_t, d_scale, d_amax, nullptr,
                     stream);
}

int amp_cast_ex(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx, void* y, int yt,
                int64_t ldy, void* y_t, int64_t ldy_t, const float* d_scale, float* d_amax,
                unsigned long long* d_sat_count, void* stream) {
  if (!al(d_scale, 4) || !al(d_amax, 4) || !al(d_sat_count, 8)) return AMP_EINVAL;
  if (rows < 0 || cols < 0) return AMP_EINVAL;
  if (!is_cast_in(xt) || !is_cast_out(yt)) return AMP_EUNSUPPORTED;
  if (rows == 0 || cols == 0) return AMP_OK;
  if (!x || (!y && !y_t)) return AMP_EINVAL;
  if (ldx < cols || (y && ldy < cols) || (y_t && ldy_t < rows)) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_cast(x, xt, rows, cols, ldx, y, yt, ldy, y_t, ldy_t, d_scale,
                                     d_amax, d_sat_count, static_cast<hipStream_t>(stream)));
}

int amp_cast_current_scaling(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                             void* y, int yt, int64_t ldy, void* y_t, int64_t ldy_t,
                             const amp_delayed_recipe* r, amp_fp8_meta* d_meta, void* stream) {
  if (!al(d_meta, alignof(amp_fp8_meta))) return AMP_EINVAL;
  if (rows < 0 || cols < 0 || !r || !d_meta) return AMP_EINVAL;
  if (!(r->fp8_max > 0.0f) || !(r->margin > 0.0f)) return AMP_EINVAL;
  if (!is_cast_in(xt) || !is_cast_out(yt)) return AMP_EUNSUPPORTED;
  if (rows == 0 || cols == 0) return AMP_OK;
  if (!x || (!y && !y_t)) return AMP_EINVAL;
  if (ldx < cols || (y && ldy < cols) || (y_t && ldy_t < rows)) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_cast_current(x, xt, rows, cols, ldx, y, yt, ldy, y_t, ldy_t,
                                             r->fp8_max, r->margin, d_meta,
                                             static_cast<hipStream_t>(stream)));
}

int amp_gemm(int opA, int opB, int64_t M, int64_t N, int64_t K, const void* A, int at,
             int64_t lda, const float* d_alphaA, const void* B, int bt, int64_t ldb,
             const float* d_alphaB, void* C, int ct, int64_t ldc, const amp_block_scales* bsA,
             const amp_block_scales* bsB, void* stream) {
  return amp_gemm_ex(opA, opB, M, N, K, A, at, lda, d_alphaA, B, bt, ldb, d_alphaB, C, ct, ldc,
                     bsA, bsB, 0, stream);
}

int amp_gemm_ex(int opA, int opB, int64_t M, int64_t N, int64_t K, const void* A, int at,
                int64_t lda, const float* d_alphaA, const void* B, int bt, int64_t ldb,
                const float* d_alphaB, void* C, int ct, int64_t ldc,
                const amp_block_scales* bsA, const amp_block_scales* bsB, int flags,
                void* stream) {
  if (!al(d_alphaA, 4) || !al(d_alphaB, 4)) return AMP_EINVAL;
  if (flags & ~(AMP_GEMM_FP8_NATIVE | AMP_GEMM_MX)) return AMP_EINVAL;
  if (M < 0 || N < 0 || K < 0) return AMP_EINVAL;
  if ((opA != AMP_OP_N && opA != AMP_OP_T) || (opB != AMP_OP_N && opB != AMP_OP_T))
    return AMP_EINVAL;
  if (ct != AMP_F32 && ct != AMP_F16 && ct != AMP_BF16) return AMP_EUNSUPPORTED;
  const bool mx = (flags & AMP_GEMM_MX) != 0;
  const bool nvfp4 = at == AMP_E2M1X2 || bt == AMP_E2M1X2;
  if (mx) {
    const bool fp4 = at == AMP_E2M1X2 && bt == AMP_E2M1X2;
    if (!fp4 && !(is_fp8(at) && is_fp8(bt))) return AMP_EUNSUPPORTED;
    if (opA != AMP_OP_N || opB != AMP_OP_T || (fp4 && (flags & AMP_GEMM_FP8_NATIVE)))
      return AMP_EINVAL;
    if (!bsA || !bsB || !bsA->scales || !bsB->scales || bsA->block2d || bsB->block2d)
      return AMP_EINVAL;
    if (K % 32 != 0) return AMP_EINVAL;
  } else if (nvfp4) {
    if (at != bt || opA != AMP_OP_N || opB != AMP_OP_T) return AMP_EUNSUPPORTED;
    if (!bsA || !bsB || !bsA->scales || !bsB->scales) return AMP_EINVAL;
    if (K % 16 != 0) return AMP_EINVAL;
  } else if (is_fp8(at) || is_fp8(bt)) {
    if (!is_fp8(at) || !is_fp8(bt) || opA != AMP_OP_N || opB != AMP_OP_T) return AMP_EUNSUPPORTED;
    if (bsA || bsB) return AMP_EINVAL;
  } else {
    if (!((at == AMP_F16 || at == AMP_BF16) && at == bt)) return AMP_EUNSUPPORTED;
    if (bsA || bsB) return AMP_EINVAL;
  }
  if (M == 0 || N == 0) return AMP_OK;
  if (!C || ldc < N) return AMP_EINVAL;
  if (K > 0) {
    if (!A || !B) return AMP_EINVAL;
    // leading dimensions in elements (NVFP4: bytes = K/2 per row)
    const int64_t kA = nvfp4 ? K / 2 : K, kB = nvfp4 ? K / 2 : K;
    if (opA == AMP_OP_N ? lda < kA : lda < M) return AMP_EINVAL;
    if (opB == AMP_OP_T ? ldb < kB : ldb < N) return AMP_EINVAL;
    if (mx && (bsA->ld < K / 32 || bsB->ld < K / 32)) return AMP_EINVAL;
    if (!mx && nvfp4 && (bsA->ld < K / 16 || bsB->ld < K / 16)) return AMP_EINVAL;
    if (!mx && nvfp4 && ((bsA->block2d && M % 16) || (bsB->block2d && N % 16))) return AMP_EINVAL;
  }
  if (int st = check_device()) return st;
  return hip_status(amp::launch_gemm(opA, opB, M, N, K, A, at, lda, d_alphaA, B, bt, ldb,
                                     d_alphaB, C, ct, ldc, bsA, bsB, flags,
                                     static_cast<hipStream_t>(stream)));
}

int amp_scaler_init(amp_scaler_state* d_state, float init_scale, void* stream) {
  if (!al(d_state, 8)) return AMP_EINVAL;
  if (!d_state || !(init_scale > 0.0f)) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_scaler_init(d_state, init_scale, static_cast<hipStream_t>(stream)));
}

int amp_check_overflow(const void* x, int xt, int64_t n, amp_scaler_state* d_state,
                       void* stream) {
  if (!al(d_state, 8)) return AMP_EINVAL;
  if (n < 0 || !d_state) return AMP_EINVAL;
  if (!is_grad(xt)) return AMP_EUNSUPPORTED;
  if (n == 0) return AMP_OK;
  if (!x) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_check_overflow(x, xt, n, d_state, static_cast<hipStream_t>(stream)));
}

int amp_found_inf_from_amax(const float* d_amax, int32_t n, int yt, const float* d_scale,
                            amp_scaler_state* d_state, void* stream) {
  if (!al(d_amax, 4) || !al(d_scale, 4) || !al(d_state, 8)) return AMP_EINVAL;
  if (n < 0 || !d_state) return AMP_EINVAL;
  if (yt != AMP_F16 && yt != AMP_BF16 && !is_fp8(yt)) return AMP_EUNSUPPORTED;
  if (n == 0) return AMP_OK;
  if (!d_amax) return AMP_EINVAL;
  if (int e = check_device()) return e;
  return hip_status(amp::launch_found_inf_from_amax(d_amax, n, yt, d_scale, d_state,
                                                    static_cast<hipStream_t>(stream)));
}

int amp_optimizer_step_ex(float* master, float* m, float* v, const void* grads, int gt,
                          void* w16, int wt, int64_t n, const amp_adamw_hparams* hp,
                          amp_scaler_state* d_state, const float* d_grad_mult, int flags,
                          void* stream) {
  if (!al(master, 4) || !al(m, 4) || !al(v, 4) || !al(d_state, 8) || !al(d_grad_mult, 4)) return AMP_EINVAL;
  if (n < 0 || !hp || !d_state) return AMP_EINVAL;
  if (!is_grad(gt)) return AMP_EUNSUPPORTED;
  if (w16 && wt != AMP_F16 && wt != AMP_BF16) return AMP_EUNSUPPORTED;
  if (flags & ~AMP_OPT_SKIP_CHECK) return AMP_EINVAL;
  if (n > 0 && (!master || !m || !v || !grads)) return AMP_EINVAL;
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0 && hp->beta2 >= 0.0 && hp->beta2 < 1.0))
    return AMP_EINVAL;
  if (int st = check_device()) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (n > 0) {
    if (!(flags & AMP_OPT_SKIP_CHECK)) {
      if (int st = hip_status(amp::launch_check_overflow(grads, gt, n, d_state, s))) return st;
    }
    if (int st = hip_status(amp::launch_optimizer_apply(master, m, v, grads, gt, w16, wt, n, *hp,
                                                        d_state, d_grad_mult, s)))
      return st;
  }
  return hip_status(amp::launch_optimizer_commit(d_state, *hp, s));
}

int amp_optimizer_step(float* master, float* m, float* v, const void* grads, int gt, void* w16,
                       int wt, int64_t n, const amp_adamw_hparams* hp,
                       amp_scaler_state* d_state, int flags, void* stream) {
  return amp_optimizer_step_ex(master, m, v, grads, gt, w16, wt, n, hp, d_state, nullptr, flags,
                               stream);
}

int amp_mx_quantize(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                    int transpose, int yt, uint8_t* q, uint8_t* scales, void* stream) {
  if (rows < 0 || cols < 0 || ldx < cols) return AMP_EINVAL;
  if (!is_cast_in(xt)) return AMP_EUNSUPPORTED;
  if (yt != AMP_E4M3 && yt != AMP_E5M2 && yt != AMP_E2M1X2) return AMP_EUNSUPPORTED;
  const int64_t K = transpose ? rows : cols;
  if (K % 32) return AMP_EINVAL;
  if (rows == 0 || cols == 0) return AMP_OK;
  if (!x || !q || !scales || !amp::aligned(q, 16)) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_mx_quantize(x, xt, rows, cols, ldx, transpose ? 1 : 0, yt, q,
                                            scales, static_cast<hipStream_t>(stream)));
}

int amp_quantize_blockwise(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                           int yt, int block, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                           uint8_t* qt, int64_t ldqt, float* st, int64_t ldst, void* stream) {
  if (!al(s, 4) || !al(st, 4)) return AMP_EINVAL;
  if (rows < 0 || cols < 0 || ldx < cols || (block != 0 && block != 1)) return AMP_EINVAL;
  if (!is_cast_in(xt)) return AMP_EUNSUPPORTED;
  if (!is_fp8(yt)) return AMP_EUNSUPPORTED;
  if (rows == 0 || cols == 0) return AMP_OK;
  if (!x || (!q && !qt) || (!q != !s) || (!qt != !st)) return AMP_EINVAL;
  const int64_t rb = (rows + 127) / 128, cb = (cols + 127) / 128;
  if (q && (ldq < cols || lds < (block ? rb : rows))) return AMP_EINVAL;
  if (qt && (ldqt < rows || ldst < (block ? cb : cols))) return AMP_EINVAL;
  if (int e = check_device()) return e;
  return hip_status(amp::launch_quantize_blockwise(x, xt, rows, cols, ldx, yt, block, q, ldq, s,
                                                   lds, qt, ldqt, st, ldst,
                                                   static_cast<hipStream_t>(stream)));
}

int amp_gemm_blockwise(int64_t M, int64_t N, int64_t K, const void* A, int at, int64_t lda,
                       const float* sA, int64_t ldsA, int a_block, const void* B, int bt,
                       int64_t ldb, const float* sB, int64_t ldsB, int b_block, void* C, int ct,
                       int64_t ldc, void* stream) {
  if (!al(sA, 4) || !al(sB, 4)) return AMP_EINVAL;
  if (M < 0 || N < 0 || K < 0) return AMP_EINVAL;
  if ((a_block != 0 && a_block != 1) || (b_block != 0 && b_block != 1)) return AMP_EINVAL;
  if (!is_fp8(at) || !is_fp8(bt)) return AMP_EUNSUPPORTED;
  if (ct != AMP_F32 && ct != AMP_F16 && ct != AMP_BF16) return AMP_EUNSUPPORTED;
  if (M == 0 || N == 0) return AMP_OK;
  if (!C || ldc < N) return AMP_EINVAL;
  if (K > 0) {
    if (!A || !B || !sA || !sB || lda < K || ldb < K) return AMP_EINVAL;
    if (ldsA < (a_block ? (M + 127) / 128 : M) || ldsB < (b_block ? (N + 127) / 128 : N))
      return AMP_EINVAL;
  }
  if (int e = check_device()) return e;
  return hip_status(amp::launch_gemm_blockwise(M, N, K, A, at, lda, sA, ldsA, a_block, B, bt, ldb,
                                               sB, ldsB, b_block, C, ct, ldc,
                                               static_cast<hipStream_t>(stream)));
}

int amp_grad_accumulate(float* acc, const void* grads, int gt, int64_t n, int first,
                        void* stream) {
  if (!al(acc, 4)) return AMP_EINVAL;
  if (n < 0) return AMP_EINVAL;
  if (!is_grad(gt)) return AMP_EUNSUPPORTED;
  if (n == 0) return AMP_OK;
  if (!acc || !grads) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_grad_accumulate(acc, grads, gt, n, first ? 1 : 0,
                                                static_cast<hipStream_t>(stream)));
}

int amp_grad_norm_init(amp_grad_norm_state* d_norm, void* stream) {
  if (!al(d_norm, 8)) return AMP_EINVAL;
  if (!d_norm) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_grad_norm_init(d_norm, static_cast<hipStream_t>(stream)));
}

int amp_grad_norm_accumulate(const void* grads, int gt, int64_t n, amp_scaler_state* d_state,
                             amp_grad_norm_state* d_norm, void* stream) {
  if (!al(d_state, 8) || !al(d_norm, 8)) return AMP_EINVAL;
  if (n < 0 || !d_state || !d_norm) return AMP_EINVAL;
  if (!is_grad(gt)) return AMP_EUNSUPPORTED;
  if (n == 0) return AMP_OK;
  if (!grads) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_grad_norm(grads, gt, n, d_state, d_norm,
                                          static_cast<hipStream_t>(stream)));
}

int amp_grad_norm_accumulate_noalloc(const void* grads, int gt, int64_t n,
                                     amp_scaler_state* d_state, double* d_sumsq, void* stream) {
  if (!al(d_state, 8) || !al(d_sumsq, 8)) return AMP_EINVAL;
  if (n < 0 || !d_state || !d_sumsq) return AMP_EINVAL;
  if (!is_grad(gt)) return AMP_EUNSUPPORTED;
  if (n == 0) return AMP_OK;
  if (!grads) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_grad_norm_noalloc(grads, gt, n, d_state, d_sumsq,
                                                  static_cast<hipStream_t>(stream)));
}

int amp_clip_coefficient(const amp_grad_norm_state* d_norm, float max_norm,
                         const amp_scaler_state* d_state, float* d_out, void* stream) {
  if (!al(d_norm, 8) || !al(d_state, 8) || !al(d_out, 4)) return AMP_EINVAL;
  if (!d_norm || !d_state || !d_out || !(max_norm > 0.0f) || !(max_norm < 3.0e38f))
    return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_clip_coefficient(d_norm, max_norm, d_state, d_out,
                                                 static_cast<hipStream_t>(stream)));
}

int amp_scaler_update(amp_scaler_state* d_state, const amp_scaler_params* p, void* stream) {
  if (!al(d_state, 8)) return AMP_EINVAL;
  if (!d_state) return AMP_EINVAL;
  amp_scaler_params q{2.0f, 0.5f, 2000};
  if (p) q = *p;
  if (q.growth_interval <= 0) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_scaler_update(d_state, q, static_cast<hipStream_t>(stream)));
}

int amp_fp8_meta_init(amp_fp8_meta* d_metas, float* d_history, int32_t n, int32_t history_len,
                      void* stream) {
  if (!al(d_metas, alignof(amp_fp8_meta)) || !al(d_history, 4)) return AMP_EINVAL;
  if (n < 0 || history_len <= 0) return AMP_EINVAL;
  if (n == 0) return AMP_OK;
  if (!d_metas || !d_history) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_meta_init(d_metas, d_history, n, history_len,
                                          static_cast<hipStream_t>(stream)));
}

int amp_delayed_scaling_update(amp_fp8_meta* d_metas, float* d_history, int32_t n,
                               const amp_delayed_recipe* r, void* stream) {
  if (!al(d_metas, alignof(amp_fp8_meta)) || !al(d_history, 4)) return AMP_EINVAL;
  if (n < 0 || !r || r->history_len <= 0) return AMP_EINVAL;
  if (r->algo != AMP_AMAX_MAX && r->algo != AMP_AMAX_MOST_RECENT) return AMP_EINVAL;
  if (!(r->fp8_max > 0.0f) || !(r->margin > 0.0f)) return AMP_EINVAL;
  if (n == 0) return AMP_OK;
  if (!d_metas || !d_history) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_delayed_update(d_metas, d_history, n, *r,
                                               static_cast<hipStream_t>(stream)));
}

int amp_nvfp4_quantize(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                       int transpose, int block2d, int rht, uint64_t rht_seed, int rnd,
                       uint64_t sr_seed, uint8_t* q, uint8_t* scales, float* d_tensor,
                       void* stream) {
  if (!al(d_tensor, 4)) return AMP_EINVAL;
  if (rows < 0 || cols < 0 || ldx < cols) return AMP_EINVAL;
  if (xt != AMP_BF16 && xt != AMP_F32) return AMP_EUNSUPPORTED;
  if (rnd != AMP_ROUND_RNE && rnd != AMP_ROUND_SR) return AMP_EINVAL;
  const int64_t R = transpose ? cols : rows, K = transpose ? rows : cols;
  if (R % 16 || K % 16) return AMP_EINVAL;
  if (!d_tensor) return AMP_EINVAL;
  if (R > 0 && K > 0 && (!x || !q || !scales)) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_nvfp4_quantize(x, xt, rows, cols, ldx, transpose, block2d, rht,
                                               rht_seed, rnd, sr_seed, q, scales, d_tensor,
                                               static_cast<hipStream_t>(stream)));
}

int amp_bias_gelu_f16(const float* acc, int64_t rows, int64_t cols, const void* b16, void* z16,
                      void* a16, void* stream) {
  if (!al(acc, 4)) return AMP_EINVAL;
  if (rows < 0 || cols < 0) return AMP_EINVAL;
  if (rows == 0 || cols == 0) return AMP_OK;
  if (!acc || !z16) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_bias_gelu(acc, rows, cols, b16, z16, a16,
                                          static_cast<hipStream_t>(stream)));
}

int amp_softmax_xent_f16(const void* logits16, const int32_t* labels, int64_t rows, int64_t cols,
                         const amp_scaler_state* d_state, float* d_loss, void* dlogits16,
                         void* stream) {
  if (!al(labels, 4) || !al(d_state, 8) || !al(d_loss, 4)) return AMP_EINVAL;
  if (rows < 0 || cols <= 0 || rows > 65536) return AMP_EINVAL;
  if (rows == 0) return AMP_OK;
  if (!logits16 || !labels) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_softmax_xent(logits16, labels, rows, cols, d_state, d_loss,
                                             dlogits16, static_cast<hipStream_t>(stream)));
}

int amp_gelu_backward_f16(const void* dA16, const void* z16, int64_t n, void* dz16, void* stream) {
  if (n < 0) return AMP_EINVAL;
  if (n == 0) return AMP_OK;
  if (!dA16 || !z16 || !dz16) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_gelu_backward(dA16, z16, n, dz16, static_cast<hipStream_t>(stream)));
}

int amp_colsum_f16(const void* x16, int64_t rows, int64_t cols, void* out16, void* stream) {
  if (rows < 0 || cols < 0) return AMP_EINVAL;
  if (cols == 0) return AMP_OK;
  if (!out16 || (rows > 0 && !x16)) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_colsum(x16, rows, cols, out16, static_cast<hipStream_t>(stream)));
}

int amp_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0) return AMP_EINVAL;
  if (bytes == 0) return AMP_OK;
  if (!src || !dst || !amp::aligned(src, 16) || !amp::aligned(dst, 16)) return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_stream_copy(src, dst, bytes, static_cast<hipStream_t>(stream)));
}

int amp_fp8_mfma_probe(int shape, int at, const void* a, const void* b, float* c, int64_t tiles,
                       void* stream) {
  if (shape < 0 || shape > 3 || tiles < 0) return AMP_EINVAL;
  if (at != AMP_E4M3 && at != AMP_E5M2) return AMP_EUNSUPPORTED;
  if (tiles == 0) return AMP_OK;
  const uintptr_t al_ab = shape <= 1 ? 8 : 32;
  if (!a || !b || !c || !amp::aligned(a, al_ab) || !amp::aligned(b, al_ab) || !amp::aligned(c, 4))
    return AMP_EINVAL;
  if (int st = check_device()) return st;
  return hip_status(amp::launch_fp8_mfma_probe(shape, at, a, b, c, tiles,
                                               static_cast<hipStream_t>(stream)));
}

}  // extern "C"
