/*
 * amp.h -- C ABI of the MI355X (gfx950) mixed-precision training hot path.
 *
 * Three parts, as the pages describe mixed-precision training:
 *   1. scaled down-casts to FP16 / BF16 / FP8 (E4M3 forward, E5M2 backward)
 *      with amax capture, delayed and current scaling, plus the NVFP4,
 *      MX and fine-grained (tile / block) FP8 quantizers;
 *   2. low-precision GEMM with FP32 accumulation (forward, dgrad, wgrad);
 *   3. the fused FP32-master AdamW step with dynamic loss scaling, with
 *      gradient accumulation and global-norm clipping.
 *
 * Conventions for every call
 * --------------------------
 *  - All tensor arguments are DEVICE pointers owned by the caller; the
 *    library never allocates, frees or retains them.  Host structs passed by
 *    pointer are read during the call only.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on that stream and never synchronises the host.
 *  - Matrices are row-major with a leading dimension (row stride) given in
 *    ELEMENTS (for AMP_E2M1X2: in bytes, i.e. pairs of elements).
 *  - Arguments are validated before anything is enqueued; on error nothing
 *    is launched and a negative amp_status is returned.  AMP_EHIP reports a
 *    failed launch; amp_last_hip_error() gives the hipError_t of the calling
 *    thread's last failure.  No C++ exception crosses this boundary.
 *  - Device pointers to state structs and scalars (amp_scaler_state,
 *    amp_grad_norm_state: 8 bytes; amp_fp8_meta, FP32 scalars and arrays:
 *    4 bytes; the 64-bit saturation counter: 8 bytes) must be naturally
 *    aligned, else AMP_EINVAL.
 *  - Numerical events (inf/NaN, saturation) are data, not errors.
 *  - Scalar state (loss scale, overflow flag, Adam step, FP8 scales) lives in
 *    device memory so that no step needs a host round trip.
 *  - Calls that share state buffers must be ordered on one stream (or
 *    synchronised by the caller); concurrent calls on distinct buffers are
 *    independent.
 */
#ifndef AMP_H_
#define AMP_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AMP_ABI_VERSION 1

typedef enum {
  AMP_OK = 0,
  AMP_EINVAL = -1,       /* bad pointer, size, stride or enum value        */
  AMP_EUNSUPPORTED = -2, /* valid but unsupported dtype/layout combination */
  AMP_EHIP = -3,         /* a HIP runtime call or kernel launch failed     */
  AMP_ENODEVICE = -4     /* the current device is not a gfx950 GPU         */
} amp_status;

typedef enum {
  AMP_F32 = 0,
  AMP_F16 = 1,   /* IEEE binary16, 1/5/10                         */
  AMP_BF16 = 2,  /* bfloat16, 1/8/7                               */
  AMP_E4M3 = 3,  /* OCP FP8 E4M3 "FN": max 448, no inf            */
  AMP_E5M2 = 4,  /* OCP FP8 E5M2: max 57344, IEEE-style inf/NaN   */
  AMP_E2M1X2 = 5 /* two FP4 E2M1 codes per byte, low nibble first */
} amp_dtype;

typedef enum { AMP_OP_N = 0, AMP_OP_T = 1 } amp_op;
typedef enum { AMP_ROUND_RNE = 0, AMP_ROUND_SR = 1 } amp_round;

/* Device-resident loss-scaler + Adam counter state (40 bytes).
 * Page "혼합 정밀도 학습" (itwiki), section "손실 스케일링": start at 2^16, halve
 * and skip on inf/NaN, double after 2000 clean steps. */
typedef struct {
  float scale;            /* loss scale S (a power of two in practice)     */
  int32_t growth_tracker; /* clean steps since the last change of S        */
  int32_t found_inf;      /* set to 1 by the overflow check, 0 by update   */
  int32_t pad_;
  int64_t adam_step;      /* applied optimizer steps                       */
  double beta1_pow;       /* beta1^adam_step (running float64 product)     */
  double beta2_pow;       /* beta2^adam_step                               */
} amp_scaler_state;

typedef struct {
  float growth_factor;     /* 2.0   */
  float backoff_factor;    /* 0.5   */
  int32_t growth_interval; /* 2000  */
} amp_scaler_params;

typedef struct {
  double lr, beta1, beta2, eps, weight_decay;
} amp_adamw_hparams;

/* Device-resident per-tensor FP8 metadata (16 bytes); the amax history is a
 * separate float array of `history_len` entries per tensor.
 * Page "FP8 혼합 정밀도 LLM 학습" (hwlabs), section "Delayed Scaling 동작 원리". */
typedef struct {
  float amax_cur;  /* max |x| accumulated by this step's casts (bit-max)   */
  float scale;     /* multiplier used by the casts of the next step        */
  float scale_inv; /* 1/scale, the dequantisation factor for GEMM epilogue */
  int32_t pos;     /* ring position of the next history entry              */
} amp_fp8_meta;

typedef enum { AMP_AMAX_MAX = 0, AMP_AMAX_MOST_RECENT = 1 } amp_amax_algo;

typedef struct {
  float fp8_max;       /* 448 (E4M3) or 57344 (E5M2)  */
  float margin;        /* 1.0 recommended             */
  int32_t history_len; /* 1024 by default             */
  int32_t algo;        /* amp_amax_algo               */
} amp_delayed_recipe;

/* NVFP4 block scales of one GEMM operand (the quantizer's output). */
typedef struct {
  const uint8_t* scales; /* E4M3 codes: [rows, K/16], or [rows/16, K/16] if block2d */
  int64_t ld;            /* row stride of `scales` in bytes                        */
  int32_t block2d;       /* 1: one scale per 16x16 tile                             */
  int32_t pad_;
} amp_block_scales;

/* Device-resident global-norm accumulator (caller-owned, 8 KiB + 8 B).
 * sumsq holds the running sum of squares of the unscaled gradients; partial
 * is the work area of one accumulation call (one float64 per work-group). */
#define AMP_NORM_PARTIALS 1024
typedef struct {
  double sumsq;
  double partial[AMP_NORM_PARTIALS];
} amp_grad_norm_state;

/* ------------------------------------------------------------------------ */

/* Library version, status text and the calling thread's last HIP error. */
int amp_abi_version(void);
const char* amp_status_string(int status);
int amp_last_hip_error(void);

/* amp_cast -- scaled down-cast with amax capture.
 * Sources: itwiki "FP16 학습 루프" (the 16-bit copy made just before each op);
 * hwlabs "FP8이 어려운 이유" (per-tensor scale, clip to [-448, 448]) and
 * "Delayed Scaling 동작 원리" (amax recorded each step, tensor read once).
 *
 *   y[i][j]   = round_yt( fl32(x[i][j] * scale) )
 *   y_t[j][i] = the same value (optional transposed copy)
 *   *d_amax   = max(*d_amax, max |x|)   (unscaled input; FP32 bit-pattern max,
 *                                        NaN dominates, canonical 0x7FC00000)
 *
 * x:      [rows, cols] of xt in {F32, F16, BF16}, row stride ldx >= cols.
 * y:      [rows, cols] of yt in {F16, BF16, E4M3, E5M2}, stride ldy; may be NULL
 *         if y_t is given.
 * y_t:    [cols, rows] of yt, stride ldy_t >= rows; NULL for none.
 * d_scale: device FP32 multiplier; NULL means 1 (no multiply).
 * d_amax:  device FP32 accumulated with max; NULL skips the reduction.  The
 *          caller (or amp_delayed_scaling_update) resets it.
 * Rounding: nearest-even.  FP16/BF16 overflow to +-inf and NaN -> canonical
 * quiet NaN; E4M3/E5M2 saturate to +-max (inf included) and NaN -> 0x7F.
 * rows or cols == 0 is a no-op. */
int amp_cast(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
             void* y, int yt, int64_t ldy, void* y_t, int64_t ldy_t,
             const float* d_scale, float* d_amax, void* stream);

/* amp_cast_ex -- amp_cast that also counts FP8 saturation.
 * Source: hwlabs "FP8이 어려운 이유" (values beyond the FP8 range are clipped to
 * it).  d_sat_count: device unsigned 64-bit counter, add-accumulated (the
 * caller zeroes it), or NULL: the number of elements whose scaled value
 * fl32(x * scale) has |t| > 448 (E4M3) or > 57344 (E5M2), infinities
 * included, NaN not.  FP16/BF16 outputs overflow to inf instead and count
 * nothing.  Every other argument and rule as amp_cast. */
int amp_cast_ex(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                void* y, int yt, int64_t ldy, void* y_t, int64_t ldy_t,
                const float* d_scale, float* d_amax, unsigned long long* d_sat_count,
                void* stream);

/* amp_gemm -- C = out_cast( alpha_A * alpha_B * op(A) @ op(B) ), FP32 accumulate.
 * Sources: itwiki "FP32 누산과 연산별 정밀도"; hwlabs "GEMM 누적 정밀도 문제";
 * marovi "La receta de precisión mixta".
 *
 * op(A) is [M, K]: opA == N: A stored [M, K] (stride lda >= K);
 *                  opA == T: A stored [K, M] (stride lda >= M).
 * op(B) is [K, N]: opB == N: B stored [K, N] (stride ldb >= N);
 *                  opB == T: B stored [N, K] (stride ldb >= K).
 * C is [M, N] of ct in {F32, F16, BF16}, stride ldc >= N.
 * Supported operand types:
 *   at == bt in {F16, BF16}           any opA/opB;
 *   at, bt in {E4M3, E5M2}            opA == N, opB == T (K-contiguous; the
 *                                      cast's transposed copy provides it);
 *   at == bt == E2M1X2 (NVFP4)        opA == N, opB == T, with bsA/bsB block
 *                                      scales; K % 16 == 0.
 * d_alphaA / d_alphaB: device FP32 factors (FP8: the tensors' scale_inv;
 * NVFP4: 1/tensor_enc); NULL means 1.  bsA/bsB must be NULL unless NVFP4.
 * M, N or K == 0 is handled (K == 0 writes zeros). */
int amp_gemm(int opA, int opB, int64_t M, int64_t N, int64_t K,
             const void* A, int at, int64_t lda, const float* d_alphaA,
             const void* B, int bt, int64_t ldb, const float* d_alphaB,
             void* C, int ct, int64_t ldc,
             const amp_block_scales* bsA, const amp_block_scales* bsB,
             void* stream);

/* amp_gemm_ex -- amp_gemm with flags.
 * AMP_GEMM_FP8_NATIVE: FP8 operands go to the CDNA4 FP8 matrix-core
 *   instruction (twice the BF16 rate).  Its 64-term dot products are formed
 *   with a reduced-precision internal sum (measured: errors near 2^-12 of the
 *   largest product in each 64-term group), the kind of limited FP8
 *   partial-sum precision hwlabs "GEMM 누적 정밀도 문제" describes for other
 *   hardware; the results between groups are accumulated in FP32.  (Every
 *   FP8 matrix-core instruction of gfx950 -- 32x32x16 and 16x16x32, and the
 *   block-scaled 32x32x64 and 16x16x128 -- measured the same way: see
 *   amp_fp8_mfma_probe.)  Without the flag (the default) FP8 operands are
 *   widened exactly to BF16 in registers before the BF16 matrix cores and
 *   every product is summed in FP32.
 * AMP_GEMM_MX: both operands are MX blocks from amp_mx_quantize (opA = N,
 *   opB = T; at = bt = AMP_E2M1X2, or at, bt in {E4M3, E5M2}); bsA / bsB hold
 *   the UE8M0 scale codes [rows, K/32] (block2d = 0, ld in bytes) and
 *   C = out_cast(alphaA * alphaB * sum_k a[m,k] 2^(sa-127) b[n,k] 2^(sb-127)).
 *   Full 256x256 tiles with K a multiple of 128 (FP8) or 256 (E2M1) run on
 *   the matrix cores, other shapes on an element-wise FP32 kernel.  FP8
 *   elements: each element times its block scale is formed exactly in BF16
 *   by the scaled conversion and summed on the BF16 matrix cores in FP32
 *   (exact products whenever the scaled elements are BF16 values: scale
 *   codes 3..246 for E4M3, 10..239 for E5M2, which amp_mx_quantize produces
 *   for every block whose maximum is at least 2^-116 / 2^-102); with
 *   AMP_GEMM_FP8_NATIVE as well they go to the block-scaled FP8 instruction
 *   instead (its reduced-precision internal sum).  E2M1 elements always use
 *   the block-scaled instruction, whose few product bits it sums exactly.
 * Other flags must be 0 (AMP_GEMM_FP8_NATIVE with E2M1 MX operands is
 * AMP_EINVAL). */
#define AMP_GEMM_FP8_NATIVE 1
#define AMP_GEMM_MX 2
int amp_gemm_ex(int opA, int opB, int64_t M, int64_t N, int64_t K,
                const void* A, int at, int64_t lda, const float* d_alphaA,
                const void* B, int bt, int64_t ldb, const float* d_alphaB,
                void* C, int ct, int64_t ldc,
                const amp_block_scales* bsA, const amp_block_scales* bsB,
                int flags, void* stream);

/* amp_scaler_init -- sets scale = init_scale, growth_tracker = found_inf = 0,
 * adam_step = 0, beta pows = 1 (GradScaler(init_scale) + fresh AdamW).
 * Source: itwiki "손실 스케일링" (dynamic loss scaling starts from a large
 * scale, 65536 with GradScaler's defaults) and "FP16 학습 루프" (the loop builds
 * GradScaler() and AdamW before training); marovi "Escalado dinámico de
 * pérdida". */
int amp_scaler_init(amp_scaler_state* d_state, float init_scale, void* stream);

/* amp_optimizer_step -- unscale by 1/S, check every gradient for inf/NaN,
 * and, only if none is found, apply AdamW to the FP32 master weights and
 * moments and re-round the 16-bit working copy.
 * Sources: itwiki "FP32 마스터 가중치" (update the FP32 copy, round16 from it;
 * 16 bytes/parameter), "손실 스케일링" (g = fp32(grad)/S; skip on inf/NaN);
 * marovi "Escalado dinámico de pérdida", "Operaciones que permanecen en FP32".
 *
 * master, m, v: [n] FP32, updated in place.
 * grads: [n] of gt in {F16, BF16, F32} (scaled by S).
 * w16:   [n] of wt in {F16, BF16}, overwritten with round(master); may be NULL.
 * flags: AMP_OPT_SKIP_CHECK -- the caller already OR-ed the overflow flag into
 *        d_state->found_inf (e.g. from its own gradient producer); no sweep.
 * Per element (FP32, no fused multiply-add):
 *   g = f32(grad) * (1/S); m = b1*m + (1-b1)*g; v = b2*v + (1-b2)*(g*g);
 *   d = sqrt(v) * rbc2 + eps; master = master*(1-lr*wd) - step*(m/d)
 * with step = lr/(1-b1^t), rbc2 = 1/sqrt(1-b2^t) from float64 state.
 * On overflow nothing is written and adam_step is unchanged.  Follow with
 * amp_scaler_update, which consumes and clears found_inf. */
#define AMP_OPT_SKIP_CHECK 1
int amp_optimizer_step(float* master, float* m, float* v, const void* grads, int gt,
                       void* w16, int wt, int64_t n, const amp_adamw_hparams* hp,
                       amp_scaler_state* d_state, int flags, void* stream);

/* amp_check_overflow -- OR (any non-finite element of x) into
 * d_state->found_inf.  x: [n] of xt in {F16, BF16, F32}.  Used when several
 * gradient buffers feed one optimizer step (then step with SKIP_CHECK).
 * Source: itwiki "손실 스케일링" (after unscaling, a step whose gradients hold
 * inf or NaN is skipped and the scale lowered); marovi "Escalado dinámico de
 * pérdida". */
int amp_check_overflow(const void* x, int xt, int64_t n, amp_scaler_state* d_state,
                       void* stream);

/* amp_found_inf_from_amax -- the overflow flag taken from the producer of the
 * gradients instead of a sweep over them (then amp_optimizer_step with
 * AMP_OPT_SKIP_CHECK is a single 28 B/parameter pass).  Source: itwiki
 * "손실 스케일링" (a step with any inf/NaN gradient is skipped).
 * d_amax: n device floats, the amax values that amp_cast recorded while
 * writing the gradients as yt in {F16, BF16, E4M3, E5M2} with the device
 * scale d_scale (NULL: 1).  Sets d_state->found_inf = 1 if an amax is inf or
 * NaN or, for F16/BF16, if round_yt(fl32(amax * scale)) is infinite --
 * exactly when some output of that cast is non-finite, since rounding is
 * monotone in |t|.  Never clears the flag. */
int amp_found_inf_from_amax(const float* d_amax, int32_t n, int yt, const float* d_scale,
                            amp_scaler_state* d_state, void* stream);

/* amp_scaler_update -- on found_inf: scale *= backoff, tracker = 0; else
 * tracker += 1 and at growth_interval: scale *= growth, tracker = 0.  Then
 * found_inf = 0.  No floor on the scale.  p == NULL uses (2, 0.5, 2000).
 * Source: itwiki "손실 스케일링" (halve on overflow, double after a run of
 * clean steps: GradScaler's update()); marovi "Escalado dinámico de pérdida"
 * and "Limitaciones y modos de fallo" (a collapsing scale is a symptom, not
 * clamped). */
int amp_scaler_update(amp_scaler_state* d_state, const amp_scaler_params* p, void* stream);

/* amp_cast_current_scaling -- current (just-in-time) scaling: one pass finds
 * amax(|x|) -> d_meta->amax_cur, then d_meta->scale = fp8_max / (margin *
 * amax) in FP32 (1 if the amax is zero or non-finite) and scale_inv = 1/scale,
 * then amp_cast with that scale (x read twice; pos and the history are not
 * touched).  Source: hwlabs "Delayed Scaling 동작 원리" (the contrast with
 * delayed scaling, which reads x once using earlier steps' amax).  Arguments
 * as amp_cast; r supplies fp8_max and margin. */
int amp_cast_current_scaling(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                             void* y, int yt, int64_t ldy, void* y_t, int64_t ldy_t,
                             const amp_delayed_recipe* r, amp_fp8_meta* d_meta, void* stream);

/* amp_fp8_meta_init -- n metas: amax_cur 0, scale = scale_inv = 1, pos 0,
 * and d_history[n * history_len] zero-filled.
 * Source: hwlabs "Delayed Scaling 동작 원리" (each FP8 tensor keeps an amax
 * history from which its scale is derived; before any history the scale is
 * the neutral 1). */
int amp_fp8_meta_init(amp_fp8_meta* d_metas, float* d_history, int32_t n,
                      int32_t history_len, void* stream);

/* amp_delayed_scaling_update -- for each of n metas (history of meta i at
 * d_history + i*history_len):
 *   history[pos] = amax_cur;
 *   amax_max = max(history) (AMP_AMAX_MAX) or history[pos] (MOST_RECENT);
 *   if amax_max is finite and > 0:
 *       scale = fp8_max / (margin * amax_max); scale_inv = 1/scale;
 *   pos = (pos + 1) % history_len; amax_cur = 0.
 * Source: hwlabs "Delayed Scaling 동작 원리" and "도입 체크리스트". */
int amp_delayed_scaling_update(amp_fp8_meta* d_metas, float* d_history, int32_t n,
                               const amp_delayed_recipe* r, void* stream);

/* amp_nvfp4_quantize -- NVFP4 two-level quantization of one GEMM operand.
 * Source: page "Pretraining Large Language Models with NVFP4", sections 2.1
 * (E2M1 elements, 16-element E4M3 block scales, FP32 tensor scale) and 2.2
 * items 2-4 (16x16 random Hadamard transform on weight-gradient inputs,
 * 16x16 weight blocks, stochastic rounding of gradients).
 *
 * x: [rows, cols] of xt in {BF16, F32}, stride ldx.  The quantized operand is
 *    op = x (transpose == 0) or x^T (transpose == 1), of shape [R, K]; blocks
 *    and the optional RHT run along K.  R and K must be multiples of 16.
 * rht: apply z = H16 diag(s) / 4 to each 16-chunk along K, s from Philox4x32-10
 *    (key rht_seed, counter (0,0,1,0), word 0).
 * block2d: one scale per 16x16 tile of op (weights) instead of per 1x16.
 * rnd: AMP_ROUND_RNE or AMP_ROUND_SR (Philox4x32-10, key sr_seed, element
 *    index idx = r*K + k: counter (idx>>2), word idx&3, u = (w>>8)*2^-24).
 * q: [R, K/2] bytes, two E2M1 codes per byte, low nibble = lower k.
 * scales: E4M3 codes [R, K/16] (or [R/16, K/16]), contiguous.
 * d_tensor: 3 device floats written as {amax of z, enc = 2688/amax (1 if the
 *    amax is 0 or not finite), dec = 1/enc}; pass &d_tensor[2] as the GEMM
 *    alpha.
 * Element: b = block amax; S = E4M3(fl32(fl32(b/6)*enc)); y = fl32(z*fl32(enc/S));
 *    code = E2M1(y) saturating at 6 (S == 0 gives code 0).
 * Range: for a tensor amax below about 2^-107 (enc = 2688/amax beyond
 *    2^118), enc/S overflows to inf and a zero element gives y = NaN; the
 *    code of such an element is that of magnitude 6 with an unspecified sign.
 *    Every other input is quantized exactly as described. */
int amp_nvfp4_quantize(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                       int transpose, int block2d, int rht, uint64_t rht_seed,
                       int rnd, uint64_t sr_seed, uint8_t* q, uint8_t* scales,
                       float* d_tensor, void* stream);

/* ---- Fine-grained FP8 scaling (tile and block scales) ----
 * Page "혼합 정밀도 학습" (itwiki), section "FP8 혼합 정밀도": DeepSeek-V3
 * computes FP8 scales on the fly per 1x128 tile of activations and per
 * 128x128 block of weights and keeps every tensor in E4M3; page hwlabs,
 * section "GEMM 누적 정밀도 문제": partial sums inside a tile, FP32 across
 * tiles.  Scales are stored K-block-major (the scales of one 128-wide K-block
 * are contiguous). */

/* amp_quantize_blockwise -- x [rows, cols] of xt in {F32, F16, BF16} (row
 * stride ldx >= cols) to yt in {E4M3, E5M2}, one FP32 scale per tile:
 *   block == 0: 1x128 tiles along the output's contiguous (K) dimension;
 *   block == 1: 128x128 blocks.
 * Outputs (device memory owned by the caller; either pair may be NULL, not
 * both):
 *   q  [rows, cols] codes of x (K = cols), row stride ldq >= cols, with
 *      s  FP32 scale_inv at s[(c/128)*lds + r] (block: r/128);
 *      lds >= rows (block: ceil(rows/128));
 *   qt [cols, rows] codes of x^T (K = rows), row stride ldqt >= rows, with
 *      st at st[(r/128)*ldst + c] (block: c/128); ldst >= cols (block:
 *      ceil(cols/128)).  Row tiles of x^T are 128x1 column tiles of x; a
 *      128x128 block has the same scale in both outputs.
 * Per tile: scale = fp8_max / amax(tile) in FP32 (448 for E4M3, 57344 for
 * E5M2; 1 if the amax is 0 or not finite); code = round(fl32(x * scale)),
 * nearest-even, saturating, NaN -> 0x7F; scale_inv = fl32(1 / scale).
 * Edge tiles may be short.  rows or cols == 0 is a no-op. */
int amp_quantize_blockwise(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                           int yt, int block, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                           uint8_t* qt, int64_t ldqt, float* st, int64_t ldst, void* stream);

/* amp_gemm_blockwise -- C = out_cast( sum_k (A[m,k] sa) (B[n,k] sb) ), the
 * GEMM of two fine-grained FP8 operands (C = A B^T; both K-contiguous, as
 * amp_quantize_blockwise writes them).
 *   A [M, K] of at in {E4M3, E5M2}, stride lda >= K; scale_inv sA[kb*ldsA +
 *     (a_block ? m/128 : m)], kb = k/128, ldsA >= M (a_block: ceil(M/128));
 *   B [N, K] of bt in {E4M3, E5M2}, stride ldb >= K; sB likewise with n;
 *   C [M, N] of ct in {F32, F16, BF16}, stride ldc >= N.
 * Each 128-K block's products are summed in FP32 (exact FP8 products) and
 * promoted as acc += P * fl32(sa * sb).  Full 256x128 tiles with K a multiple
 * of 128, per-row A scales (16-byte aligned, ldsA % 4 == 0) and bt == E4M3
 * run on the matrix cores; other shapes on an element-wise kernel.  M or
 * N == 0 is a no-op; K == 0 writes zeros. */
int amp_gemm_blockwise(int64_t M, int64_t N, int64_t K,
                       const void* A, int at, int64_t lda, const float* sA, int64_t ldsA,
                       int a_block, const void* B, int bt, int64_t ldb, const float* sB,
                       int64_t ldsB, int b_block, void* C, int ct, int64_t ldc, void* stream);

/* ---- FP16 AMP training step of a two-layer MLP: the element-wise glue ----
 * Page "혼합 정밀도 학습" (itwiki), section "FP16 학습 루프": Linear(512, 2048)
 * -> GELU -> Linear(2048, 10) under FP16 autocast with cross-entropy in FP32
 * and the backward pass started from S * loss; marovi "Operaciones que
 * permanecen en FP32" (softmax / cross-entropy in FP32).  FP16 tensors are
 * passed as raw 16-bit codes (void*).  The GEMMs of the step are amp_gemm
 * calls; these kernels cover what sits between them. */

/* z = round16(fl32(acc + b)) and, if a16 != NULL, a = round16(gelu(z)) with
 * the exact-erf GELU evaluated in FP32.  acc: [rows, cols] FP32 (contiguous);
 * b16: [cols] FP16 or NULL; z16, a16: [rows, cols] FP16. */
int amp_bias_gelu_f16(const float* acc, int64_t rows, int64_t cols, const void* b16,
                      void* z16, void* a16, void* stream);

/* Cross-entropy of FP16 logits [rows, cols] (contiguous) against int32
 * labels in [0, cols): *d_loss = mean over rows, in FP32 (NULL: not written);
 * dlogits16 = round16(S * (softmax - onehot) / rows) with S read from
 * d_state->scale (d_state NULL: S = 1; dlogits16 NULL: not written).
 * Runs as one work-group (meant for classifier heads, rows <= 65536).
 * labels are device int32 in 0..cols-1; a row whose label lies outside that
 * range adds NaN to the loss and gets an all-zero dlogits row (the kernel
 * reads no logit for it), so a bad label shows up as a NaN loss rather than
 * as a memory fault. */
int amp_softmax_xent_f16(const void* logits16, const int32_t* labels, int64_t rows,
                         int64_t cols, const amp_scaler_state* d_state, float* d_loss,
                         void* dlogits16, void* stream);

/* dz = round16(fl32(dA * fl32(gelu'(z)))), element-wise over n FP16 values. */
int amp_gelu_backward_f16(const void* dA16, const void* z16, int64_t n, void* dz16,
                          void* stream);

/* out[c] = round16(fl32(sum_r x[r][c])) (sequential FP32 sum; bias grads). */
int amp_colsum_f16(const void* x16, int64_t rows, int64_t cols, void* out16, void* stream);

/* amp_mx_quantize -- MX block quantization of one GEMM operand.
 * Source: itwiki "FP8 혼합 정밀도" (MX formats: one power-of-two scale per 32
 * elements), gist 2.1 (MXFP4: 32-element blocks, UE8M0 scales), with the OCP
 * microscaling conversion the page points to.
 * x: [rows, cols] of xt in {F32, F16, BF16}, stride ldx; op = x (transpose 0)
 *    or x^T (1), shape [R, K], K a multiple of 32, blocks along K.
 * yt: AMP_E4M3 / AMP_E5M2 (q: [R, K] bytes) or AMP_E2M1X2 (q: [R, K/2], two
 *    codes per byte, lower K in the low nibble).
 * scales: UE8M0 codes [R, K/32]: e = floor(log2(block amax)) - emax (8, 15,
 *    2 for E4M3, E5M2, E2M1) clamped to [-127, 127], stored as e + 127; 0 for
 *    an all-zero block, 0xFF for a block holding inf/NaN (its elements are
 *    then encoded unscaled).  Elements: x * 2^-e to the element format,
 *    nearest-even, saturating.  q and scales rows are contiguous; q 16-byte
 *    aligned. */
int amp_mx_quantize(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                    int transpose, int yt, uint8_t* q, uint8_t* scales, void* stream);

/* ---- gradient accumulation and global-norm clipping ----------------------
 * Page "혼합 정밀도 학습" (itwiki), section "FP16 학습 루프": the loop unscales
 * (unscale_) and only then clips the global gradient norm to max_norm = 1.0,
 * so that the norm is measured on gradients of their true size; section
 * "함께 쓰는 기법과 주의점": with gradient accumulation over micro-batches
 * the loss-scale adjustment and the inf check run once per effective batch.
 * Page "Mixed Precision Training/es" (marovi), "Operaciones que permanecen
 * en FP32": reductions such as gradient norms stay in (at least) FP32; page
 * hwlabs, "도입 체크리스트": keep gradient clipping (max_norm 1.0).
 *
 * Typical step: amp_grad_accumulate per micro-batch into an FP32 buffer;
 * amp_grad_norm_init; amp_grad_norm_accumulate over every gradient buffer
 * (it also sets found_inf, replacing amp_check_overflow); amp_clip_coefficient;
 * amp_optimizer_step_ex(..., d_coef, AMP_OPT_SKIP_CHECK); amp_scaler_update. */

/* acc[i] = f32(g[i]) if first, else fl32(acc[i] + f32(g[i])).  acc: [n] FP32
 * (in place); grads: [n] of gt in {F16, BF16, F32}.  inf and NaN propagate,
 * so one check of acc per effective batch sees every micro-batch. */
int amp_grad_accumulate(float* acc, const void* grads, int gt, int64_t n, int first,
                        void* stream);

/* d_norm->sumsq = 0. */
int amp_grad_norm_init(amp_grad_norm_state* d_norm, void* stream);

/* d_norm->sumsq += sum_i (f32(g[i]) * (1/S))^2 over the finite elements, the
 * squares exact in float64 and the sum in float64 (work-group partials added
 * in a fixed order, so the result is reproducible); S = d_state->scale.  Any
 * non-finite element sets d_state->found_inf = 1.  Calls on one d_norm must
 * not overlap. */
int amp_grad_norm_accumulate(const void* grads, int gt, int64_t n, amp_scaler_state* d_state,
                             amp_grad_norm_state* d_norm, void* stream);

/* amp_grad_norm_accumulate_noalloc -- amp_grad_norm_accumulate for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same kernels and the
 * same result bit for bit, but the running sum is one caller float64
 * (*d_sumsq += ..., the caller zeroes it) and the per-work-group partials
 * live in a file-scope device array of the library (1024 float64 = 8 KiB per
 * GPU, kept until the process ends; the pass never uses more work-groups, so
 * every n fits).  The call allocates nothing.  All calls on one GPU share
 * that array: calls that overlap on one GPU (other streams, other threads)
 * race and must be serialised by the caller.  d_sumsq: device, 8-byte
 * aligned. */
int amp_grad_norm_accumulate_noalloc(const void* grads, int gt, int64_t n,
                                     amp_scaler_state* d_state, double* d_sumsq, void* stream);

/* d_out[0] = coef = min(1, fl32(max_norm / fl32(norm + 1e-6))) and d_out[1] =
 * norm, with norm = fl32(sqrt(sumsq)) (float64 square root); if found_inf is
 * set: d_out = {1, +inf} (the step will be skipped).  max_norm > 0. */
int amp_clip_coefficient(const amp_grad_norm_state* d_norm, float max_norm,
                         const amp_scaler_state* d_state, float* d_out, void* stream);

/* amp_optimizer_step with an optional device FP32 gradient multiplier (the
 * clip coefficient): g = f32(grad) * (1/S), then g = fl32(g * *d_grad_mult)
 * when d_grad_mult != NULL; the rest as amp_optimizer_step. */
int amp_optimizer_step_ex(float* master, float* m, float* v, const void* grads, int gt,
                          void* w16, int wt, int64_t n, const amp_adamw_hparams* hp,
                          amp_scaler_state* d_state, const float* d_grad_mult, int flags,
                          void* stream);

/* amp_stream_copy -- a plain device copy dst[0..bytes) = src[0..bytes), the
 * reference for the HBM roofline of the element-wise kernels (not a step of
 * the training path).  The optimizer pass reads as many bytes as it writes, so
 * the rate of a plain copy (16-byte non-temporal loads and stores, four in
 * flight per thread, one contiguous 256 KiB range per work-group: the fastest
 * copy form measured on this part) is its practical ceiling on a given part.
 * src and dst: device memory, 16-byte aligned, not
 * overlapping; bytes == 0 is a no-op; misaligned or NULL pointers give
 * AMP_EINVAL. */
int amp_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* amp_fp8_mfma_probe -- one FP8 matrix-core instruction per wave on given
 * operand bytes, C_in = 0: the measurement behind AMP_GEMM_FP8_NATIVE's
 * precision note (hwlabs "GEMM 누적 정밀도 문제": FP8 matrix units may keep
 * limited precision in their partial sums); not a step of the training path.
 * shape: 0 = 32x32x16 FP8, 1 = 16x16x32 FP8, 2 = block-scaled 32x32x64
 * f8f6f4, 3 = block-scaled 16x16x128 f8f6f4 (neutral scales, 2^0).
 * at: format of A, AMP_E4M3 or AMP_E5M2; B is E4M3.
 * Layout, per tile t (tiles of them) and lane l = 0..63, with D = 32 (shapes
 * 0, 2) or 16 (1, 3), P = 8 (shapes 0, 1) or 32 (2, 3) bytes per lane and
 * R = 16 (32x32) or 4 (16x16) outputs per lane:
 *   a[(t*64 + l)*P + j], b[(t*64 + l)*P + j]: lane l holds row l % D of A
 *   and column l % D of B; A's byte j of lane l meets B's byte j of every
 *   lane with the same l / D (the same K index on both sides), so
 *   C[i][n] = sum over groups q < 64/D and bytes j of
 *             a[q*D + i][j] * b[q*D + n][j];
 *   c[(t*64 + l)*R + r] = C[row][l % D] with row = 8*(r/4) + 4*(l/32) + r%4
 *   (32x32) or 4*(l/16) + r (16x16).
 * a, b: device, 8-byte (shapes 0, 1) or 32-byte (2, 3) aligned; c: device,
 * 4-byte aligned.  tiles == 0 is a no-op. */
int amp_fp8_mfma_probe(int shape, int at, const void* a, const void* b, float* c,
                       int64_t tiles, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* AMP_H_ */
