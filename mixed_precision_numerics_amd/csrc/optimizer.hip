// Fused FP32-master AdamW step with dynamic loss scaling, the loss-scaler
// update and the delayed-scaling (amax history) update (gfx950).
//
// Sources: page "혼합 정밀도 학습" (itwiki), sections "FP32 마스터 가중치" (the
// update goes to the FP32 copy, the 16-bit copy is re-rounded from it) and
// "손실 스케일링" (unscale by 1/S in FP32; check every step for inf/NaN, skip
// the update and halve S on overflow, double S after 2000 clean steps); page
// "Mixed Precision Training/es" (marovi), sections "Escalado dinámico de
// pérdida" and "Operaciones que permanecen en FP32" (Adam moments stay FP32);
// page "FP8 혼합 정밀도 LLM 학습" (hwlabs), section "Delayed Scaling 동작 원리"
// (amax history, scale = fp8_max / (margin * amax_max)).  AdamW itself is
// only named on the pages; the update is the decoupled-weight-decay form.
//
// Skip semantics: an overflowing step must leave master, m, v, the 16-bit
// copy and the step count untouched, so an in-place update cannot begin
// before every gradient is checked.  The step is therefore two sweeps:
//   check  -- reads the 16-bit gradients (2 B/param) and sets found_inf;
//   apply  -- gated on found_inf, one fused pass over the state
//             (read g, master, m, v; write master, m, v, w16: 28 B/param).
// A producer that already knows the overflow flag skips the check sweep.
// The per-element arithmetic is FP32 without contraction (-ffp-contract=off):
//   g = f32(g16)*invS; m = b1*m + c1*g; v = b2*v + c2*(g*g);
//   d = sqrt(v)*rbc2 + eps; theta = theta*decay - step*(m/d); w16 = rne(theta).
#include <mutex>

#include "common.hpp"
#include "formats.hpp"

namespace amp {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- check ---
// 1 if the word holds a non-finite value (branch-free).
template <int GT>
__device__ __forceinline__ uint32_t nonfinite_word(uint32_t w) {
  if constexpr (GT == AMP_F32) {
    return static_cast<uint32_t>((w & 0x7f800000u) == 0x7f800000u);
  } else {
    constexpr uint32_t kMask = GT == AMP_F16 ? 0x7c007c00u : 0x7f807f80u;
    const uint32_t t = (w & kMask) ^ kMask;     // a half is non-finite iff its part is 0
    return static_cast<uint32_t>((t & 0xffffu) == 0) | static_cast<uint32_t>((t >> 16) == 0);
  }
}

// Vector path: work-group b scans the contiguous 16-byte words
// [b * chunk, (b + 1) * chunk) with four non-temporal loads in flight per
// thread (a grid-stride loop over the same grid ran at 6.5 TB/s).
template <int GT, bool VEC>
__global__ __launch_bounds__(kThreads) void check_kernel(const void* __restrict__ g, int64_t n,
                                                         int64_t chunk,
                                                         amp_scaler_state* __restrict__ st) {
  // a block that starts after the flag is already set has nothing to add;
  // one thread reads the flag so that the whole block leaves together
  __shared__ int done;
  if (threadIdx.x == 0)
    done = __hip_atomic_load(&st->found_inf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (done) return;
  const int eb = GT == AMP_F32 ? 4 : 2;
  const int64_t nvec = VEC ? n * eb / 16 : 0;
  const u32x4* gv = static_cast<const u32x4*>(g);
  uint32_t bad = 0;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t nthr = static_cast<int64_t>(gridDim.x) * kThreads;
  if constexpr (VEC) {
    const int64_t b0 = static_cast<int64_t>(blockIdx.x) * chunk;
    const int64_t b1 = b0 + chunk < nvec ? b0 + chunk : nvec;
    int64_t i = b0 + threadIdx.x;
    for (; i + 3 * kThreads < b1; i += 4 * kThreads) {
      u32x4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = __builtin_nontemporal_load(gv + i + u * kThreads);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        bad |= nonfinite_word<GT>(w[u].x) | nonfinite_word<GT>(w[u].y) |
               nonfinite_word<GT>(w[u].z) | nonfinite_word<GT>(w[u].w);
    }
    for (; i < b1; i += kThreads) {
      const u32x4 w = __builtin_nontemporal_load(gv + i);
      bad |= nonfinite_word<GT>(w.x) | nonfinite_word<GT>(w.y) | nonfinite_word<GT>(w.z) |
             nonfinite_word<GT>(w.w);
    }
  }
  // tail elements (n not a multiple of 16 bytes)
  for (int64_t e = nvec * 16 / eb + tid; e < n; e += nthr) {
    if constexpr (GT == AMP_F32) {
      bad |= nonfinite_word<GT>(static_cast<const uint32_t*>(g)[e]);
    } else {
      const uint32_t h = static_cast<const uint16_t*>(g)[e];
      bad |= nonfinite_word<GT>(h | (h << 16));
    }
  }
  if (__syncthreads_or(static_cast<int>(bad)) && threadIdx.x == 0) atomicOr(&st->found_inf, 1);
}

// ---------------------------------------------------------------- apply ---
struct StepScalars {
  float inv_s, b1, b2, c1, c2, eps, rbc2, decay, step;
  float mult;      // gradient multiplier (the clip coefficient) when MULT
};

__device__ __forceinline__ StepScalars make_scalars(const amp_scaler_state& st,
                                                    const amp_adamw_hparams& hp) {
  StepScalars k;
  const double b1p = st.beta1_pow * hp.beta1;
  const double b2p = st.beta2_pow * hp.beta2;
  k.step = static_cast<float>(hp.lr / (1.0 - b1p));
  k.rbc2 = static_cast<float>(1.0 / sqrt(1.0 - b2p));
  k.decay = static_cast<float>(1.0 - hp.lr * hp.weight_decay);
  k.c1 = static_cast<float>(1.0 - hp.beta1);
  k.c2 = static_cast<float>(1.0 - hp.beta2);
  k.b1 = static_cast<float>(hp.beta1);
  k.b2 = static_cast<float>(hp.beta2);
  k.eps = static_cast<float>(hp.eps);
  k.inv_s = 1.0f / st.scale;
  return k;
}

template <int GT>
__device__ __forceinline__ float grad_at(const void* g, int64_t i) {
  if constexpr (GT == AMP_F32) return static_cast<const float*>(g)[i];
  else if constexpr (GT == AMP_BF16) return bf16_to_f32(static_cast<const uint16_t*>(g)[i]);
  else return f16_to_f32(static_cast<const uint16_t*>(g)[i]);
}

template <int WT>
__device__ __forceinline__ uint32_t w16_code(float t) {
  if constexpr (WT == AMP_BF16) return f32_to_bf16(t);
  else return f32_to_f16(t);
}

template <bool MULT>
__device__ __forceinline__ void adam_elem(const StepScalars& k, float g16, float& th, float& m,
                                          float& v) {
  float g = g16 * k.inv_s;
  if constexpr (MULT) g = g * k.mult;
  m = k.b1 * m + k.c1 * g;
  v = k.b2 * v + k.c2 * (g * g);
  const float d = sqrtf(v) * k.rbc2 + k.eps;
  th = th * k.decay - k.step * (m / d);
}

// Vector path, in units of four parameters (a quad: 16 bytes of each FP32
// array, 8 bytes of 16-bit gradient or copy).  Work-group b owns the
// contiguous quads [b * kApplyQuads, (b + 1) * kApplyQuads); thread t takes
// quads t, t + 256, t + 512 and t + 768 of that range, all four loaded before
// the first store, so every load and store instruction of a wave covers one
// contiguous span (1 KiB of a state array).  The once-read gradients and the
// write-only 16-bit copy use non-temporal accesses, the state plain ones.
// Measured on MI355X for the same 28 B/param stream: 4.91 TB/s for a
// grid-stride loop over 8-parameter vectors, 5.22 with 4096-parameter ranges
// of 8-parameter vectors (each store instruction then covers every other
// 16 bytes of its span, and HBM writes ran 6 % above the algorithmic bytes).
constexpr int64_t kApplyQuads = 1024;
constexpr int kApplyUnroll = 4;

template <int GT>
__device__ __forceinline__ void load_g4(const void* __restrict__ g_p, int64_t q, float (&gg)[4]) {
  if constexpr (GT == AMP_F32) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g_p) + q);
    gg[0] = a.x; gg[1] = a.y; gg[2] = a.z; gg[3] = a.w;
  } else {
    const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(g_p) + q);
    const uint32_t ww[2] = {w.x, w.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if constexpr (GT == AMP_BF16) {
        gg[2 * h] = bitsf(ww[h] << 16);
        gg[2 * h + 1] = bitsf(ww[h] & 0xffff0000u);
      } else {
        gg[2 * h] = f16_to_f32(ww[h] & 0xffffu);
        gg[2 * h + 1] = f16_to_f32(ww[h] >> 16);
      }
    }
  }
}

__device__ __forceinline__ void load_f4(const float* __restrict__ p, int64_t q, float (&x)[4]) {
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[q];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}

__device__ __forceinline__ void store_f4(float* __restrict__ p, int64_t q, const float (&x)[4]) {
  reinterpret_cast<f32x4*>(p)[q] = f32x4{x[0], x[1], x[2], x[3]};
}

template <int GT, int WT, bool HAS_W, bool MULT>
__global__ __launch_bounds__(kThreads) void apply_kernel(float* __restrict__ th_p,
                                                         float* __restrict__ m_p,
                                                         float* __restrict__ v_p,
                                                         const void* __restrict__ g_p,
                                                         void* __restrict__ w_p, int64_t n,
                                                         amp_adamw_hparams hp,
                                                         const amp_scaler_state* __restrict__ st_p,
                                                         const float* __restrict__ mult_p) {
  const amp_scaler_state st = *st_p;
  if (st.found_inf) return;
  StepScalars k = make_scalars(st, hp);
  if constexpr (MULT) k.mult = *mult_p;
  const int64_t nq = n / 4;
  const int64_t q0 = static_cast<int64_t>(blockIdx.x) * kApplyQuads;
  const int64_t q1 = q0 + kApplyQuads < nq ? q0 + kApplyQuads : nq;
  auto update = [&](int64_t q, float (&gg)[4], float (&th)[4], float (&mm)[4], float (&vv)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) adam_elem<MULT>(k, gg[e], th[e], mm[e], vv[e]);
    store_f4(th_p, q, th);
    store_f4(m_p, q, mm);
    store_f4(v_p, q, vv);
    if constexpr (HAS_W) {
      const u32x2 w = {w16_code<WT>(th[0]) | (w16_code<WT>(th[1]) << 16),
                       w16_code<WT>(th[2]) | (w16_code<WT>(th[3]) << 16)};
      __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(w_p) + q);
    }
  };
  int64_t q = q0 + threadIdx.x;
  for (; q + (kApplyUnroll - 1) * kThreads < q1; q += kApplyUnroll * kThreads) {
    float gg[kApplyUnroll][4], th[kApplyUnroll][4], mm[kApplyUnroll][4], vv[kApplyUnroll][4];
#pragma unroll
    for (int u = 0; u < kApplyUnroll; ++u) {
      load_g4<GT>(g_p, q + u * kThreads, gg[u]);
      load_f4(th_p, q + u * kThreads, th[u]);
      load_f4(m_p, q + u * kThreads, mm[u]);
      load_f4(v_p, q + u * kThreads, vv[u]);
    }
#pragma unroll
    for (int u = 0; u < kApplyUnroll; ++u) update(q + u * kThreads, gg[u], th[u], mm[u], vv[u]);
  }
  for (; q < q1; q += kThreads) {
    float gg[4], th[4], mm[4], vv[4];
    load_g4<GT>(g_p, q, gg);
    load_f4(th_p, q, th);
    load_f4(m_p, q, mm);
    load_f4(v_p, q, vv);
    update(q, gg, th, mm, vv);
  }
  // the elements past the last whole quad belong to the last work-group
  if (blockIdx.x + 1 == gridDim.x) {
    for (int64_t i = nq * 4 + threadIdx.x; i < n; i += kThreads) {
      float th = th_p[i], m = m_p[i], v = v_p[i];
      adam_elem<MULT>(k, grad_at<GT>(g_p, i), th, m, v);
      th_p[i] = th; m_p[i] = m; v_p[i] = v;
      if constexpr (HAS_W) static_cast<uint16_t*>(w_p)[i] = static_cast<uint16_t>(w16_code<WT>(th));
    }
  }
}

// Scalar path for buffers that are not 16-byte aligned.
template <int GT, int WT, bool HAS_W, bool MULT>
__global__ __launch_bounds__(kThreads) void apply_kernel_scalar(float* __restrict__ th_p,
                                                                float* __restrict__ m_p,
                                                                float* __restrict__ v_p,
                                                                const void* __restrict__ g_p,
                                                                void* __restrict__ w_p, int64_t n,
                                                                amp_adamw_hparams hp,
                                                                const amp_scaler_state* __restrict__ st_p,
                                                                const float* __restrict__ mult_p) {
  const amp_scaler_state st = *st_p;
  if (st.found_inf) return;
  StepScalars k = make_scalars(st, hp);
  if constexpr (MULT) k.mult = *mult_p;
  const int64_t nthr = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n; i += nthr) {
    float th = th_p[i], m = m_p[i], v = v_p[i];
    adam_elem<MULT>(k, grad_at<GT>(g_p, i), th, m, v);
    th_p[i] = th; m_p[i] = m; v_p[i] = v;
    if constexpr (HAS_W) static_cast<uint16_t*>(w_p)[i] = static_cast<uint16_t>(w16_code<WT>(th));
  }
}

__global__ void commit_kernel(amp_scaler_state* st, amp_adamw_hparams hp) {
  if (threadIdx.x == 0 && !st->found_inf) {
    st->adam_step += 1;
    st->beta1_pow *= hp.beta1;
    st->beta2_pow *= hp.beta2;
  }
}

// --------------------------------------------------------------- scaler ---
__global__ void scaler_init_kernel(amp_scaler_state* st, float init_scale) {
  if (threadIdx.x == 0) {
    st->scale = init_scale;
    st->growth_tracker = 0;
    st->found_inf = 0;
    st->pad_ = 0;
    st->adam_step = 0;
    st->beta1_pow = 1.0;
    st->beta2_pow = 1.0;
  }
}

__global__ void scaler_update_kernel(amp_scaler_state* st, amp_scaler_params p) {
  if (threadIdx.x != 0) return;
  if (st->found_inf) {
    st->scale = st->scale * p.backoff_factor;
    st->growth_tracker = 0;
  } else {
    const int32_t t = st->growth_tracker + 1;
    if (t == p.growth_interval) {
      st->scale = st->scale * p.growth_factor;
      st->growth_tracker = 0;
    } else {
      st->growth_tracker = t;
    }
  }
  st->found_inf = 0;
}

// --------------------------------------------------------- FP8 recipe ---
__global__ __launch_bounds__(kThreads) void meta_init_kernel(amp_fp8_meta* metas, float* hist,
                                                             int32_t len) {
  const int i = blockIdx.x;
  for (int j = threadIdx.x; j < len; j += kThreads) hist[static_cast<int64_t>(i) * len + j] = 0.0f;
  if (threadIdx.x == 0) {
    metas[i].amax_cur = 0.0f;
    metas[i].scale = 1.0f;
    metas[i].scale_inv = 1.0f;
    metas[i].pos = 0;
  }
}

__global__ __launch_bounds__(kThreads) void delayed_update_kernel(amp_fp8_meta* metas, float* hist,
                                                                  amp_delayed_recipe r) {
  __shared__ uint32_t red[kThreads / kWave];
  const int i = blockIdx.x;
  amp_fp8_meta* mt = metas + i;
  float* h = hist + static_cast<int64_t>(i) * r.history_len;
  const int32_t pos = mt->pos;
  const uint32_t cur = fbits(mt->amax_cur);
  uint32_t mx = 0;
  if (r.algo == AMP_AMAX_MOST_RECENT) {
    mx = cur;
  } else {
    for (int j = threadIdx.x; j < r.history_len; j += kThreads) {
      const uint32_t b = j == pos ? cur : fbits(h[j]);
      mx = mx > b ? mx : b;
    }
    mx = block_max_u32<kThreads>(mx, red);
  }
  __syncthreads();   // every thread has read h[] before thread 0 rewrites it
  if (threadIdx.x == 0) {
    h[pos] = bitsf(cur);
    const float amax = bitsf(mx);
    if (mx < 0x7f800000u && mx != 0u) {
      const float denom = r.margin * amax;
      const float scale = r.fp8_max / denom;
      mt->scale = scale;
      mt->scale_inv = 1.0f / scale;
    }
    mt->pos = pos + 1 == r.history_len ? 0 : pos + 1;
    mt->amax_cur = 0.0f;
  }
}


// ------------------------------------------- accumulation, norm, clip ---
// Page "혼합 정밀도 학습" (itwiki), section "FP16 학습 루프" (clip the global
// norm after unscaling) and section "함께 쓰는 기법과 주의점" (with gradient
// accumulation, scale changes and the inf check once per effective batch).

template <int GT>
__device__ __forceinline__ void widen8(const void* g, int64_t j, float (&x)[8]) {
  // gradients are read once: non-temporal loads (as in the overflow sweep)
  if constexpr (GT == AMP_F32) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g) + 2 * j);
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g) + 2 * j + 1);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(g) + j);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (GT == AMP_BF16) {
        x[2 * q] = bitsf(ww[q] << 16);
        x[2 * q + 1] = bitsf(ww[q] & 0xffff0000u);
      } else {
        x[2 * q] = f16_to_f32(ww[q] & 0xffffu);
        x[2 * q + 1] = f16_to_f32(ww[q] >> 16);
      }
    }
  }
}

// Four consecutive gradients from element e (8- or 16-byte aligned), widened.
template <int GT>
__device__ __forceinline__ void widen4(const void* g, int64_t e, float* x) {
  if constexpr (GT == AMP_F32) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(static_cast<const float*>(g) + e));
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  } else {
    const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(g) + e));
    const uint32_t ww[2] = {w.x, w.y};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if constexpr (GT == AMP_BF16) {
        x[2 * q] = bitsf(ww[q] << 16);
        x[2 * q + 1] = bitsf(ww[q] & 0xffff0000u);
      } else {
        x[2 * q] = f16_to_f32(ww[q] & 0xffffu);
        x[2 * q + 1] = f16_to_f32(ww[q] >> 16);
      }
    }
  }
}

// acc = first ? f32(g) : fl32(acc + f32(g)).  Vector path (every buffer
// 16-byte aligned): work-group b owns the contiguous 8-element vectors
// [b * kAccChunk, (b + 1) * kAccChunk), each thread with two vectors' loads
// in flight before its stores, all accesses non-temporal (the accumulator is
// next touched by the following micro-batch's pass); the last work-group also
// does the n % 8 trailing elements (5.35 TB/s for 2^30 FP16 gradients, against
// 5.24 for a grid-stride loop and 4.87 with 16384-vector ranges).  In the
// unrolled steps a wave's 8 vectors are its 512 consecutive elements, lane l
// taking elements 4l .. 4l+3 and 256+4l .. 256+4l+3, so that every load and
// store instruction covers one contiguous span (with 8 consecutive elements
// per lane, each of a lane's two 16-byte accumulator accesses covered every
// other 16 bytes of a 2 KiB span, and the counters showed 9 % more bytes
// written than the accumulator holds).  Scalar path: a grid-stride loop.
constexpr int64_t kAccChunk = 512;
constexpr int kAccUnroll = 2;

template <int GT, bool VEC>
__global__ __launch_bounds__(kThreads) void accumulate_kernel(float* __restrict__ acc,
                                                              const void* __restrict__ g,
                                                              int64_t n, int first) {
  if constexpr (VEC) {
    const int64_t nv = n / 8;
    f32x4* a4 = reinterpret_cast<f32x4*>(acc);
    const int64_t b0 = static_cast<int64_t>(blockIdx.x) * kAccChunk;
    const int64_t b1 = b0 + kAccChunk < nv ? b0 + kAccChunk : nv;
    auto load = [&](int64_t j, float (&x)[8], f32x4& p, f32x4& q) __attribute__((always_inline)) {
      widen8<GT>(g, j, x);
      if (!first) {
        p = __builtin_nontemporal_load(a4 + 2 * j);
        q = __builtin_nontemporal_load(a4 + 2 * j + 1);
      }
    };
    auto store = [&](int64_t j, const float (&x)[8], f32x4 p, f32x4 q) __attribute__((always_inline)) {
      f32x4 lo = f32x4{x[0], x[1], x[2], x[3]}, hi = f32x4{x[4], x[5], x[6], x[7]};
      if (!first) {
        lo = f32x4{p.x + lo.x, p.y + lo.y, p.z + lo.z, p.w + lo.w};
        hi = f32x4{q.x + hi.x, q.y + hi.y, q.z + hi.z, q.w + hi.w};
      }
      __builtin_nontemporal_store(lo, a4 + 2 * j);
      __builtin_nontemporal_store(hi, a4 + 2 * j + 1);
    };
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    int64_t jb = b0;   // the block's first vector of the step
    for (; jb + kAccUnroll * kThreads <= b1; jb += kAccUnroll * kThreads) {
      float x[kAccUnroll][8];
      f32x4 p[kAccUnroll] = {}, q[kAccUnroll] = {};
#pragma unroll
      for (int u = 0; u < kAccUnroll; ++u) {
        const int64_t e = (jb + u * kThreads) * 8 + 512 * wv + 4 * lane;
        widen4<GT>(g, e, x[u]);
        widen4<GT>(g, e + 256, x[u] + 4);
        if (!first) {
          p[u] = __builtin_nontemporal_load(a4 + e / 4);
          q[u] = __builtin_nontemporal_load(a4 + (e + 256) / 4);
        }
      }
#pragma unroll
      for (int u = 0; u < kAccUnroll; ++u) {
        const int64_t e = (jb + u * kThreads) * 8 + 512 * wv + 4 * lane;
        f32x4 lo = f32x4{x[u][0], x[u][1], x[u][2], x[u][3]}, hi = f32x4{x[u][4], x[u][5], x[u][6], x[u][7]};
        if (!first) {
          lo = f32x4{p[u].x + lo.x, p[u].y + lo.y, p[u].z + lo.z, p[u].w + lo.w};
          hi = f32x4{q[u].x + hi.x, q[u].y + hi.y, q[u].z + hi.z, q[u].w + hi.w};
        }
        __builtin_nontemporal_store(lo, a4 + e / 4);
        __builtin_nontemporal_store(hi, a4 + (e + 256) / 4);
      }
    }
    for (int64_t j = jb + threadIdx.x; j < b1; j += kThreads) {
      float x[8];
      f32x4 p = {}, q = {};
      load(j, x, p, q);
      store(j, x, p, q);
    }
    if (blockIdx.x == gridDim.x - 1)
      for (int64_t i = nv * 8 + threadIdx.x; i < n; i += kThreads) {
        const float x = grad_at<GT>(g, i);
        acc[i] = first ? x : acc[i] + x;
      }
  } else {
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t nthr = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t i = tid; i < n; i += nthr) {
      const float x = grad_at<GT>(g, i);
      acc[i] = first ? x : acc[i] + x;
    }
  }
}

constexpr int kNormThreads = 512;

// Fixed-order float64 block sum (wave xor-tree, then waves in order).
template <int NT>
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  if (lane == 0) red[wid] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0)
    for (int w = 0; w < NT / kWave; ++w) t += red[w];
  return t;
}

// Sum of squares of the finite gradients (float64; a float32 square is exact
// in float64), one partial per work-group; non-finite elements set found_inf.
// Vector path: work-group b sums the contiguous 8-element vectors
// [b * chunk, (b + 1) * chunk) with four 16-byte loads in flight per thread
// (a grid-stride loop over the same grid ran 11 % slower), and the last
// work-group adds the n % 8 trailing elements.  Scalar path: grid-stride.
template <int GT, bool VEC>
__global__ __launch_bounds__(kNormThreads) void norm_kernel(const void* __restrict__ g, int64_t n,
                                                            int64_t chunk,
                                                            amp_scaler_state* __restrict__ st,
                                                            double* __restrict__ partial) {
  __shared__ double red[kNormThreads / kWave];
  __shared__ uint32_t bad_any;
  if (threadIdx.x == 0) bad_any = 0;
  double accs[4] = {0.0, 0.0, 0.0, 0.0};   // independent chains, summed in a fixed order
  uint32_t bad = 0;
  auto add = [&](float x, int c) {
    const uint32_t fin = static_cast<uint32_t>((fbits(x) & 0x7f800000u) != 0x7f800000u);
    bad |= fin ^ 1u;
    const double d = fin ? static_cast<double>(x) : 0.0;
    accs[c] = __builtin_fma(d, d, accs[c]);
  };
  if constexpr (VEC) {
    const int64_t nv = n / 8;
    const int64_t b0 = static_cast<int64_t>(blockIdx.x) * chunk;
    const int64_t b1 = b0 + chunk < nv ? b0 + chunk : nv;
    // FP32 input: a wave's 8 vectors of a step are its 512 consecutive
    // elements, lane l taking 4l .. 4l+3 and 256+4l .. 256+4l+3 (one
    // contiguous span per load instruction, as in the accumulation pass)
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    int64_t jb = b0;   // the block's first vector of the step
    for (; jb + 4 * kNormThreads <= b1; jb += 4 * kNormThreads) {
      float x[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if constexpr (GT == AMP_F32) {
          const int64_t e = (jb + u * kNormThreads) * 8 + 512 * wv + 4 * lane;
          widen4<GT>(g, e, x[u]);
          widen4<GT>(g, e + 256, x[u] + 4);
        } else {
          widen8<GT>(g, jb + u * kNormThreads + threadIdx.x, x[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) add(x[u][q], q & 3);
    }
    for (int64_t j = jb + threadIdx.x; j < b1; j += kNormThreads) {
      float x[8];
      widen8<GT>(g, j, x);
#pragma unroll
      for (int q = 0; q < 8; ++q) add(x[q], q & 3);
    }
    if (blockIdx.x == gridDim.x - 1)
      for (int64_t i = nv * 8 + threadIdx.x; i < n; i += kNormThreads) add(grad_at<GT>(g, i), 0);
  } else {
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * kNormThreads + threadIdx.x;
    const int64_t nthr = static_cast<int64_t>(gridDim.x) * kNormThreads;
    for (int64_t i = tid; i < n; i += nthr) add(grad_at<GT>(g, i), 0);
  }
  __syncthreads();
  if (bad) bad_any = 1u;
  const double t = block_sum_f64<kNormThreads>((accs[0] + accs[1]) + (accs[2] + accs[3]), red);
  __syncthreads();
  if (threadIdx.x == 0) {
    partial[blockIdx.x] = t;
    if (bad_any) st->found_inf = 1;
  }
}

// sumsq += (sum of the partials) * (1/S)^2 -- exact scaling by a power of
// two.  One wave: lane l adds partials l, l + 64, ... in order, then a fixed
// xor tree, so the result does not depend on timing.
__global__ __launch_bounds__(kWave) void norm_finalize(const double* __restrict__ partial,
                                                       double* __restrict__ sumsq, int nb,
                                                       const amp_scaler_state* st) {
  double t = 0.0;
  for (int b = threadIdx.x; b < nb; b += kWave) t += partial[b];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off, kWave);
  if (threadIdx.x == 0) {
    const double inv = static_cast<double>(1.0f / st->scale);
    *sumsq += t * inv * inv;
  }
}

__global__ void norm_init_kernel(amp_grad_norm_state* ns) {
  if (threadIdx.x == 0) ns->sumsq = 0.0;
}

__global__ void clip_kernel(const amp_grad_norm_state* ns, float max_norm,
                            const amp_scaler_state* st, float* out) {
  if (threadIdx.x != 0) return;
  if (st->found_inf) {
    out[0] = 1.0f;
    out[1] = __builtin_inff();
    return;
  }
  const float norm = static_cast<float>(__builtin_sqrt(ns->sumsq));
  const float c = max_norm / (norm + 1e-6f);
  out[0] = c < 1.0f ? c : 1.0f;
  out[1] = norm;
}

// Grid-stride launches: up to 64 blocks per CU keeps enough 16-byte requests
// in flight to saturate HBM (measured).
int64_t grid_for(int64_t work_items) {
  int64_t b = (work_items + kThreads - 1) / kThreads;
  if (b > 256 * 64) b = 256 * 64;
  return b < 1 ? 1 : b;
}

// One work-group per kApplyQuads quads (at least one, for the tail).
int64_t apply_blocks(int64_t n) {
  const int64_t b = (n / 4 + kApplyQuads - 1) / kApplyQuads;
  return b < 1 ? 1 : b;
}

template <int GT, int WT, bool HAS_W, bool MULT>
hipError_t launch_apply_t(float* th, float* m, float* v, const void* g, void* w, int64_t n,
                          const amp_adamw_hparams& hp, amp_scaler_state* st, const float* mult,
                          hipStream_t s) {
  const bool vec = aligned(th, 16) && aligned(m, 16) && aligned(v, 16) && aligned(g, 16) &&
                   (!HAS_W || aligned(w, 16));
  if (vec)
    apply_kernel<GT, WT, HAS_W, MULT><<<dim3(static_cast<unsigned>(apply_blocks(n))), kThreads, 0, s>>>(
        th, m, v, g, w, n, hp, st, mult);
  else
    apply_kernel_scalar<GT, WT, HAS_W, MULT><<<dim3(static_cast<unsigned>(grid_for(n))), kThreads, 0, s>>>(
        th, m, v, g, w, n, hp, st, mult);
  return hipGetLastError();
}

template <int GT, bool MULT>
hipError_t launch_apply_m(float* th, float* m, float* v, const void* g, void* w, int wt, int64_t n,
                          const amp_adamw_hparams& hp, amp_scaler_state* st, const float* mult,
                          hipStream_t s) {
  if (w == nullptr) return launch_apply_t<GT, AMP_F16, false, MULT>(th, m, v, g, w, n, hp, st, mult, s);
  if (wt == AMP_BF16) return launch_apply_t<GT, AMP_BF16, true, MULT>(th, m, v, g, w, n, hp, st, mult, s);
  return launch_apply_t<GT, AMP_F16, true, MULT>(th, m, v, g, w, n, hp, st, mult, s);
}

template <int GT>
hipError_t launch_apply_g(float* th, float* m, float* v, const void* g, void* w, int wt, int64_t n,
                          const amp_adamw_hparams& hp, amp_scaler_state* st, const float* mult,
                          hipStream_t s) {
  if (mult) return launch_apply_m<GT, true>(th, m, v, g, w, wt, n, hp, st, mult, s);
  return launch_apply_m<GT, false>(th, m, v, g, w, wt, n, hp, st, mult, s);
}

// Overflow flag from the amax values a producing cast recorded: one thread
// per value.  Rounding is monotone in |t|, so the largest magnitude decides
// whether any output of that cast is non-finite.
template <int YT>
__global__ void flag_from_amax_kernel(const float* __restrict__ amax, int32_t n,
                                      const float* __restrict__ d_scale,
                                      amp_scaler_state* __restrict__ st) {
  const int i = static_cast<int>(blockIdx.x) * 64 + static_cast<int>(threadIdx.x);
  if (i >= n) return;
  const uint32_t b = fbits(amax[i]) & 0x7fffffffu;
  bool bad = b >= 0x7f800000u;                    // an inf or NaN input
  if constexpr (YT == AMP_F16 || YT == AMP_BF16) {
    if (!bad) {
      const float t = d_scale ? bitsf(b) * *d_scale : bitsf(b);
      if constexpr (YT == AMP_F16) bad = (f32_to_f16(t) & 0x7c00u) == 0x7c00u;
      else bad = (f32_to_bf16(t) & 0x7f80u) == 0x7f80u;
    }
  }
  if (bad) st->found_inf = 1;
}

}  // namespace

hipError_t launch_found_inf_from_amax(const float* amax, int32_t n, int yt, const float* d_scale,
                                      amp_scaler_state* st, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((n + 63) / 64));
  switch (yt) {
    case AMP_F16: flag_from_amax_kernel<AMP_F16><<<grid, 64, 0, s>>>(amax, n, d_scale, st); break;
    case AMP_BF16: flag_from_amax_kernel<AMP_BF16><<<grid, 64, 0, s>>>(amax, n, d_scale, st); break;
    default: flag_from_amax_kernel<AMP_E4M3><<<grid, 64, 0, s>>>(amax, n, d_scale, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_check_overflow(const void* g, int gt, int64_t n, amp_scaler_state* st,
                                 hipStream_t s) {
  // the vector loop reads 16-byte words; an unaligned buffer uses the element loop
  const bool vec = aligned(g, 16);
  const int64_t nvec = n * dtype_bytes(gt) / 16;
  const int64_t blocks = grid_for(vec ? (n * dtype_bytes(gt) + 15) / 16 : n);
  const int64_t chunk = (nvec + blocks - 1) / blocks;      // 16-byte words per work-group
  const dim3 grid(static_cast<unsigned>(blocks));
#define AMP_CHECK(T)                                                              \
  if (vec) check_kernel<T, true><<<grid, kThreads, 0, s>>>(g, n, chunk, st);      \
  else check_kernel<T, false><<<grid, kThreads, 0, s>>>(g, n, 0, st);
  switch (gt) {
    case AMP_F32: AMP_CHECK(AMP_F32) break;
    case AMP_BF16: AMP_CHECK(AMP_BF16) break;
    default: AMP_CHECK(AMP_F16) break;
  }
#undef AMP_CHECK
  return hipGetLastError();
}

hipError_t launch_optimizer_apply(float* th, float* m, float* v, const void* g, int gt, void* w,
                                  int wt, int64_t n, const amp_adamw_hparams& hp,
                                  amp_scaler_state* st, const float* mult, hipStream_t s) {
  switch (gt) {
    case AMP_F32: return launch_apply_g<AMP_F32>(th, m, v, g, w, wt, n, hp, st, mult, s);
    case AMP_BF16: return launch_apply_g<AMP_BF16>(th, m, v, g, w, wt, n, hp, st, mult, s);
    default: return launch_apply_g<AMP_F16>(th, m, v, g, w, wt, n, hp, st, mult, s);
  }
}

hipError_t launch_grad_accumulate(float* acc, const void* g, int gt, int64_t n, int first,
                                  hipStream_t s) {
  const bool vec = aligned(acc, 16) && aligned(g, 16);
  int64_t blocks = vec ? (n / 8 + kAccChunk - 1) / kAccChunk : grid_for(n);
  if (blocks < 1) blocks = 1;
  const dim3 grid(static_cast<unsigned>(blocks));
#define AMP_ACC(T)                                                                      \
  if (vec) accumulate_kernel<T, true><<<grid, kThreads, 0, s>>>(acc, g, n, first);      \
  else accumulate_kernel<T, false><<<grid, kThreads, 0, s>>>(acc, g, n, first);
  switch (gt) {
    case AMP_F32: AMP_ACC(AMP_F32) break;
    case AMP_BF16: AMP_ACC(AMP_BF16) break;
    default: AMP_ACC(AMP_F16) break;
  }
#undef AMP_ACC
  return hipGetLastError();
}

hipError_t launch_grad_norm_init(amp_grad_norm_state* ns, hipStream_t s) {
  norm_init_kernel<<<1, 64, 0, s>>>(ns);
  return hipGetLastError();
}

namespace {

// Work-groups of one norm pass: one float64 partial each, at most
// AMP_NORM_PARTIALS whatever n is (each then sums a longer range).
int64_t norm_blocks(int64_t n) {
  int64_t nb = (n + 8 * kNormThreads - 1) / (8 * kNormThreads);
  if (nb > AMP_NORM_PARTIALS) nb = AMP_NORM_PARTIALS;
  return nb < 1 ? 1 : nb;
}

hipError_t launch_norm_pass(const void* g, int gt, int64_t n, amp_scaler_state* st,
                            double* partial, double* sumsq, int64_t nb, hipStream_t s) {
  const bool vec = aligned(g, 16);
  const dim3 grid(static_cast<unsigned>(nb));
  const int64_t chunk = (n / 8 + nb - 1) / nb;     // vectors per work-group (vector path)
#define AMP_NORM(T)                                                                          \
  if (vec) norm_kernel<T, true><<<grid, kNormThreads, 0, s>>>(g, n, chunk, st, partial);      \
  else norm_kernel<T, false><<<grid, kNormThreads, 0, s>>>(g, n, 0, st, partial);
  switch (gt) {
    case AMP_F32: AMP_NORM(AMP_F32) break;
    case AMP_BF16: AMP_NORM(AMP_BF16) break;
    default: AMP_NORM(AMP_F16) break;
  }
#undef AMP_NORM
  norm_finalize<<<1, kWave, 0, s>>>(partial, sumsq, static_cast<int>(nb), st);
  return hipGetLastError();
}

}  // namespace

// Scratch of the no-allocation norm entry point: the per-work-group float64
// partials that amp_grad_norm_accumulate keeps in the caller's state struct.
// One copy per GPU, held until the process ends (8 KiB); every pass writes the
// slots it reads, so nothing needs clearing between calls.
constexpr int kNormScratchPartials = AMP_NORM_PARTIALS;   // 1024 float64 = 8 KiB
constexpr int kMaxScratchDevices = 64;
static __device__ __align__(256) double scratch[kNormScratchPartials];

namespace {

// Device address of `scratch` on the current GPU, looked up once per device
// with that device current (the array's name is only a host-side stand-in).
hipError_t scratch_on_current_device(double** out) {
  static std::mutex mu;
  static double* ptr[kMaxScratchDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = static_cast<double*>(p);
  }
  *out = ptr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_grad_norm(const void* g, int gt, int64_t n, amp_scaler_state* st,
                            amp_grad_norm_state* ns, hipStream_t s) {
  return launch_norm_pass(g, gt, n, st, ns->partial, &ns->sumsq, norm_blocks(n), s);
}

hipError_t launch_grad_norm_noalloc(const void* g, int gt, int64_t n, amp_scaler_state* st,
                                    double* sumsq, hipStream_t s) {
  const int64_t nb = norm_blocks(n);
  if (nb > kNormScratchPartials) return hipErrorInvalidValue;   // never: the grid is capped
  double* partial = nullptr;
  if (hipError_t e = scratch_on_current_device(&partial)) return e;
  return launch_norm_pass(g, gt, n, st, partial, sumsq, nb, s);
}

hipError_t launch_clip_coefficient(const amp_grad_norm_state* ns, float max_norm,
                                   const amp_scaler_state* st, float* out, hipStream_t s) {
  clip_kernel<<<1, 64, 0, s>>>(ns, max_norm, st, out);
  return hipGetLastError();
}

hipError_t launch_optimizer_commit(amp_scaler_state* st, const amp_adamw_hparams& hp,
                                   hipStream_t s) {
  commit_kernel<<<1, 64, 0, s>>>(st, hp);
  return hipGetLastError();
}

hipError_t launch_scaler_init(amp_scaler_state* st, float init_scale, hipStream_t s) {
  scaler_init_kernel<<<1, 64, 0, s>>>(st, init_scale);
  return hipGetLastError();
}

hipError_t launch_scaler_update(amp_scaler_state* st, const amp_scaler_params& p, hipStream_t s) {
  scaler_update_kernel<<<1, 64, 0, s>>>(st, p);
  return hipGetLastError();
}

hipError_t launch_meta_init(amp_fp8_meta* metas, float* hist, int32_t n, int32_t len,
                            hipStream_t s) {
  meta_init_kernel<<<dim3(static_cast<unsigned>(n)), kThreads, 0, s>>>(metas, hist, len);
  return hipGetLastError();
}

hipError_t launch_delayed_update(amp_fp8_meta* metas, float* hist, int32_t n,
                                 const amp_delayed_recipe& r, hipStream_t s) {
  delayed_update_kernel<<<dim3(static_cast<unsigned>(n)), kThreads, 0, s>>>(metas, hist, r);
  return hipGetLastError();
}

}  // namespace amp
