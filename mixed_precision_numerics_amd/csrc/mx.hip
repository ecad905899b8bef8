// MX (microscaling) block quantizer (gfx950): 32 elements along K share one
// power-of-two scale stored as a UE8M0 byte.
//
// Page "혼합 정밀도 학습" (itwiki), section "FP8 혼합 정밀도" (MXFP8 / MXFP6 /
// MXFP4: one power-of-two scale per 32 elements) and page "Pretraining Large
// Language Models with NVFP4", section 2.1 (MXFP4 uses 32-element blocks with
// UE8M0 scales).  Per block of the operand op = x or x^T ([R, K], K along the
// blocks):
//   e  = floor(log2(amax)) - emax   (emax 8 for E4M3, 15 for E5M2, 2 for E2M1)
//   sc = clamp(e, -127, 127) + 127;  0 for an all-zero block, 0xFF if the
//        block holds inf or NaN (then the elements are encoded unscaled)
//   q  = element format of x * 2^-(sc - 127), nearest-even, saturating.
// E2M1 codes are packed two per byte, the lower K index in the low nibble.
//
// One thread per (op row, block).  Plain operand: a thread reads its block's
// 32 contiguous elements with 16-byte loads (neighbouring threads take the
// next block).  Transposed operand: neighbouring threads take neighbouring op
// rows (x columns), so each of the 32 element loads is contiguous across the
// wave.
#include "common.hpp"
#include "formats.hpp"

namespace amp {
namespace {

constexpr int kMxThreads = 256;

template <int XT>
__device__ __forceinline__ float ld_elem(const void* x, int64_t i) {
  if constexpr (XT == AMP_F32) return static_cast<const float*>(x)[i];
  else if constexpr (XT == AMP_BF16) return bf16_to_f32(static_cast<const uint16_t*>(x)[i]);
  else return f16_to_f32(static_cast<const uint16_t*>(x)[i]);
}

template <int XT>
__device__ __forceinline__ void ld8(const void* x, int64_t i, float (&v)[8]) {
  if constexpr (XT == AMP_F32) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + i);
    const f32x4 b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + i);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (XT == AMP_BF16) {
        v[2 * q] = bitsf(ww[q] << 16);
        v[2 * q + 1] = bitsf(ww[q] & 0xffff0000u);
      } else {
        v[2 * q] = f16_to_f32(ww[q] & 0xffffu);
        v[2 * q + 1] = f16_to_f32(ww[q] >> 16);
      }
    }
  }
}

template <int YT> struct MxElem;
template <> struct MxElem<AMP_E4M3> { static constexpr int kEmax = 8; };
template <> struct MxElem<AMP_E5M2> { static constexpr int kEmax = 15; };
template <> struct MxElem<AMP_E2M1X2> { static constexpr int kEmax = 2; };

template <int YT>
__device__ __forceinline__ uint32_t elem_code(float t) {
  if constexpr (YT == AMP_E4M3) return f32_to_e4m3(t);
  else if constexpr (YT == AMP_E5M2) return f32_to_e5m2(t);
  else return e2m1_rne(t);
}

// UE8M0 block scale code from the block's |x| bit-max.
template <int YT>
__device__ __forceinline__ uint32_t scale_code(uint32_t amax_bits) {
  if (amax_bits >= 0x7f800000u) return 0xffu;
  if (amax_bits == 0u) return 0u;
  const int ef = static_cast<int>(amax_bits >> 23);
  const int fl = ef > 0 ? ef - 127 : (31 - __builtin_clz(amax_bits)) - 149;   // floor(log2)
  int e = fl - MxElem<YT>::kEmax;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  return static_cast<uint32_t>(e + 127);
}

template <int XT, int YT, bool TRANS, bool VEC>
__global__ __launch_bounds__(kMxThreads) void mx_quantize_kernel(
    const void* __restrict__ x, int64_t ldx, int64_t R, int64_t K, uint8_t* __restrict__ q,
    uint8_t* __restrict__ scales) {
  const int64_t nb = K / 32;
  const int64_t id = static_cast<int64_t>(blockIdx.x) * kMxThreads + threadIdx.x;
  if (id >= R * nb) return;
  // plain: neighbouring threads take neighbouring blocks of one row;
  // transposed: neighbouring threads take neighbouring rows of one block
  const int64_t r = TRANS ? id % R : id / nb;
  const int64_t b = TRANS ? id / R : id % nb;
  float v[32];
  if constexpr (TRANS) {
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = ld_elem<XT>(x, (32 * b + j) * ldx + r);
  } else if constexpr (VEC) {
#pragma unroll
    for (int j = 0; j < 32; j += 8) {
      float w[8];
      ld8<XT>(x, r * ldx + 32 * b + j, w);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[j + k] = w[k];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = ld_elem<XT>(x, r * ldx + 32 * b + j);
  }
  uint32_t am = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint32_t a = fbits(v[j]) & 0x7fffffffu;
    am = am > a ? am : a;
  }
  const uint32_t sc = scale_code<YT>(am);
  // x * 2^(127 - sc) exactly (two power-of-two factors keep every step in range)
  const int sh = 127 - static_cast<int>(sc);
  const float f1 = bitsf(static_cast<uint32_t>(127 + (sh >> 1)) << 23);
  const float f2 = bitsf(static_cast<uint32_t>(127 + (sh - (sh >> 1))) << 23);
  const bool nan_block = sc == 0xffu;
  uint32_t c[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) c[j] = elem_code<YT>(nan_block ? v[j] : (v[j] * f1) * f2);
  if constexpr (YT == AMP_E2M1X2) {
    u32x4 w;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t word = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) word |= (c[8 * d + k] & 0xfu) << (4 * k);
      w[d] = word;
    }
    *reinterpret_cast<u32x4*>(q + r * (K / 2) + 16 * b) = w;
  } else {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 16 * d + 4 * e;
        w[e] = c[j] | (c[j + 1] << 8) | (c[j + 2] << 16) | (c[j + 3] << 24);
      }
      *reinterpret_cast<u32x4*>(q + r * K + 32 * b + 16 * d) = w;
    }
  }
  scales[r * nb + b] = static_cast<uint8_t>(sc);
}

// Plain operand with contiguous rows (ldx == K): the blocks are consecutive
// runs of 32 elements of one flat stream.  Lane-piece layout: a piece is 16
// bytes of x (kPE = 8 16-bit or 4 FP32 elements) and the kLB = 32 / kPE
// consecutive lanes that hold one block exchange their maxima, so that every
// load and store instruction of a wave covers one contiguous span (one
// thread per block, as above, makes each instruction touch every fourth
// 16-byte piece of its span).  Four pieces per thread are loaded before the
// first is encoded; the source is read once (non-temporal loads).  The block
// maximum crosses the lanes by DPP quad permutes (one exchange through the
// LDS crossbar per step, as a plain shuffle compiles, had made this layout
// 6-10 % slower than one thread per block).
constexpr int kMxUnroll = 4;

template <int XT, int YT>
__global__ __launch_bounds__(kMxThreads) void mx_quantize_flat(const void* __restrict__ x, int64_t np,
                                                               uint8_t* __restrict__ q,
                                                               uint8_t* __restrict__ scales) {
  constexpr int kPE = XT == AMP_F32 ? 4 : 8;
  constexpr int kLB = 32 / kPE;
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * (kMxThreads * kMxUnroll) + threadIdx.x;
  float v[kMxUnroll][kPE];
#pragma unroll
  for (int u = 0; u < kMxUnroll; ++u) {
    const int64_t p = p0 + u * kMxThreads;
    if (p < np) {
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + p);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (XT == AMP_F32) {
          v[u][e] = bitsf(ww[e]);
        } else if constexpr (XT == AMP_BF16) {
          v[u][2 * e] = bitsf(ww[e] << 16);
          v[u][2 * e + 1] = bitsf(ww[e] & 0xffff0000u);
        } else {
          v[u][2 * e] = f16_to_f32(ww[e] & 0xffffu);
          v[u][2 * e + 1] = f16_to_f32(ww[e] >> 16);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kPE; ++j) v[u][j] = 0.0f;
    }
  }
#pragma unroll
  for (int u = 0; u < kMxUnroll; ++u) {
    const int64_t p = p0 + u * kMxThreads;
    uint32_t am = 0;
#pragma unroll
    for (int j = 0; j < kPE; ++j) {
      const uint32_t a = fbits(v[u][j]) & 0x7fffffffu;
      am = am > a ? am : a;
    }
    // the block's lanes are an aligned group of kLB (np and every group
    // start are multiples of kLB, so a group is wholly in or out of range)
    {
      // within the quad by DPP (quad_perm [1,0,3,2], then [2,3,0,1]); FP32's
      // 8-lane groups take one more step across quads
      uint32_t o = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(am), 0xB1, 0xF, 0xF, false));
      am = am > o ? am : o;
      o = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(am), 0x4E, 0xF, 0xF, false));
      am = am > o ? am : o;
      if constexpr (kLB == 8) {
        o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(am), 4, kWave));
        am = am > o ? am : o;
      }
    }
    const uint32_t sc = scale_code<YT>(am);
    const int sh = 127 - static_cast<int>(sc);
    const float f1 = bitsf(static_cast<uint32_t>(127 + (sh >> 1)) << 23);
    const float f2 = bitsf(static_cast<uint32_t>(127 + (sh - (sh >> 1))) << 23);
    const bool nan_block = sc == 0xffu;
    uint32_t c[kPE];
#pragma unroll
    for (int j = 0; j < kPE; ++j) c[j] = elem_code<YT>(nan_block ? v[u][j] : (v[u][j] * f1) * f2);
    if (p < np) {
      if constexpr (YT == AMP_E2M1X2) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < kPE; ++j) word |= (c[j] & 0xfu) << (4 * j);
        if constexpr (kPE == 8) __builtin_nontemporal_store(word, reinterpret_cast<uint32_t*>(q) + p);
        else reinterpret_cast<uint16_t*>(q)[p] = static_cast<uint16_t>(word);
      } else if constexpr (kPE == 8) {
        const u32x2 w = {c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                         c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(q) + p);
      } else {
        __builtin_nontemporal_store(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                                    reinterpret_cast<uint32_t*>(q) + p);
      }
      if ((threadIdx.x & (kLB - 1)) == 0) scales[p / kLB] = static_cast<uint8_t>(sc);
    }
  }
}

template <int XT, int YT>
hipError_t run(const void* x, int64_t ldx, int64_t R, int64_t K, bool trans, uint8_t* q,
               uint8_t* sc, hipStream_t s) {
  const int64_t work = R * (K / 32);
  const dim3 grid(static_cast<unsigned>((work + kMxThreads - 1) / kMxThreads));
  const int64_t eb = XT == AMP_F32 ? 4 : 2;
  const bool vec = aligned(x, 16) && (ldx * eb) % 16 == 0;
  // FP8 codes take the lane-piece layout (FP8 weight 5.63 -> 6.01-6.04 TB/s,
  // activation 4.72 -> 4.83-4.85); E2M1 keeps one thread per block, whose
  // 16-byte code stores are already one contiguous span per instruction (the
  // lane-piece layout's 4-byte stores made the 8192 x 4096 activation 6 %
  // slower while the weight gained 2-7 %)
  const int64_t qb = 16 / eb;   // code bytes one lane stores in the lane-piece layout
  if (YT != AMP_E2M1X2 && !trans && vec && ldx == K && aligned(q, static_cast<size_t>(qb))) {
    const int64_t np = R * K * eb / 16;
    const int64_t per = static_cast<int64_t>(kMxThreads) * kMxUnroll;
    mx_quantize_flat<XT, YT><<<dim3(static_cast<unsigned>((np + per - 1) / per)), kMxThreads, 0, s>>>(
        x, np, q, sc);
    return hipGetLastError();
  }
  if (trans) mx_quantize_kernel<XT, YT, true, false><<<grid, kMxThreads, 0, s>>>(x, ldx, R, K, q, sc);
  else if (vec) mx_quantize_kernel<XT, YT, false, true><<<grid, kMxThreads, 0, s>>>(x, ldx, R, K, q, sc);
  else mx_quantize_kernel<XT, YT, false, false><<<grid, kMxThreads, 0, s>>>(x, ldx, R, K, q, sc);
  return hipGetLastError();
}

template <int XT>
hipError_t run_y(int yt, const void* x, int64_t ldx, int64_t R, int64_t K, bool trans,
                 uint8_t* q, uint8_t* sc, hipStream_t s) {
  if (yt == AMP_E4M3) return run<XT, AMP_E4M3>(x, ldx, R, K, trans, q, sc, s);
  if (yt == AMP_E5M2) return run<XT, AMP_E5M2>(x, ldx, R, K, trans, q, sc, s);
  return run<XT, AMP_E2M1X2>(x, ldx, R, K, trans, q, sc, s);
}

}  // namespace

hipError_t launch_mx_quantize(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                              int transpose, int yt, uint8_t* q, uint8_t* scales, hipStream_t s) {
  const int64_t R = transpose ? cols : rows, K = transpose ? rows : cols;
  if (R == 0 || K == 0) return hipSuccess;
  if (xt == AMP_F32) return run_y<AMP_F32>(yt, x, ldx, R, K, transpose, q, scales, s);
  if (xt == AMP_BF16) return run_y<AMP_BF16>(yt, x, ldx, R, K, transpose, q, scales, s);
  return run_y<AMP_F16>(yt, x, ldx, R, K, transpose, q, scales, s);
}

}  // namespace amp
