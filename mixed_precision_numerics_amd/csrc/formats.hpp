// Device-side number-format conversions for gfx950.
//
// Every conversion rounds to nearest with ties to the even code, keeps
// gradual underflow and the sign of zero, and is written with integer and
// exact FP32 operations so that it is bit-identical on every input:
//   * FP16 / BF16 (IEEE): overflow gives +-inf, NaN gives the canonical quiet
//     NaN (0x7E00 / 0x7FC0).
//   * FP8 E4M3 (OCP, max 448) and E5M2 (max 57344): values are clipped to
//     [-max, max] first (inf included), the page's clip(x, -448, 448) of
//     "FP8 혼합 정밀도 LLM 학습" (hwlabs), section "FP8이 어려운 이유"; NaN -> 0x7F.
//   * FP4 E2M1 (NVFP4 element, page "Pretraining Large Language Models with
//     NVFP4", section 2.1): clipped to [-6, 6]; nearest-even or stochastic.
// Subnormal targets use one exact FP32 addition of a power of two whose ulp
// equals the target's subnormal spacing, so the FPU does the tie-to-even.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace amp {

__device__ __forceinline__ uint32_t fbits(float x) { return __float_as_uint(x); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __uint_as_float(u); }

// All conversions below are branch-free: both the normal-range and the
// subnormal-range result are formed and selected, so a wave never diverges.

// ---- FP32 -> FP16 / BF16 ---------------------------------------------------
// Round to nearest even (FP16 subnormal results kept, |x| >= 65520 gives inf),
// NaN gives the canonical 0x7E00 / 0x7FC0.  gfx950's conversions round to
// nearest even and keep NaN payloads, hence the NaN select.  Compared on MI355X
// with bit-manipulation encoders: equal on all 2^32 FP32 patterns.
__device__ __forceinline__ uint32_t f32_to_f16(float x) {
  const uint32_t c = __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  return x != x ? 0x7e00u : c;
}

__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  const uint32_t c = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  return x != x ? 0x7fc0u : c;
}

// ---- FP32 -> E4M3 / E5M2 (saturating) ------------------------------------
// Round to nearest even, magnitudes beyond the largest finite value (448,
// 57344) and infinities saturate to it, NaN gives 0x7F.  gfx950's conversion
// instruction rounds to nearest even but turns out-of-range inputs into NaN,
// so the input is first clamped to the format's range with a median-of-three
// (which returns a bound for a NaN input, hence the NaN select).  Compared on
// MI355X with bit-manipulation encoders (mantissa rounded at the format's last
// bit for normal results, an aligning addition for subnormal ones, a
// saturation threshold): equal on all 2^32 FP32 patterns for both formats.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const float y = __builtin_amdgcn_fmed3f(x, -448.0f, 448.0f);
  const uint32_t c = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false)) & 0xffu;
  return x != x ? 0x7fu : c;
}

__device__ __forceinline__ uint32_t f32_to_e5m2(float x) {
  const float y = __builtin_amdgcn_fmed3f(x, -57344.0f, 57344.0f);
  const uint32_t c = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_bf8_f32(y, y, 0, false)) & 0xffu;
  return x != x ? 0x7fu : c;
}

// ---- widening (exact) -----------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t c) { return bitsf(c << 16); }

// FP16 -> FP32 with the hardware conversion: exact for every code (FP16
// subnormals are kept), NaN stays NaN.
__device__ __forceinline__ float f16_to_f32(uint32_t c) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(c)));
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xfu;
  const uint32_t m = c & 0x7u;
  const uint32_t sub = fbits(static_cast<float>(m) * 0.001953125f);
  const uint32_t nrm = ((e + 120u) << 23) | (m << 20);
  const uint32_t r = s | (e == 0 ? sub : nrm);
  return bitsf((e == 0xfu && m == 0x7u) ? 0x7fc00000u : r);
}

__device__ __forceinline__ float e5m2_to_f32(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 24;
  const uint32_t e = (c >> 2) & 0x1fu;
  const uint32_t m = c & 0x3u;
  const uint32_t sub = fbits(static_cast<float>(m) * 1.52587890625e-5f);
  const uint32_t nrm = ((e + 112u) << 23) | (m << 21);
  const uint32_t spec = 0x7f800000u | (m << 21);
  return bitsf(s | (e == 0 ? sub : (e == 0x1fu ? spec : nrm)));
}

// ---- E2M1 (FP4) -----------------------------------------------------------
// Magnitude codes 0..7 = {0, 0.5, 1, 1.5, 2, 3, 4, 6}; bit 3 is the sign.
// From [1, 8) up the E2M1 grid is the FP32 grid cut to one fraction bit, so
// code = (FP32 bits >> 22) - 252 there; below 1 the spacing is 0.5.
// Round to nearest even, ties to the even code (5 gives 4); magnitudes above
// 5 give 6, including everything beyond 6 (saturation); NaN gives +0 (E2M1
// has no NaN).  gfx950's FP4 conversion
// (scale 1) rounds to nearest even and saturates; only NaN needs the select.
// Compared on MI355X with a bit-manipulation encoder (the FP32 pattern cut to
// one fraction bit from 1 up, midpoint compares below): equal on all 2^32 FP32
// patterns.
__device__ __forceinline__ uint32_t e2m1_rne(float y) {
  const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y, y, 1.0f, 0) & 0xfu;
  return y != y ? 0u : c;
}

// Stochastic rounding driven by the element's 32-bit random word w: the
// magnitude rounds up iff u < frac with u = (w >> 8) * 2^-24 and
// frac = (|y| - lower neighbour) / gap (exact in FP32).  Both ranges are
// evaluated as a carry: adding the complement of the word's top bits to the
// part of |y| below the E2M1 step carries into the kept part exactly when the
// rounding goes up.
//  * |y| >= 1: the step is one unit of FP32 bit 22, the part below it is the
//    low 22 pattern bits m, and u < frac  <=>  (w >> 10) < m
//    <=>  m + (~w >> 10) >= 2^22; the carry runs on into the exponent, so the
//    code is (pattern >> 22) - 252 after the addition (6 is the largest
//    magnitude and has m = 0, so nothing carries past it).
//  * |y| < 1: the step is 0.5; with C = ceil(|y| * 2^25) (integer units of
//    2^-25; for the integer X = w >> 8, X < F <=> X < ceil(F)), the code is
//    (C + (~w >> 8)) >> 24.
// A NaN y is taken as magnitude 6 (code 7 with y's sign bit).  In the
// quantizer y is NaN only if the input block holds a NaN, and then the block
// scale is NaN and the whole block is zeroed, or if enc / S overflows (a
// tensor amax below about 2^-107) and an element is zero.
__device__ __forceinline__ uint32_t e2m1_sr(float y, uint32_t w) {
  const float a = fminf(fabsf(y), 6.0f);
  const uint32_t b = fbits(a);
  const uint32_t nw = ~w;
  const uint32_t cn = (b + (nw >> 10) - 0x3f000000u) >> 22;          // (pattern >> 22) - 252
  const uint32_t cs = (static_cast<uint32_t>(ceilf(a * 33554432.0f)) + (nw >> 8)) >> 24;
  return (b >= 0x3f800000u ? cn : cs) | ((fbits(y) >> 28) & 0x8u);
}

__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t m = c & 7u;
  const float v = m < 4 ? 0.5f * static_cast<float>(m)
                        : (m == 4 ? 2.0f : (m == 5 ? 3.0f : (m == 6 ? 4.0f : 6.0f)));
  return (c & 8u) ? -v : v;
}

// ---- Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) ---------------------
struct ctr4 { uint32_t x, y, z, w; };

// a ^ b ^ c in one instruction (gfx950's three-input bit operation; 0x96 is
// the truth table of the three-input parity).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ ctr4 philox4x32_10(ctr4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c.x;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c.z;
    const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
    const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
    c = ctr4{xor3(hi1, c.y, k0), lo1, xor3(hi0, c.w, k1), lo0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

}  // namespace amp
