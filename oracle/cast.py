"""Scaled down-cast with amax capture (oracle).

Test infrastructure only (see ``oracle/__init__``).

What is computed (page "FP8 혼합 정밀도 LLM 학습" (hwlabs), sections
"FP8이 어려운 이유" and "Delayed Scaling 동작 원리"; page "혼합 정밀도 학습"
(itwiki), section "FP16 학습 루프", where the 16-bit working copy is made just
before each op):

* ``amax = max_i |x_i|`` of the *unscaled* input, recorded for the
  delayed-scaling history.  It is computed as an unsigned maximum over the
  FP32 bit patterns with the sign bit cleared, so the result is exact and
  independent of reduction order, and NaN > inf > any finite value.  Every NaN
  is first replaced by the canonical quiet NaN 0x7FC00000 (reading: the pages
  are silent on NaN).  The result is max-accumulated into the caller's value.
* ``t_i = fl32(x_i * scale)`` with ``scale`` an FP32 value -- one FP32 multiply (16-bit inputs widen to FP32
  exactly first).  Reading of the page's contradictory formula: the scale is a
  multiplier, because ``scale = fp8_max / (margin * amax)`` only brings a
  tensor into range as a multiplier.
* ``y_i = round_fmt(t_i)``: FP16/BF16 round to nearest even and overflow to
  +-inf (an overflowing FP16 gradient must surface as inf so that the step is
  skipped); E4M3/E5M2 saturate, i.e. ``clip(t, -max, max)`` then round.
"""
from __future__ import annotations

import numpy as np

from . import formats as F

CANON_NAN_BITS = np.uint32(0x7FC00000)


def widen_to_f32_bits(codes, in_fmt: F.Fmt) -> np.ndarray:
    """FP32 bit patterns of 16/32-bit input codes (exact widening)."""
    codes = np.asarray(codes)
    if in_fmt is F.F32:
        return codes.astype(np.uint32)
    if in_fmt is F.BF16:
        # BF16 is the upper half of the FP32 bit layout (1/8/7 vs 1/8/23)
        return codes.astype(np.uint32) << np.uint32(16)
    v = F.decode(codes, in_fmt)
    return F.encode_exact(v, F.F32)


def amax_bits(f32_bits) -> np.uint32:
    """Unsigned max of |x| bit patterns, NaN canonicalised (0 for empty)."""
    a = np.asarray(f32_bits, dtype=np.uint32) & np.uint32(0x7FFFFFFF)
    a = np.where(a > np.uint32(0x7F800000), CANON_NAN_BITS, a)
    return np.uint32(a.max()) if a.size else np.uint32(0)


def cast(codes, in_fmt: F.Fmt, out_fmt: F.Fmt, scale: float | None = None,
         amax_prior_bits: int = 0):
    """Scaled cast of an array of input codes.

    Returns ``(out_codes, amax_bits)`` where ``amax_bits`` is
    ``max(amax_prior_bits, amax(|x|))`` as an FP32 bit pattern.
    """
    bits = widen_to_f32_bits(codes, in_fmt)
    am = np.uint32(max(int(amax_prior_bits), int(amax_bits(bits))))
    x = F.decode(bits, F.F32)
    # the scale is an FP32 value (a device-resident FP32 multiplier)
    t = x if scale is None else F.f32(x * F.f32(np.float64(scale)))
    return F.encode(t, out_fmt), am


def cast_values(x_f32_values, out_fmt: F.Fmt, scale: float | None = None):
    """Convenience: cast FP32 values (float64 holding FP32-representable
    numbers) and return the rounded output values (float64)."""
    x = np.asarray(x_f32_values, dtype=np.float64)
    t = x if scale is None else F.f32(x * F.f32(np.float64(scale)))
    return F.round_to(t, out_fmt)


def saturated_count(codes, in_fmt: F.Fmt, out_fmt: F.Fmt, scale: float | None = None) -> int:
    """Number of elements the saturating cast clips.

    Saturation is data, not an error (hwlabs "FP8이 어려운 이유": values
    beyond the format's range are clipped to it).  Reading: an element is
    saturated when its scaled value
    ``t = fl32(x * scale)`` has ``|t| > max_finite`` of the saturating output
    format (E4M3, E5M2), infinities included; NaN is not a saturation; the
    IEEE-mode 16-bit formats overflow to inf instead and count nothing."""
    if not out_fmt.saturate:
        return 0
    bits = widen_to_f32_bits(codes, in_fmt)
    x = F.decode(bits, F.F32)
    t = x if scale is None else F.f32(x * F.f32(np.float64(scale)))
    with np.errstate(invalid="ignore"):
        return int(np.count_nonzero(np.abs(t) > out_fmt.max_finite))


def found_inf_from_amax(amax_bits_list, out_fmt: F.Fmt, scale: float | None = None) -> bool:
    """Overflow flag of gradients that a scaled cast produced, from the amax
    values that cast recorded, so that the optimizer needs no sweep of its own
    (itwiki "손실 스케일링": a step with any inf/NaN gradient is skipped).

    Reading: rounding is monotone in |t|, so some output of the cast is
    non-finite exactly when the largest input magnitude gives one: the flag is
    set if an amax is NaN or inf, or, for the IEEE-mode 16-bit formats, if
    ``round_fmt(fl32(amax * scale))`` is infinite.  Saturating formats (FP8)
    clip finite values, so only a non-finite amax sets it there."""
    for ab in amax_bits_list:
        a = float(F.from_f32_bits(np.uint32(int(ab))))
        if not np.isfinite(a):
            return True
        if not out_fmt.saturate:
            t = a if scale is None else float(F.f32(a * float(F.f32(np.float64(scale)))))
            if not np.isfinite(F.round_to(np.array([t]), out_fmt)[0]):
                return True
    return False

