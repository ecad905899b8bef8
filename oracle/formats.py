"""Bit-exact number formats (oracle).

Test infrastructure only (see ``oracle/__init__``).

Formats and their bit splits
----------------------------
* FP32 1/8/23 -- page "Mixed Precision Training/es" (marovi), section
  "Formatos de coma flotante".
* FP16 1/5/10, max 65504, min normal 2^-14, subnormal floor 2^-24 -- page
  "혼합 정밀도 학습" (itwiki), section "왜 그냥 FP16으로는 안 되는가".
* BF16 1/8/7 -- marovi "Formatos de coma flotante".
* FP8 E4M3 (range [-448, 448]) and E5M2 -- itwiki section "FP8 혼합 정밀도";
  page "FP8 혼합 정밀도 LLM 학습" (hwlabs), sections "FP8이 어려운 이유" and
  "두 FP8 서브포맷의 선택 이유" (the two formats treat NaN/inf differently).
  E4M3 here is the OCP "FN" variant: no infinities, NaN = S.1111.111, so the
  largest finite value is 1.75*2^8 = 448 as the page states.  E5M2 keeps
  IEEE-style inf/NaN; its largest finite value 1.75*2^15 = 57344 follows from
  1/5/2 (the page does not print it).
* E2M1 (the 4-bit element of NVFP4) -- page "Pretraining Large Language Models
  with NVFP4" (gist.science), section "2.1 NVFP4 포맷의 특징".  1/2/1 with bias
  1, no specials: magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.

Rounding (reading, the pages only say "round")
----------------------------------------------
* Round to nearest, ties to the even code, gradual underflow, signed zero kept.
* IEEE formats (FP32, FP16, BF16): a value whose correctly rounded magnitude
  exceeds the largest finite value becomes +-inf; NaN becomes the canonical
  quiet NaN (sign 0, top mantissa bit set).
* Saturating formats (E4M3, E5M2, E2M1): clip to [-max, max] first (+-inf go to
  +-max), then round.  This is the page's ``clip(x, -448, 448)`` (hwlabs,
  "FP8이 어려운 이유").  NaN encodes as 0x7F for both FP8 formats; E2M1 has no
  NaN and a NaN input encodes as +0 (documented reading).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Fmt:
    name: str
    ebits: int
    mbits: int
    bias: int
    saturate: bool        # True: clip to +-max before rounding (no overflow to inf)
    has_inf: bool         # True: the all-ones exponent encodes inf/NaN (IEEE style)
    max_finite: float
    nan_code: int | None  # canonical NaN code (None: format has no NaN)

    @property
    def nbits(self) -> int:
        return 1 + self.ebits + self.mbits

    @property
    def emin(self) -> int:      # exponent of the smallest normal
        return 1 - self.bias

    @property
    def min_normal(self) -> float:
        return float(np.ldexp(1.0, self.emin))

    @property
    def min_subnormal(self) -> float:
        return float(np.ldexp(1.0, self.emin - self.mbits))


def _maxf(ebits, mbits, bias, top_exp_reserved, top_mant_reserved):
    """Largest finite value from the bit split.

    top_exp_reserved: the all-ones exponent is inf/NaN (IEEE style).
    top_mant_reserved: only the all-ones mantissa of the all-ones exponent is
    NaN (OCP E4M3 style)."""
    emax_field = (1 << ebits) - 1 - (1 if top_exp_reserved else 0)
    mant = (1 << mbits) - 1 - (1 if top_mant_reserved else 0)
    return float(np.ldexp(1.0 + mant / (1 << mbits), emax_field - bias))


F32 = Fmt("f32", 8, 23, 127, False, True, _maxf(8, 23, 127, True, False), 0x7FC00000)
F16 = Fmt("f16", 5, 10, 15, False, True, _maxf(5, 10, 15, True, False), 0x7E00)
BF16 = Fmt("bf16", 8, 7, 127, False, True, _maxf(8, 7, 127, True, False), 0x7FC0)
E4M3 = Fmt("e4m3", 4, 3, 7, True, False, _maxf(4, 3, 7, False, True), 0x7F)
E5M2 = Fmt("e5m2", 5, 2, 15, True, True, _maxf(5, 2, 15, True, False), 0x7F)
E2M1 = Fmt("e2m1", 2, 1, 1, True, False, _maxf(2, 1, 1, False, False), None)

FORMATS = {f.name: f for f in (F32, F16, BF16, E4M3, E5M2, E2M1)}


def round_to(x, fmt: Fmt) -> np.ndarray:
    """Round float64 values to the nearest value of ``fmt`` (ties to even).

    Returns float64 values that are exactly representable in ``fmt`` (or
    +-inf / NaN for the IEEE formats).  The rounding is done on the exact
    float64 input: the spacing (ulp) of the target at the input's binade is a
    power of two, so ``x / ulp`` is exact and ``rint`` (ties to even) rounds the
    significand once.
    """
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    if not fmt.saturate:
        xc = x
    else:
        xc = np.clip(np.where(nan, 0.0, x), -fmt.max_finite, fmt.max_finite)
    a = np.abs(np.where(nan, 0.0, xc))
    finite = np.isfinite(a)
    af = np.where(finite, a, 0.0)
    _, e = np.frexp(af)                       # af = f * 2^e, f in [0.5, 1)
    binade = e.astype(np.int64) - 1           # floor(log2 af) for af > 0
    q = np.maximum(binade, fmt.emin) - fmt.mbits   # log2 of the spacing
    y = np.ldexp(np.rint(np.ldexp(af, -q)), q)
    if not fmt.saturate:
        y = np.where(y > fmt.max_finite, np.inf, y)
    y = np.where(finite, y, np.inf)
    y = np.copysign(y, xc)
    return np.where(nan, np.nan, y)


def encode(x, fmt: Fmt) -> np.ndarray:
    """Round float64 values to ``fmt`` and return the integer codes."""
    y = round_to(x, fmt)
    return encode_exact(y, fmt)


def encode_exact(y, fmt: Fmt) -> np.ndarray:
    """Integer codes of values already representable in ``fmt``."""
    y = np.asarray(y, dtype=np.float64)
    nan = np.isnan(y)
    inf = np.isinf(y)
    sign = np.signbit(y).astype(np.int64)
    a = np.abs(np.where(nan | inf, 0.0, y))
    _, e = np.frexp(a)
    binade = e.astype(np.int64) - 1
    sub = a < fmt.min_normal
    exp_field = np.where(sub, 0, binade + fmt.bias)
    q = np.where(sub, fmt.emin, binade) - fmt.mbits
    sig = np.ldexp(a, -q).astype(np.int64)    # exact: a is representable
    mant = np.where(sub, sig, sig - (1 << fmt.mbits))
    code = (sign << (fmt.ebits + fmt.mbits)) | (exp_field << fmt.mbits) | mant
    code = np.where(a == 0, sign << (fmt.ebits + fmt.mbits), code)
    if fmt.has_inf:
        inf_code = (sign << (fmt.ebits + fmt.mbits)) | (((1 << fmt.ebits) - 1) << fmt.mbits)
        code = np.where(inf, inf_code, code)
    elif inf.any():
        raise ValueError(f"{fmt.name} has no infinity")
    if fmt.nan_code is not None:
        code = np.where(nan, fmt.nan_code, code)
    elif nan.any():
        code = np.where(nan, 0, code)
    dt = {8: np.uint8, 16: np.uint16, 32: np.uint32}.get(fmt.nbits, np.uint8)
    return code.astype(dt)


def decode(code, fmt: Fmt) -> np.ndarray:
    """float64 value of each integer code of ``fmt``."""
    c = np.asarray(code).astype(np.int64) & ((1 << fmt.nbits) - 1)
    sign = (c >> (fmt.ebits + fmt.mbits)) & 1
    ef = (c >> fmt.mbits) & ((1 << fmt.ebits) - 1)
    mf = c & ((1 << fmt.mbits) - 1)
    sub = ef == 0
    mag = np.where(sub,
                   np.ldexp(mf.astype(np.float64), fmt.emin - fmt.mbits),
                   np.ldexp((mf + (1 << fmt.mbits)).astype(np.float64),
                            ef - fmt.bias - fmt.mbits))
    top = ef == (1 << fmt.ebits) - 1
    if fmt.has_inf:
        mag = np.where(top & (mf == 0), np.inf, mag)
        mag = np.where(top & (mf != 0), np.nan, mag)
    elif fmt.nan_code is not None:     # OCP E4M3: only S.1111.111 is NaN
        mag = np.where(top & (mf == (1 << fmt.mbits) - 1), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


# --------------------------------------------------------------------------
# FP32 helpers: the oracle's "FP32 operation" = exact/float64 op, then one RNE.
# --------------------------------------------------------------------------

def f32(x) -> np.ndarray:
    """Round to FP32 (RNE, IEEE overflow), returned as float64."""
    return round_to(x, F32)


def f32_bits(x) -> np.ndarray:
    """FP32 bit patterns (uint32) of values already representable in FP32."""
    return encode_exact(x, F32)


def from_f32_bits(u) -> np.ndarray:
    return decode(np.asarray(u, dtype=np.uint32), F32)


def ulp_distance(code_a, code_b, fmt: Fmt) -> np.ndarray:
    """Distance in units of last place between two codes of ``fmt``, using the
    monotone integer ordering of sign-magnitude codes (+0 and -0 coincide)."""
    n = fmt.nbits
    sb = 1 << (n - 1)

    def ordered(c):
        c = np.asarray(c).astype(np.int64)
        return np.where(c & sb, -(c & (sb - 1)), c)

    return np.abs(ordered(code_a) - ordered(code_b))
