"""Gradient accumulation and global-norm clipping (oracle).

Test infrastructure only (see ``oracle/__init__``).

Sources
-------
* Page "혼합 정밀도 학습" (itwiki), section "FP16 학습 루프": the loop calls
  ``scaler.unscale_`` and then ``clip_grad_norm_(max_norm=1.0)``; clipping must
  come after unscaling so that the norm is that of the true gradients.
* Same page, section "함께 쓰는 기법과 주의점": when gradients of several
  micro-batches are accumulated, the scale adjustment and the inf check happen
  once per effective batch.
* Page "Mixed Precision Training/es" (marovi), "Operaciones que permanecen en
  FP32": long reductions such as gradient norms for clipping stay in FP32.

Readings (the pages name the operations, not their arithmetic):
* Accumulation is into an FP32 buffer: ``acc = fl32(acc + f32(g))`` per
  micro-batch (the first micro-batch is copied).  inf/NaN propagate, so one
  check of the accumulated buffer covers every micro-batch.
* The global norm is the Euclidean norm of all unscaled gradients,
  ``sqrt(sum (f32(g) / S)^2)``, taken over finite elements (a non-finite one
  means the step is skipped anyway).  Its sum of squares is formed at least in
  FP32; here it is exact (every FP32 square is exact in float64 and the sum is
  correctly rounded with ``math.fsum``), so an implementation that sums in
  float64 in any order lies within n * 2^-53 of it.
* The coefficient is PyTorch's documented formula with its 1e-6 guard,
  evaluated in FP32: ``coef = min(1, fl32(max_norm / fl32(norm32 + 1e-6)))``
  with ``norm32 = fl32(sqrt(sumsq))``; the clipped gradient is ``fl32(g * coef)``
  (see ``adamw.apply(grad_mult=...)``).
"""
from __future__ import annotations

import math

import numpy as np

from . import formats as F


def accumulate(acc, g_codes, g_fmt: F.Fmt, first: bool):
    """One micro-batch into the FP32 accumulator (float64 arrays of FP32 values)."""
    g = F.f32(F.decode(g_codes, g_fmt))
    if first:
        return g
    return F.f32(np.asarray(acc, dtype=np.float64) + g)


def norm_sq(g_codes, g_fmt: F.Fmt, loss_scale: float):
    """Exact (correctly rounded) sum of squares of the finite unscaled gradients,
    and whether a non-finite gradient was seen."""
    x = F.f32(F.decode(np.asarray(g_codes).ravel(), g_fmt))
    finite = np.isfinite(x)
    inv = float(F.f32(1.0 / loss_scale))
    y = x[finite] * inv                 # exact: 1/S is a power of two
    return math.fsum((y * y).tolist()), bool((~finite).any())


def coefficient_from_norm(norm32: float, max_norm: float) -> float:
    """min(1, fl32(max_norm / fl32(norm32 + 1e-6))), all in FP32."""
    mx = float(F.f32(max_norm))
    c = float(F.f32(mx / float(F.f32(norm32 + float(F.f32(1e-6))))))
    return min(1.0, c)


def clip_coefficient(sumsq: float, max_norm: float):
    """(coef, norm32) from the sum of squares of the unscaled gradients."""
    norm32 = float(F.f32(math.sqrt(sumsq)))
    return coefficient_from_norm(norm32, max_norm), norm32
