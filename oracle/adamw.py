"""Unscale + overflow check + skip-or-apply AdamW on FP32 master weights (oracle).

Test infrastructure only (see ``oracle/__init__``).

Sources
-------
* FP32 master weights: page "혼합 정밀도 학습" (itwiki), section
  "FP32 마스터 가중치" -- the update is applied to the FP32 copy and the 16-bit
  working copy is re-rounded from it; optimizer state (Adam moments) is FP32
  (page "Mixed Precision Training/es" (marovi), section "Operaciones que
  permanecen en FP32"; page hwlabs, section "도입 체크리스트").
* Unscale by 1/S in FP32 just before the update: itwiki section "손실 스케일링"
  (equation g = (1/S) fp32(grad of S*L)); marovi "La receta de precisión mixta".
* inf/NaN check with skip: itwiki "손실 스케일링"; marovi "Escalado dinámico de
  pérdida".
* AdamW is only named (itwiki "FP16 학습 루프" uses torch.optim.AdamW with
  lr=1e-3).  Reading: decoupled weight decay (Loshchilov & Hutter, "Decoupled
  Weight Decay Regularization", ICLR 2019) in the form PyTorch documents for
  AdamW; unstated hyper-parameters take PyTorch's documented defaults.

FP32 operation order (no fused multiply-add), per element::

    g = f32(g16) * invS                      (exact: S is a power of two)
    m = b1*m + c1*g
    v = b2*v + c2*(g*g)
    d = sqrt(v)*rbc2 + eps
    theta = theta*decay - step*(m/d)
    w16 = round16(theta)

with the scalars computed once per applied step in float64 and rounded once to
FP32: ``t += 1``, running products ``b1p *= beta1``, ``b2p *= beta2``,
``step = lr/(1-b1p)``, ``rbc2 = 1/sqrt(1-b2p)``, ``decay = 1-lr*wd``,
``c1 = 1-beta1``, ``c2 = 1-beta2``.  When any gradient is non-finite nothing is
written and the step count is unchanged.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import formats as F


@dataclass
class AdamWHParams:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01


@dataclass
class AdamCounters:
    step: int = 0
    beta1_pow: float = 1.0
    beta2_pow: float = 1.0


def nonfinite_16(codes, fmt: F.Fmt) -> np.ndarray:
    """True where a 16-bit (or FP32) gradient code is inf or NaN: its exponent
    field is all ones.  Integer codes are tested in their own width."""
    c = np.asarray(codes)
    if c.dtype.kind not in "ui":
        c = c.astype(np.int64)
    ef_mask = ((1 << fmt.ebits) - 1) << fmt.mbits
    return (c & ef_mask) == ef_mask


def found_inf(codes, fmt: F.Fmt) -> bool:
    return bool(nonfinite_16(codes, fmt).any())


def scalars(hp: AdamWHParams, ctr: AdamCounters, loss_scale: float):
    """Per-step scalars for the step that would be applied next."""
    b1p = ctr.beta1_pow * hp.beta1
    b2p = ctr.beta2_pow * hp.beta2
    return dict(
        b1p=b1p, b2p=b2p,
        step=float(F.f32(hp.lr / (1.0 - b1p))),
        rbc2=float(F.f32(1.0 / np.sqrt(1.0 - b2p))),
        decay=float(F.f32(1.0 - hp.lr * hp.weight_decay)),
        c1=float(F.f32(1.0 - hp.beta1)),
        c2=float(F.f32(1.0 - hp.beta2)),
        b1=float(F.f32(hp.beta1)),
        b2=float(F.f32(hp.beta2)),
        eps=float(F.f32(hp.eps)),
        inv_s=float(F.f32(1.0 / loss_scale)),
    )


def apply(theta, m, v, g_codes, g_fmt: F.Fmt, hp: AdamWHParams,
          ctr: AdamCounters, loss_scale: float, w_fmt: F.Fmt = F.F16,
          skip: bool | None = None, grad_mult: float | None = None):
    """One optimizer step on float64 arrays holding FP32 values.

    Returns ``(theta, m, v, w_codes, applied)``; the inputs are not modified.
    ``skip`` overrides the overflow decision (used when a caller checks a
    larger buffer than the sample it passes here).  ``grad_mult`` (an FP32
    value, e.g. the clip coefficient) multiplies the unscaled gradient in FP32
    before the update: itwiki "FP16 학습 루프" clips after ``unscale_``.
    """
    theta = np.asarray(theta, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if skip is None:
        skip = found_inf(g_codes, g_fmt)
    if skip:
        return theta.copy(), m.copy(), v.copy(), F.encode(theta, w_fmt), False
    s = scalars(hp, ctr, loss_scale)
    f32 = F.f32
    g = f32(F.decode(g_codes, g_fmt) * s["inv_s"])
    if grad_mult is not None:
        g = f32(g * float(F.f32(grad_mult)))
    m1 = f32(f32(s["b1"] * m) + f32(s["c1"] * g))
    v1 = f32(f32(s["b2"] * v) + f32(s["c2"] * f32(g * g)))
    d = f32(f32(f32(np.sqrt(v1)) * s["rbc2"]) + s["eps"])
    th1 = f32(f32(theta * s["decay"]) - f32(s["step"] * f32(m1 / d)))
    ctr.step += 1
    ctr.beta1_pow = s["b1p"]
    ctr.beta2_pow = s["b2p"]
    return th1, m1, v1, F.encode(th1, w_fmt), True
