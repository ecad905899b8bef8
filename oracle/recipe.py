"""Delayed-scaling recipe for FP8 tensors (oracle).

Test infrastructure only (see ``oracle/__init__``).

Page "FP8 혼합 정밀도 LLM 학습" (hwlabs), section "Delayed Scaling 동작 원리":
at the end of each step the tensor's amax is stored in ``amax_history``;
before the next step the maximum over the last N entries (default 1024) gives
``scale = fp8_max / (margin * amax_max)``; the tensor is then cast with that
scale.  Section "도입 체크리스트" adds ``amax_compute_algo = most_recent`` (use
the latest amax only) and the default history length 1024; margin 1.0 is the
recommended value.

Readings (the pages are silent):
* ``margin`` multiplies amax literally, as the printed formula says.
* amax values are compared as FP32 bit patterns (NaN dominates).
* If ``amax_max`` is not finite or is zero, the previous scale is kept.
* ``scale_inv = fl32(1 / scale)``, used to dequantise in the GEMM epilogue.
* Initial state: history all zero, ``pos = 0``, ``scale = scale_inv = 1``.

Current (just-in-time) scaling, the alternative the same section contrasts
with delayed scaling: the tensor is read once to find its amax and then cast
with ``scale = fp8_max / (margin * amax)`` from that amax (two reads instead of
one).  Reading: with a zero or non-finite amax there is no history to fall
back on, so the scale is 1.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import formats as F

E4M3_MAX = 448.0
E5M2_MAX = 57344.0


@dataclass
class FP8Meta:
    history_len: int = 1024
    amax_cur_bits: int = 0
    scale: float = 1.0
    scale_inv: float = 1.0
    pos: int = 0
    history_bits: np.ndarray = field(default=None)

    def __post_init__(self):
        if self.history_bits is None:
            self.history_bits = np.zeros(self.history_len, dtype=np.uint32)

    def record(self, amax_bits: int):
        """Max-accumulate a cast's amax into the current step's amax."""
        self.amax_cur_bits = max(self.amax_cur_bits, int(amax_bits))


def update(meta: FP8Meta, fp8_max: float, margin: float = 1.0,
           algo: str = "max") -> FP8Meta:
    """One end-of-step update: record, reduce the window, derive the scale."""
    meta.history_bits[meta.pos] = np.uint32(meta.amax_cur_bits)
    if algo == "max":
        amax_max_bits = int(meta.history_bits.max())
    elif algo == "most_recent":
        amax_max_bits = int(meta.history_bits[meta.pos])
    else:
        raise ValueError(algo)
    amax_max = float(F.from_f32_bits(np.uint32(amax_max_bits)))
    if np.isfinite(amax_max) and amax_max > 0.0:
        denom = float(F.f32(np.float64(F.f32(margin)) * amax_max))
        scale = float(F.f32(np.float64(F.f32(fp8_max)) / denom))
        meta.scale = scale
        meta.scale_inv = float(F.f32(1.0 / scale))
    meta.pos = (meta.pos + 1) % meta.history_len
    meta.amax_cur_bits = 0
    return meta


def current_scale(amax_bits: int, fp8_max: float, margin: float = 1.0):
    """(scale, scale_inv) of current scaling from this tensor's amax bits."""
    amax = float(F.from_f32_bits(np.uint32(amax_bits)))
    if np.isfinite(amax) and amax > 0.0:
        denom = float(F.f32(np.float64(F.f32(margin)) * amax))
        scale = float(F.f32(np.float64(F.f32(fp8_max)) / denom))
        return scale, float(F.f32(1.0 / scale))
    return 1.0, 1.0
