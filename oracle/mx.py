"""Microscaling (MX) block formats: quantize, dequantize, GEMM reference
(oracle).

Test infrastructure only (see ``oracle/__init__``).

Sources
-------
* Page "혼합 정밀도 학습" (itwiki), section "FP8 혼합 정밀도": MX formats keep
  one power-of-two scale per block of 32 elements (MXFP8, MXFP6, MXFP4); the
  page points to the OCP microscaling specification for the details.
* Page "Pretraining Large Language Models with NVFP4" (gist), section 2.1:
  MXFP4 uses 32-element blocks with UE8M0 scales (NVFP4 changes both).

Reading (the OCP MX v1.0 conversion, restated):
* A block is 32 consecutive elements along K of one row.  Its scale is
  ``X = 2^e`` with ``e = floor(log2(amax)) - emax_elem`` (``emax_elem`` is the
  exponent of the element format's largest normal: 8 for E4M3, 15 for E5M2,
  2 for E2M1), clamped to the UE8M0 range [-127, 127] and stored as the byte
  ``e + 127``.
* Elements are ``round(x / X)`` to the element format, nearest-even, with
  saturation at the format's largest magnitude.
* An all-zero block gets ``e = -127`` (code 0); a block holding inf or NaN
  gets the NaN scale code 0xFF and its elements are encoded from ``x`` as they
  are (NaN codes where the format has them, 0 for E2M1).
* Dequantized element = decode(code) * 2^(code_X - 127).
"""
from __future__ import annotations

import math

import numpy as np

from . import formats as F

EMAX = {"e4m3": 8, "e5m2": 15, "e2m1": 2}
BLOCK = 32
SCALE_NAN = 0xFF


def _floor_log2(a: float) -> int:
    m, e = math.frexp(a)          # a = m * 2^e, m in [0.5, 1)
    return e - 1


def block_scale_code(amax: float, fmt: F.Fmt) -> int:
    if not math.isfinite(amax):
        return SCALE_NAN
    if amax == 0.0:
        return 0
    e = _floor_log2(amax) - EMAX[fmt.name]
    e = max(-127, min(127, e))
    return e + 127


def quantize(x, fmt: F.Fmt, transpose: bool = False):
    """x: [rows, cols] values (float64 holding the input's exact values); the
    operand is ``x`` (blocks along cols) or ``x^T`` (blocks along rows).
    Returns (codes [R, K] uint8 -- one code per element, E2M1 in the low
    nibble), scale codes [R, K/32] uint8)."""
    op = np.asarray(x, dtype=np.float64)
    if transpose:
        op = op.T
    R, K = op.shape
    assert K % BLOCK == 0
    blocks = op.reshape(R, K // BLOCK, BLOCK)
    codes = np.zeros((R, K // BLOCK, BLOCK), dtype=np.uint8)
    scales = np.zeros((R, K // BLOCK), dtype=np.uint8)
    for r in range(R):
        for b in range(K // BLOCK):
            v = blocks[r, b]
            amax = float(np.max(np.abs(v))) if np.all(np.isfinite(v)) else math.inf
            sc = block_scale_code(amax, fmt)
            scales[r, b] = sc
            if sc == SCALE_NAN:
                t = v
            else:
                t = v * math.ldexp(1.0, 127 - sc)          # exact: a power of two
            codes[r, b] = F.encode(t, fmt).astype(np.uint8)
    return codes.reshape(R, K), scales


def dequantize(codes, scales, fmt: F.Fmt):
    codes = np.asarray(codes)
    R, K = codes.shape
    vals = F.decode(codes, fmt).reshape(R, K // BLOCK, BLOCK)
    sc = np.asarray(scales).astype(np.int64)
    mult = np.where(sc == SCALE_NAN, np.nan, np.ldexp(1.0, sc - 127))
    return (vals * mult[:, :, None]).reshape(R, K)


def pack_e2m1(codes):
    """Two E2M1 codes per byte, the lower K index in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)
