"""Fine-grained FP8 scaling (1x128 tiles, 128x128 blocks) and its GEMM
(oracle).

Test infrastructure only (see ``oracle/__init__``).

Sources
-------
* Page "혼합 정밀도 학습" (itwiki), section "FP8 혼합 정밀도": DeepSeek-V3
  computes scales on the fly, per 1x128 tile for activations and per 128x128
  block for weights, and stores every tensor in E4M3 (relative loss error
  against BF16 under 0.25 %).
* Page "FP8 혼합 정밀도 LLM 학습" (hwlabs), section "DeepSeek-V3 FP8 학습 사례":
  FP8 forward and backward on every linear layer; section "GEMM 누적 정밀도
  문제": partial sums inside a tile may be low precision, the sum across
  tiles is FP32.

Readings (the pages give the granularity only):
* An operand ``O`` is ``[R, K]`` with K contiguous (``x`` or ``x^T``).  Its
  scaling tiles are 1x128 (one row, 128 consecutive K) or 128x128 (128 rows x
  128 K); the last tile along K, and in block mode along R, may be shorter.
* "On the fly" is current scaling tile by tile: the tile's amax (the FP32
  bit-pattern maximum of ``cast.amax_bits``) gives ``(scale, scale_inv)`` by
  ``recipe.current_scale`` with the element format's maximum (448 for E4M3,
  57344 for E5M2) and margin 1, i.e. ``scale = fl32(fmax / amax)``, or 1 when
  amax is 0 or not finite; ``scale_inv = fl32(1 / scale)``.
* Elements: ``round_fmt(fl32(x * scale))``, saturating (``cast.cast``).
* Scales are stored K-block-major: ``s[kb, r]`` (1x128) or ``s[kb, r // 128]``
  (128x128), so that the scales of one K-block are contiguous.
* GEMM: ``C[m, n] = sum_k (A[m,k] * sa(m,k)) * (B[n,k] * sb(n,k))`` with the
  dequantized operands (code value times its tile's ``scale_inv``), summed
  exactly (float64 matrix product of the dequantized values).
"""
from __future__ import annotations

import numpy as np

from . import cast as C
from . import formats as F
from . import recipe

TILE = 128
FMAX = {"e4m3": recipe.E4M3_MAX, "e5m2": recipe.E5M2_MAX}


def _ceil(a: int, b: int) -> int:
    return -(-a // b)


def quantize(x_codes, in_fmt: F.Fmt, out_fmt: F.Fmt, block: bool,
             transpose: bool = False):
    """Quantize the operand ``x`` (``transpose=False``) or ``x^T``.

    x_codes: [rows, cols] input codes (F32 bit patterns, BF16 or F16 codes).
    Returns (codes [R, K] uint8, scale_inv [ceil(K/128), R or ceil(R/128)]
    float64 holding FP32 values)."""
    bits = C.widen_to_f32_bits(np.asarray(x_codes), in_fmt)
    op = bits.T if transpose else bits
    R, K = op.shape
    KB = _ceil(K, TILE)
    RB = _ceil(R, TILE) if block else R
    fmax = FMAX[out_fmt.name]
    codes = np.zeros((R, K), dtype=np.uint8)
    s_inv = np.ones((KB, RB), dtype=np.float64)
    for rb in range(RB):
        rows = slice(rb * TILE, min(R, (rb + 1) * TILE)) if block else slice(rb, rb + 1)
        for kb in range(KB):
            cols = slice(kb * TILE, min(K, (kb + 1) * TILE))
            tile = op[rows, cols]
            am = C.amax_bits(tile)
            scale, scale_inv = recipe.current_scale(int(am), fmax)
            y, _ = C.cast(tile, F.F32, out_fmt, scale)
            codes[rows, cols] = y
            s_inv[kb, rb] = scale_inv
    return codes, s_inv


def dequantize(codes, s_inv, fmt: F.Fmt, block: bool):
    """Code value times its tile's scale_inv (float64, exact)."""
    v = F.decode(np.asarray(codes), fmt)
    R, K = v.shape
    kb = np.arange(K) // TILE
    r = np.arange(R) // (TILE if block else 1)
    return v * np.asarray(s_inv, dtype=np.float64)[kb[None, :], r[:, None]]


def gemm(a_codes, sa, a_fmt: F.Fmt, a_block: bool, b_codes, sb, b_fmt: F.Fmt,
         b_block: bool):
    """C = deq(A) deq(B)^T for A [M, K] and B [N, K]; also returns the
    magnitude sum_k |a||b| that bounds FP32 accumulation error."""
    A = dequantize(a_codes, sa, a_fmt, a_block)
    B = dequantize(b_codes, sb, b_fmt, b_block)
    return A @ B.T, np.abs(A) @ np.abs(B).T
