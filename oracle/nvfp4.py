"""NVFP4 two-level quantizer (oracle).

Test infrastructure only (see ``oracle/__init__``).

Page "Pretraining Large Language Models with NVFP4" (gist.science):
* section "2.1 NVFP4 포맷의 특징": 4-bit E2M1 elements in blocks of 16, one E4M3
  block scale per block, and a tensor-level FP32 scale on top (two levels);
* section "2.2", item 2: 16x16 random Hadamard transform on the weight-gradient
  GEMM inputs only;
* item 3: weights use 16x16 two-dimensional blocks, activations and gradients
  1x16 blocks;
* item 4: gradients are stochastically rounded, forward tensors are not.

Readings (the page gives the structure, not the arithmetic):
1. Operand orientation: the quantized operand has ``rows x K`` with K the
   reduction dimension; blocks run along K.  ``transpose=True`` quantizes
   ``x.T`` (the weight-gradient GEMM reduces over tokens, the leading dim).
2. RHT (optional) along K, see ``oracle.hadamard``.
3. Tensor scale: ``A = max |z|``; ``enc = fl32(2688 / A)`` (2688 = 448 * 6, the
   E4M3 max times the E2M1 max) if A is finite and > 0, else 1.
4. Block scale: ``b = max |z|`` over the block; stored E4M3 code
   ``s_blk = E4M3_sat(fl32(fl32(b / 6) * enc))``; ``S = decode(s_blk)``.
5. Element: if ``S == 0`` the code is +0; else ``y = fl32(z * fl32(enc / S))``
   and the code is ``E2M1_sat(y)`` with round-to-nearest-even (forward tensors)
   or stochastic rounding (gradients).
6. Stochastic rounding: ``lo <= |y| < hi`` are the neighbouring E2M1
   magnitudes, ``frac = (|y| - lo) / (hi - lo)`` (exact in FP32),
   ``u = (w >> 8) * 2^-24`` with ``w`` the Philox word for the element's
   row-major index ``idx = row * K + k``; the magnitude rounds up iff
   ``u < frac``; ``|y| >= 6`` gives 6; the sign is kept.
7. Packing: two codes per byte, the lower K index in the low nibble.
8. Dequantised value: ``e2m1(q) * S / enc``.
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from . import hadamard
from .philox import stream_words

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
TENSOR_NUM = 2688.0


def tensor_enc(amax: float) -> float:
    """Reading 3: ``enc = fl32(2688 / A)`` for a finite A > 0, else 1."""
    a = float(amax)
    if np.isfinite(a) and a > 0.0:
        return float(F.f32(TENSOR_NUM / a))
    return 1.0


def _tensor_enc(z) -> float:
    return tensor_enc(float(np.max(np.abs(z))) if z.size else 0.0)


def _sr_e2m1(y, u):
    """Stochastic rounding of FP32 values y (float64) with uniforms u."""
    a = np.minimum(np.abs(y), 6.0)
    lo_i = np.searchsorted(E2M1_MAG, a, side="right") - 1
    lo_i = np.clip(lo_i, 0, 7)
    lo = E2M1_MAG[lo_i]
    hi = E2M1_MAG[np.minimum(lo_i + 1, 7)]
    gap = np.where(hi > lo, hi - lo, 1.0)
    frac = F.f32((a - lo) / gap)
    up = (u < frac) & (hi > lo)
    mag = np.where(up, hi, lo)
    return np.copysign(mag, y)


def quantize(x, transpose: bool = False, block2d: bool = False,
             rht: bool = False, rht_seed: int = 0, sr: bool = False,
             sr_seed: int = 0, tensor_amax: float | None = None, row_ids=None):
    """Quantize a 2-D float64 array (FP32/BF16-representable values).

    Returns ``(q_packed uint8 [rows, K/2], scale_codes uint8, enc float)``;
    ``scale_codes`` is ``[rows, K/16]`` (1x16 blocks) or ``[rows/16, K/16]``
    (16x16 blocks).

    To quantize some rows of a larger operand: ``tensor_amax`` is the whole
    (transformed) operand's ``max |z|`` (reading 3 takes the tensor's amax,
    not the slice's) and ``row_ids`` the rows' indices in it (the stochastic
    rounding index of reading 6 is ``row * K + k`` in the whole operand).
    """
    op = np.asarray(x, dtype=np.float64)
    if transpose:
        op = op.T
    rows, K = op.shape
    if K % 16 or (block2d and rows % 16):
        raise ValueError("dimensions must be multiples of 16")
    z = hadamard.rht16(op, hadamard.sign_vector(rht_seed)) if rht else op.copy()
    enc = _tensor_enc(z) if tensor_amax is None else tensor_enc(tensor_amax)
    az = np.abs(z)
    if block2d:
        b = az.reshape(rows // 16, 16, K // 16, 16).max(axis=(1, 3))
    else:
        b = az.reshape(rows, K // 16, 16).max(axis=2)
    s_code = F.encode(F.f32(F.f32(b / 6.0) * enc), F.E4M3)
    S = F.decode(s_code, F.E4M3)
    S_el = (np.repeat(np.repeat(S, 16, axis=0), 16, axis=1) if block2d
            else np.repeat(S, 16, axis=1))
    with np.errstate(divide="ignore", invalid="ignore"):
        mult = np.where(S_el > 0, F.f32(enc / np.where(S_el > 0, S_el, 1.0)), 0.0)
    y = F.f32(z * mult)
    if sr:
        r = (np.arange(rows, dtype=np.uint64) if row_ids is None
             else np.asarray(row_ids, dtype=np.uint64))
        idx = (r[:, None] * np.uint64(K) + np.arange(K, dtype=np.uint64)[None, :]).ravel()
        w = stream_words(sr_seed, idx).reshape(rows, K).astype(np.float64)
        u = np.floor(w / 256.0) * 2.0 ** -24
        yq = _sr_e2m1(y, u)
    else:
        yq = F.round_to(y, F.E2M1)
    codes = F.encode_exact(yq, F.E2M1).astype(np.uint8)
    codes = np.where(S_el > 0, codes, 0).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, s_code.astype(np.uint8), enc


def unpack(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def dequantize(packed, scale_codes, enc: float, block2d: bool = False):
    """float64 values ``e2m1(q) * S / enc`` of a quantized operand."""
    codes = unpack(packed)
    rows, K = codes.shape
    S = F.decode(scale_codes, F.E4M3)
    S_el = (np.repeat(np.repeat(S, 16, axis=0), 16, axis=1) if block2d
            else np.repeat(S, 16, axis=1))
    return F.decode(codes, F.E2M1) * S_el / enc
