"""16-point random Hadamard transform (oracle).

Test infrastructure only (see ``oracle/__init__``).

Page "Pretraining Large Language Models with NVFP4" (gist.science), section
"2.2 학습 방법론의 핵심 구성 요소", item 2: a 16x16 random Hadamard transform is
applied to the inputs of the weight-gradient GEMM (not to forward or
activation-gradient GEMMs) to spread outliers.

Readings (the page gives no formula):
* Transform ``H~ = H16 diag(s) / 4`` with the Sylvester matrix
  ``H16[i][j] = (-1)^popcount(i & j)`` and a seeded sign vector ``s``
  (``s_j = 1 - 2*bit_j`` of Philox word 0 at counter (0,0,1,0)).  ``H~`` is
  orthogonal, so applying the same ``H~`` along K to both wgrad operands leaves
  the product unchanged.
* Evaluation order (fixes FP32 rounding so that both sides agree bit for bit):
  sign flip (exact); butterflies ``(a, b) -> (a + b, a - b)`` at strides 1, 2,
  4, 8 in that order, each result rounded to FP32; finally multiply by 0.25
  (rounded to FP32, exact unless the result is subnormal).
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from .philox import philox4x32_10


def sylvester16() -> np.ndarray:
    i = np.arange(16)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def sign_vector(seed: int) -> np.ndarray:
    w0 = int(philox4x32_10(0, 0, 1, 0, seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)[0])
    bits = np.array([(w0 >> j) & 1 for j in range(16)], dtype=np.float64)
    return 1.0 - 2.0 * bits


def rht16(x, signs) -> np.ndarray:
    """Apply H~ to every 16-element chunk along the last axis.

    ``x``: float64 array of FP32-representable values, last dim % 16 == 0.
    """
    x = np.asarray(x, dtype=np.float64)
    shp = x.shape
    z = (x.reshape(-1, 16) * signs[None, :]).copy()
    for h in (1, 2, 4, 8):
        for blk in range(0, 16, 2 * h):
            for i in range(blk, blk + h):
                a = z[:, i].copy()
                b = z[:, i + h].copy()
                z[:, i] = F.f32(a + b)
                z[:, i + h] = F.f32(a - b)
    z = F.f32(z * 0.25)
    return z.reshape(shp)


def rht16_dense(x, signs) -> np.ndarray:
    """The same transform as one float64 matrix product (no FP32 rounding)."""
    x = np.asarray(x, dtype=np.float64)
    h = sylvester16() * signs[None, :] / 4.0
    return (x.reshape(-1, 16) @ h.T).reshape(x.shape)
