"""Low-precision GEMM with FP32 accumulation: float64 reference (oracle).

Test infrastructure only (see ``oracle/__init__``).

Page "혼합 정밀도 학습" (itwiki), section "FP32 누산과 연산별 정밀도": 16-bit
products are accumulated in FP32 and the result is written out in 16 bits.
Page hwlabs, section "GEMM 누적 정밀도 문제": FP8 products, FP32 accumulation,
output cast.  Page marovi, "La receta de precisión mixta": matrix units consume
low-precision inputs, accumulate in FP32, write low-precision outputs.

The pages fix no summation order (and marovi "Limitaciones y modos de fallo"
notes that bit-level results differ across hardware), so the reference is the
exact-as-possible float64 sum ``C_ref = alpha * sum_k a_ik b_kj`` together with
``bound = |alpha| * sum_k |a_ik| |b_kj|``.  A GPU result passes when
``|C_gpu - C_ref| <= rtol * bound`` (rtol = 1e-5) before output rounding, and
when a rounded output lies within one output-format ulp of that band.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from . import formats as F

RTOL = 1e-5


def reference(a, b, alpha: float = 1.0):
    """(C_ref, bound) for C = alpha * a @ b with a [M,K], b [K,N] float64."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    c = np.matmul(a, b) * alpha
    bound = np.matmul(np.abs(a), np.abs(b)) * abs(alpha)
    return c, bound


def exact(a, b):
    """Exact rational product for tiny shapes (brute force)."""
    M, K = len(a), len(a[0])
    N = len(b[0])
    fa = [[Fraction(float(a[i][k])) for k in range(K)] for i in range(M)]
    fb = [[Fraction(float(b[k][j])) for j in range(N)] for k in range(K)]
    return [[sum((fa[i][k] * fb[k][j] for k in range(K)), Fraction(0))
             for j in range(N)] for i in range(M)]


def check_f32(c_gpu, c_ref, bound, rtol: float = RTOL):
    """Boolean mask of elements within the FP32-accumulation tolerance."""
    c_gpu = np.asarray(c_gpu, dtype=np.float64)
    return np.abs(c_gpu - c_ref) <= rtol * bound


def check_rounded(out_codes, out_fmt: F.Fmt, c_ref, bound, rtol: float = RTOL):
    """Boolean mask: a rounded output passes if it lies within one ulp of the
    tolerance band ``[c_ref - rtol*bound, c_ref + rtol*bound]``, i.e. it is a
    value that rounding some admissible FP32 accumulator could give, or its
    neighbour."""
    val = F.decode(out_codes, out_fmt)
    tol = rtol * bound
    lo = F.encode(c_ref - tol, out_fmt)
    hi = F.encode(c_ref + tol, out_fmt)
    ord_ = lambda c: _ordered(c, out_fmt)
    o = ord_(out_codes)
    ok = (o >= ord_(lo) - 1) & (o <= ord_(hi) + 1)
    return ok & ~np.isnan(val)


def _ordered(codes, fmt: F.Fmt):
    c = np.asarray(codes).astype(np.int64)
    sb = 1 << (fmt.nbits - 1)
    return np.where(c & sb, -(c & (sb - 1)), c)
