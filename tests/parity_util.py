"""Host-side helpers for the full-size parity tests.

They only spread the oracle's own functions over row chunks of large arrays
(a worker pool sized to the host's share of cores) and decode codes through
tables the oracle builds; none of them holds arithmetic of its own.  Row
chunks do not change any result: every oracle function used here is
element-wise or, for amax, an order-free maximum.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import cast as OC
from oracle import formats as F
from oracle import gemm as OG

WORKERS = max(1, min(16, int(os.environ.get("OMP_NUM_THREADS", "8") or 8)))
_POOL = ThreadPoolExecutor(WORKERS)
_LUT: dict = {}


def lut(fmt: F.Fmt) -> np.ndarray:
    """float64 value of every code of an 8- or 16-bit format (oracle decode)."""
    if fmt.name not in _LUT:
        _LUT[fmt.name] = F.decode(np.arange(1 << fmt.nbits, dtype=np.int64), fmt)
    return _LUT[fmt.name]


def values(codes, fmt: F.Fmt) -> np.ndarray:
    """float64 values of 8/16-bit codes, or of FP32 bit patterns."""
    c = np.asarray(codes)
    if fmt is F.F32:
        # an FP32 bit pattern read as FP32 is exact in float64
        return c.astype(np.uint32).view(np.float32).astype(np.float64)
    return lut(fmt)[c.astype(np.int64) if c.dtype.itemsize > 2 else c]


def _chunks(n: int, parts: int):
    step = max(1, -(-n // parts))
    return [(o, min(n, o + step)) for o in range(0, n, step)]


def submit_rows(fn, *arrays, parts: int | None = None):
    """Futures of fn(a[r0:r1], b[r0:r1], ...) for each row chunk, on the pool."""
    n = arrays[0].shape[0]
    parts = parts or 4 * WORKERS
    return [_POOL.submit(fn, *(a[r0:r1] for a in arrays)) for r0, r1 in _chunks(n, parts)]


def map_rows(fn, *arrays, parts: int | None = None):
    """[fn(a[r0:r1], b[r0:r1], ...) for each row chunk], run on the pool."""
    n = arrays[0].shape[0]
    parts = parts or 4 * WORKERS
    futs = [_POOL.submit(fn, *(a[r0:r1] for a in arrays)) for r0, r1 in _chunks(n, parts)]
    return [f.result() for f in futs]


def cast(codes, in_fmt: F.Fmt, out_fmt: F.Fmt, scale: float | None = None):
    """The oracle's scaled cast of a large 2-D array: (codes, amax bits)."""
    res = map_rows(lambda c: OC.cast(c, in_fmt, out_fmt, scale), np.asarray(codes))
    out = np.concatenate([r[0] for r in res]).reshape(np.asarray(codes).shape)
    return out, max(int(r[1]) for r in res)


def amax(codes, in_fmt: F.Fmt) -> int:
    """The oracle's amax (unsigned max of |x| FP32 bit patterns)."""
    res = map_rows(lambda c: int(OC.amax_bits(OC.widen_to_f32_bits(c, in_fmt))),
                   np.asarray(codes))
    return max(res)


def check_full(out_codes, out_fmt: F.Fmt, a, b, alpha: float = 1.0, what=""):
    """Every output of C = alpha * a @ b against the oracle's float64 reference
    within the FP32-accumulation bound (one output ulp after rounding).
    a [M, K], b [K, N] float64."""
    cref, bound = OG.reference(a, b, alpha=alpha)
    if out_fmt is F.F32:
        oks = map_rows(lambda o, c, bd: OG.check_f32(values(o, F.F32), c, bd), out_codes,
                       cref, bound)
    else:
        oks = map_rows(lambda o, c, bd: OG.check_rounded(o, out_fmt, c, bd), out_codes, cref,
                       bound)
    ok = np.concatenate(oks)
    bad = np.argwhere(~ok)
    assert bad.size == 0, (what, bad.shape[0], bad[:5], cref[tuple(bad[0])], bound[tuple(bad[0])])
    return ok.size


def check_entries(out_codes, out_fmt: F.Fmt, a_rows, b_cols, alpha: float = 1.0, what=""):
    """Sampled outputs: out_codes[s] = alpha * sum_k a_rows[s, k] * b_cols[s, k]."""
    a_rows = np.asarray(a_rows, dtype=np.float64)
    b_cols = np.asarray(b_cols, dtype=np.float64)
    ref = [OG.reference(a_rows[s][None, :], b_cols[s][:, None], alpha=alpha)
           for s in range(a_rows.shape[0])]
    cref = np.array([r[0][0, 0] for r in ref])
    bound = np.array([r[1][0, 0] for r in ref])
    if out_fmt is F.F32:
        ok = OG.check_f32(values(out_codes, F.F32), cref, bound)
    else:
        ok = OG.check_rounded(out_codes, out_fmt, cref, bound)
    bad = np.flatnonzero(~ok)
    assert bad.size == 0, (what, bad.size, bad[:5])
    return ok.size
