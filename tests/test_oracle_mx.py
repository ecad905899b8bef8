"""Pins for oracle/mx.py (MX block formats) against the format's definition:
power-of-two block scales placing the block maximum in the element format's
top binade, exact round trips, nearest-even with saturation, and exact GEMM
sums of the dequantized operands."""
from fractions import Fraction
import math

import numpy as np
import pytest

from oracle import formats as F
from oracle import gemm as G
from oracle import mx
import synth

FMTS = [(F.E4M3, 8, 448.0), (F.E5M2, 15, 57344.0), (F.E2M1, 2, 6.0)]


@pytest.mark.parametrize("fmt,emax,fmax", FMTS)
def test_scale_puts_block_max_in_top_binade(fmt, emax, fmax):
    x = synth.student_t_f32(3, (64, 256), scale=5.0).astype(np.float64)
    x[5, :32] *= 2.0 ** -60            # a block of tiny values
    x[6, 32:64] *= 2.0 ** 60           # and of huge ones
    codes, sc = mx.quantize(x, fmt)
    blocks = np.abs(x).reshape(64, 8, 32).max(axis=2)
    X = np.ldexp(1.0, sc.astype(np.int64) - 127)
    r = blocks / X
    assert np.all((r >= 2.0 ** emax) & (r < 2.0 ** (emax + 1)))
    deq = mx.dequantize(codes, sc, fmt)
    assert np.all(np.abs(deq) <= fmax * np.repeat(X, 32, axis=1))


@pytest.mark.parametrize("fmt,emax,fmax", FMTS)
def test_round_trip_of_representable_blocks(fmt, emax, fmax):
    rng = np.random.default_rng(1)
    grid = np.unique(np.abs(F.decode(np.arange(1 << fmt.nbits), fmt)))
    grid = grid[np.isfinite(grid)]
    for t in range(20):
        e = int(rng.integers(-100, 100))
        v = rng.choice(grid, size=32) * rng.choice([-1.0, 1.0], size=32)
        v[0] = fmax                         # the block maximum sets the scale
        X = 2.0 ** e
        x = (v * X)[None, :]
        codes, sc = mx.quantize(x, fmt)
        # amax = fmax * 2^e lies in [2^emax, 2^(emax+1)) * 2^e
        assert sc[0, 0] == e + 127
        assert np.array_equal(mx.dequantize(codes, sc, fmt), x)


@pytest.mark.parametrize("fmt,emax,fmax", FMTS)
def test_elements_nearest_even_with_saturation(fmt, emax, fmax):
    x = synth.normal_f32(4, (16, 64), 1.0).astype(np.float64)
    codes, sc = mx.quantize(x, fmt)
    X = np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=1)
    grid = F.decode(np.arange(1 << fmt.nbits), fmt)
    grid = np.unique(grid[np.isfinite(grid)])
    for i in range(16):
        for k in range(64):
            t = x[i, k] / X[i, k]
            got = F.decode(np.array([codes[i, k]]), fmt)[0]
            if abs(t) >= fmax:
                assert got == math.copysign(fmax, t)
                continue
            d = np.abs(grid - t)
            best = grid[d == d.min()]
            if best.size == 1:
                assert got == best[0]
            else:                           # a tie: the even code
                cands = [int(F.encode(np.array([b]), fmt)[0]) for b in best]
                assert int(codes[i, k]) in cands and int(codes[i, k]) % 2 == 0


def test_zero_and_non_finite_blocks():
    x = np.zeros((3, 32))
    x[1, 7] = np.inf
    x[2, 3] = np.nan
    x[2, 4] = 1.0
    for fmt in (F.E4M3, F.E2M1):
        codes, sc = mx.quantize(x, fmt)
        assert sc[0, 0] == 0 and not codes[0].any()
        assert sc[1, 0] == mx.SCALE_NAN and sc[2, 0] == mx.SCALE_NAN


def test_transpose_and_packing():
    x = synth.normal_f32(5, (64, 96), 1.0).astype(np.float64)
    c1, s1 = mx.quantize(x, F.E2M1, transpose=True)
    c2, s2 = mx.quantize(x.T.copy(), F.E2M1)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    p = mx.pack_e2m1(np.array([[1, 2, 3, 4]], np.uint8))
    assert p.tolist() == [[0x21, 0x43]]


def test_gemm_reference_exact_on_mx_operands():
    """Sums of products of dequantized MX values: the float64 reference equals
    the Fraction-exact sum within its stated error bound."""
    a = synth.normal_f32(6, (4, 64), 1.0).astype(np.float64)
    b = synth.normal_f32(7, (5, 64), 1.0).astype(np.float64)
    ca, sa = mx.quantize(a, F.E2M1)
    cb, sb = mx.quantize(b, F.E4M3)
    A = mx.dequantize(ca, sa, F.E2M1)
    B = mx.dequantize(cb, sb, F.E4M3)
    c, bound = G.reference(A, B.T)
    ex = G.exact(A, B.T)
    for i in range(4):
        for j in range(5):
            assert abs(Fraction(c[i, j]) - ex[i][j]) <= Fraction(bound[i, j]) * Fraction(1, 2 ** 40)
