"""Pins for oracle/blockwise.py (fine-grained FP8 scaling and its GEMM) against
what the method fixes: every tile's largest element lands on the format's
maximum, dequantized values lie within half a code step of the input, tiles
are independent of one another, closed-form scales of constant tiles (which
also fix the K-block-major scale layout and the tile orientation), block
scales are orientation-free, and the GEMM equals an exact rational sum."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import blockwise as BW
from oracle import formats as F
from oracle import gemm as G
import synth

FMT_MAX = [(F.E4M3, 448.0), (F.E5M2, 57344.0)]


def _tiles(R, K, block):
    rb_n = -(-R // 128) if block else R
    for rb in range(rb_n):
        rows = slice(rb * 128, min(R, rb * 128 + 128)) if block else slice(rb, rb + 1)
        for kb in range(-(-K // 128)):
            yield rb, kb, rows, slice(kb * 128, min(K, kb * 128 + 128))


@pytest.mark.parametrize("fmt,fmax", FMT_MAX)
@pytest.mark.parametrize("block", [False, True])
@pytest.mark.parametrize("transpose", [False, True])
def test_tile_max_hits_format_max_and_half_step_error(fmt, fmax, block, transpose):
    x = synth.student_t_f32(11, (200, 300), 3.0, 2.0)
    x[3, :] *= 1e3                       # one loud row: other row tiles must not see it
    x[:, 7] *= 1e-3                      # one quiet column
    codes, s = BW.quantize(synth.f32_bits(x), F.F32, fmt, block, transpose)
    op = (x.T if transpose else x).astype(np.float64)
    deq = BW.dequantize(codes, s, fmt, block)
    R, K = op.shape
    half = 2.0 ** -(fmt.mbits + 1)
    sub = fmt.min_subnormal / 2
    for rb, kb, rows, cols in _tiles(R, K, block):
        t, d = op[rows, cols], deq[rows, cols]
        sinv = s[kb, rb]
        i = np.unravel_index(np.argmax(np.abs(t)), t.shape)
        assert abs(d[i]) == fmax * sinv                 # the tile maximum maps to +-fmax
        assert np.all(np.abs(d - t) <= half * np.abs(t) + sub * sinv)


@pytest.mark.parametrize("fmt,fmax", FMT_MAX)
def test_constant_tiles_closed_form_layout(fmt, fmax):
    # row-tile mode: row r, K-block kb holds 2^(r%5 + 2kb); scale_inv is
    # fl32(2^e / fmax) at s[kb, r]; block mode: 2^(rb + 3kb) at s[kb, rb]
    R, K = 260, 384
    e_row = (np.arange(R)[:, None] % 5) + 2 * (np.arange(K)[None, :] // 128)
    x = np.ldexp(1.0, e_row).astype(np.float32)
    x[1::2] *= -1
    codes, s = BW.quantize(synth.f32_bits(x), F.F32, fmt, block=False)
    assert s.shape == (3, R)
    for r in range(R):
        for kb in range(3):
            assert s[kb, r] == F.f32(2.0 ** (r % 5 + 2 * kb) / fmax)
    assert np.array_equal(np.abs(F.decode(codes, fmt)), np.full((R, K), fmax))
    e_blk = (np.arange(R)[:, None] // 128) + 3 * (np.arange(K)[None, :] // 128)
    xb = np.ldexp(1.0, e_blk).astype(np.float32)
    codes, s = BW.quantize(synth.f32_bits(xb), F.F32, fmt, block=True)
    assert s.shape == (3, 3)
    for rb in range(3):
        for kb in range(3):
            assert s[kb, rb] == F.f32(2.0 ** (rb + 3 * kb) / fmax)
    # the same data read as x^T: row tiles of x^T are 128x1 column tiles of x
    # x[k, r] = 2^(r%5 + 2*(k//128)): x^T has the row-tile pattern above
    xt = np.ldexp(1.0, (np.arange(K)[:, None] // 128) * 2 + (np.arange(R)[None, :] % 5)).astype(np.float32)
    codes, s = BW.quantize(synth.f32_bits(xt), F.F32, fmt, block=False, transpose=True)
    assert s.shape == (3, R) and codes.shape == (R, K)
    for r in range(R):
        for kb in range(3):
            assert s[kb, r] == F.f32(2.0 ** (r % 5 + 2 * kb) / fmax)


@pytest.mark.parametrize("block", [False, True])
def test_tiles_are_independent(block):
    x = synth.normal_f32(12, (256, 256), 1.0)
    c0, s0 = BW.quantize(synth.f32_bits(x), F.F32, F.E4M3, block)
    y = x.copy()
    y[0:128, 128:256] *= 2.0 ** 9 if block else 1.0
    if not block:
        y[5, 128:256] *= 2.0 ** 9
    c1, s1 = BW.quantize(synth.f32_bits(y), F.F32, F.E4M3, block)
    assert np.array_equal(c0, c1)
    changed = (1, 0) if block else (1, 5)
    ratio = s1 / s0
    assert ratio[changed] == 2.0 ** 9
    ratio[changed] = 1.0
    assert np.all(ratio == 1.0)


def test_block_scales_are_orientation_free():
    x = synth.student_t_f32(13, (300, 200), 3.0)
    c, s = BW.quantize(synth.f32_bits(x), F.F32, F.E4M3, block=True)
    ct, st = BW.quantize(synth.f32_bits(x), F.F32, F.E4M3, block=True, transpose=True)
    assert np.array_equal(ct, c.T) and np.array_equal(st, s.T)


def test_zero_and_non_finite_tiles():
    x = np.ones((3, 256), dtype=np.float32)
    x[0, :128] = 0.0
    x[1, 5] = np.inf
    x[2, 200] = np.nan
    c, s = BW.quantize(synth.f32_bits(x), F.F32, F.E4M3, block=False)
    inv448 = F.f32(1.0 / 448.0)
    # zero tile: scale 1, codes 0; a tile of ones: scale 448
    assert s[0, 0] == 1.0 and not c[0, :128].any()
    assert s[1, 0] == inv448 and s[0, 2] == inv448 and s[1, 1] == inv448
    # inf tile: scale 1, inf saturates to 448, the other elements unscaled
    assert s[0, 1] == 1.0
    assert F.decode(c[1, 5:7], F.E4M3).tolist() == [448.0, 1.0]
    # NaN tile: scale 1, NaN code 0x7F
    assert s[1, 2] == 1.0 and c[2, 200] == 0x7F and F.decode(c[2, 201:202], F.E4M3)[0] == 1.0
    # BF16 input and E5M2 output: inf saturates to 57344
    c5, _ = BW.quantize(synth.to_bf16_codes(x), F.BF16, F.E5M2, block=False)
    assert F.decode(c5[1, 5:6], F.E5M2)[0] == 57344.0


def test_dequantize_index_map():
    R, K = 260, 300
    one = int(F.encode(np.array([1.0]), F.E4M3)[0])
    codes = np.full((R, K), one, dtype=np.uint8)
    s_row = np.ldexp(1.0, np.arange(3)[:, None] * 10 + (np.arange(R)[None, :] % 7))
    d = BW.dequantize(codes, s_row, F.E4M3, block=False)
    exp = np.ldexp(1.0, (np.arange(K)[None, :] // 128) * 10 + (np.arange(R)[:, None] % 7))
    assert np.array_equal(d, exp)
    s_blk = np.ldexp(1.0, np.arange(3)[:, None] * 10 + np.arange(3)[None, :])
    d = BW.dequantize(codes, s_blk, F.E4M3, block=True)
    exp = np.ldexp(1.0, (np.arange(K)[None, :] // 128) * 10 + (np.arange(R)[:, None] // 128))
    assert np.array_equal(d, exp)


@pytest.mark.parametrize("b_block", [False, True])
def test_gemm_equals_exact_rational_sum(b_block):
    M, N, K = 5, 130, 260
    a = synth.student_t_f32(14, (M, K), 3.0)
    b = synth.normal_f32(15, (N, K), 0.02)
    ca, sa = BW.quantize(synth.f32_bits(a), F.F32, F.E5M2, block=False)
    cb, sb = BW.quantize(synth.f32_bits(b), F.F32, F.E4M3, block=b_block)
    c, mag = BW.gemm(ca, sa, F.E5M2, False, cb, sb, F.E4M3, b_block)
    va, vb = F.decode(ca, F.E5M2), F.decode(cb, F.E4M3)
    for m in range(M):
        for n in range(0, N, 13):
            tot = Fraction(0)
            for k in range(K):
                fa = Fraction(float(va[m, k])) * Fraction(float(sa[k // 128, m]))
                fb = Fraction(float(vb[n, k])) * Fraction(float(sb[k // 128, n // 128 if b_block else n]))
                tot += fa * fb
            assert abs(float(tot) - c[m, n]) <= 2.0 ** -48 * mag[m, n]


def test_gemm_unit_scales_reduce_to_plain_fp8_gemm():
    M, N, K = 7, 9, 384
    rng = np.random.default_rng(3)
    ca = rng.integers(0, 256, (M, K)).astype(np.uint8)
    cb = rng.integers(0, 256, (N, K)).astype(np.uint8)
    ca[(ca & 0x7F) == 0x7F] = 0x10            # no NaN codes
    cb[(cb & 0x7F) == 0x7F] = 0x11
    ones_a, ones_b = np.ones((3, M)), np.ones((3, 1))
    c, _ = BW.gemm(ca, ones_a, F.E4M3, False, cb, ones_b, F.E4M3, True)
    ref, _ = G.reference(F.decode(ca, F.E4M3), F.decode(cb, F.E4M3).T)
    assert np.array_equal(c, ref)
