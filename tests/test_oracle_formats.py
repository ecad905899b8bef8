"""Pins for the oracle's number formats (no GPU).

Each format is checked against what the pages print (golden constants), an
independent library conversion (NumPy FP32, PyTorch CPU FP16/BF16/FP8) over a
structured sweep of FP32 inputs, and brute force (E2M1, where no library cast
exists)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def test_page_constants_fp16():
    assert F.F16.max_finite == GOLD["fp16_max"]["value"]
    assert F.F16.min_normal == 2.0 ** GOLD["fp16_min_normal_log2"]["value"]
    assert F.F16.min_subnormal == 2.0 ** GOLD["fp16_subnormal_floor_log2"]["value"]
    assert [1, F.F16.ebits, F.F16.mbits] == GOLD["fp16_bits"]["value"]
    assert [1, F.BF16.ebits, F.BF16.mbits] == GOLD["bf16_bits"]["value"]
    assert [1, F.F32.ebits, F.F32.mbits] == GOLD["fp32_bits"]["value"]
    # just below the floor underflows to zero, the floor itself survives
    assert F.round_to(2.0 ** -24, F.F16) == 2.0 ** -24
    assert F.round_to(2.0 ** -26, F.F16) == 0.0
    assert F.round_to(70000.0, F.F16) == np.inf


def test_page_constants_fp8():
    assert F.E4M3.max_finite == GOLD["e4m3_range"]["value"]
    assert [1, F.E4M3.ebits, F.E4M3.mbits] == GOLD["e4m3_bits"]["value"]
    assert [1, F.E5M2.ebits, F.E5M2.mbits] == GOLD["e5m2_bits"]["value"]
    # clip(x, -448, 448): everything beyond the range saturates
    assert F.round_to(1e6, F.E4M3) == 448.0
    assert F.round_to(-np.inf, F.E4M3) == -448.0
    assert F.round_to(1e9, F.E5M2) == 57344.0


@pytest.mark.parametrize("fmt", [F.F16, F.BF16, F.E4M3, F.E5M2, F.E2M1])
def test_all_codes_roundtrip(fmt):
    codes = np.arange(1 << fmt.nbits, dtype=np.uint32)
    vals = F.decode(codes, fmt)
    finite = np.isfinite(vals)
    back = F.encode_exact(vals[finite], fmt).astype(np.uint32)
    assert np.array_equal(back, codes[finite])
    # decode is strictly monotone over the positive finite codes
    pos = vals[finite & (codes < (1 << (fmt.nbits - 1)))]
    assert np.all(np.diff(pos) > 0)


def _structured_f32(low_patterns, low_bits, seed=0):
    """All sign/exponent/top-mantissa combinations with chosen low bits."""
    top = np.arange(1 << (32 - low_bits), dtype=np.uint64) << np.uint64(low_bits)
    rnd = np.random.default_rng(seed).integers(0, 1 << low_bits, size=top.size, dtype=np.uint64)
    parts = [top | np.uint64(p) for p in low_patterns] + [top | rnd]
    return np.concatenate(parts).astype(np.uint32).view(np.float32)


def test_f32_rounding_vs_numpy():
    x = np.random.default_rng(1).standard_normal(200000) * np.exp(
        np.random.default_rng(2).uniform(-100, 100, 200000))
    x = np.concatenate([x, [1e-310, -1e-320, 3.5e38, 3.4028235677973366e38,
                            3.4028235677973362e38, np.inf, -np.inf]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).astype(np.float64)
    assert np.array_equal(F.f32(x), ref)


def test_f16_vs_torch_structured():
    x = _structured_f32([0, 1, 0xFFF, 0x1000, 0x1001, 0x1FFF], 13)
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x).half().float().numpy().astype(np.float64)
    assert np.array_equal(F.round_to(x.astype(np.float64), F.F16), ref)


def test_bf16_vs_torch_structured():
    x = _structured_f32([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], 16)
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x).bfloat16().float().numpy().astype(np.float64)
    assert np.array_equal(F.round_to(x.astype(np.float64), F.BF16), ref)


@pytest.mark.parametrize("fmt,tdt,lim", [(F.E4M3, torch.float8_e4m3fn, 464.0),
                                         (F.E5M2, torch.float8_e5m2, 61440.0)])
def test_fp8_vs_torch_in_non_saturating_range(fmt, tdt, lim):
    x = _structured_f32([0, 1, 0xFFFFF, 0x100000, 0x100001], 20)
    x = x[np.isfinite(x) & (np.abs(x) < lim)]
    ref = torch.from_numpy(x).to(tdt).float().numpy().astype(np.float64)
    assert np.array_equal(F.round_to(x.astype(np.float64), fmt), ref)


def test_nan_and_inf_encodings():
    assert int(F.encode(np.nan, F.F16)) == 0x7E00
    assert int(F.encode(np.nan, F.BF16)) == 0x7FC0
    assert int(F.encode(np.nan, F.E4M3)) == 0x7F
    assert int(F.encode(np.nan, F.E5M2)) == 0x7F
    assert int(F.encode(np.inf, F.F16)) == 0x7C00
    assert int(F.encode(-np.inf, F.BF16)) == 0xFF80
    assert int(F.encode(np.inf, F.E4M3)) == 0x7E
    assert int(F.encode(-np.inf, F.E5M2)) == 0xFB
    assert int(F.encode(-0.0, F.F16)) == 0x8000
    assert int(F.encode(-1e-30, F.E4M3)) == 0x80   # negative underflow keeps the sign


def _brute_nearest_even(x, fmt):
    codes = np.arange(1 << fmt.nbits)
    vals = F.decode(codes, fmt)
    keep = np.isfinite(vals)
    codes, vals = codes[keep], vals[keep]
    fx = Fraction(float(x))
    best = None
    for c, v in zip(codes, vals):
        d = abs(Fraction(float(v)) - fx)
        key = (d, int(c) & 1)        # ties: prefer the even code
        if best is None or key < best[0]:
            best = (key, float(v))
    return best[1]


def test_e2m1_brute_force():
    xs = np.concatenate([np.linspace(-7.0, 7.0, 561), np.arange(-8, 8.25, 0.25)])
    xs = F.f32(xs)
    got = F.round_to(xs, F.E2M1)
    want = np.array([_brute_nearest_even(min(max(x, -6.0), 6.0), F.E2M1) for x in xs])
    assert np.array_equal(np.abs(got), np.abs(want))
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for k, v in ties.items():
        assert F.round_to(k, F.E2M1) == v


def test_e4m3_brute_force_small():
    xs = F.f32(np.random.default_rng(3).standard_normal(400) * 20.0)
    got = F.round_to(xs, F.E4M3)
    want = np.array([_brute_nearest_even(min(max(x, -448.0), 448.0), F.E4M3) for x in xs])
    assert np.array_equal(got, want)


def test_master_weight_necessity():
    """An FP16 update below ~2^-11 of the weight vanishes in an FP16 add, while
    an FP32 master keeps it (itwiki, table in 왜 그냥 FP16으로는 안 되는가;
    marovi, La receta: spacing 2^-10 near 1)."""
    r16 = lambda v: float(F.round_to(v, F.F16))
    r32 = lambda v: float(F.f32(v))
    u = 2.0 ** -12
    w16 = 1.0
    for _ in range(3):
        w16 = r16(w16 + u)
    assert w16 == 1.0                        # pure FP16: all three updates lost
    w32 = 1.0
    seen = []
    for _ in range(3):
        w32 = r32(w32 + u)
        seen.append(r16(w32))
    assert seen == [1.0, 1.0, 1.0 + 2.0 ** -10]   # tie-to-even at 2 updates
    assert r16(1.0 - 2.0 ** -12) == 1.0           # tie below 1 vanishes too
    assert r16(1.0 - 2.0 ** -11) == 1.0 - 2.0 ** -11
    assert r16(1.0 + 2.0 ** GOLD["fp16_spacing_near_one_log2"]["value"]) != 1.0
    ratio = 2.0 ** GOLD["fp16_update_vanish_ratio_log2"]["value"]
    for w in (1.0, 3.0, 1000.0):
        wq = r16(w)
        assert r16(wq + 0.49 * ratio * wq) == wq or r16(wq + 0.99 * ratio * wq) == wq


def test_ulp_distance():
    a = F.encode([1.0, -1.0, 0.0], F.BF16)
    b = F.encode([1.0078125, -1.0, -0.0], F.BF16)
    assert list(F.ulp_distance(a, b, F.BF16)) == [1, 0, 0]
