"""Pins for the oracle's optimizer step and GEMM reference."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import adamw as A
from oracle import formats as F
from oracle import gemm as G
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def test_memory_contract_16_bytes_per_param():
    d_in, d_h, d_out = GOLD["mlp_shapes"]["value"]
    n = d_in * d_h + d_h + d_h * d_out + d_out
    assert n == 1_071_114
    per = GOLD["bytes_per_param_adam"]
    # 16-bit weight + 16-bit grad + FP32 master, m, v
    layout = {"w16": 2, "g16": 2, "master": 4, "m": 4, "v": 4}
    assert sum(layout.values()) == per["value"] == sum(per["parts"])
    assert n * per["value"] == 17_137_824
    assert (1 << 31) * per["value"] == 34_359_738_368


def test_unscale_is_exact_for_power_of_two_scales():
    codes = synth.to_f16_codes(synth.normal_f32(1, 20000, std=100.0))
    g16 = F.decode(codes, F.F16)
    for k in (0, 5, 16, 24, -3):
        S = 2.0 ** k
        g = F.f32(g16 * float(F.f32(1.0 / S)))
        assert np.array_equal(g * S, g16)


def test_overflow_detection():
    codes = synth.to_f16_codes(np.array([1.0, 2.0, 65504.0], np.float32))
    assert not A.found_inf(codes, F.F16)
    for bad in (np.inf, -np.inf, np.nan):
        c = synth.to_f16_codes(np.array([1.0, bad], np.float32))
        assert A.found_inf(c, F.F16)
    c = synth.to_bf16_codes(np.array([3e38, np.nan], np.float32))
    assert A.found_inf(c, F.BF16)


def test_nonfinite_mask_over_every_16bit_code():
    """The per-code test flags exactly the codes NumPy / PyTorch read as inf
    or NaN (FP16 through NumPy's float16, BF16 through PyTorch's bfloat16),
    in any integer width the codes arrive in."""
    import torch
    c = np.arange(1 << 16, dtype=np.uint16)
    f16 = ~np.isfinite(c.view(np.float16).astype(np.float64))
    bf = ~torch.isfinite(torch.from_numpy(c.view(np.int16)).view(torch.bfloat16).float()).numpy()
    for codes in (c, c.view(np.int16), c.astype(np.int64)):
        assert np.array_equal(A.nonfinite_16(codes, F.F16), f16)
        assert np.array_equal(A.nonfinite_16(codes, F.BF16), bf)
    assert f16.sum() == 2 * 1024 and bf.sum() == 2 * 128


def test_first_step_closed_form():
    hp = A.AdamWHParams(lr=1e-3, weight_decay=0.0, eps=0.0)
    ctr = A.AdamCounters()
    g = np.array([0.5, -2.0, 1e-3, 3.0], np.float32)
    theta = np.array([1.0, -1.0, 0.25, 0.0])
    codes = synth.to_f16_codes(g)
    gq = F.decode(codes, F.F16)
    th, m, v, w, ok = A.apply(theta, np.zeros(4), np.zeros(4), codes, F.F16, hp, ctr, 1.0)
    assert ok and ctr.step == 1
    c1 = float(F.f32(0.1)); c2 = float(F.f32(1 - 0.999))
    assert np.array_equal(m, F.f32(c1 * gq))
    assert np.array_equal(v, F.f32(c2 * F.f32(gq ** 2)))
    # with zero eps and wd the first step is theta - lr * sign(g), up to FP32 rounding
    err = np.abs(th - (theta - 1e-3 * np.sign(g)))
    assert np.all(err <= 4e-7 * (1 + np.abs(theta))), err
    assert np.array_equal(w, F.encode(th, F.F16))


def test_skip_leaves_state_bit_identical():
    hp = A.AdamWHParams()
    ctr = A.AdamCounters(step=3, beta1_pow=0.9 ** 3, beta2_pow=0.999 ** 3)
    theta = synth.normal_f32(2, 16, 0.02).astype(np.float64)
    m = synth.normal_f32(3, 16, 1e-3).astype(np.float64)
    v = np.abs(synth.normal_f32(4, 16, 1e-6)).astype(np.float64)
    g = synth.normal_f32(5, 16).copy()
    g[7] = np.nan
    th1, m1, v1, _, ok = A.apply(theta, m, v, synth.to_f16_codes(g), F.F16, hp, ctr, 1024.0)
    assert not ok and ctr.step == 3
    assert np.array_equal(th1, theta) and np.array_equal(m1, m) and np.array_equal(v1, v)


def test_multi_step_vs_torch_adamw():
    """Library cross-check: torch.optim.AdamW (FP32, different op order)."""
    n = 4096
    hp = A.AdamWHParams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    theta0 = synth.normal_f32(11, n, 0.02)
    p = torch.nn.Parameter(torch.from_numpy(theta0.copy()))
    opt = torch.optim.AdamW([p], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps,
                            weight_decay=hp.weight_decay, foreach=False)
    th = theta0.astype(np.float64); m = np.zeros(n); v = np.zeros(n)
    ctr = A.AdamCounters()
    for t in range(12):
        g = synth.normal_f32(100 + t, n, 1e-3)
        codes = synth.to_f16_codes(g * 1024.0)
        th, m, v, _, ok = A.apply(th, m, v, codes, F.F16, hp, ctr, 1024.0)
        p.grad = torch.from_numpy((F.decode(codes, F.F16) / 1024.0).astype(np.float32))
        opt.step()
    ref = p.detach().numpy().astype(np.float64)
    # ulps measured at the larger of |theta| and the step size lr (an element
    # that crosses zero has a tiny spacing unrelated to the update's rounding)
    unit = np.spacing(np.maximum(np.abs(ref), hp.lr).astype(np.float32)).astype(np.float64)
    ulps = np.abs(th - ref) / unit
    # a dropped or wrong term (bias correction, decay, eps) would be ~2^20 ulps
    assert ulps.max() <= 64, ulps.max()
    assert np.quantile(ulps, 0.99) <= 4
    assert np.mean(ulps == 0) > 0.5


def test_gemm_reference_vs_exact_brute_force():
    rng = np.random.default_rng(0)
    for fmt in (F.E4M3, F.E5M2, F.BF16, F.F16):
        M, N, K = 5, 7, 32
        a = F.decode(rng.integers(0, 1 << fmt.nbits, (M, K)), fmt)
        b = F.decode(rng.integers(0, 1 << fmt.nbits, (K, N)), fmt)
        a = np.where(np.isfinite(a), a, 1.0); b = np.where(np.isfinite(b), b, -2.0)
        c, bound = G.reference(a, b)
        ex = G.exact(a, b)
        for i in range(M):
            for j in range(N):
                assert abs(float(ex[i][j]) - c[i, j]) <= 2.0 ** -50 * bound[i, j] + 1e-300


def test_gemm_power_of_two_scale_invariance_and_transpose():
    rng = np.random.default_rng(1)
    a = F.round_to(rng.standard_normal((9, 16)), F.BF16)
    b = F.round_to(rng.standard_normal((16, 11)), F.BF16)
    c, _ = G.reference(a, b)
    c2, _ = G.reference(a * 8.0, b * 0.25, alpha=0.5)
    assert np.array_equal(c, c2)
    ct, _ = G.reference(b.T, a.T)
    assert np.array_equal(ct.T, c)


def test_gemm_checks():
    c_ref = np.array([[1.0, -2.0, 1e-3]])
    bound = np.array([[10.0, 10.0, 100.0]])
    assert G.check_f32(c_ref + 9e-5, c_ref, bound).all()
    assert not G.check_f32(c_ref + 2e-4, c_ref, bound)[0, 0]
    out = F.encode(c_ref, F.BF16)
    assert G.check_rounded(out, F.BF16, c_ref, bound).all()
    wrong = F.encode(c_ref * 1.05, F.BF16)
    assert not G.check_rounded(wrong, F.BF16, c_ref, bound)[0, :2].any()
