"""Gradient accumulation, global-norm clipping and the clipped optimizer step
(HIP) against oracle/clip.py and oracle/adamw.py.

Bars: accumulation and the optimizer bit-exact; the float64 sum of squares
within n * 2^-53 of the exact one (its summation order is the kernel's); the
FP32 norm and clip coefficient exact unless the exact value sits within that
bound of an FP32 rounding boundary (then either neighbour is accepted)."""
import math

import numpy as np
import pytest
import torch

import mixed_precision_numerics_amd as amp
from oracle import adamw as OA
from oracle import clip as OC
from oracle import formats as F
import synth
from gpu_util import dev, empty, host, scaler_state

pytestmark = pytest.mark.gpu

GF = {amp.F16: F.F16, amp.BF16: F.BF16, amp.F32: F.F32}


def grads(gt, n, seed, scale):
    x = synth.normal_f32(seed, n, 1.0) * np.float32(scale)
    if gt == amp.F16:
        return synth.to_f16_codes(x)
    if gt == amp.BF16:
        return synth.to_bf16_codes(x)
    return synth.f32_bits(x).copy()


def gpu_norm(bufs, S):
    st = empty(40)
    amp.amp_scaler_init(st, S)
    ns = empty(amp.NORM_STATE_BYTES)
    amp.amp_grad_norm_init(ns)
    for codes, gt in bufs:
        amp.amp_grad_norm_accumulate(dev(codes), gt, codes.size, st, ns)
    out = torch.empty(2, device="cuda")
    amp.amp_clip_coefficient(ns, 1.0, st, out)
    return float(host(ns, np.float64)[0]), host(out, np.float32).copy(), scaler_state(st)


def check_coef(got, sumsq_exact, n, max_norm=1.0):
    """Exact FP32 (coef, norm) unless the exact sum lies within the float64
    summation bound of a point where they change."""
    want = OC.clip_coefficient(sumsq_exact, max_norm)
    lo = OC.clip_coefficient(sumsq_exact * (1 - n * 2.0 ** -52), max_norm)
    hi = OC.clip_coefficient(sumsq_exact * (1 + n * 2.0 ** -52), max_norm)
    ok = {tuple(np.float32(v) for v in w) for w in (want, lo, hi)}
    assert (np.float32(got[0]), np.float32(got[1])) in ok, (got, want)


@pytest.mark.parametrize("gt", [amp.F16, amp.BF16, amp.F32])
@pytest.mark.parametrize("offset", [0, 1])
def test_accumulate_bit_exact(gt, offset):
    n = (1 << 18) + 13
    eb = 4 if gt == amp.F32 else 2
    acc_d = empty(4 * (n + 4))
    acc_p = acc_d.data_ptr() + 4 * offset          # offset 1: not 16-byte aligned
    acc = None
    for k in range(4):
        codes = grads(gt, n + 1, 10 + k, 300.0)
        if k == 2:
            codes[5], codes[9] = ({amp.F16: 0x7C00, amp.BF16: 0x7F80, amp.F32: 0x7F800000}[gt],
                                  {amp.F16: 0x7E00, amp.BF16: 0x7FC0, amp.F32: 0x7FC00000}[gt])
        g_d = dev(codes)
        amp.amp_grad_accumulate(acc_p, g_d.data_ptr() + eb * offset, gt, n, k == 0)
        acc = OC.accumulate(acc, codes[offset:offset + n], GF[gt], k == 0)
    got = host(acc_d, np.float32)[offset:offset + n].astype(np.float64)
    assert np.array_equal(got, acc, equal_nan=True)


@pytest.mark.parametrize("gt,S", [(amp.F16, 1024.0), (amp.BF16, 1.0), (amp.F32, 65536.0)])
def test_norm_and_clip_coefficient(gt, S):
    n1, n2 = (1 << 22) + 3, 777
    a, b = grads(gt, n1, 20, 0.05 * S), grads(gt, n2, 21, 2.0 * S)
    sumsq, out, st = gpu_norm([(a, gt), (b, gt)], S)
    e1, bad1 = OC.norm_sq(a, GF[gt], S)
    e2, bad2 = OC.norm_sq(b, GF[gt], S)
    exact = math.fsum([e1, e2])
    n = n1 + n2
    assert not (bad1 or bad2) and int(st["found_inf"]) == 0
    assert abs(sumsq - exact) <= n * 2.0 ** -53 * exact, (sumsq, exact)
    check_coef(out, exact, n)


def test_norm_sets_found_inf_and_no_clip():
    codes = grads(amp.F16, 100000, 22, 1.0)
    codes[4321] = 0xFC00
    _, out, st = gpu_norm([(codes, amp.F16)], 1.0)
    assert int(st["found_inf"]) == 1
    assert out[0] == 1.0 and np.isinf(out[1])


def test_small_norm_is_not_clipped():
    codes = grads(amp.F16, 4096, 23, 1e-3)
    sumsq, out, _ = gpu_norm([(codes, amp.F16)], 1.0)
    exact, _ = OC.norm_sq(codes, F.F16, 1.0)
    assert out[0] == 1.0
    check_coef(out, exact, 4096)


def test_optimizer_with_clip_multiplier_bit_exact():
    n = (1 << 20) + 5
    hp_o = OA.AdamWHParams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    hp = amp.AdamWHParams(hp_o.lr, hp_o.beta1, hp_o.beta2, hp_o.eps, hp_o.weight_decay)
    theta0 = synth.normal_f32(30, n, 0.02)
    th_d, m_d, v_d = dev(theta0), dev(np.zeros(n, np.float32)), dev(np.zeros(n, np.float32))
    w_d = empty(2 * n)
    st = empty(40)
    amp.amp_scaler_init(st, 512.0)
    th, m, v = theta0.astype(np.float64), np.zeros(n), np.zeros(n)
    ctr = OA.AdamCounters()
    for t, coef in enumerate((0.3712, 1.0, 0.05)):
        codes = grads(amp.F16, n, 40 + t, 512.0 * 0.01)
        c32 = np.float32(coef)
        amp.amp_optimizer_step_ex(th_d, m_d, v_d, dev(codes), amp.F16, w_d, amp.F16, n, hp, st,
                                  d_grad_mult=dev(np.array([c32])))
        th, m, v, w, ok = OA.apply(th, m, v, codes, F.F16, hp_o, ctr, 512.0,
                                   grad_mult=float(c32))
        amp.amp_scaler_update(st)
        assert ok
        assert np.array_equal(host(th_d, np.float32).astype(np.float64), th), t
        assert np.array_equal(host(m_d, np.float32).astype(np.float64), m), t
        assert np.array_equal(host(v_d, np.float32).astype(np.float64), v), t
        assert np.array_equal(host(w_d, np.uint16), w), t


def test_effective_batch_step_with_accumulation_and_clipping():
    """Three effective batches of 4 FP16 micro-batches: accumulate in FP32,
    norm + inf check once, clip, AdamW, scaler update; an inf in one
    micro-batch of the second batch skips that step."""
    n = (1 << 20) + 3
    S = 4096.0
    hp_o = OA.AdamWHParams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    hp = amp.AdamWHParams(hp_o.lr, hp_o.beta1, hp_o.beta2, hp_o.eps, hp_o.weight_decay)
    theta0 = synth.normal_f32(50, n, 0.02)
    th_d, m_d, v_d = dev(theta0), dev(np.zeros(n, np.float32)), dev(np.zeros(n, np.float32))
    acc_d = empty(4 * n)
    st = empty(40)
    ns = empty(amp.NORM_STATE_BYTES)
    coef_d = torch.empty(2, device="cuda")
    amp.amp_scaler_init(st, S)
    th, m, v = theta0.astype(np.float64), np.zeros(n), np.zeros(n)
    ctr = OA.AdamCounters()
    scale = S
    for step in range(3):
        acc = None
        for k in range(4):
            codes = grads(amp.F16, n, 100 + 4 * step + k, scale * 2e-3)
            if step == 1 and k == 2:
                codes[777] = 0x7C00
            amp.amp_grad_accumulate(acc_d, dev(codes), amp.F16, n, k == 0)
            acc = OC.accumulate(acc, codes, F.F16, k == 0)
        acc_bits = synth.f32_bits(acc.astype(np.float32))
        assert np.array_equal(host(acc_d, np.uint32), acc_bits), step
        amp.amp_grad_norm_init(ns)
        amp.amp_grad_norm_accumulate(acc_d, amp.F32, n, st, ns)
        amp.amp_clip_coefficient(ns, 1.0, st, coef_d)
        exact, bad = OC.norm_sq(acc_bits, F.F32, scale)
        want_coef, _ = OC.clip_coefficient(exact, 1.0)
        got = host(coef_d, np.float32).copy()
        assert bool(scaler_state(st)["found_inf"]) == bad, step
        if not bad:
            check_coef(got, exact, n)
            if np.float32(got[0]) != np.float32(want_coef):
                pytest.skip("coefficient on an FP32 rounding boundary: trajectories split")
        amp.amp_optimizer_step_ex(th_d, m_d, v_d, acc_d, amp.F32, None, amp.F16, n, hp, st,
                                  d_grad_mult=coef_d, flags=amp.OPT_SKIP_CHECK)
        th, m, v, _, ok = OA.apply(th, m, v, acc_bits, F.F32, hp_o, ctr, scale, skip=bad,
                                   grad_mult=want_coef)
        amp.amp_scaler_update(st)
        if bad:
            scale *= 0.5
        assert float(scaler_state(st)["scale"]) == scale
        assert ok == (not bad)
        assert np.array_equal(host(th_d, np.float32).astype(np.float64), th), step
        assert np.array_equal(host(m_d, np.float32).astype(np.float64), m), step
        assert np.array_equal(host(v_d, np.float32).astype(np.float64), v), step
