"""Parity of the fused optimizer step, the loss scaler and the delayed-scaling
recipe (HIP) with the oracle."""
import numpy as np
import pytest
import torch

import mixed_precision_numerics_amd as amp
from oracle import adamw as OA
from oracle import formats as F
from oracle import recipe as OR
from oracle import scaler as OS
import synth
from gpu_util import dev, empty, f32_dev, host, metas, scaler_state

pytestmark = pytest.mark.gpu

GFMT = {amp.F16: (F.F16, np.uint16), amp.BF16: (F.BF16, np.uint16), amp.F32: (F.F32, np.uint32)}


def _grads(gt, n, seed, S):
    g = synth.normal_f32(seed, n, 1e-4) * np.exp(2.0 * synth.normal_f32(seed + 1, n)).astype(np.float32)
    g = (g * np.float32(S)).astype(np.float32)
    if gt == amp.F16:
        return synth.to_f16_codes(np.clip(g, -65504, 65504))
    if gt == amp.BF16:
        return synth.to_bf16_codes(g)
    return synth.f32_bits(g).copy()


@pytest.mark.parametrize("gt,wt", [(amp.F16, amp.F16), (amp.BF16, amp.BF16), (amp.F32, amp.F16)])
def test_adamw_steps_bit_exact_with_skip(gt, wt):
    n = (1 << 20) + 5
    hp_o = OA.AdamWHParams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    hp = amp.AdamWHParams(hp_o.lr, hp_o.beta1, hp_o.beta2, hp_o.eps, hp_o.weight_decay)
    theta0 = synth.normal_f32(1, n, 0.02)
    th_d = dev(theta0); m_d = dev(np.zeros(n, np.float32)); v_d = dev(np.zeros(n, np.float32))
    w_d = empty(2 * n)
    st_d = empty(40)
    amp.amp_scaler_init(st_d, 1024.0)
    th = theta0.astype(np.float64); m = np.zeros(n); v = np.zeros(n)
    ctr = OA.AdamCounters()
    sst = OS.ScalerState(scale=1024.0)
    gfmt, gdt = GFMT[gt]
    wfmt = F.F16 if wt == amp.F16 else F.BF16
    for t in range(5):
        S = sst.scale
        codes = _grads(gt, n, 100 + t, S)
        if t == 2:
            codes = codes.copy()
            codes[n // 3] = {amp.F16: 0x7E00, amp.BF16: 0x7FC0, amp.F32: 0x7FC00000}[gt]
        g_d = dev(codes)
        amp.amp_optimizer_step(th_d, m_d, v_d, g_d, gt, w_d, wt, n, hp, st_d)
        st = scaler_state(st_d)
        th, m, v, w, applied = OA.apply(th, m, v, codes, gfmt, hp_o, ctr, S, w_fmt=wfmt)
        assert bool(st["found_inf"]) == (not applied)
        amp.amp_scaler_update(st_d, amp.ScalerParams(2.0, 0.5, 3))
        OS.update(sst, not applied, 2.0, 0.5, 3)
        st = scaler_state(st_d)
        assert st["scale"] == sst.scale and st["growth_tracker"] == sst.growth_tracker
        assert st["found_inf"] == 0 and st["adam_step"] == ctr.step
        assert st["beta1_pow"] == ctr.beta1_pow and st["beta2_pow"] == ctr.beta2_pow
        gth = host(th_d, np.float32).astype(np.float64)
        assert np.array_equal(gth, th), (t, np.nonzero(gth != th)[0][:5])
        assert np.array_equal(host(m_d, np.float32).astype(np.float64), m)
        assert np.array_equal(host(v_d, np.float32).astype(np.float64), v)
        if applied:
            assert np.array_equal(host(w_d, np.uint16), w)


@pytest.mark.parametrize("n", [1, 3, 4, 7, 4096, 4096 * 3 + 6])
def test_adamw_sizes_at_range_edges(n):
    """Vector path below one 4-parameter unit (the trailing loop only), one
    work-group range exactly, and several ranges with a ragged end."""
    hp_o = OA.AdamWHParams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    hp = amp.AdamWHParams(hp_o.lr, hp_o.beta1, hp_o.beta2, hp_o.eps, hp_o.weight_decay)
    theta0 = synth.normal_f32(7, n, 0.02)
    m0 = synth.normal_f32(8, n, 1e-3)
    v0 = np.abs(synth.normal_f32(9, n, 1e-6)).astype(np.float32)
    th_d, m_d, v_d = dev(theta0), dev(m0), dev(v0)
    w_d = empty(2 * n)
    st_d = empty(40)
    amp.amp_scaler_init(st_d, 256.0)
    codes = _grads(amp.BF16, n, 11, 256.0)
    amp.amp_optimizer_step(th_d, m_d, v_d, dev(codes), amp.BF16, w_d, amp.BF16, n, hp, st_d)
    th, m, v, w, applied = OA.apply(theta0.astype(np.float64), m0.astype(np.float64),
                                    v0.astype(np.float64), codes, F.BF16, hp_o, OA.AdamCounters(),
                                    256.0, w_fmt=F.BF16)
    assert applied
    assert np.array_equal(host(th_d, np.float32).astype(np.float64), th)
    assert np.array_equal(host(m_d, np.float32).astype(np.float64), m)
    assert np.array_equal(host(v_d, np.float32).astype(np.float64), v)
    assert np.array_equal(host(w_d, np.uint16)[:n], w)


def test_skip_check_flag_and_external_overflow():
    n = 4096
    hp = amp.AdamWHParams(1e-3, 0.9, 0.999, 1e-8, 0.01)
    th_d = dev(synth.normal_f32(2, n)); m_d = dev(np.zeros(n, np.float32))
    v_d = dev(np.zeros(n, np.float32)); w_d = empty(2 * n)
    st_d = empty(40)
    amp.amp_scaler_init(st_d, 65536.0)
    good = _grads(amp.F16, n, 5, 65536.0)
    bad = good.copy(); bad[7] = 0x7C00
    # overflow seen in another gradient buffer: skip applies to the whole step
    amp.amp_check_overflow(dev(bad), amp.F16, n, st_d)
    before = host(th_d, np.float32).copy()
    amp.amp_optimizer_step(th_d, m_d, v_d, dev(good), amp.F16, w_d, amp.F16, n, hp, st_d,
                           flags=amp.OPT_SKIP_CHECK)
    assert np.array_equal(host(th_d, np.float32), before)
    assert scaler_state(st_d)["adam_step"] == 0
    amp.amp_scaler_update(st_d)
    assert scaler_state(st_d)["scale"] == 32768.0


def test_unaligned_buffers_match_aligned():
    n = 1000
    hp = amp.AdamWHParams(1e-3, 0.9, 0.999, 1e-8, 0.01)
    theta = synth.normal_f32(3, n + 1)
    codes = _grads(amp.F16, n + 1, 9, 1.0)
    outs = []
    for off in (0, 1):
        th_d = dev(theta); m_d = dev(np.zeros(n + 1, np.float32)); v_d = dev(np.zeros(n + 1, np.float32))
        g_d = dev(codes); w_d = empty(2 * (n + 1)); st_d = empty(40)
        amp.amp_scaler_init(st_d, 1.0)
        amp.amp_optimizer_step(th_d.data_ptr() + 4 * off, m_d.data_ptr() + 4 * off,
                               v_d.data_ptr() + 4 * off, g_d.data_ptr() + 2 * off, amp.F16,
                               w_d.data_ptr() + 2 * off, amp.F16, n, hp, st_d)
        outs.append(host(th_d, np.float32)[off:off + n].copy())
    ctr = OA.AdamCounters()
    th, *_ = OA.apply(theta[1:].astype(np.float64), np.zeros(n), np.zeros(n), codes[1:], F.F16,
                      OA.AdamWHParams(), ctr, 1.0)
    assert np.array_equal(outs[1].astype(np.float64), th)


def test_scaler_long_sequence():
    st_d = empty(40)
    amp.amp_scaler_init(st_d, 65536.0)
    rng = np.random.default_rng(4)
    flags = rng.random(300) < 0.05
    o = OS.ScalerState()
    n = 16
    g_ok = dev(np.zeros(n, np.uint16))
    g_bad = dev(np.full(n, 0x7C00, np.uint16))
    for f in flags:
        amp.amp_check_overflow(g_bad if f else g_ok, amp.F16, n, st_d)
        amp.amp_scaler_update(st_d, amp.ScalerParams(2.0, 0.5, 7))
        OS.update(o, bool(f), 2.0, 0.5, 7)
    st = scaler_state(st_d)
    assert st["scale"] == o.scale and st["growth_tracker"] == o.growth_tracker


@pytest.mark.parametrize("algo", [amp.AMAX_MAX, amp.AMAX_MOST_RECENT])
@pytest.mark.parametrize("hist_len", [16, 1024])
def test_delayed_scaling_update(algo, hist_len):
    nm = 3
    md = empty(16 * nm)
    hd = empty(4 * nm * hist_len)
    amp.amp_fp8_meta_init(md, hd, nm, hist_len)
    om = [OR.FP8Meta(history_len=hist_len) for _ in range(nm)]
    rng = np.random.default_rng(hist_len + algo)
    recipe = amp.DelayedRecipe(448.0, 1.0, hist_len, algo)
    algo_s = "max" if algo == amp.AMAX_MAX else "most_recent"
    for step in range(40):
        vals = np.exp(rng.normal(0, 3, nm)).astype(np.float32)
        if step == 5:
            vals[1] = np.inf
        if step == 9:
            vals[2] = 0.0
        # max-accumulate through a cast of a small tensor whose amax is vals[i]
        for i in range(nm):
            x = np.array([vals[i] * 0.5, -vals[i]], np.float32)
            amp.amp_cast(dev(x), amp.F32, 1, 2, 2, empty(2), amp.E4M3, 2,
                         d_scale=md.data_ptr() + 16 * i + 4, d_amax=md.data_ptr() + 16 * i)
            om[i].record(int(synth.f32_bits(np.array([abs(vals[i])], np.float32))[0]))
        amp.amp_delayed_scaling_update(md, hd, nm, recipe)
        for i in range(nm):
            OR.update(om[i], 448.0, 1.0, algo_s)
        got = metas(md, nm)
        for i in range(nm):
            assert got[i]["scale"] == np.float32(om[i].scale), (step, i)
            assert got[i]["scale_inv"] == np.float32(om[i].scale_inv)
            assert got[i]["pos"] == om[i].pos and got[i]["amax_cur"] == 0.0
    hist = host(hd, np.uint32).reshape(nm, hist_len)
    for i in range(nm):
        assert np.array_equal(hist[i], om[i].history_bits)


@pytest.mark.parametrize("yt", [amp.F16, amp.BF16, amp.E4M3])
@pytest.mark.parametrize("scale", [None, 0.5, 2.0])
def test_found_inf_from_amax_matches_the_cast_outputs(yt, scale):
    """amp_found_inf_from_amax on the amax values amp_cast recorded equals the
    oracle's check of the oracle's cast outputs of the same inputs."""
    yf = {amp.F16: F.F16, amp.BF16: F.BF16, amp.E4M3: F.E4M3}[yt]
    from oracle import cast as OC
    for peak in (1.0, 65519.0, 65520.0, 7e4, 3.4e38, np.inf, np.nan):
        tensors = [synth.normal_f32(300 + k, 4099, 10.0) for k in range(3)]
        tensors[1] = tensors[1].copy()
        tensors[1][77] = peak
        amax = empty(4 * len(tensors))
        amax.zero_()
        st_d = empty(40)
        amp.amp_scaler_init(st_d, 1.0)
        want = False
        for k, x in enumerate(tensors):
            y = empty(x.size * 2)
            amp.amp_cast(dev(x), amp.F32, 1, x.size, x.size, y, yt, x.size, None, 0,
                         None if scale is None else dev(np.array([scale], np.float32)),
                         amax[4 * k:4 * k + 4])
            codes, _ = OC.cast(synth.f32_bits(x), F.F32, yf, scale)
            want |= OA.found_inf(codes, yf) if yt != amp.E4M3 else not np.all(np.isfinite(x))
        amp.amp_found_inf_from_amax(amax, len(tensors), yt,
                                    None if scale is None else dev(np.array([scale], np.float32)), st_d)
        assert bool(scaler_state(st_d)["found_inf"]) == want, (peak, scale)


@pytest.mark.parametrize("overflow", [False, True])
def test_single_pass_step_with_the_producer_flag(overflow):
    """FP32 gradients cast to FP16 by amp_cast (recording amax), the flag from
    that amax, and one optimizer pass with SKIP_CHECK: the same state as the
    oracle's checked step on the oracle's cast of the same gradients."""
    from oracle import cast as OC
    n = (1 << 18) + 3
    S = 1024.0
    hp_o = OA.AdamWHParams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    hp = amp.AdamWHParams(hp_o.lr, hp_o.beta1, hp_o.beta2, hp_o.eps, hp_o.weight_decay)
    theta0 = synth.normal_f32(11, n, 0.02)
    g32 = (synth.normal_f32(12, n, 1e-3) * np.float32(S)).astype(np.float32)
    if overflow:
        g32[n // 2] = 7e4                      # finite in FP32, inf in FP16
    th_d = dev(theta0); m_d = dev(np.zeros(n, np.float32)); v_d = dev(np.zeros(n, np.float32))
    w_d = empty(2 * n); g16_d = empty(2 * n); amax = empty(4); amax.zero_()
    st_d = empty(40)
    amp.amp_scaler_init(st_d, S)
    amp.amp_cast(dev(g32), amp.F32, 1, n, n, g16_d, amp.F16, n, None, 0, None, amax)
    amp.amp_found_inf_from_amax(amax, 1, amp.F16, None, st_d)
    amp.amp_optimizer_step(th_d, m_d, v_d, g16_d, amp.F16, w_d, amp.F16, n, hp, st_d,
                           flags=amp.OPT_SKIP_CHECK)
    codes, _ = OC.cast(synth.f32_bits(g32), F.F32, F.F16, None)
    th, m, v, w, applied = OA.apply(theta0.astype(np.float64), np.zeros(n), np.zeros(n), codes,
                                    F.F16, hp_o, OA.AdamCounters(), S)
    assert applied == (not overflow)
    assert bool(scaler_state(st_d)["found_inf"]) == overflow
    assert np.array_equal(host(th_d, np.float32).astype(np.float64), th)
    assert np.array_equal(host(m_d, np.float32).astype(np.float64), m)
    assert np.array_equal(host(v_d, np.float32).astype(np.float64), v)
    if applied:
        assert np.array_equal(host(w_d, np.uint16), w)
