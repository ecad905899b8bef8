"""Workload-level parity: the fused optimizer over 200 steps with dynamic loss
scaling and injected overflows (at 2^24 with a 2^16 sample, and at the full
2^31 with every decision scanned by the oracle), and the NVFP4 weight-gradient
GEMM at its full size on random codes (12B-style layer: hidden 5120, FFN
20480, 16384 tokens) and the quantizer on full-length column slices.  The
transformer-block workloads at full size are in test_gpu_workloads.py."""
import numpy as np
import pytest
import torch

import mixed_precision_numerics_amd as amp
from oracle import adamw as OA
from oracle import cast as OC
from oracle import formats as F
from oracle import gemm as OG
from oracle import nvfp4 as ON
from oracle import recipe as OR
from oracle import scaler as OS
import synth
import parity_util as PU
from gpu_util import dev, empty, host, metas, scaler_state

pytestmark = pytest.mark.gpu


def _optimizer_run(n, steps, seed, sample, check_every):
    d = "cuda"
    gen = torch.Generator(device=d).manual_seed(seed)
    theta = torch.empty(n, device=d).normal_(0.0, 0.02, generator=gen)
    m = torch.zeros(n, device=d)
    v = torch.zeros(n, device=d)
    w16 = torch.empty(n, device=d, dtype=torch.float16)
    st = torch.empty(40, device=d, dtype=torch.uint8)
    amp.amp_scaler_init(st, 65536.0)
    hp = amp.AdamWHParams(3e-4, 0.9, 0.95, 1e-8, 0.1)
    ohp = OA.AdamWHParams(3e-4, 0.9, 0.95, 1e-8, 0.1)
    inj = synth.injection_schedule(seed, n_steps=steps, n_inject=4, n_params=n) if steps >= 50 else []
    inj_at = {s: (i, val) for s, i, val in inj}
    idx = np.unique(np.concatenate([synth.rng(seed + 1).integers(0, n, sample),
                                    np.array([i for _, i, _ in inj], dtype=np.int64)]))
    idx_d = torch.from_numpy(idx).to(d)
    o_th = theta[idx_d].cpu().numpy().astype(np.float64)
    o_m = np.zeros(idx.size); o_v = np.zeros(idx.size)
    ctr = OA.AdamCounters()
    osc = OS.ScalerState()
    skips = 0
    for t in range(steps):
        S = osc.scale
        assert scaler_state(st)["scale"] == np.float32(S), t
        g16 = synth.adam_grads_f16(gen, n, S)
        if t in inj_at:
            i, val = inj_at[t]
            g16[i] = float(val)
        codes = g16.view(torch.int16).cpu().numpy().view(np.uint16)
        found = any(OA.found_inf(codes[o:o + (1 << 26)], F.F16)   # full scan, oracle side
                    for o in range(0, n, 1 << 26))
        amp.amp_optimizer_step(theta, m, v, g16, amp.F16, w16, amp.F16, n, hp, st)
        gs = scaler_state(st)
        assert bool(gs["found_inf"]) == found, t
        amp.amp_scaler_update(st)
        o_th, o_m, o_v, o_w, ok = OA.apply(o_th, o_m, o_v, codes[idx], F.F16, ohp, ctr, S,
                                           skip=found)
        OS.update(osc, found)
        skips += int(found)
        if t % 20 == 0:
            print(f"optimizer step {t}: scale {S}, skipped so far {skips}", flush=True)
        if t % check_every == 0 or t == steps - 1:
            assert np.array_equal(theta[idx_d].cpu().numpy().astype(np.float64), o_th), t
            assert np.array_equal(m[idx_d].cpu().numpy().astype(np.float64), o_m), t
            assert np.array_equal(v[idx_d].cpu().numpy().astype(np.float64), o_v), t
            if ok:
                assert np.array_equal(w16[idx_d].view(torch.int16).cpu().numpy().view(np.uint16),
                                      o_w), t
    gs = scaler_state(st)
    assert gs["scale"] == np.float32(osc.scale) and gs["growth_tracker"] == osc.growth_tracker
    assert gs["adam_step"] == ctr.step
    return skips, osc.scale


def test_optimizer_200_steps_dynamic_scaling_with_injections():
    skips, final_scale = _optimizer_run(1 << 24, 200, seed=2, sample=1 << 16, check_every=10)
    # the live scale backs off from 2^16 until the heavy-tailed gradients fit,
    # then the 4 injected overflows are skipped too
    assert skips >= 4 and final_scale < 65536.0
    print(f"optimizer 200 steps: {skips} skipped, final scale {final_scale}")


@pytest.mark.timeout(400)
def test_optimizer_full_size_2pow31_200_steps():
    """The optimizer workload at its stated size: 2^31 parameters, 200 steps,
    live loss scale from 65536, 4 seeded injected non-finite steps.  Every
    step's skip decision is checked against the oracle's scan of the whole
    FP16 gradient buffer (copied to pinned host memory; the scan runs over row
    chunks on the host cores), and the oracle carries the AdamW state of a
    seeded 2^20-index sample plus every injected index through all 200 steps
    (its step t-1 runs while step t's gradients are scanned); θ, m, v and the
    FP16 copy of the sample are compared bit for bit after every step."""
    n, steps, seed = 1 << 31, 200, 5
    d = "cuda"
    gen = torch.Generator(device=d).manual_seed(seed)
    theta = torch.empty(n, device=d).normal_(0.0, 0.02, generator=gen)
    m = torch.zeros(n, device=d)
    v = torch.zeros(n, device=d)
    w16 = torch.empty(n, device=d, dtype=torch.float16)
    st = torch.empty(40, device=d, dtype=torch.uint8)
    amp.amp_scaler_init(st, 65536.0)
    hp = amp.AdamWHParams(3e-4, 0.9, 0.95, 1e-8, 0.1)
    ohp = OA.AdamWHParams(3e-4, 0.9, 0.95, 1e-8, 0.1)
    inj = synth.injection_schedule(seed, n_steps=steps, n_inject=4, n_params=n)
    inj_at = {s_: (i, val) for s_, i, val in inj}
    idx = np.unique(np.concatenate([synth.rng(seed + 1).integers(0, n, 1 << 20),
                                    np.array([i for _, i, _ in inj], dtype=np.int64)]))
    idx_d = torch.from_numpy(idx).to(d)
    host_g = torch.empty(n, dtype=torch.int16, pin_memory=True)
    hg = host_g.numpy().view(np.uint16)
    o = dict(th=theta[idx_d].cpu().numpy().astype(np.float64), m=np.zeros(idx.size),
             v=np.zeros(idx.size))
    ctr = OA.AdamCounters()
    osc = OS.ScalerState()
    pending = None               # (S, found, sample codes, GPU snapshot) of the last step
    skips = 0

    def oracle_step(rec):
        S, found, codes, snap = rec
        o["th"], o["m"], o["v"], ow, ok = OA.apply(o["th"], o["m"], o["v"], codes, F.F16, ohp,
                                                   ctr, S, skip=found)
        assert np.array_equal(snap[0], o["th"]) and np.array_equal(snap[1], o["m"])
        assert np.array_equal(snap[2], o["v"])
        if ok:
            assert np.array_equal(snap[3], ow)

    for t in range(steps):
        S = osc.scale
        assert scaler_state(st)["scale"] == np.float32(S), t
        g16 = synth.adam_grads_f16(gen, n, S)
        if t in inj_at:
            i, val = inj_at[t]
            g16[i] = float(val)
        host_g.copy_(g16.view(torch.int16), non_blocking=True)
        codes = g16.view(torch.int16)[idx_d].cpu().numpy().view(np.uint16)
        amp.amp_optimizer_step(theta, m, v, g16, amp.F16, w16, amp.F16, n, hp, st)
        # oracle: scan the whole buffer while it carries the sample through step t-1
        futs = PU.submit_rows(lambda c: OA.found_inf(c, F.F16), hg, parts=64)
        if pending is not None:
            oracle_step(pending)
        found = any(f.result() for f in futs)
        gs = scaler_state(st)
        assert bool(gs["found_inf"]) == found, t
        amp.amp_scaler_update(st)
        snap = (theta[idx_d].cpu().numpy().astype(np.float64),
                m[idx_d].cpu().numpy().astype(np.float64),
                v[idx_d].cpu().numpy().astype(np.float64),
                w16[idx_d].view(torch.int16).cpu().numpy().view(np.uint16))
        pending = (S, found, codes, snap)
        OS.update(osc, found)
        skips += int(found)
        if t % 20 == 0:
            print(f"optimizer 2^31 step {t}: scale {S}, skipped so far {skips}", flush=True)
    oracle_step(pending)
    gs = scaler_state(st)
    assert gs["scale"] == np.float32(osc.scale) and gs["growth_tracker"] == osc.growth_tracker
    assert gs["adam_step"] == ctr.step
    assert skips >= 4 and osc.scale < 65536.0
    print(f"optimizer 2^31, 200 steps: {skips} skipped, final scale {osc.scale}")


def test_nvfp4_wgrad_full_size_gemm_sampled():
    """dW [20480 x 5120] = dY^T X over 16384 tokens with NVFP4 operands."""
    O, I, T = 20480, 5120, 16384
    qa, sa, enca = synth.nvfp4_operand(1, O, T)
    qb, sb, encb = synth.nvfp4_operand(2, I, T)
    d = "cuda"
    qa_d, qb_d, sa_d, sb_d = dev(qa), dev(qb), dev(sa), dev(sb)
    deca = np.float32(1.0) / np.float32(enca); decb = np.float32(1.0) / np.float32(encb)
    c = torch.empty(O, I, device=d, dtype=torch.bfloat16)
    amp.amp_gemm(amp.OP_N, amp.OP_T, O, I, T, qa_d, amp.E2M1X2, T // 2, dev(np.array([deca])),
                 qb_d, amp.E2M1X2, T // 2, dev(np.array([decb])), c, amp.BF16, I,
                 amp.BlockScales(sa_d.data_ptr(), T // 16, 0, 0),
                 amp.BlockScales(sb_d.data_ptr(), T // 16, 0, 0))
    rng = np.random.default_rng(3)
    ii = rng.integers(0, O, 256); jj = rng.integers(0, I, 256)
    A = ON.dequantize(qa[ii], sa[ii], 1.0) * float(deca)
    B = ON.dequantize(qb[jj], sb[jj], 1.0) * float(decb)
    cref = np.sum(A * B, axis=1)
    bound = np.sum(np.abs(A) * np.abs(B), axis=1)
    out = c.view(torch.int16)[torch.from_numpy(ii).to(d), torch.from_numpy(jj).to(d)]
    assert OG.check_rounded(out.cpu().numpy().view(np.uint16), F.BF16, cref, bound).all()


@pytest.mark.parametrize("which", ["dY", "X"])
def test_nvfp4_quantize_full_length_column_slices(which):
    """The wgrad operands at full token length (16384): quantize 64-column
    slices of dY [16384 x 20480] / X [16384 x 5120] (strided input) and
    compare bit for bit with the oracle."""
    T = 16384
    C = 20480 if which == "dY" else 5120
    d = "cuda"
    gen = torch.Generator(device=d).manual_seed(6 if which == "dY" else 7)
    x = torch.randn(T, C, generator=gen, device=d)
    mask = torch.rand(T, C, generator=gen, device=d) < 1e-3
    x = torch.where(mask, torch.sign(x) * 50.0, x).to(torch.bfloat16)
    sr = which == "dY"
    for c0 in (0, C // 2 + 64, C - 64):
        q = empty(64 * T // 2); s = empty(64 * T // 16); ts = empty(12)
        amp.amp_nvfp4_quantize(x.data_ptr() + 2 * c0, amp.BF16, T, 64, C, 1, 0, 1, 99, amp.ROUND_SR if sr else amp.ROUND_RNE,
                               1234, q, s, ts)
        xs = x[:, c0:c0 + 64].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        wq, ws, enc = ON.quantize(F.decode(xs, F.BF16), transpose=True, rht=True, rht_seed=99,
                                  sr=sr, sr_seed=1234)
        assert host(ts, np.float32)[1] == np.float32(enc)
        assert np.array_equal(host(s, np.uint8).reshape(ws.shape), ws)
        assert np.array_equal(host(q, np.uint8).reshape(wq.shape), wq)
