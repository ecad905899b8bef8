"""Pins for oracle/clip.py (gradient accumulation, global-norm clipping) and
the clip multiplier of oracle/adamw.py, against closed forms and independent
library routines (NumPy float32 arithmetic, torch.nn.utils.clip_grad_norm_,
torch.optim.AdamW)."""
import math

import numpy as np
import torch

from oracle import adamw as A
from oracle import clip as C
from oracle import formats as F
import synth


def test_accumulate_matches_float32_addition():
    """Four FP16 micro-batches summed in FP32: NumPy's float32 adds."""
    n = 20000
    acc = None
    ref = None
    for k in range(4):
        codes = synth.to_f16_codes(synth.normal_f32(30 + k, n) * 1000.0)
        acc = C.accumulate(acc, codes, F.F16, first=(k == 0))
        g32 = F.decode(codes, F.F16).astype(np.float32)
        ref = g32.copy() if k == 0 else (ref + g32).astype(np.float32)
    assert np.array_equal(acc, ref.astype(np.float64))


def test_accumulate_propagates_non_finite():
    a = C.accumulate(None, np.array([0x3C00, 0x3C00, 0x3C00], np.uint16), F.F16, True)
    a = C.accumulate(a, np.array([0x7C00, 0x7E00, 0x3C00], np.uint16), F.F16, False)
    a = C.accumulate(a, np.array([0x3C00, 0x3C00, 0xFC00], np.uint16), F.F16, False)
    assert a[0] == np.inf and np.isnan(a[1]) and a[2] == -np.inf


def test_norm_closed_form_and_scale():
    """n equal FP16 gradients c at loss scale S: sumsq = n (c/S)^2 exactly."""
    c = 1.5 * 2.0 ** -3
    for n, S in ((1000, 1024.0), (4096, 65536.0), (7, 1.0)):
        codes = synth.to_f16_codes(np.full(n, c * S, np.float32))
        s, bad = C.norm_sq(codes, F.F16, S)
        assert not bad and s == n * c * c
        coef, norm = C.clip_coefficient(s, 1.0)
        assert norm == np.float32(math.sqrt(n) * c)


def test_norm_skips_and_flags_non_finite():
    codes = np.array([0x3C00, 0x7C00, 0x4000, 0x7E01], np.uint16)
    s, bad = C.norm_sq(codes, F.F16, 1.0)
    assert bad and s == 1.0 + 4.0


def test_norm_vs_numpy_linalg():
    x = synth.normal_f32(40, 100003, 3e-2)
    s, bad = C.norm_sq(synth.f32_bits(x), F.F32, 1.0)
    assert not bad
    ref = np.linalg.norm(x.astype(np.float64))
    assert abs(math.sqrt(s) - ref) <= 1e-13 * ref


def test_clip_coefficient_vs_torch_clip_grad_norm():
    """torch's clip_grad_norm_ on the unscaled FP32 gradients: given torch's
    own (FP32-summed) norm, the coefficient formula reproduces torch's clipped
    gradients bit for bit; the exact norm agrees with torch's to FP32
    summation accuracy."""
    for seed, scale, max_norm in ((50, 1e-2, 1.0), (51, 1e-4, 1.0), (52, 3.0, 0.25)):
        g32 = (synth.normal_f32(seed, 50000) * scale).astype(np.float32)
        s, _ = C.norm_sq(synth.f32_bits(g32), F.F32, 1.0)
        coef, norm = C.clip_coefficient(s, max_norm)
        p = torch.nn.Parameter(torch.zeros(g32.size))
        p.grad = torch.from_numpy(g32.copy())
        tn = float(torch.nn.utils.clip_grad_norm_([p], max_norm))
        assert abs(norm - tn) <= 1e-5 * tn
        c_t = C.coefficient_from_norm(tn, max_norm)
        theirs = p.grad.numpy().astype(np.float64)
        assert np.array_equal(F.f32(g32.astype(np.float64) * c_t), theirs)
        if norm <= max_norm:
            assert coef == 1.0


def test_clip_coefficient_closed_forms():
    coef, norm = C.clip_coefficient(4.0, 1.0)                 # norm 2
    assert norm == 2.0
    assert coef == float(np.float32(np.float32(1.0) / np.float32(np.float32(2.0) + np.float32(1e-6))))
    assert C.clip_coefficient(0.25, 1.0)[0] == 1.0             # norm 0.5: no clipping
    assert C.clip_coefficient(0.0, 1.0) == (1.0, 0.0)


def test_adamw_with_clip_multiplier_vs_torch():
    """AdamW on clipped unscaled gradients: torch.optim.AdamW fed fl32(g*coef)."""
    n = 4096
    hp = A.AdamWHParams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    theta0 = synth.normal_f32(61, n, 0.02)
    p = torch.nn.Parameter(torch.from_numpy(theta0.copy()))
    opt = torch.optim.AdamW([p], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps,
                            weight_decay=hp.weight_decay, foreach=False)
    th = theta0.astype(np.float64); m = np.zeros(n); v = np.zeros(n)
    ctr = A.AdamCounters()
    for t in range(8):
        codes = synth.to_f16_codes(synth.normal_f32(200 + t, n, 0.05) * 1024.0)
        s, _ = C.norm_sq(codes, F.F16, 1024.0)
        coef, _ = C.clip_coefficient(s, 1.0)
        assert coef < 1.0                                     # these gradients are clipped
        th, m, v, _, ok = A.apply(th, m, v, codes, F.F16, hp, ctr, 1024.0, grad_mult=coef)
        g = F.f32(F.f32(F.decode(codes, F.F16) / 1024.0) * coef)
        p.grad = torch.from_numpy(g.astype(np.float32))
        opt.step()
    ref = p.detach().numpy().astype(np.float64)
    unit = np.spacing(np.maximum(np.abs(ref), hp.lr).astype(np.float32)).astype(np.float64)
    ulps = np.abs(th - ref) / unit
    assert ulps.max() <= 64 and np.quantile(ulps, 0.99) <= 4
