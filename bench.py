"""Benchmark of the mixed-precision training hot path on one MI355X.

Headline workload (the fused AMP optimizer step over a 2^31-parameter shard):
  FP32 master ~ N(0, 0.02), FP32 Adam moments from zero, FP16 gradients
  g16 = round16(S * 1e-4 * N(0,1) * exp(2 Z)) at loss scale S = 2^10 (clipped
  to the FP16 range so that every timed step is applied), AdamW lr 3e-4,
  betas (0.9, 0.95), wd 0.1, eps 1e-8, FP16 working copy written.
One step = amp_check_overflow (2 B/param) + amp_optimizer_step with the check
already done (apply: read g16, master, m, v; write master, m, v, w16 =
28 B/param) + amp_scaler_update.  value = 28 B/param * n / step time.  The
single-pass variant (the overflow flag taken from the amax that the casting
producer of the gradients recorded, amp_found_inf_from_amax) is reported
under "components".

Also measured in the same run (reported under "components"):
  * the BF16 and FP8 (delayed-scaling, E4M3 fwd / E5M2 bwd) GEMMs of one
    transformer block's linear layers at hidden 4096, FFN 14336, 8192 tokens
    (fwd, dgrad, wgrad of QKV, O, up/gate, down: 10.72 TFLOP per block step),
    the FP8 step both on the exact BF16 route and on the native FP8
    instruction;
  * the NVFP4 weight-gradient GEMM 20480 x 5120 x 16384 and its two
    quantizer calls (RHT on both operands, stochastic rounding on dY);
  * the scaled casts (BF16 -> E4M3 flat 2^31, BF16 -> E5M2 [8192 x 28672]
    with its transposed copy), and delayed against current scaling;
  * the global-norm pass (2^31 FP16 gradients) and FP32 gradient
    accumulation;
  * MXFP4 and MXFP8 GEMMs of the FFN up projection on the block-scaled
    matrix cores, with their quantizer;
  * fine-grained FP8 (1x128 activation / gradient tiles, 128x128 weight
    blocks): the three quantizer passes and the forward, dgrad and wgrad
    GEMMs of the FFN up projection.
The CPU oracle is timed on a bounded sample of the optimizer workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-components]
                       [--components name,name,...] [--no-cpu-baseline] [--calibrate-copy]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
FP4_PEAK_TFLOPS = 10100.0
N_PARAMS = 1 << 31
BYTES_PER_PARAM = 28


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class StreamTimer:
    """HIP events on the stream the kernels are launched on."""

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e

    def stop(self, s):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs.append((s, e))

    def mean_ms(self):
        self.torch.cuda.synchronize()
        return sum(s.elapsed_time(e) for s, e in self.pairs) / max(1, len(self.pairs))


def optimizer_workload(torch, amp, n, steps, warmup, calibrate_copy):
    dev = "cuda"
    gen = torch.Generator(device=dev).manual_seed(1)
    log(f"allocating optimizer state for n = {n}")
    theta = torch.empty(n, device=dev, dtype=torch.float32)
    theta.normal_(0.0, 0.02, generator=gen)
    m = torch.zeros(n, device=dev, dtype=torch.float32)
    v = torch.zeros(n, device=dev, dtype=torch.float32)
    S = 1024.0
    g16 = torch.empty(n, device=dev, dtype=torch.float16)
    chunk = 1 << 28
    for o in range(0, n, chunk):
        k = min(chunk, n - o)
        z = torch.randn(k, device=dev, generator=gen)
        g = torch.randn(k, device=dev, generator=gen) * 1e-4 * torch.exp(2.0 * z) * S
        g16[o:o + k] = g.clamp_(-65504.0, 65504.0).half()
        del z, g
    w16 = torch.empty(n, device=dev, dtype=torch.float16)
    st = torch.empty(40, device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    amp.amp_scaler_init(st, S)
    hp = amp.AdamWHParams(3e-4, 0.9, 0.95, 1e-8, 0.1)
    if calibrate_copy:
        # a plain copy of known size for scaling the HBM byte counters
        a = torch.empty(1 << 28, device=dev, dtype=torch.float32)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("calibration copy: 1 GiB read + 1 GiB written")
        del a, b

    def step(timer=None):
        amp.amp_check_overflow(g16, amp.F16, n, st)
        t0 = timer.start() if timer else None
        amp.amp_optimizer_step(theta, m, v, g16, amp.F16, w16, amp.F16, n, hp, st,
                               flags=amp.OPT_SKIP_CHECK)
        if timer:
            timer.stop(t0)
        amp.amp_scaler_update(st)

    for i in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({warmup} steps)")
    timer = StreamTimer(torch, stream)
    t0 = time.perf_counter()
    for i in range(steps):
        step(timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    apply_ms = timer.mean_ms()
    state = st.cpu().numpy().view(amp.SCALER_STATE_DTYPE)[0]
    if int(state["adam_step"]) != warmup + steps:
        raise RuntimeError(f"expected every step applied, adam_step = {int(state['adam_step'])}")
    log(f"timed {steps} steps: {wall * 1e3 / steps:.3f} ms/step, apply kernel {apply_ms:.3f} ms")

    # The producer-flag variant: when a cast of ours wrote the gradients, the
    # amax it recorded decides the overflow flag and the step is one 28 B/param
    # pass.  Stand-in for that record: the bit-exact max |g16| (the same
    # decision as the producing cast's input amax for these gradients).
    amax = g16.abs().max().float().reshape(1)

    def step1():
        amp.amp_found_inf_from_amax(amax, 1, amp.F16, None, st)
        amp.amp_optimizer_step(theta, m, v, g16, amp.F16, w16, amp.F16, n, hp, st,
                               flags=amp.OPT_SKIP_CHECK)
        amp.amp_scaler_update(st)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step1()
    torch.cuda.synchronize()
    wall1 = time.perf_counter() - t0
    state = st.cpu().numpy().view(amp.SCALER_STATE_DTYPE)[0]
    if int(state["adam_step"]) != warmup + 2 * steps:
        raise RuntimeError(f"expected every step applied, adam_step = {int(state['adam_step'])}")
    log(f"single-pass variant: {wall1 * 1e3 / steps:.3f} ms/step")

    # A step that overflows: one +inf among the gradients.  The check sweep
    # sets the flag, the apply kernel reads it and writes nothing, the scaler
    # halves S.  Timed separately (median of 20 steps); state must not move.
    g16[n // 3] = float("inf")
    step_before = int(st.cpu().numpy().view(amp.SCALER_STATE_DTYPE)[0]["adam_step"])
    th_probe = theta[: 1 << 20].clone()
    skip_ms = _median_ms(torch, step, 20, warm=2)
    state = st.cpu().numpy().view(amp.SCALER_STATE_DTYPE)[0]
    if int(state["adam_step"]) != step_before or not torch.equal(th_probe, theta[: 1 << 20]):
        raise RuntimeError("a skipped step changed the optimizer state")
    g16[n // 3] = 0.0
    del th_probe
    log(f"skipped (overflowing) step: {skip_ms:.3f} ms")

    # The same-run HBM ceiling for a read-as-much-as-written stream: a plain
    # 16-byte copy of 4 GiB (4 GiB read + 4 GiB written).
    cb = 1 << 32
    src = torch.empty(cb, device=dev, dtype=torch.uint8)
    src.fill_(1)
    dst = torch.empty_like(src)
    copy_ms = _median_ms(torch, lambda: amp.amp_stream_copy(src, dst, cb), 20)
    if not torch.equal(src[: 1 << 20], dst[: 1 << 20]):
        raise RuntimeError("stream copy mismatch")
    del src, dst
    torch.cuda.empty_cache()
    copy_gbs = 2 * cb / copy_ms / 1e6
    log(f"stream copy 4 GiB: {copy_ms:.3f} ms = {copy_gbs:.1f} GB/s")
    return wall * 1e3 / steps, apply_ms, wall1 * 1e3 / steps, skip_ms, copy_ms, copy_gbs


def gemm_block_workload(torch, amp, fp8: bool, reps: int = 20, native: bool = False):
    """12 GEMMs of one transformer block (fwd, dgrad, wgrad of 4 linears),
    median of ``reps`` block steps.  BF16: the FP32 master weights are cast to
    BF16 (amp_cast) at the start of the step, then the 12 GEMMs; each GEMM is
    also timed alone (median of ``reps``).  FP8: E4M3 activations/weights,
    E5M2 output gradients, delayed-scaling casts (row-major + transposed FP8
    copies) before the GEMMs.  native: the FP8 GEMMs on the FP8 matrix-core
    instruction (AMP_GEMM_FP8_NATIVE, its reduced-precision 64-term sums)
    instead of the exact BF16 route."""
    gflags = amp.GEMM_FP8_NATIVE if native else 0
    T = 8192
    layers = [("qkv", 4096, 6144), ("o", 4096, 4096), ("up", 4096, 28672), ("down", 14336, 4096)]
    dev = "cuda"
    gen = torch.Generator(device=dev).manual_seed(3)
    flops = 0
    bufs = []
    for name, din, dout in layers:
        X = torch.randn(T, din, device=dev, generator=gen).to(torch.bfloat16)
        W32 = torch.randn(dout, din, device=dev, generator=gen) * 0.02
        W = W32.to(torch.bfloat16)
        dY = torch.randn(T, dout, device=dev, generator=gen).to(torch.bfloat16)
        Y = torch.empty(T, dout, device=dev, dtype=torch.bfloat16)
        dX = torch.empty(T, din, device=dev, dtype=torch.bfloat16)
        dW = torch.empty(dout, din, device=dev, dtype=torch.bfloat16)
        d = dict(X=X, W=W, dY=dY, Y=Y, dX=dX, dW=dW, din=din, dout=dout, name=name)
        if not fp8:
            d["W32"] = W32
        else:
            del W32
        if fp8:
            d.update(X8=torch.empty(T * din, device=dev, dtype=torch.uint8),
                     X8t=torch.empty(T * din, device=dev, dtype=torch.uint8),
                     W8=torch.empty(dout * din, device=dev, dtype=torch.uint8),
                     W8t=torch.empty(dout * din, device=dev, dtype=torch.uint8),
                     G8=torch.empty(T * dout, device=dev, dtype=torch.uint8),
                     G8t=torch.empty(T * dout, device=dev, dtype=torch.uint8))
        bufs.append(d)
        flops += 3 * 2 * T * din * dout
    if fp8:
        nm = 3 * len(layers)
        metas = torch.empty(16 * nm, device=dev, dtype=torch.uint8)
        hist = torch.empty(4 * nm * 1024, device=dev, dtype=torch.uint8)
        amp.amp_fp8_meta_init(metas, hist, nm, 1024)
        r43 = amp.DelayedRecipe(448.0, 1.0, 1024, amp.AMAX_MAX)
        r52 = amp.DelayedRecipe(57344.0, 1.0, 1024, amp.AMAX_MAX)
    mp = lambda i, off: metas.data_ptr() + 16 * i + off

    def bf16_gemms(d):
        din, dout = d["din"], d["dout"]
        return (
            ("fwd", 2 * T * din * dout, lambda: amp.amp_gemm(
                amp.OP_N, amp.OP_T, T, dout, din, d["X"], amp.BF16, din, None, d["W"], amp.BF16,
                din, None, d["Y"], amp.BF16, dout)),
            ("dgrad", 2 * T * din * dout, lambda: amp.amp_gemm(
                amp.OP_N, amp.OP_N, T, din, dout, d["dY"], amp.BF16, dout, None, d["W"], amp.BF16,
                din, None, d["dX"], amp.BF16, din)),
            ("wgrad", 2 * T * din * dout, lambda: amp.amp_gemm(
                amp.OP_T, amp.OP_N, dout, din, T, d["dY"], amp.BF16, dout, None, d["X"], amp.BF16,
                din, None, d["dW"], amp.BF16, din)))

    def run():
        if not fp8:
            for d in bufs:           # FP32 master weights -> BF16 working copies
                amp.amp_cast(d["W32"], amp.F32, d["dout"], d["din"], d["din"], d["W"], amp.BF16,
                             d["din"])
        for li, d in enumerate(bufs):
            din, dout = d["din"], d["dout"]
            if not fp8:
                for _, _, f in bf16_gemms(d):
                    f()
            else:
                ix, iw, ig = 3 * li, 3 * li + 1, 3 * li + 2
                amp.amp_cast(d["X"], amp.BF16, T, din, din, d["X8"], amp.E4M3, din, d["X8t"], T,
                             mp(ix, 4), mp(ix, 0))
                amp.amp_cast(d["W"], amp.BF16, dout, din, din, d["W8"], amp.E4M3, din, d["W8t"],
                             dout, mp(iw, 4), mp(iw, 0))
                amp.amp_gemm_ex(amp.OP_N, amp.OP_T, T, dout, din, d["X8"], amp.E4M3, din, mp(ix, 8),
                                d["W8"], amp.E4M3, din, mp(iw, 8), d["Y"], amp.BF16, dout,
                                flags=gflags)
                amp.amp_cast(d["dY"], amp.BF16, T, dout, dout, d["G8"], amp.E5M2, dout, d["G8t"],
                             T, mp(ig, 4), mp(ig, 0))
                amp.amp_gemm_ex(amp.OP_N, amp.OP_T, T, din, dout, d["G8"], amp.E5M2, dout, mp(ig, 8),
                                d["W8t"], amp.E4M3, dout, mp(iw, 8), d["dX"], amp.BF16, din,
                                flags=gflags)
                amp.amp_gemm_ex(amp.OP_N, amp.OP_T, dout, din, T, d["G8t"], amp.E5M2, T, mp(ig, 8),
                                d["X8t"], amp.E4M3, T, mp(ix, 8), d["dW"], amp.BF16, din,
                                flags=gflags)
        if fp8:
            # E4M3 metas (X, W) and E5M2 metas (dY) are updated by role
            for li in range(len(layers)):
                amp.amp_delayed_scaling_update(mp(3 * li, 0), hist.data_ptr() + 4 * 1024 * 3 * li,
                                               2, r43)
                amp.amp_delayed_scaling_update(mp(3 * li + 2, 0),
                                               hist.data_ptr() + 4 * 1024 * (3 * li + 2), 1, r52)

    ms = _median_ms(torch, run, reps)
    per = None
    if not fp8:
        per = {}
        for d in bufs:
            for pname, fl, f in bf16_gemms(d):
                g_ms = _median_ms(torch, f, reps)
                per[f"{d['name']}_{pname}"] = {
                    "mnk": [T, d["dout"], d["din"]] if pname == "fwd" else
                           [T, d["din"], d["dout"]] if pname == "dgrad" else [d["dout"], d["din"], T],
                    "ms": round(g_ms, 4), "tflops": round(fl / g_ms / 1e9, 1),
                    "frac": round(fl / g_ms / 1e9 / BF16_PEAK_TFLOPS, 4)}
    del bufs
    torch.cuda.empty_cache()
    # the FP8 block runs the BF16-rate instruction on the exact route: its
    # fraction is also given against the BF16 peak
    peak = FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS
    tf = flops / ms / 1e9
    out = {"ms": round(ms, 4), "tflops": round(tf, 1), "peak_tflops": peak,
           "frac": round(tf / peak, 4), "tflop_per_step": round(flops / 1e12, 3),
           "timing": f"median of {reps} block steps",
           "includes": ("6 delayed-scaling FP8 casts per layer + amax-history updates + 12 GEMMs"
                        if fp8 else "4 FP32->BF16 weight casts + 12 GEMMs")}
    if fp8 and not native:
        out["frac_of_bf16_peak"] = round(tf / BF16_PEAK_TFLOPS, 4)
    if native:
        out["fp8_instruction"] = "native (reduced-precision 64-term sums)"
    if per is not None:
        out["per_gemm"] = per
    return out


def cast_workload(torch, amp):
    """The two flat casts of the cast-only workload, 2^31 elements each with
    amax capture: BF16 -> E4M3 with a scale (3 B/elem) and FP32 -> FP16, the
    master-weight recast (6 B/elem)."""
    n = 1 << 31
    x = torch.randn(n, device="cuda").to(torch.bfloat16)
    y = torch.empty(n, device="cuda", dtype=torch.uint8)
    sc = torch.ones(1, device="cuda")
    am = torch.zeros(1, device="cuda")
    f = lambda: amp.amp_cast(x, amp.BF16, 1, n, n, y, amp.E4M3, n, None, 0, sc, am)
    ms = _median_ms(torch, f, 20)
    del x, y
    torch.cuda.empty_cache()
    gbs = 3 * n / ms / 1e6
    x32 = torch.randn(n, device="cuda")
    y16 = torch.empty(n, device="cuda", dtype=torch.float16)
    f32 = lambda: amp.amp_cast(x32, amp.F32, 1, n, n, y16, amp.F16, n, None, 0, None, am)
    ms32 = _median_ms(torch, f32, 20)
    del x32, y16
    torch.cuda.empty_cache()
    gbs32 = 6 * n / ms32 / 1e6
    return {"what": "BF16->E4M3 flat 2^31 with amax", "ms": round(ms, 4), "gbs": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "f32_to_f16": {"what": "FP32->FP16 flat 2^31 with amax (6 B/elem)", "ms": round(ms32, 4),
                           "gbs": round(gbs32, 1), "frac": round(gbs32 / HBM_PEAK_GBS, 4)}}


def _median_ms(torch, f, reps=20, warm=3):
    """Median over ``reps`` runs of f, each bracketed by its own pair of HIP
    events on the current stream, after ``warm`` untimed runs."""
    for _ in range(warm):
        f()
    torch.cuda.synchronize()
    evs = []
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        f()
        e.record()
        evs.append((s, e))
    torch.cuda.synchronize()
    ts = sorted(s.elapsed_time(e) for s, e in evs)
    return ts[len(ts) // 2]


def _timed(torch, f, reps):
    """Median of at least 20 individually timed runs."""
    return _median_ms(torch, f, max(20, reps))


def _timed_rot(torch, fns, reps):
    """Mean time of one call when the calls rotate over the given closures
    (distinct buffers totalling more than the 256 MB Infinity Cache, so that
    every call reads from HBM)."""
    for f in fns:
        f()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(reps):
        fns[i % len(fns)]()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def _copies(need_bytes, each_bytes, lo=4):
    """Number of buffer sets needed for a working set above 1 GiB."""
    return max(lo, -(-need_bytes // each_bytes))


def cast_t_workload(torch, amp):
    """BF16 -> E5M2 of an FFN output gradient [8192 x 28672] with its
    transposed copy (the dgrad and wgrad operands) and amax: 4 B/elem."""
    R, C = 8192, 28672
    gen = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randn(R, C, device="cuda", generator=gen).to(torch.bfloat16)
    y = torch.empty(R * C, device="cuda", dtype=torch.uint8)
    yt = torch.empty(R * C, device="cuda", dtype=torch.uint8)
    sc = torch.ones(1, device="cuda")
    am = torch.zeros(1, device="cuda")
    ms = _timed(torch, lambda: amp.amp_cast(x, amp.BF16, R, C, C, y, amp.E5M2, C, yt, R, sc, am),
                5)
    del x, y, yt
    torch.cuda.empty_cache()
    gbs = 4 * R * C / ms / 1e6
    return {"what": "BF16->E5M2 [8192 x 28672] + transposed copy + amax", "ms": round(ms, 4),
            "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}


def nvfp4_workload(torch, amp):
    """NVFP4 weight-gradient step of a 12B-style FFN up projection (hidden
    5120, FFN 20480, 16384 tokens): quantize dY^T (RHT + stochastic rounding)
    and X^T (RHT, round to nearest) along the token axis, then
    dW[20480 x 5120] = dY^T X in BF16."""
    T, I, O = 16384, 5120, 20480
    dev = "cuda"
    gen = torch.Generator(device=dev).manual_seed(7)

    def outliers(rows, cols):
        x = torch.randn(rows, cols, device=dev, generator=gen)
        hit = torch.rand(rows, cols, device=dev, generator=gen) < 1e-3
        sgn = torch.where(torch.rand(rows, cols, device=dev, generator=gen) < 0.5, -50.0, 50.0)
        return torch.where(hit, sgn, x).to(torch.bfloat16)

    dY = outliers(T, O)
    X = outliers(T, I)
    qa = torch.empty(O * T // 2, device=dev, dtype=torch.uint8)
    sa = torch.empty(O * T // 16, device=dev, dtype=torch.uint8)
    qb = torch.empty(I * T // 2, device=dev, dtype=torch.uint8)
    sb = torch.empty(I * T // 16, device=dev, dtype=torch.uint8)
    ta = torch.empty(3, device=dev)
    tb = torch.empty(3, device=dev)
    dW = torch.empty(O, I, device=dev, dtype=torch.bfloat16)

    def quant():
        amp.amp_nvfp4_quantize(dY, amp.BF16, T, O, O, 1, 0, 1, 11, amp.ROUND_SR, 12, qa, sa, ta)
        amp.amp_nvfp4_quantize(X, amp.BF16, T, I, I, 1, 0, 1, 11, amp.ROUND_RNE, 0, qb, sb, tb)

    def gemm():
        amp.amp_gemm(amp.OP_N, amp.OP_T, O, I, T, qa, amp.E2M1X2, T // 2, ta.data_ptr() + 8,
                     qb, amp.E2M1X2, T // 2, tb.data_ptr() + 8, dW, amp.BF16, I,
                     amp.BlockScales(sa.data_ptr(), T // 16, 0, 0),
                     amp.BlockScales(sb.data_ptr(), T // 16, 0, 0))

    q_ms = _timed(torch, quant, 5)
    g_ms = _timed(torch, gemm, 5)
    del dY, X, qa, sa, qb, sb, dW
    torch.cuda.empty_cache()
    flops = 2 * O * I * T
    tf = flops / g_ms / 1e9
    # quantizer traffic: amax pass reads BF16, encode pass reads BF16 and
    # writes 0.5 B of codes + 1/16 B of scales per element
    qbytes = (T * O + T * I) * (2 + 2 + 0.5 + 1.0 / 16)
    return {"gemm_ms": round(g_ms, 4), "gemm_tflops": round(tf, 1),
            "peak_tflops_fp4": FP4_PEAK_TFLOPS, "frac_fp4": round(tf / FP4_PEAK_TFLOPS, 4),
            "frac_bf16_mfma": round(tf / BF16_PEAK_TFLOPS, 4),
            "mfma": "f16 (E2M1 x E4M3 decoded exactly to F16 per register fragment)",
            "quantize_ms": round(q_ms, 4), "quantize_gbs": round(qbytes / q_ms / 1e6, 1),
            "tflop_per_step": round(flops / 1e12, 3)}


def scaling_workload(torch, amp):
    """Delayed scaling (one read: the scale comes from earlier steps) against
    current scaling (amax pass, then the cast) on the FP8 block's activation
    [8192 x 4096] and FFN output gradient [8192 x 28672], each with its
    transposed copy."""
    out = {}
    gen = torch.Generator(device="cuda").manual_seed(9)
    for name, R, C, yt, fmax in (("x_e4m3", 8192, 4096, amp.E4M3, 448.0),
                                 ("dy_e5m2", 8192, 28672, amp.E5M2, 57344.0)):
        # rotate over enough input/output sets to exceed 1 GiB
        k = _copies(1 << 30, 4 * R * C)
        xs = [torch.randn(R, C, device="cuda", generator=gen).to(torch.bfloat16) for _ in range(k)]
        ys = [torch.empty(R * C, device="cuda", dtype=torch.uint8) for _ in range(k)]
        yts = [torch.empty(R * C, device="cuda", dtype=torch.uint8) for _ in range(k)]
        meta = torch.empty(16, device="cuda", dtype=torch.uint8)
        hist = torch.empty(4 * 1024, device="cuda", dtype=torch.uint8)
        amp.amp_fp8_meta_init(meta, hist, 1, 1024)
        r = amp.DelayedRecipe(fmax, 1.0, 1024, amp.AMAX_MAX)
        mp = meta.data_ptr()
        dl = [lambda i=i: amp.amp_cast(xs[i], amp.BF16, R, C, C, ys[i], yt, C, yts[i], R, mp + 4, mp)
              for i in range(k)]
        cl = [lambda i=i: amp.amp_cast_current_scaling(xs[i], amp.BF16, R, C, C, ys[i], yt, C, yts[i],
                                                       R, r, meta) for i in range(k)]
        d_ms = _timed_rot(torch, dl, 4 * k)
        c_ms = _timed_rot(torch, cl, 4 * k)
        out[name] = {"delayed_ms": round(d_ms, 4), "current_ms": round(c_ms, 4),
                     "current_over_delayed": round(c_ms / d_ms, 3),
                     "working_set_gib": round(k * 4 * R * C / 2**30, 2)}
        del xs, ys, yts
    torch.cuda.empty_cache()
    return out


def clip_workload(torch, amp):
    """Global-norm pass over 2^31 FP16 gradients (2 B/param read; also the
    overflow check) and FP32 micro-batch accumulation of 2^30 FP16 gradients
    (10 B/param)."""
    n = 1 << 31
    g = torch.randn(n, device="cuda", dtype=torch.float16)
    st = torch.empty(40, device="cuda", dtype=torch.uint8)
    amp.amp_scaler_init(st, 1024.0)
    ns = torch.empty(amp.NORM_STATE_BYTES, device="cuda", dtype=torch.uint8)
    amp.amp_grad_norm_init(ns)
    n_ms = _timed(torch, lambda: amp.amp_grad_norm_accumulate(g, amp.F16, n, st, ns), 5)
    na = 1 << 30
    acc = torch.empty(na, device="cuda", dtype=torch.float32)
    amp.amp_grad_accumulate(acc, g, amp.F16, na, True)
    a_ms = _timed(torch, lambda: amp.amp_grad_accumulate(acc, g, amp.F16, na, False), 5)
    del g, acc
    torch.cuda.empty_cache()
    return {"norm_2pow31_f16": {"ms": round(n_ms, 4), "gbs": round(2 * n / n_ms / 1e6, 1),
                                "frac": round(2 * n / n_ms / 1e6 / HBM_PEAK_GBS, 4)},
            "accumulate_2pow30_f16_to_f32": {"ms": round(a_ms, 4),
                                            "gbs": round(10 * na / a_ms / 1e6, 1),
                                            "frac": round(10 * na / a_ms / 1e6 / HBM_PEAK_GBS, 4)}}


def mx_workload(torch, amp):
    """MX GEMMs on the block-scaled matrix cores at the FFN up projection
    (8192 x 28672 x 4096, K-contiguous operands as the forward pass has them),
    plus the MX quantizer of the activation and of the weight: MXFP4 (E2M1) and
    MXFP8 (E4M3)."""
    T, I, O = 8192, 4096, 28672
    gen = torch.Generator(device="cuda").manual_seed(11)
    X = torch.randn(T, I, device="cuda", generator=gen).to(torch.bfloat16)
    W = (torch.randn(O, I, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    out = {}
    flops = 2 * T * O * I
    for name, yt, peak in (("mxfp4", amp.E2M1X2, FP4_PEAK_TFLOPS), ("mxfp8", amp.E4M3, FP8_PEAK_TFLOPS),
                           ("mxfp8_native", amp.E4M3, FP8_PEAK_TFLOPS)):
        gflags = amp.GEMM_MX | (amp.GEMM_FP8_NATIVE if name == "mxfp8_native" else 0)
        div = 2 if yt == amp.E2M1X2 else 1
        qx = torch.empty(T * I // div, device="cuda", dtype=torch.uint8)
        qw = torch.empty(O * I // div, device="cuda", dtype=torch.uint8)
        sx = torch.empty(T * I // 32, device="cuda", dtype=torch.uint8)
        sw = torch.empty(O * I // 32, device="cuda", dtype=torch.uint8)
        k = _copies(1 << 30, T * I * 2)
        Xs = [X] + [X.clone() for _ in range(k - 1)]
        qs = [qx] + [torch.empty_like(qx) for _ in range(k - 1)]
        ss = [sx] + [torch.empty_like(sx) for _ in range(k - 1)]
        q_ms = _timed_rot(torch, [lambda i=i: amp.amp_mx_quantize(Xs[i], amp.BF16, T, I, I, 0, yt, qs[i],
                                                                   ss[i]) for i in range(k)], 4 * k)
        del Xs[1:], qs[1:], ss[1:]
        # the weight (28672 x 4096, 3.5x the activation's elements)
        kw = _copies(1 << 30, O * I * 2)
        Ws = [W] + [W.clone() for _ in range(kw - 1)]
        qws = [qw] + [torch.empty_like(qw) for _ in range(kw - 1)]
        sws = [sw] + [torch.empty_like(sw) for _ in range(kw - 1)]
        qw_ms = _timed_rot(torch, [lambda i=i: amp.amp_mx_quantize(Ws[i], amp.BF16, O, I, I, 0, yt, qws[i],
                                                                    sws[i]) for i in range(kw)], 4 * kw)
        del Ws[1:], qws[1:], sws[1:]
        Y = torch.empty(T, O, device="cuda", dtype=torch.bfloat16)
        bsx = amp.BlockScales(sx.data_ptr(), I // 32, 0, 0)
        bsw = amp.BlockScales(sw.data_ptr(), I // 32, 0, 0)
        g_ms = _timed(torch, lambda: amp.amp_gemm_ex(amp.OP_N, amp.OP_T, T, O, I, qx, yt, I // div,
                                                     None, qw, yt, I // div, None, Y, amp.BF16, O,
                                                     bsx, bsw, flags=gflags), 10)
        tf = flops / g_ms / 1e9
        qbytes = T * I * (2 + 1.0 / div + 1.0 / 32)
        wbytes = O * I * (2 + 1.0 / div + 1.0 / 32)
        out[name] = {"gemm_ms": round(g_ms, 4), "gemm_tflops": round(tf, 1), "peak_tflops": peak,
                     "frac": round(tf / peak, 4), "quantize_ms": round(q_ms, 4),
                     "quantize_gbs": round(qbytes / q_ms / 1e6, 1),
                     "quantize_weight_ms": round(qw_ms, 4),
                     "quantize_weight_gbs": round(wbytes / qw_ms / 1e6, 1)}
        if name == "mxfp8":
            out[name]["mfma"] = "bf16 (FP8 x UE8M0 block scale widened exactly; FP32 sums)"
            out[name]["frac_bf16_mfma"] = round(tf / BF16_PEAK_TFLOPS, 4)
        if name == "mxfp8_native":
            out[name]["mfma"] = "block-scaled FP8 (reduced-precision 64-term sums)"
        del qx, qw, sx, sw, Y
    del X, W
    torch.cuda.empty_cache()
    return out


def blockwise_workload(torch, amp):
    """Fine-grained FP8 (1x128 activation / gradient tiles, 128x128 weight
    blocks, E4M3 everywhere) through one FFN up projection (8192 tokens,
    hidden 4096, 28672 outputs): quantize X, W and dY (each with its
    transposed operand in the same pass), then the forward, dgrad and wgrad
    GEMMs with per-128-K promotion."""
    T, I, O = 8192, 4096, 28672
    d = "cuda"
    gen = torch.Generator(device=d).manual_seed(13)
    X = torch.randn(T, I, device=d, generator=gen).to(torch.bfloat16)
    W = (torch.randn(O, I, device=d, generator=gen) * 0.02).to(torch.bfloat16)
    dY = (torch.randn(T, O, device=d, generator=gen) * 1e-3).to(torch.bfloat16)
    u8, f32 = torch.uint8, torch.float32
    qx, qxt = torch.empty(T, I, dtype=u8, device=d), torch.empty(I, T, dtype=u8, device=d)
    sx, sxt = torch.empty(I // 128, T, dtype=f32, device=d), torch.empty(T // 128, I, dtype=f32, device=d)
    qw, qwt = torch.empty(O, I, dtype=u8, device=d), torch.empty(I, O, dtype=u8, device=d)
    sw, swt = (torch.empty(I // 128, O // 128, dtype=f32, device=d),
               torch.empty(O // 128, I // 128, dtype=f32, device=d))
    qd, qdt = torch.empty(T, O, dtype=u8, device=d), torch.empty(O, T, dtype=u8, device=d)
    sd, sdt = torch.empty(O // 128, T, dtype=f32, device=d), torch.empty(T // 128, O, dtype=f32, device=d)
    Y = torch.empty(T, O, dtype=torch.bfloat16, device=d)
    dX = torch.empty(T, I, dtype=torch.bfloat16, device=d)
    dW = torch.empty(O, I, dtype=f32, device=d)
    E4 = amp.E4M3

    def quant():
        amp.amp_quantize_blockwise(X, amp.BF16, T, I, I, E4, 0, qx, I, sx, T, qxt, T, sxt, I)
        amp.amp_quantize_blockwise(W, amp.BF16, O, I, I, E4, 1, qw, I, sw, O // 128, qwt, O, swt, I // 128)
        amp.amp_quantize_blockwise(dY, amp.BF16, T, O, O, E4, 0, qd, O, sd, T, qdt, T, sdt, O)

    def fprop():
        amp.amp_gemm_blockwise(T, O, I, qx, E4, I, sx, T, 0, qw, E4, I, sw, O // 128, 1, Y, amp.BF16, O)

    def dgrad():
        amp.amp_gemm_blockwise(T, I, O, qd, E4, O, sd, T, 0, qwt, E4, O, swt, I // 128, 1, dX,
                               amp.BF16, I)

    def wgrad():
        amp.amp_gemm_blockwise(O, I, T, qdt, E4, T, sdt, O, 0, qxt, E4, T, sxt, I, 0, dW, amp.F32, I)

    q_ms = _timed(torch, quant, 5)
    out = {"quantize_ms": round(q_ms, 4),
           "quantize_gbs": round((T * I + O * I + T * O) * 4 / q_ms / 1e6, 1)}
    flops = 2 * T * I * O
    total = q_ms
    for name, f in (("fprop", fprop), ("dgrad", dgrad), ("wgrad", wgrad)):
        ms = _timed(torch, f, 10)
        total += ms
        tf = flops / ms / 1e9
        out[name] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                     "frac_bf16_mfma": round(tf / BF16_PEAK_TFLOPS, 4)}
    out["layer_ms"] = round(total, 4)
    out["layer_tflops"] = round(3 * flops / total / 1e9, 1)
    out["mfma"] = "bf16 (E4M3 widened exactly; per-128-K FP32 promotion)"
    del X, W, dY, qx, qxt, qw, qwt, qd, qdt, Y, dX, dW
    torch.cuda.empty_cache()
    return out


def measured_traffic():
    """HBM bytes per launch of the apply kernel, from the committed rocprofv3
    counter summary, or None when the kernel sources changed since then."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "apply_kernel_adamw_2pow31_hbm_bytes.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_bytes = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    m_sha = re.search(r"source_sha256_16: (\w+)", text)
    m_src = re.search(r"sources: (.*)", text)
    if not (m_bytes and m_sha and m_src):
        return None
    h = hashlib.sha256()
    for rel in m_src.group(1).split(", "):
        h.update(open(os.path.join(ROOT, rel.strip()), "rb").read())
    if h.hexdigest()[:16] != m_sha.group(1):
        return None
    return int(m_bytes.group(1))


def _oracle_optimizer_worker(args):
    """One host process: the oracle's optimizer step (check + AdamW + FP16
    recast) on its own sample, ``steps`` times; returns the loop time."""
    seed, sample, steps = args
    import numpy as np
    from oracle import adamw as OA
    from oracle import formats as F
    import synth
    theta = synth.normal_f32(seed, sample, 0.02).astype(np.float64)
    g = synth.normal_f32(seed + 1, sample, 1e-4) * np.exp(2.0 * synth.normal_f32(seed + 2, sample))
    codes = synth.to_f16_codes(np.clip(g * 1024.0, -65504, 65504).astype(np.float32))
    m = np.zeros(sample)
    v = np.zeros(sample)
    hp = OA.AdamWHParams(3e-4, 0.9, 0.95, 1e-8, 0.1)
    ctr = OA.AdamCounters()
    t0 = time.perf_counter()
    for _ in range(steps):
        found = OA.found_inf(codes, F.F16)
        theta, m, v, w, ok = OA.apply(theta, m, v, codes, F.F16, hp, ctr, 1024.0, skip=found)
    return time.perf_counter() - t0


def cpu_baseline(sample: int = 1 << 20, steps: int = 8, gemm_mnk=(8192, 6144, 4096)):
    """The oracle as it stands, timed on this host's cores before the GPU is
    touched: the optimizer step under multiprocessing (one process per
    available core, at most 16, each on its own 2^20-parameter sample), and
    the oracle's GEMM reference (float64 C_ref and the sum |a||b| bound, BLAS
    threads) on the QKV forward shape of the transformer block."""
    import multiprocessing
    import numpy as np
    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(16, affinity))
    ctx = multiprocessing.get_context("fork")
    with ctx.Pool(workers) as pool:
        times = pool.map(_oracle_optimizer_worker, [(100 + 3 * i, sample, steps)
                                                    for i in range(workers)])
    dt = max(times)
    gbs = BYTES_PER_PARAM * sample * steps * workers / dt / 1e9
    try:
        import threadpoolctl
        blas = max((i.get("num_threads", 0) for i in threadpoolctl.threadpool_info()
                    if i.get("user_api") == "blas"), default=None)
    except Exception:
        blas = None
    from oracle import gemm as OG
    M, N, K = gemm_mnk
    rng = np.random.default_rng(0)
    a = rng.standard_normal((M, K))
    b = rng.standard_normal((K, N)) * 0.02
    t0 = time.perf_counter()
    OG.reference(a, b)
    g_s = time.perf_counter() - t0
    del a, b
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": f"{workers} processes x {sample} params x {steps} optimizer steps "
                      f"(check + AdamW + FP16 recast, NumPy); slowest process "
                      f"{dt / steps * 1e3:.1f} ms/step; same 28 B/param accounting",
            "host": {"os_cpu_count": os.cpu_count(), "affinity": affinity,
                     "blas_threads": blas},
            "gemm": {"shape": [M, N, K], "what": "oracle GEMM reference on the QKV forward "
                     "shape: float64 C_ref and the sum |a||b| bound (two float64 matmuls)",
                     "s": round(g_s, 3), "gflops": round(2 * M * N * K / g_s / 1e9, 1),
                     "blas_threads": blas}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-components", action="store_true")
    ap.add_argument("--components", default="all",
                    help="comma-separated component names to run (default all; 'none' = none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the hot path here runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding is a design note, not an implemented path.", file=sys.stderr)
        sys.exit(2)

    cpu = None
    if not args.no_cpu_baseline:
        # before anything touches the GPU (the workers are forked)
        log("cpu baseline (oracle)")
        cpu = cpu_baseline()

    import torch
    import mixed_precision_numerics_amd as amp
    amp.load()
    torch.cuda.set_device(0)

    ms_step, apply_ms, ms_single, skip_ms, copy_ms, copy_gbs = optimizer_workload(
        torch, amp, N_PARAMS, args.steps, args.warmup, args.calibrate_copy)
    value = BYTES_PER_PARAM * N_PARAMS / ms_step / 1e6
    achieved = BYTES_PER_PARAM * N_PARAMS / apply_ms / 1e6
    comps = {"optimizer_single_pass": {
        "what": "flag from the producing cast's amax + AdamW pass (SKIP_CHECK) + scaler update",
        "ms": round(ms_single, 4),
        "gbs": round(BYTES_PER_PARAM * N_PARAMS / ms_single / 1e6, 1)},
        "optimizer_skipped_step": {
        "what": "an overflowing step (one +inf gradient): check sweep sets the flag, the AdamW "
                "pass writes nothing, S halves; median of 20",
        "ms": round(skip_ms, 4)}}
    table = (
        ("gemm_bf16_block", "BF16 block GEMMs", lambda: gemm_block_workload(torch, amp, fp8=False)),
        ("gemm_fp8_block", "FP8 delayed-scaling block", lambda: gemm_block_workload(torch, amp, fp8=True)),
        ("gemm_fp8_native_block", "FP8 block on the native FP8 instruction",
         lambda: gemm_block_workload(torch, amp, fp8=True, native=True)),
        ("cast", "cast", lambda: cast_workload(torch, amp)),
        ("cast_t", "cast with transposed copy", lambda: cast_t_workload(torch, amp)),
        ("nvfp4_wgrad", "NVFP4 weight-gradient quantize + GEMM", lambda: nvfp4_workload(torch, amp)),
        ("mx", "MX GEMMs", lambda: mx_workload(torch, amp)),
        ("blockwise_fp8", "fine-grained FP8 (1x128 / 128x128 scales) FFN up projection",
         lambda: blockwise_workload(torch, amp)),
        ("scaling", "delayed vs current scaling casts", lambda: scaling_workload(torch, amp)),
        ("clip", "gradient norm and accumulation", lambda: clip_workload(torch, amp)))
    wanted = set() if (args.no_components or args.components == "none") else (
        {n for n, _, _ in table} if args.components == "all" else set(args.components.split(",")))
    unknown = wanted - {n for n, _, _ in table}
    if unknown:
        raise SystemExit(f"bench.py: unknown components {sorted(unknown)}")
    for name, what, fn in table:
        if name in wanted:
            log(f"components: {what}")
            comps[name] = fn()
    traffic = measured_traffic()

    out = {
        "metric": "scaled GEMM TFLOP/s (bf16/fp8) + fused AMP step GB/s, % of MI355X peak",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "fused AMP optimizer step (unscale + inf/NaN check + AdamW on "
                               "FP32 master + FP16 recast + loss-scale update), 2^31 params",
                   "n_params": N_PARAMS, "grad_dtype": "f16", "bytes_per_param": BYTES_PER_PARAM},
        "skipped_step_ms": round(skip_ms, 4),
        "copy_ceiling_gbs": round(copy_gbs, 1),
        "roofline": {"bound": "hbm", "kernel": "apply_kernel (fused AdamW pass)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "copy_ceiling": {"gbs": round(copy_gbs, 1), "ms": round(copy_ms, 4),
                                      "what": "amp_stream_copy of 4 GiB (read + write), same run",
                                      "apply_over_copy": round(achieved / copy_gbs, 4)},
                     "traffic": None if traffic is None else round(traffic / 1e9, 3),
                     "traffic_unit": "GB per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "copy-calibrated)",
                     "algorithmic": round(BYTES_PER_PARAM * N_PARAMS / 1e9, 3)},
        "components": comps,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
