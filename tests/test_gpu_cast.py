"""Parity of amp_cast (HIP) with the oracle: bit-exact codes and amax."""
import numpy as np
import pytest
import torch

import mixed_precision_numerics_amd as amp
from oracle import cast as OC
from oracle import formats as F
import synth
from gpu_util import dev, empty, f32_dev, host

pytestmark = pytest.mark.gpu

IN = {amp.F32: (F.F32, np.uint32), amp.F16: (F.F16, np.uint16), amp.BF16: (F.BF16, np.uint16)}
OUT = {amp.F16: (F.F16, np.uint16), amp.BF16: (F.BF16, np.uint16),
       amp.E4M3: (F.E4M3, np.uint8), amp.E5M2: (F.E5M2, np.uint8)}


def make_input(xt, n, seed):
    """Heavy-tailed values plus every edge value, as codes of the input type."""
    x = synth.student_t_f32(seed, n, scale=30.0)
    e = synth.edge_f32_values()
    x[: min(n, e.size)] = e[: min(n, e.size)]
    if xt == amp.F32:
        return synth.f32_bits(x).copy()
    if xt == amp.BF16:
        return synth.to_bf16_codes(x)
    return synth.to_f16_codes(np.clip(x, -65504, 65504))


@pytest.mark.parametrize("xt", list(IN))
@pytest.mark.parametrize("yt", list(OUT))
@pytest.mark.parametrize("scaled", [False, True])
def test_flat_cast_bit_exact(xt, yt, scaled):
    n = 100_003                                    # ragged: not a multiple of 8
    codes = make_input(xt, n, seed=10 + xt + 3 * yt)
    scale = 448.0 / 300.0 if scaled else None
    fin, ndt = IN[xt]
    fout, odt = OUT[yt]
    want, want_amax = OC.cast(codes, fin, fout, scale, amax_prior_bits=0)
    x = dev(codes)
    y = empty(n * np.dtype(odt).itemsize)
    amax = f32_dev([0.0])
    sc = f32_dev([scale]) if scaled else None
    amp.amp_cast(x, xt, 1, n, n, y, yt, n, d_scale=sc, d_amax=amax)
    got = host(y, odt)[:n]
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (bad[:10], got[bad[:10]], want[bad[:10]])
    assert host(amax, np.uint32)[0] == want_amax


@pytest.mark.parametrize("n", [1, 2, 7, 8, 9, 8 * 1024, 8 * 1024 + 3, 8 * 1024 * 13 + 5])
def test_flat_cast_sizes_at_range_edges(n):
    """Flat vector path: fewer than 8 elements (the trailing loop only), one
    block pass exactly, and ragged multi-range inputs."""
    codes = make_input(amp.BF16, n, seed=n)
    want, want_amax = OC.cast(codes, F.BF16, F.E4M3, 2.0, amax_prior_bits=0)
    y = empty(n)
    amax = f32_dev([0.0])
    amp.amp_cast(dev(codes), amp.BF16, 1, n, n, y, amp.E4M3, n, d_scale=f32_dev([2.0]), d_amax=amax)
    assert np.array_equal(host(y, np.uint8)[:n], want)
    assert host(amax, np.uint32)[0] == want_amax


def test_flat_cast_multi_pass_ranges():
    """2^29 + 4141 elements: more 2048-vector ranges than work-groups, so every
    work-group converts two or three ranges.  Codes are checked on a sample
    (the range edges, the tail and random indices); amax against three planted
    elements whose magnitude exceeds every other element's by construction."""
    nv = 2 * 16384 * 2048 + 517
    n = 8 * nv + 5
    rng = np.random.default_rng(2024)
    # random sign and mantissa, exponent field 120..127: |x| < 2
    codes = (rng.integers(0, 1 << 16, size=n, dtype=np.uint16) & np.uint16(0x83FF)) | np.uint16(0x3C00)
    planted = np.array([5, n // 2 + 3, n - 2])
    codes[planted] = np.array([0x4480, 0xC5A3, 0x4520], np.uint16)   # 1024, -5216, 2560
    y = empty(n)
    amax = f32_dev([0.0])
    amp.amp_cast(dev(codes), amp.BF16, 1, n, n, y, amp.E4M3, n, d_scale=f32_dev([0.25]),
                 d_amax=amax)
    got = host(y, np.uint8)[:n]
    range_el = 8 * 2048
    edges = np.arange(0, n, range_el)
    idx = np.unique(np.concatenate([
        np.arange(0, 2 * range_el), (edges[:, None] + np.arange(-4, 4)).ravel(),
        np.arange(n - 3 * range_el, n), rng.integers(0, n, size=200_000), planted]))
    idx = idx[(idx >= 0) & (idx < n)]
    want, _ = OC.cast(codes[idx], F.BF16, F.E4M3, 0.25, amax_prior_bits=0)
    bad = np.nonzero(got[idx] != want)[0]
    assert bad.size == 0, (idx[bad[:10]], got[idx[bad[:10]]], want[bad[:10]])
    _, want_amax = OC.cast(codes[planted], F.BF16, F.E4M3, 0.25, amax_prior_bits=0)
    assert host(amax, np.uint32)[0] == want_amax


@pytest.mark.parametrize("xt,yt,scale", [(amp.BF16, amp.E4M3, 64.0), (amp.F32, amp.F16, None)])
def test_flat_cast_full_size_2pow31_sampled(xt, yt, scale):
    """The cast-only workload at its full size, 2^31 elements: BF16 -> E4M3
    with a scale and FP32 -> FP16 (the master-weight recast), both with amax.
    Inputs are generated on the device (uniform in [-2, 2) from a seeded
    generator, then five planted values: three beyond every other magnitude,
    one past the FP16 range, one below its normal range); the oracle gets the
    same input bytes at the sampled indices by a device-to-host gather: every
    range edge of the flat kernel's first and last ranges, a window around
    each of 4096 evenly spaced range starts, the tail, 200,000 random indices
    and the planted ones.  amax is checked against the planted values, which
    exceed every other element's magnitude by construction."""
    n = 1 << 31
    gen = torch.Generator(device="cuda").manual_seed(31)
    x = torch.rand(n, device="cuda", generator=gen)
    x.mul_(4.0).sub_(2.0)
    planted = torch.tensor([5, n // 2 + 3, n - 2, 777777, n - 99], device="cuda")
    x[planted] = torch.tensor([1024.0, -5216.0, 2560.0, 70000.0, 1e-8], device="cuda")
    if xt == amp.BF16:
        x = x.to(torch.bfloat16)
        xbits, ndt = x.view(torch.int16), np.uint16
    else:
        xbits, ndt = x.view(torch.int32), np.uint32
    fin = IN[xt][0]
    fout, odt = OUT[yt]
    y = torch.empty(n * np.dtype(odt).itemsize, device="cuda", dtype=torch.uint8)
    amax = f32_dev([0.0])
    sc = f32_dev([scale]) if scale is not None else None
    amp.amp_cast(x, xt, 1, n, n, y, yt, n, d_scale=sc, d_amax=amax)
    rng = np.random.default_rng(31)
    range_el = 8 * 2048
    starts = np.linspace(0, n - range_el, 4096).astype(np.int64) // range_el * range_el
    idx = np.unique(np.concatenate([
        np.arange(0, 2 * range_el), (starts[:, None] + np.arange(-8, 8)).ravel(),
        np.arange(n - 2 * range_el, n), rng.integers(0, n, size=200_000),
        planted.cpu().numpy()]))
    idx = idx[(idx >= 0) & (idx < n)]
    it = torch.from_numpy(idx).to("cuda")
    xs = xbits[it].cpu().numpy().view(ndt)
    ybits = y.view(torch.int16) if odt == np.uint16 else y
    ys = ybits[it].cpu().numpy().view(odt)
    want, _ = OC.cast(xs, fin, fout, scale, amax_prior_bits=0)
    bad = np.nonzero(ys != want)[0]
    assert bad.size == 0, (idx[bad[:10]], ys[bad[:10]], want[bad[:10]])
    pl = np.searchsorted(idx, planted.cpu().numpy())
    _, want_amax = OC.cast(xs[pl], fin, fout, scale, amax_prior_bits=0)
    assert host(amax, np.uint32)[0] == want_amax
    del x, xbits, y


@pytest.mark.parametrize("xt,yt", [(amp.BF16, amp.E4M3), (amp.BF16, amp.E5M2),
                                   (amp.F32, amp.E4M3), (amp.F32, amp.BF16),
                                   (amp.F16, amp.F16)])
@pytest.mark.parametrize("rows,cols,ldx_pad", [(300, 260, 3), (256, 384, 0), (1, 17, 0),
                                               (129, 127, 8), (304, 264, 0)])
def test_tile_cast_with_transpose(xt, yt, rows, cols, ldx_pad):
    """(304, 264, 0): every row 16-byte aligned on all three operands, so the
    16-byte path runs with partial edge tiles; the other shapes take the
    element path ((300, 260, 3), (1, 17, 0), (129, 127, 8)) or full tiles."""
    fin, ndt = IN[xt]
    fout, odt = OUT[yt]
    ldx = cols + ldx_pad
    codes = make_input(xt, rows * ldx, seed=rows + cols).reshape(rows, ldx)
    scale = 2.0 ** 3 * 1.1
    want, want_amax = OC.cast(codes[:, :cols], fin, fout, scale)
    ldy, ldyt = cols + 16, rows + 32
    x = dev(codes)
    y = empty(rows * ldy * np.dtype(odt).itemsize, fill=0xAB)
    yt_buf = empty(cols * ldyt * np.dtype(odt).itemsize, fill=0xCD)
    amax = f32_dev([0.5])
    amp.amp_cast(x, xt, rows, cols, ldx, y, yt, ldy, yt_buf, ldyt, f32_dev([scale]), amax)
    gy = host(y, odt).reshape(rows, ldy)
    gt = host(yt_buf, odt).reshape(cols, ldyt)
    assert np.array_equal(gy[:, :cols], want)
    assert np.array_equal(gt[:, :rows], want.T)
    # padding untouched
    pad = 0xAB if odt == np.uint8 else 0xABAB
    assert np.all(gy[:, cols:] == pad)
    prior = int(synth.f32_bits(np.array([0.5], np.float32))[0])
    assert host(amax, np.uint32)[0] == max(prior, int(want_amax))


def test_transpose_only_output_and_no_amax():
    rows, cols = 512, 1024
    codes = synth.bf16_codes_normal(3, (rows, cols))
    want, _ = OC.cast(codes, F.BF16, F.E5M2, 1000.0)
    yt_buf = empty(cols * rows)
    amp.amp_cast(dev(codes), amp.BF16, rows, cols, cols, None, amp.E5M2, 0, yt_buf, rows,
                 f32_dev([1000.0]), None)
    assert np.array_equal(host(yt_buf, np.uint8).reshape(cols, rows), want.T)


def test_unaligned_pointers_use_scalar_path():
    n = 4097
    codes = make_input(amp.F32, n + 1, 77)
    x = dev(codes)
    y = empty(2 * (n + 1))
    want, am = OC.cast(codes[1:], F.F32, F.F16, None)
    amax = f32_dev([0.0])
    amp.amp_cast(x.data_ptr() + 4, amp.F32, 1, n, n, y.data_ptr() + 2, amp.F16, n, d_amax=amax)
    assert np.array_equal(host(y, np.uint16)[1:n + 1], want)
    assert host(amax, np.uint32)[0] == am


def test_amax_is_order_free_and_deterministic():
    n = 1 << 22
    codes = synth.bf16_codes_normal(9, n)
    x = dev(codes)
    y = empty(n)
    res = []
    for _ in range(3):
        amax = f32_dev([0.0])
        amp.amp_cast(x, amp.BF16, 1, n, n, y, amp.E4M3, n, d_scale=f32_dev([64.0]), d_amax=amax)
        res.append(int(host(amax, np.uint32)[0]))
    want = int(OC.amax_bits(OC.widen_to_f32_bits(codes, F.BF16)))
    assert res == [want] * 3


def _structured_f32_bits(low_bits, patterns, seed=0):
    """Every sign/exponent/top-mantissa combination with chosen low bits."""
    top = np.arange(1 << (32 - low_bits), dtype=np.uint64) << np.uint64(low_bits)
    rnd = np.random.default_rng(seed).integers(0, 1 << low_bits, size=top.size, dtype=np.uint64)
    parts = [top | np.uint64(p) for p in patterns] + [top | rnd]
    return np.concatenate(parts).astype(np.uint32)


@pytest.mark.parametrize("yt,low,pats", [
    (amp.F16, 13, [0, 1, 0xFFF, 0x1000, 0x1001, 0x1FFF]),
    (amp.BF16, 16, [0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF]),
    (amp.E4M3, 20, [0, 1, 0x7FFFF, 0x80000, 0x80001, 0xFFFFF]),
    (amp.E5M2, 21, [0, 1, 0xFFFFF, 0x100000, 0x100001, 0x1FFFFF])])
def test_cast_structured_sweep_of_all_binades(yt, low, pats):
    """All FP32 exponents and leading mantissa bits, each with the rounding-
    critical low bit patterns (exact ties, one above, one below, random)."""
    bits = _structured_f32_bits(low, pats, seed=yt)
    fout, odt = OUT[yt]
    want, want_amax = OC.cast(bits, F.F32, fout, None)
    n = bits.size
    y = empty(n * np.dtype(odt).itemsize)
    amax = f32_dev([0.0])
    amp.amp_cast(dev(bits), amp.F32, 1, n, n, y, yt, n, d_amax=amax)
    got = host(y, odt)[:n]
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (bad[:8], bits[bad[:8]], got[bad[:8]], want[bad[:8]])
    assert host(amax, np.uint32)[0] == want_amax


@pytest.mark.parametrize("xt,yt,ld_pad,transposed", [
    (amp.BF16, amp.E4M3, 0, True), (amp.F32, amp.E4M3, 5, True), (amp.BF16, amp.E5M2, 0, False),
    (amp.F16, amp.E5M2, 3, False), (amp.F32, amp.E5M2, 0, False)])
def test_current_scaling_cast(xt, yt, ld_pad, transposed):
    """amp_cast_current_scaling: amax of this tensor, scale from it, cast with
    it -- meta and codes bit-exact (oracle recipe.current_scale + cast)."""
    from oracle import recipe as OR
    rows, cols = 515, 389
    ldx = cols + ld_pad
    x = synth.student_t_f32(60 + xt, rows * ldx, scale=7.0).reshape(rows, ldx)
    if xt == amp.F32:
        codes = synth.f32_bits(x).copy()
    elif xt == amp.BF16:
        codes = synth.to_bf16_codes(x)
    else:
        codes = synth.to_f16_codes(np.clip(x, -65504, 65504))
    fin, _ = IN[xt]
    fout, odt = OUT[yt]
    fmax = 448.0 if yt == amp.E4M3 else 57344.0
    r = amp.DelayedRecipe(fmax, 1.0, 1024, amp.AMAX_MAX)
    meta = empty(16)
    y = empty(rows * cols, fill=0xAB)
    yt_buf = empty(rows * cols, fill=0xAB) if transposed else None
    amp.amp_cast_current_scaling(dev(codes), xt, rows, cols, ldx, y, yt, cols, yt_buf, rows, r, meta)
    view = codes[:, :cols]
    am = int(OC.amax_bits(OC.widen_to_f32_bits(view.ravel(), fin)))
    sc, inv = OR.current_scale(am, fmax, 1.0)
    m = host(meta, amp.FP8_META_DTYPE)[0]
    assert int(np.float32(m["amax_cur"]).view(np.uint32)) == am
    assert m["scale"] == np.float32(sc) and m["scale_inv"] == np.float32(inv)
    want, _ = OC.cast(view.ravel(), fin, fout, sc)
    assert np.array_equal(host(y, odt)[:rows * cols], want)
    if transposed:
        assert np.array_equal(host(yt_buf, odt)[:rows * cols].reshape(cols, rows),
                              want.reshape(rows, cols).T)


def test_current_scaling_amax_over_many_ranges():
    """The amax pass of current scaling over 2^29 + 4141 BF16 elements (more
    2048-vector ranges than work-groups, a ragged tail), generated on the
    device: uniform in [-2, 2) plus three planted values, the largest in the
    tail.  amax_cur and the scale equal the oracle's from the planted values;
    the codes are checked at range edges, the tail and random indices."""
    from oracle import recipe as OR
    nv = 2 * 16384 * 2048 + 517
    n = 8 * nv + 5
    gen = torch.Generator(device="cuda").manual_seed(41)
    x = torch.rand(n, device="cuda", generator=gen)
    x.mul_(4.0).sub_(2.0)
    planted = torch.tensor([3, n // 3, n - 1], device="cuda")
    x[planted] = torch.tensor([-300.0, 700.0, -1500.0], device="cuda")
    x = x.to(torch.bfloat16)
    r = amp.DelayedRecipe(448.0, 1.0, 1024, amp.AMAX_MAX)
    meta = empty(16)
    y = torch.empty(n, device="cuda", dtype=torch.uint8)
    amp.amp_cast_current_scaling(x, amp.BF16, 1, n, n, y, amp.E4M3, n, None, 0, r, meta)
    pl = planted.cpu().numpy()
    xb = x.view(torch.int16)
    am = int(OC.amax_bits(OC.widen_to_f32_bits(xb[planted].cpu().numpy().view(np.uint16), F.BF16)))
    sc, inv = OR.current_scale(am, 448.0, 1.0)
    m = host(meta, amp.FP8_META_DTYPE)[0]
    assert int(np.float32(m["amax_cur"]).view(np.uint32)) == am
    assert m["scale"] == np.float32(sc) and m["scale_inv"] == np.float32(inv)
    rng = np.random.default_rng(41)
    range_el = 8 * 2048
    idx = np.unique(np.concatenate([
        np.arange(0, 2 * range_el), (np.arange(0, n, 64 * range_el)[:, None] + np.arange(-4, 4)).ravel(),
        np.arange(n - 2 * range_el, n), rng.integers(0, n, size=100_000), pl]))
    idx = idx[(idx >= 0) & (idx < n)]
    it = torch.from_numpy(idx).to("cuda")
    xs = xb[it].cpu().numpy().view(np.uint16)
    want, _ = OC.cast(xs, F.BF16, F.E4M3, sc)
    got = y[it].cpu().numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (idx[bad[:10]], got[bad[:10]], want[bad[:10]])


@pytest.mark.parametrize("fill", ["zero", "nan"])
def test_current_scaling_degenerate(fill):
    from oracle import recipe as OR
    n = 4096
    codes = np.zeros(n, np.uint16) if fill == "zero" else np.full(n, 0x3C00, np.uint16)
    if fill == "nan":
        codes[100] = 0x7FC1
    r = amp.DelayedRecipe(448.0, 1.0, 1024, amp.AMAX_MAX)
    meta = empty(16)
    y = empty(n)
    amp.amp_cast_current_scaling(dev(codes), amp.BF16, 1, n, n, y, amp.E4M3, n, None, 0, r, meta)
    m = host(meta, amp.FP8_META_DTYPE)[0]
    assert m["scale"] == 1.0 and m["scale_inv"] == 1.0
    want, _ = OC.cast(codes, F.BF16, F.E4M3, 1.0)
    assert np.array_equal(host(y, np.uint8)[:n], want)


@pytest.mark.parametrize("yt", [amp.E4M3, amp.E5M2, amp.F16])
@pytest.mark.parametrize("layout", ["flat", "tile", "tile_t"])
def test_cast_saturation_count(yt, layout):
    """amp_cast_ex counts the clipped elements (oracle.cast.saturated_count):
    flat path, strided tile path, and tile path with the transposed copy."""
    rows, cols = 300, 200
    x = synth.student_t_f32(140 + yt, (rows, cols), 3.0, 150.0)
    x[3, 5] = np.inf
    x[4, 6] = np.nan
    x[7, :] = 448.0
    xc = synth.to_bf16_codes(x)
    ldx = cols if layout == "flat" else cols + 8
    buf = np.zeros((rows, ldx), np.uint16)
    buf[:, :cols] = xc
    scale = np.float32(1.5)
    yb = 1 if yt != amp.F16 else 2
    y = empty(rows * ldx * yb)
    y_t = empty(rows * cols * yb) if layout == "tile_t" else None
    sat = empty(8)
    amp.amp_cast_ex(dev(buf), amp.BF16, rows, cols, ldx, y, yt, ldx, y_t, rows if y_t is not None else 0,
                    dev(np.array([scale])), None, sat)
    want = OC.saturated_count(xc, F.BF16, {amp.E4M3: F.E4M3, amp.E5M2: F.E5M2, amp.F16: F.F16}[yt],
                              float(scale))
    assert int(host(sat, np.uint64)[0]) == want
    if yt == amp.E4M3:
        assert want > 100

