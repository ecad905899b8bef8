"""MX block formats on the GPU: amp_mx_quantize bit-exact against oracle/mx.py
and the MX GEMM (E2M1 on CDNA4's block-scaled matrix cores, FP8 elements
widened exactly to BF16 times their block scale, or on the block-scaled FP8
instruction on request) against the float64 product of the dequantized
operands."""
import numpy as np
import pytest

import mixed_precision_numerics_amd as amp
from oracle import formats as F
from oracle import gemm as OG
from oracle import mx as OM
import synth
from gpu_util import dev, empty, host

pytestmark = pytest.mark.gpu

YF = {amp.E4M3: F.E4M3, amp.E5M2: F.E5M2, amp.E2M1X2: F.E2M1}


def mx_input(seed, rows, cols, xt):
    x = synth.student_t_f32(seed, (rows, cols), scale=3.0)
    x[1, :] = 0.0                                 # zero blocks (plain and transposed)
    x[:, 2] *= 2.0 ** 40                          # huge and tiny columns
    x[:, 3] *= 2.0 ** -40
    x[5, 7] = np.nan
    x[9, 40] = -np.inf
    if xt == amp.F32:
        return synth.f32_bits(x).copy(), F.decode(synth.f32_bits(x), F.F32)
    codes = synth.to_bf16_codes(x)
    return codes, F.decode(codes, F.BF16)


@pytest.mark.parametrize("xt", [amp.BF16, amp.F32])
@pytest.mark.parametrize("yt", [amp.E4M3, amp.E5M2, amp.E2M1X2])
@pytest.mark.parametrize("transpose", [False, True])
def test_mx_quantize_bit_exact(xt, yt, transpose):
    rows, cols = 96, 160
    codes, vals = mx_input(70 + xt + yt, rows, cols, xt)
    R, K = (cols, rows) if transpose else (rows, cols)
    qbytes = R * K // 2 if yt == amp.E2M1X2 else R * K
    q = empty(qbytes, fill=0xEE)
    sc = empty(R * K // 32, fill=0xEE)
    amp.amp_mx_quantize(dev(codes), xt, rows, cols, cols, transpose, yt, q, sc)
    wq, ws = OM.quantize(vals, YF[yt], transpose=transpose)
    if yt == amp.E2M1X2:
        wq = OM.pack_e2m1(wq)
    assert np.array_equal(host(sc, np.uint8)[:R * K // 32].reshape(ws.shape), ws)
    got = host(q, np.uint8)[:qbytes].reshape(wq.shape)
    bad = np.argwhere(got != wq)
    assert bad.size == 0, (bad[:5], got[tuple(bad[0])], wq[tuple(bad[0])])


@pytest.mark.parametrize("xt", [amp.BF16, amp.F32])
@pytest.mark.parametrize("yt", [amp.E4M3, amp.E2M1X2])
@pytest.mark.parametrize("rows,cols,ld_pad", [(257, 4096, 0), (96, 160, 32), (10, 64, 0)])
def test_mx_quantize_plain_layouts(xt, yt, rows, cols, ld_pad):
    """Plain operand: contiguous rows (one flat stream of blocks, many
    work-groups and a ragged last one; a single block row) and padded rows
    (per-block threads)."""
    codes, vals = mx_input(90 + xt + yt + rows, rows, cols, xt)
    ldx = cols + ld_pad
    padded = np.zeros((rows, ldx), codes.dtype)
    padded[:, :cols] = codes
    qbytes = rows * cols // 2 if yt == amp.E2M1X2 else rows * cols
    q = empty(qbytes, fill=0xEE)
    sc = empty(rows * cols // 32, fill=0xEE)
    amp.amp_mx_quantize(dev(padded), xt, rows, cols, ldx, 0, yt, q, sc)
    wq, ws = OM.quantize(vals, YF[yt], transpose=False)
    if yt == amp.E2M1X2:
        wq = OM.pack_e2m1(wq)
    assert np.array_equal(host(sc, np.uint8)[:rows * cols // 32].reshape(ws.shape), ws)
    got = host(q, np.uint8)[:qbytes].reshape(wq.shape)
    bad = np.argwhere(got != wq)
    assert bad.size == 0, (bad[:5], got[tuple(bad[0])], wq[tuple(bad[0])])


def mx_operand(seed, rows, k, yt):
    """Random MX operand: element codes and UE8M0 scales around 2^0."""
    g = synth.rng(seed)
    if yt == amp.E2M1X2:
        q = g.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
        codes = np.stack([q & 0xF, q >> 4], axis=2).reshape(rows, k)
    else:
        codes = g.integers(0, 256, size=(rows, k), dtype=np.uint8)
        nan = 0x7F if yt == amp.E4M3 else None
        fin = np.isfinite(F.decode(codes, YF[yt]))
        codes = np.where(fin, codes, 0x38).astype(np.uint8)      # replace inf/NaN codes by 1.0
        q = codes
    sc = g.integers(120, 135, size=(rows, k // 32), dtype=np.uint8)
    return q, codes.astype(np.uint8), sc


def run_mx_gemm(M, N, K, at, bt, ct=amp.F32, seed=0, native=False, scales=None, edit=None):
    qa, ca, sa = mx_operand(seed + 1, M, K, at)
    qb, cb, sb = mx_operand(seed + 2, N, K, bt)
    if scales is not None:                  # ((A lo, A hi), (B lo, B hi)) inclusive code ranges
        g = synth.rng(seed + 3)
        (alo, ahi), (blo, bhi) = scales
        sa = g.integers(alo, ahi + 1, size=sa.shape, dtype=np.uint8)
        sb = g.integers(blo, bhi + 1, size=sb.shape, dtype=np.uint8)
    if edit is not None:
        edit(sa, sb)
    lda = K // 2 if at == amp.E2M1X2 else K
    ldb = K // 2 if bt == amp.E2M1X2 else K
    c = empty(M * N * 4)
    sa_d, sb_d = dev(sa), dev(sb)
    amp.amp_gemm_ex(amp.OP_N, amp.OP_T, M, N, K, dev(qa), at, lda, None, dev(qb), bt, ldb, None,
                    c, ct, N, amp.BlockScales(sa_d.data_ptr(), K // 32, 0, 0),
                    amp.BlockScales(sb_d.data_ptr(), K // 32, 0, 0),
                    flags=amp.GEMM_MX | (amp.GEMM_FP8_NATIVE if native else 0))
    A = OM.dequantize(ca, sa, YF[at])
    B = OM.dequantize(cb, sb, YF[bt])
    cref, bound = OG.reference(A, B.T)
    return host(c, np.float32).reshape(M, N).astype(np.float64), cref, bound


@pytest.mark.parametrize("M,N,K", [(512, 768, 512), (256, 512, 768), (256, 256, 256), (256, 512, 1280),
                                   (200, 100, 96)])
def test_mxfp4_gemm_within_fp32_accumulation_bound(M, N, K):
    """E2M1 x E2M1 with UE8M0 scales: full tiles on the block-scaled matrix
    cores (products of E2M1 values are short, so the per-instruction sums are
    exact), ragged shapes on the element-wise kernel: both within the FP32
    accumulation bound."""
    out, cref, bound = run_mx_gemm(M, N, K, amp.E2M1X2, amp.E2M1X2)
    ok = OG.check_f32(out, cref, bound)
    assert ok.all(), (np.argwhere(~ok)[:5], np.max(np.abs(out - cref) / np.maximum(bound, 1e-300)))


@pytest.mark.parametrize("K", [1024, 384])          # an even and an odd number of K-steps
@pytest.mark.parametrize("at,bt", [(amp.E4M3, amp.E4M3), (amp.E5M2, amp.E4M3),
                                   (amp.E4M3, amp.E5M2), (amp.E5M2, amp.E5M2)])
def test_mxfp8_gemm_within_fp32_accumulation_bound(at, bt, K):
    """FP8 elements widened to BF16 times their block scale (exact) on the
    BF16 matrix cores: every output within 1e-5 * sum|ab|."""
    out, cref, bound = run_mx_gemm(512, 512, K, at, bt, seed=5)
    ok = OG.check_f32(out, cref, bound)
    assert ok.all(), (np.argwhere(~ok)[:5], np.max(np.abs(out - cref) / np.maximum(bound, 1e-300)))


@pytest.mark.parametrize("at,bt,scales", [
    (amp.E4M3, amp.E4M3, ((3, 40), (210, 246))),       # E4M3 exact range: codes 3..246
    (amp.E5M2, amp.E4M3, ((200, 239), (15, 54))),      # E5M2 exact range: codes 10..239
    (amp.E5M2, amp.E5M2, ((10, 50), (200, 239)))])
def test_mxfp8_gemm_extreme_block_scales(at, bt, scales):
    """Block scales at both ends of the widened route's exact range (every
    scaled element still a BF16 value), paired so that the products stay in
    FP32's range: within the FP32-accumulation bound."""
    out, cref, bound = run_mx_gemm(256, 256, 256, at, bt, seed=11, scales=scales)
    ok = OG.check_f32(out, cref, bound)
    fin = (bound < 2.0 ** 120) & (bound > 2.0 ** -100)
    assert fin.mean() > 0.99
    assert ok[fin].all(), (np.argwhere(~ok & fin)[:5])


def test_mxfp8_gemm_nan_block_scale():
    """A UE8M0 scale of 0xFF makes its block NaN, and every output that block
    reaches NaN; the others are unaffected."""
    def edit(sa, sb):
        sa[3, 1] = 0xFF          # row 3 of A, K block 1
        sb[7, 0] = 0xFF          # column 7 of B, K block 0
    out, cref, bound = run_mx_gemm(256, 256, 256, amp.E4M3, amp.E4M3, seed=13, edit=edit)
    nan = np.isnan(out)
    assert nan[3, :].all() and nan[:, 7].all()
    keep = np.ones_like(nan)
    keep[3, :] = False
    keep[:, 7] = False
    assert not nan[keep].any()
    assert OG.check_f32(out[keep], cref[keep], bound[keep]).all()


@pytest.mark.parametrize("K", [1024, 384])
@pytest.mark.parametrize("at,bt", [(amp.E4M3, amp.E4M3), (amp.E5M2, amp.E4M3)])
def test_mxfp8_native_instruction_precision_report(at, bt, K):
    """FP8 elements on the block-scaled FP8 matrix cores (AMP_GEMM_FP8_NATIVE):
    the 64-term sums have the reduced internal precision of the FP8
    instruction (documented); assert the measured bound and report how many
    outputs meet 1e-5 * sum|ab|."""
    out, cref, bound = run_mx_gemm(512, 512, K, at, bt, seed=5, native=True)
    rel = np.abs(out - cref) / np.maximum(bound, 1e-300)
    frac = float(np.mean(rel <= OG.RTOL))
    print(f"MXFP8 {at}x{bt}: max |err|/sum|ab| = {rel.max():.3g}, within 1e-5: {frac:.4f}")
    assert rel.max() <= 2.0 ** -10


def test_mxfp8_gemm_ragged_is_exact_route():
    out, cref, bound = run_mx_gemm(100, 130, 64, amp.E4M3, amp.E5M2, seed=9)
    assert OG.check_f32(out, cref, bound).all()


def test_mx_quantize_then_gemm_matches_oracle_quantization():
    """X [512 x 1024] and W [768 x 1024] (BF16) quantized to MXFP4 on the GPU,
    multiplied on the block-scaled matrix cores; the oracle quantizes the same
    inputs and forms the float64 product."""
    M, N, K = 512, 768, 1024
    xc = synth.outlier_bf16_codes(81, (M, K))
    wc = synth.to_bf16_codes(synth.normal_f32(82, (N, K), 0.05))
    qx, sx = empty(M * K // 2), empty(M * K // 32)
    qw, sw = empty(N * K // 2), empty(N * K // 32)
    amp.amp_mx_quantize(dev(xc), amp.BF16, M, K, K, 0, amp.E2M1X2, qx, sx)
    amp.amp_mx_quantize(dev(wc), amp.BF16, N, K, K, 0, amp.E2M1X2, qw, sw)
    c = empty(M * N * 2)
    amp.amp_gemm_ex(amp.OP_N, amp.OP_T, M, N, K, qx, amp.E2M1X2, K // 2, None, qw, amp.E2M1X2,
                    K // 2, None, c, amp.BF16, N, amp.BlockScales(sx.data_ptr(), K // 32, 0, 0),
                    amp.BlockScales(sw.data_ptr(), K // 32, 0, 0), flags=amp.GEMM_MX)
    cx, scx = OM.quantize(F.decode(xc, F.BF16), F.E2M1)
    cw, scw = OM.quantize(F.decode(wc, F.BF16), F.E2M1)
    cref, bound = OG.reference(OM.dequantize(cx, scx, F.E2M1), OM.dequantize(cw, scw, F.E2M1).T)
    ok = OG.check_rounded(host(c, np.uint16).reshape(M, N), F.BF16, cref, bound)
    assert ok.all(), np.argwhere(~ok)[:5]
