"""Parity of amp_gemm (HIP, MFMA) with the float64 oracle.

Tolerance (stated by the workload definition): per element
|C_gpu - C_ref| <= 1e-5 * sum_k |a_ik| |b_kj| before output rounding, and a
rounded output within one output-format ulp of that band."""
import numpy as np
import pytest
import torch

import mixed_precision_numerics_amd as amp
from oracle import cast as OC
from oracle import formats as F
from oracle import gemm as OG
import synth
from gpu_util import dev, empty, f32_dev, host

pytestmark = pytest.mark.gpu

FMT = {amp.BF16: F.BF16, amp.F16: F.F16, amp.E4M3: F.E4M3, amp.E5M2: F.E5M2}
CT = {amp.F32: (F.F32, np.uint32, 4), amp.BF16: (F.BF16, np.uint16, 2), amp.F16: (F.F16, np.uint16, 2)}


def run_gemm(opA, opB, M, N, K, a_codes, at, lda, b_codes, bt, ldb, ct, alphaA=None,
             alphaB=None, flags=0, ldc=None):
    ldc = ldc or N
    c = empty(M * ldc * CT[ct][2], fill=0x7F)
    amp.amp_gemm_ex(opA, opB, M, N, K, dev(a_codes), at, lda,
                    f32_dev([alphaA]) if alphaA is not None else None, dev(b_codes), bt, ldb,
                    f32_dev([alphaB]) if alphaB is not None else None, c, ct, ldc, flags=flags)
    return host(c, CT[ct][1]).reshape(M, ldc)[:, :N]


def ref_values(opA, opB, M, N, K, a_codes, at, b_codes, bt):
    a = F.decode(a_codes, FMT[at]).reshape(a_codes.shape)
    b = F.decode(b_codes, FMT[bt]).reshape(b_codes.shape)
    A = a if opA == amp.OP_N else a.T
    B = b if opB == amp.OP_N else b.T
    return A[:M, :K], B[:K, :N]


def check(out, ct, cref, bound, what):
    fmt = CT[ct][0]
    if ct == amp.F32:
        ok = OG.check_f32(out.view(np.float32).astype(np.float64), cref, bound)
    else:
        ok = OG.check_rounded(out, fmt, cref, bound)
    bad = np.argwhere(~ok)
    assert bad.size == 0, (what, bad[:5], out[tuple(bad[0])], cref[tuple(bad[0])], bound[tuple(bad[0])])


def codes_16(et, shape, seed, std=1.0):
    x = synth.normal_f32(seed, shape, std)
    return synth.to_bf16_codes(x) if et == amp.BF16 else synth.to_f16_codes(x)


@pytest.mark.parametrize("et", [amp.BF16, amp.F16])
@pytest.mark.parametrize("opA,opB", [(amp.OP_N, amp.OP_T), (amp.OP_N, amp.OP_N),
                                     (amp.OP_T, amp.OP_N), (amp.OP_T, amp.OP_T)])
@pytest.mark.parametrize("ct", [amp.F32, amp.BF16])
def test_gemm_16bit_layouts_ragged(et, opA, opB, ct):
    M, N, K = 300, 520, 200          # several 256-tiles, ragged in M, N and K
    a_shape = (M, K) if opA == amp.OP_N else (K, M)
    b_shape = (K, N) if opB == amp.OP_N else (N, K)
    a = codes_16(et, a_shape, 1)
    b = codes_16(et, b_shape, 2, 0.02)
    out = run_gemm(opA, opB, M, N, K, a, et, a_shape[1], b, et, b_shape[1], ct, alphaA=0.5,
                   alphaB=3.0)
    A, B = ref_values(opA, opB, M, N, K, a, et, b, et)
    cref, bound = OG.reference(A, B, alpha=1.5)
    check(out, ct, cref, bound, (opA, opB))


@pytest.mark.parametrize("M,N,K,opA,opB", [(64, 10, 2048, amp.OP_N, amp.OP_T),
                                           (64, 2048, 10, amp.OP_N, amp.OP_N),
                                           (10, 2048, 64, amp.OP_T, amp.OP_N),
                                           (7, 13, 5, amp.OP_T, amp.OP_T)])
def test_gemm_small_odd_shapes(M, N, K, opA, opB):
    a_shape = (M, K) if opA == amp.OP_N else (K, M)
    b_shape = (K, N) if opB == amp.OP_N else (N, K)
    a = codes_16(amp.F16, a_shape, 3)
    b = codes_16(amp.F16, b_shape, 4)
    out = run_gemm(opA, opB, M, N, K, a, amp.F16, a_shape[1], b, amp.F16, b_shape[1], amp.F16)
    A, B = ref_values(opA, opB, M, N, K, a, amp.F16, b, amp.F16)
    cref, bound = OG.reference(A, B)
    check(out, amp.F16, cref, bound, "small")


def test_gemm_k_zero_and_padded_ldc():
    M, N = 40, 24
    a = np.zeros((M, 8), np.uint16); b = np.zeros((N, 8), np.uint16)
    out = run_gemm(amp.OP_N, amp.OP_T, M, N, 0, a, amp.BF16, 8, b, amp.BF16, 8, amp.F32, ldc=N + 5)
    assert np.all(out.view(np.float32) == 0.0)


@pytest.mark.parametrize("kind", ["bf16", "f16", "fp8", "fp8_native", "nvfp4", "mx4", "mx8"])
@pytest.mark.parametrize("ct", [amp.F32, amp.BF16])
def test_gemm_k_zero_full_tiles(kind, ct):
    """K == 0 on whole 256x256 tiles (the shapes that reach the direct-to-LDS
    kernels otherwise): C is zero and no operand or scale is read (all the
    operand pointers given are one-byte buffers and lda = ldb = 0 is valid)."""
    M, N = 512, 256
    at = {"bf16": amp.BF16, "f16": amp.F16, "fp8": amp.E4M3, "fp8_native": amp.E4M3,
          "nvfp4": amp.E2M1X2, "mx4": amp.E2M1X2, "mx8": amp.E5M2}[kind]
    flags = {"fp8_native": amp.GEMM_FP8_NATIVE, "mx4": amp.GEMM_MX, "mx8": amp.GEMM_MX}.get(kind, 0)
    one = empty(16)
    bs = amp.BlockScales(one.data_ptr(), 0, 0) if kind in ("nvfp4", "mx4", "mx8") else None
    c = empty(M * N * CT[ct][2], fill=0x7F)
    amp.amp_gemm_ex(amp.OP_N, amp.OP_T, M, N, 0, one, at, 0, None, one, at, 0, None, c, ct, N,
                    bsA=bs, bsB=bs, flags=flags)
    assert np.all(host(c, CT[ct][1]) == 0)


def fp8_operands(seed, M, N, K, fa, fb):
    x = synth.student_t_f32(seed, (M, K), scale=3.0)
    w = synth.normal_f32(seed + 1, (N, K), 0.02)
    sx = 448.0 / float(np.abs(x).max()) if fa == amp.E4M3 else 57344.0 / float(np.abs(x).max())
    sw = 448.0 / float(np.abs(w).max())
    a, _ = OC.cast(synth.f32_bits(x), F.F32, FMT[fa], sx)
    b, _ = OC.cast(synth.f32_bits(w), F.F32, FMT[fb], sw)
    return a.reshape(M, K), b.reshape(N, K), float(np.float32(1 / np.float32(sx))), float(np.float32(1 / np.float32(sw)))


@pytest.mark.parametrize("fa,fb", [(amp.E4M3, amp.E4M3), (amp.E5M2, amp.E4M3)])
@pytest.mark.parametrize("ct", [amp.F32, amp.BF16])
def test_gemm_fp8_exact_path(fa, fb, ct):
    M, N, K = 272, 300, 384
    a, b, ia, ib = fp8_operands(5, M, N, K, fa, fb)
    out = run_gemm(amp.OP_N, amp.OP_T, M, N, K, a, fa, K, b, fb, K, ct, alphaA=ia, alphaB=ib)
    A, B = ref_values(amp.OP_N, amp.OP_T, M, N, K, a, fa, b, fb)
    alpha = float(np.float32(np.float32(ia) * np.float32(ib)))
    cref, bound = OG.reference(A, B, alpha=alpha)
    check(out, ct, cref, bound, "fp8 exact")


@pytest.mark.parametrize("fmt", [amp.E4M3, amp.E5M2])
def test_fp8_decode_every_code_via_identity(fmt):
    """C = A @ I reproduces every FP8 code exactly (checks the widening)."""
    K = N = 256
    codes = np.arange(256, dtype=np.uint8)
    vals = F.decode(codes, FMT[fmt])
    codes = np.where(np.isfinite(vals), codes, 0).astype(np.uint8)
    a = np.stack([np.roll(codes, 17 * r) for r in range(16)])
    eye = np.where(np.eye(N, K, dtype=bool), np.uint8(0x38), np.uint8(0)).astype(np.uint8)
    out = run_gemm(amp.OP_N, amp.OP_T, 16, N, K, a, fmt, K, eye, amp.E4M3, K, amp.F32)
    assert np.array_equal(out.view(np.float32).astype(np.float64), F.decode(a, FMT[fmt]))


@pytest.mark.parametrize("K", [4096, 384])          # an even and an odd number of K-steps
def test_gemm_fp8_native_precision_report(K):
    """The FP8 matrix-core path: report its error against the bound (its
    64-term partial sums have reduced internal precision); require 2^-10."""
    M, N = 512, 512
    a, b, ia, ib = fp8_operands(7, M, N, K, amp.E4M3, amp.E4M3)
    out = run_gemm(amp.OP_N, amp.OP_T, M, N, K, a, amp.E4M3, K, b, amp.E4M3, K, amp.F32,
                   flags=amp.GEMM_FP8_NATIVE)
    A, B = ref_values(amp.OP_N, amp.OP_T, M, N, K, a, amp.E4M3, b, amp.E4M3)
    cref, bound = OG.reference(A, B)
    rel = np.abs(out.view(np.float32).astype(np.float64) - cref) / bound
    print(f"fp8 native: max |err|/bound {rel.max():.3e}, mean {rel.mean():.3e}, "
          f"frac > 1e-5: {(rel > 1e-5).mean():.4f}")
    assert rel.max() < 2.0 ** -10


@pytest.mark.parametrize("name,M,N,K,opA,opB", [
    ("qkv_fwd", 8192, 6144, 4096, amp.OP_N, amp.OP_T),
    ("qkv_dgrad", 8192, 4096, 6144, amp.OP_N, amp.OP_N),
    ("qkv_wgrad", 6144, 4096, 8192, amp.OP_T, amp.OP_N),
])
def test_gemm_bf16_full_size_sampled(name, M, N, K, opA, opB):
    """Transformer-block shapes (hidden 4096, 8192 tokens): sampled entries."""
    a_shape = (M, K) if opA == amp.OP_N else (K, M)
    b_shape = (K, N) if opB == amp.OP_N else (N, K)
    g = torch.Generator(device="cuda").manual_seed(11)
    a_d = torch.randn(a_shape, generator=g, device="cuda").to(torch.bfloat16)
    b_d = (torch.randn(b_shape, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    amp.amp_gemm(opA, opB, M, N, K, a_d, amp.BF16, a_shape[1], None, b_d, amp.BF16, b_shape[1],
                 None, c, amp.BF16, N)
    torch.cuda.synchronize()
    a = a_d.view(torch.int16).cpu().numpy().view(np.uint16)
    b = b_d.view(torch.int16).cpu().numpy().view(np.uint16)
    out = c.view(torch.int16).cpu().numpy().view(np.uint16)
    rng = np.random.default_rng(0)
    ii = rng.integers(0, M, 512); jj = rng.integers(0, N, 512)
    av = F.decode(a, F.BF16); bv = F.decode(b, F.BF16)
    rows = av[ii, :] if opA == amp.OP_N else av[:, ii].T
    cols = bv[:, jj].T if opB == amp.OP_N else bv[jj, :]
    cref = np.sum(rows * cols, axis=1)
    bound = np.sum(np.abs(rows) * np.abs(cols), axis=1)
    ok = OG.check_rounded(out[ii, jj], F.BF16, cref, bound)
    assert ok.all(), np.nonzero(~ok)[0][:5]


@pytest.mark.parametrize("et,ct", [(amp.F16, amp.F32), (amp.BF16, amp.F16), (amp.BF16, amp.BF16)])
@pytest.mark.parametrize("opA,opB", [(amp.OP_N, amp.OP_T), (amp.OP_N, amp.OP_N),
                                     (amp.OP_T, amp.OP_N), (amp.OP_T, amp.OP_T)])
def test_gemm_interior_direct_to_lds_path(et, ct, opA, opB):
    """Full 256x256 tiles and K a multiple of the K-step: the direct-to-LDS
    kernel, with K-contiguous operands read as 16-byte rows and M/N-
    contiguous ones through transposing LDS reads; padded leading dimensions."""
    M, N, K = 512, 768, 320
    a_shape = (M, K) if opA == amp.OP_N else (K, M)
    b_shape = (K, N) if opB == amp.OP_N else (N, K)
    pad = 8
    a = codes_16(et, (a_shape[0], a_shape[1] + pad), 21 + opA)
    b = codes_16(et, (b_shape[0], b_shape[1] + pad), 22 + opB, 0.05)
    out = run_gemm(opA, opB, M, N, K, a, et, a_shape[1] + pad, b, et, b_shape[1] + pad, ct,
                   alphaA=2.0)
    A, B = ref_values(opA, opB, M, N, K, a[:, :a_shape[1]], et, b[:, :b_shape[1]], et)
    cref, bound = OG.reference(A, B, alpha=2.0)
    check(out, ct, cref, bound, "d2l")


@pytest.mark.parametrize("ct", [amp.F32, amp.BF16, amp.F16])
@pytest.mark.parametrize("ldc_pad", [8, 3])
def test_gemm_interior_padded_output_rows(ct, ldc_pad):
    """Full tiles with output rows longer than N: 16-byte aligned rows (pad 8)
    leave through the LDS-staged row stores, others (pad 3) through element
    stores; the columns past N keep their fill."""
    M, N, K = 512, 256, 192
    ldc = N + ldc_pad
    a = codes_16(amp.BF16, (M, K), 31)
    b = codes_16(amp.BF16, (N, K), 32, 0.05)
    c = empty(M * ldc * CT[ct][2], fill=0x7F)
    amp.amp_gemm_ex(amp.OP_N, amp.OP_T, M, N, K, dev(a), amp.BF16, K, f32_dev([0.5]), dev(b),
                    amp.BF16, K, None, c, ct, ldc)
    full = host(c, CT[ct][1]).reshape(M, ldc)
    A, B = ref_values(amp.OP_N, amp.OP_T, M, N, K, a, amp.BF16, b, amp.BF16)
    cref, bound = OG.reference(A, B, alpha=0.5)
    check(full[:, :N], ct, cref, bound, ("padded ldc", ldc_pad))
    fill = 0x7F7F7F7F if ct == amp.F32 else 0x7F7F
    assert np.all(full[:, N:] == fill), "columns past N were written"


@pytest.mark.parametrize("fa,fb", [(amp.E4M3, amp.E4M3), (amp.E5M2, amp.E4M3)])
def test_gemm_fp8_exact_interior(fa, fb):
    M, N, K = 256, 512, 512
    a, b, ia, ib = fp8_operands(31, M, N, K, fa, fb)
    out = run_gemm(amp.OP_N, amp.OP_T, M, N, K, a, fa, K, b, fb, K, amp.F32, alphaA=ia, alphaB=ib)
    A, B = ref_values(amp.OP_N, amp.OP_T, M, N, K, a, fa, b, fb)
    alpha = float(np.float32(np.float32(ia) * np.float32(ib)))
    cref, bound = OG.reference(A, B, alpha=alpha)
    check(out, amp.F32, cref, bound, "fp8 exact interior")


# lanes hold rows (A) / columns (B) l % D; P bytes per lane; R outputs per lane
PROBE = {0: (32, 8, 16, "32x32x16 FP8"), 1: (16, 8, 4, "16x16x32 FP8"),
         2: (32, 32, 16, "block-scaled 32x32x64 f8f6f4"),
         3: (16, 32, 4, "block-scaled 16x16x128 f8f6f4")}


def _probe_codes(seed, n, fmt, kind):
    if kind == "all-codes":
        c = synth.rng(seed).integers(0, 256, size=n, dtype=np.uint8)
        return np.where(np.isfinite(F.decode(c, fmt)), c, 0x38).astype(np.uint8)
    x = synth.student_t_f32(seed, n, scale=1.0)
    return OC.cast(synth.f32_bits(x), F.F32, fmt, float(fmt.max_finite) / float(np.abs(x).max()))[0]


@pytest.mark.parametrize("at", [amp.E4M3, amp.E5M2])
@pytest.mark.parametrize("shape", [0, 1, 2, 3])
def test_fp8_instruction_precision_report(shape, at):
    """Each FP8 matrix-core instruction of gfx950 on random operands (every
    finite code; Student-t activations scaled to the format's range) against
    the exact sums: report the largest |err| / sum|ab| and the share of
    outputs within 1e-5 * sum|ab|; assert the documented reduced-precision
    bound (2^-10) and that the lane layout is the documented one (no gross
    errors)."""
    D, P, R, name = PROBE[shape]
    G, tiles = 64 // D, 1024
    lanes, r = np.arange(64), np.arange(R)
    if D == 32:
        row = 8 * (r // 4)[None, :] + 4 * (lanes // 32)[:, None] + (r % 4)[None, :]
    else:
        row = 4 * (lanes // 16)[:, None] + r[None, :]
    col = np.broadcast_to((lanes % D)[:, None], row.shape)
    for kind in ("all-codes", "activations"):
        a = _probe_codes(100 + shape, tiles * 64 * P, FMT[at], kind)
        b = _probe_codes(200 + shape, tiles * 64 * P, F.E4M3, kind)
        c = empty(tiles * 64 * R * 4)
        amp.amp_fp8_mfma_probe(shape, at, dev(a), dev(b), c, tiles)
        got = host(c, np.float32).reshape(tiles, 64, R).astype(np.float64)
        # byte j of lane q*D + i meets byte j of lane q*D + n: K index (q, j)
        Av = F.decode(a, FMT[at]).reshape(tiles, G, D, P).transpose(0, 2, 1, 3).reshape(tiles, D, G * P)
        Bv = F.decode(b, F.E4M3).reshape(tiles, G, D, P).transpose(0, 2, 1, 3).reshape(tiles, D, G * P)
        cref, bound = OG.reference(Av, Bv.transpose(0, 2, 1))
        want, bd = cref[:, row, col], bound[:, row, col]
        rel = np.abs(got - want) / np.maximum(bd, 1e-300)
        within = float(np.mean(rel <= OG.RTOL))
        print(f"{name} {'E5M2' if at == amp.E5M2 else 'E4M3'}xE4M3 {kind}: "
              f"max |err|/sum|ab| = {rel.max():.3g}, within 1e-5: {within:.4f}")
        assert rel.max() <= 2.0 ** -10, (name, kind)
