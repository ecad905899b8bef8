"""Parity of amp_nvfp4_quantize (HIP) with the oracle (bit-exact codes, block
scales and tensor scale), and of the NVFP4 GEMM with the float64 reference of
the dequantised operands."""
import numpy as np
import pytest

import mixed_precision_numerics_amd as amp
from oracle import formats as F
from oracle import gemm as OG
from oracle import nvfp4 as ON
import synth
from gpu_util import dev, empty, host

pytestmark = pytest.mark.gpu


def quantize_gpu(xc, xt, rows, cols, transpose, block2d, rht, rht_seed, sr, sr_seed):
    R, K = (cols, rows) if transpose else (rows, cols)
    q = empty(R * K // 2, fill=0xEE)
    nsc = (R // 16 if block2d else R) * (K // 16)
    s = empty(nsc, fill=0xEE)
    ts = empty(12)
    amp.amp_nvfp4_quantize(dev(xc), xt, rows, cols, cols, transpose, block2d, rht, rht_seed,
                           amp.ROUND_SR if sr else amp.ROUND_RNE, sr_seed, q, s, ts)
    return (host(q, np.uint8).reshape(R, K // 2), host(s, np.uint8)[:nsc],
            host(ts, np.float32)[:3])


@pytest.mark.parametrize("transpose", [False, True])
@pytest.mark.parametrize("block2d", [False, True])
@pytest.mark.parametrize("rht", [False, True])
@pytest.mark.parametrize("sr", [False, True])
def test_nvfp4_quantize_bit_exact(transpose, block2d, rht, sr):
    rows, cols = 320, 272            # ragged against the 64 x 256 tiles
    xc = synth.outlier_bf16_codes(40 + 8 * transpose + 4 * block2d + 2 * rht + sr, (rows, cols))
    x = F.decode(xc, F.BF16)
    wq, ws, enc = ON.quantize(x, transpose=transpose, block2d=block2d, rht=rht, rht_seed=77,
                              sr=sr, sr_seed=0x1234_5678_9ABC)
    q, s, ts = quantize_gpu(xc, amp.BF16, rows, cols, transpose, block2d, rht, 77, sr,
                            0x1234_5678_9ABC)
    assert ts[1] == np.float32(enc)
    assert ts[2] == np.float32(1.0 / np.float32(enc))
    assert np.array_equal(s, ws.reshape(-1)), np.nonzero(s != ws.reshape(-1))[0][:8]
    bad = np.argwhere(q != wq)
    assert bad.size == 0, (bad[:5], q[tuple(bad[0])], wq[tuple(bad[0])])


def test_nvfp4_f32_input_and_specials():
    x = synth.normal_f32(5, (64, 48)).astype(np.float32)
    x[3, 5] = np.inf
    x[10:26, 16:32] = 0.0            # an all-zero block
    wq, ws, enc = ON.quantize(x.astype(np.float64))
    q, s, ts = quantize_gpu(synth.f32_bits(x).copy(), amp.F32, 64, 48, False, False, False, 0,
                            False, 0)
    assert ts[1] == np.float32(enc)
    assert np.array_equal(s, ws.reshape(-1))
    assert np.array_equal(q, wq)


def test_nvfp4_wgrad_gemm_parity():
    """wgrad dW = dY^T X with both operands NVFP4 (RHT, SR on dY): the GEMM
    on the dequantised operands within the FP32-accumulation tolerance."""
    T, O, I = 512, 256, 320
    dy = synth.outlier_bf16_codes(91, (T, O))
    xx = synth.outlier_bf16_codes(92, (T, I))
    qa, sa, ta = quantize_gpu(dy, amp.BF16, T, O, True, False, True, 5, True, 17)
    qb, sb, tb = quantize_gpu(xx, amp.BF16, T, I, True, False, True, 5, False, 0)
    A = ON.dequantize(qa, sa.reshape(O, T // 16), float(ta[1]))
    B = ON.dequantize(qb, sb.reshape(I, T // 16), float(tb[1]))
    c = empty(O * I * 4)
    ta_d, tb_d = dev(ta), dev(tb)
    sa_d = dev(sa); sb_d = dev(sb)
    bsA = amp.BlockScales(sa_d.data_ptr(), T // 16, 0, 0)
    bsB = amp.BlockScales(sb_d.data_ptr(), T // 16, 0, 0)
    amp.amp_gemm(amp.OP_N, amp.OP_T, O, I, T, dev(qa), amp.E2M1X2, T // 2, ta_d.data_ptr() + 8,
                 dev(qb), amp.E2M1X2, T // 2, tb_d.data_ptr() + 8, c, amp.F32, I, bsA, bsB)
    out = host(c, np.float32).reshape(O, I).astype(np.float64)
    # dequantised values already include 1/enc exactly; the kernel multiplies by
    # fl32(1/enc_A) * fl32(1/enc_B), a relative 2^-23 difference, inside rtol
    cref, bound = OG.reference(A, B.T)
    assert OG.check_f32(out, cref, bound).all()
    # the quantized product approximates the unquantised one (context)
    full, _ = OG.reference(F.decode(dy, F.BF16).T, F.decode(xx, F.BF16))
    rel = np.linalg.norm(out - full) / np.linalg.norm(full)
    print(f"nvfp4 wgrad relative error vs unquantised: {rel:.3f}")
    # 4-bit elements give ~0.2 relative error here; a wrong transform, scale
    # or operand pairing gives ~1 or more
    assert rel < 0.3


@pytest.mark.parametrize("ct", [amp.F32, amp.BF16])
@pytest.mark.parametrize("b2d", [False, True])
def test_nvfp4_gemm_direct_to_lds_path(ct, b2d):
    """Full 256x256 tiles, K a multiple of 256 and 16-byte scale rows: the
    codes travel to LDS by direct loads and each fragment is decoded in
    registers (E2M1 -> F16 times its E4M3 block scale); B with 16x16 weight
    blocks or 1x16 blocks; subnormal, zero and maximal block scales; tensor
    scales in the epilogue."""
    M, N, K = 512, 256, 768                    # 2 x 1 tiles, 3 K-steps
    qa, sa, enca = synth.nvfp4_operand(201, M, K)
    qb, sb, encb = synth.nvfp4_operand(202, N, K)
    sa[0, :4] = [0x01, 0x07, 0x7E, 0x00]        # 2^-9, 7*2^-9, 448, 0
    sa[300, 40:44] = [0x08, 0x7E, 0x01, 0x3F]
    if b2d:
        sb = sb[: N // 16].copy()
        sb[3, 10:12] = [0x7E, 0x02]
    deca = np.float32(1.0) / np.float32(enca)
    decb = np.float32(1.0) / np.float32(encb)
    c = empty(M * N * 4)
    sa_d, sb_d = dev(sa), dev(sb)
    amp.amp_gemm(amp.OP_N, amp.OP_T, M, N, K, dev(qa), amp.E2M1X2, K // 2, dev(np.array([deca])),
                 dev(qb), amp.E2M1X2, K // 2, dev(np.array([decb])), c, ct, N,
                 amp.BlockScales(sa_d.data_ptr(), K // 16, 0, 0),
                 amp.BlockScales(sb_d.data_ptr(), K // 16, int(b2d), 0))
    A = ON.dequantize(qa, sa, 1.0) * float(deca)
    B = ON.dequantize(qb, sb, 1.0, block2d=b2d) * float(decb)
    cref, bound = OG.reference(A, B.T)
    if ct == amp.F32:
        ok = OG.check_f32(host(c, np.float32)[:M * N].reshape(M, N), cref, bound)
    else:
        ok = OG.check_rounded(host(c, np.uint16)[:M * N].reshape(M, N), F.BF16, cref, bound)
    bad = np.argwhere(~ok)
    assert bad.size == 0, bad[:5]


def test_nvfp4_decode_every_code_and_scale_via_identity():
    """C = A @ I over all 16 E2M1 codes times many E4M3 block scales."""
    K = 256
    M = 16
    codes = np.tile(np.arange(16, dtype=np.uint8), K // 16)
    a_codes = np.stack([np.roll(codes, r) for r in range(M)])
    qa = (a_codes[:, 0::2] | (a_codes[:, 1::2] << 4)).astype(np.uint8)
    sa = np.arange(M * K // 16, dtype=np.uint8).reshape(M, K // 16) % 0x7F
    # identity with value 1.0 = code 2, block scale 1.0 = 0x38
    eye = np.zeros((K, K), np.uint8)
    eye[np.arange(K), np.arange(K)] = 2
    qb = (eye[:, 0::2] | (eye[:, 1::2] << 4)).astype(np.uint8)
    sb = np.full((K, K // 16), 0x38, np.uint8)
    c = empty(M * K * 4)
    sa_d, sb_d = dev(sa), dev(sb)
    amp.amp_gemm(amp.OP_N, amp.OP_T, M, K, K, dev(qa), amp.E2M1X2, K // 2, None, dev(qb),
                 amp.E2M1X2, K // 2, None, c, amp.F32, K,
                 amp.BlockScales(sa_d.data_ptr(), K // 16, 0, 0),
                 amp.BlockScales(sb_d.data_ptr(), K // 16, 0, 0))
    want = F.decode(a_codes, F.E2M1) * np.repeat(F.decode(sa, F.E4M3), 16, axis=1)
    assert np.array_equal(host(c, np.float32).reshape(M, K).astype(np.float64), want)


@pytest.mark.parametrize("xt", ["bf16", "f32"])
@pytest.mark.parametrize("transpose", [False, True])
@pytest.mark.parametrize("unaligned", [False, True])
@pytest.mark.parametrize("opts", [(False, True, True), (True, True, False), (False, False, False)])
def test_nvfp4_layouts_and_strides(xt, transpose, unaligned, opts):
    """Both load paths: 16-byte aligned rows (vector cells) and rows that
    start off a 16-byte boundary (the LDS-staged path), in BF16 and FP32, with
    a padded leading dimension; ragged against every tile shape."""
    block2d, rht, sr = opts
    rows, cols = 112, 304
    ldx = cols + (1 if unaligned else 8)
    seed = 300 + 16 * transpose + 8 * unaligned + 2 * (xt == "f32") + block2d + 4 * rht
    xc = synth.outlier_bf16_codes(seed, (rows, cols))
    x = F.decode(xc, F.BF16)
    if xt == "f32":
        x = x * 1.001                      # values off the BF16 grid
        x32 = x.astype(np.float32)
        x = x32.astype(np.float64)
        buf = np.zeros((rows, ldx), dtype=np.uint32)
        buf[:, :cols] = synth.f32_bits(x32)
        esize, code = 4, amp.F32
    else:
        buf = np.zeros((rows, ldx), dtype=np.uint16)
        buf[:, :cols] = xc
        esize, code = 2, amp.BF16
    flat = np.concatenate([np.zeros(1, dtype=buf.dtype), buf.reshape(-1)])
    xd = dev(flat)
    ptr = xd.data_ptr() + esize            # one element in: 16-byte aligned only via ldx
    if not unaligned:
        xd = dev(buf.reshape(-1))
        ptr = xd.data_ptr()
    R, K = (cols, rows) if transpose else (rows, cols)
    q = empty(R * K // 2, fill=0xEE)
    nsc = (R // 16 if block2d else R) * (K // 16)
    s = empty(nsc, fill=0xEE)
    ts = empty(12)
    amp.amp_nvfp4_quantize(ptr, code, rows, cols, ldx, transpose, block2d, rht, 91,
                           amp.ROUND_SR if sr else amp.ROUND_RNE, 0xC0FFEE, q, s, ts)
    wq, ws, enc = ON.quantize(x, transpose=transpose, block2d=block2d, rht=rht, rht_seed=91,
                              sr=sr, sr_seed=0xC0FFEE)
    assert host(ts, np.float32)[1] == np.float32(enc)
    assert np.array_equal(host(s, np.uint8)[:nsc], ws.reshape(-1))
    assert np.array_equal(host(q, np.uint8).reshape(R, K // 2), wq)
