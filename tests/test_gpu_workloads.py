"""Full-size parity of the transformer-block workloads.

* BF16 block (hidden 4096, FFN 14336, 8192 tokens): every output of all 12
  GEMMs (QKV, O, up/gate, down x forward, dgrad, wgrad; BF16 in, FP32
  accumulate, BF16 out) against the oracle's float64 product, so every
  output tile of every grid shape is checked.
* FP8 delayed scaling on the same shapes, 64 steps per layer: amax and scales
  bit-exact every step, E4M3 activations/weights and E5M2 gradients with their
  transposed copies bit-exact at the GEMM steps, 4096 sampled outputs of each
  GEMM at those steps and every output of all three GEMMs at step 63.
* NVFP4 weight gradient of the 12B-style layer (hidden 5120, FFN 20480, 16384
  tokens): both operands quantized on the GPU at full size (RHT; stochastic
  rounding for dY, nearest for X), then the GEMM of those codes; tensor scales
  bit-exact, sampled operand rows bit-exact against the oracle's quantization
  of the same slices with the whole tensor's scale, and sampled outputs
  against the oracle's product of the dequantized rows.
* Fine-grained FP8 FFN up projection: dgrad and wgrad at full size.

Inputs are seeded draws of the workload laws (activations N(0,1) or
sigma_t * Student-t(3), weights N(0, 0.02) FP32 masters, gradients N(0,1) or
1e-3 * Student-t(3), NVFP4 inputs N(0,1) with 0.1 % outliers at 50)."""
import numpy as np
import pytest
import torch

import mixed_precision_numerics_amd as amp
from oracle import blockwise as OB
from oracle import formats as F
from oracle import hadamard as OH
from oracle import nvfp4 as ON
from oracle import recipe as OR
import parity_util as PU
import synth
from gpu_util import empty, metas

pytestmark = pytest.mark.gpu

T = 8192
LAYERS = {"qkv": (4096, 6144), "o": (4096, 4096), "up_gate": (4096, 28672),
          "down": (14336, 4096)}                      # (in, out) features


def u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def u8(t):
    return t.cpu().numpy().view(np.uint8)


def gemm_pass(p, X, W, dY, din, dout, out, at=amp.BF16, wt=amp.BF16, gt=amp.BF16,
              Wt=None, Xt=None, dYt=None, aX=None, aW=None, adY=None):
    """Launch one pass of a linear layer.  16-bit operands use the
    transposing layouts; FP8 operands are K-contiguous (the casts' transposed
    copies Wt [in, out], Xt [in, T], dYt [out, T])."""
    if p == "fwd":                 # Y [T, out] = X W^T
        amp.amp_gemm(amp.OP_N, amp.OP_T, T, dout, din, X, at, din, aX, W, wt, din, aW,
                     out, amp.BF16, dout)
    elif p == "dgrad":             # dX [T, in] = dY W
        if Wt is None:
            amp.amp_gemm(amp.OP_N, amp.OP_N, T, din, dout, dY, gt, dout, adY, W, wt, din, aW,
                         out, amp.BF16, din)
        else:
            amp.amp_gemm(amp.OP_N, amp.OP_T, T, din, dout, dY, gt, dout, adY, Wt, wt, dout, aW,
                         out, amp.BF16, din)
    else:                          # dW [out, in] = dY^T X
        if dYt is None:
            amp.amp_gemm(amp.OP_T, amp.OP_N, dout, din, T, dY, gt, dout, adY, X, at, din, aX,
                         out, amp.BF16, din)
        else:
            amp.amp_gemm(amp.OP_N, amp.OP_T, dout, din, T, dYt, gt, T, adY, Xt, at, T, aX,
                         out, amp.BF16, din)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("p", ["fwd", "dgrad", "wgrad"])
@pytest.mark.parametrize("layer", list(LAYERS))
def test_bf16_block_gemm_every_output(layer, p):
    din, dout = LAYERS[layer]
    d = "cuda"
    gen = torch.Generator(device=d).manual_seed(3)
    X = torch.randn(T, din, generator=gen, device=d).to(torch.bfloat16)
    W32 = torch.randn(dout, din, generator=gen, device=d) * 0.02
    dY = torch.randn(T, dout, generator=gen, device=d).to(torch.bfloat16)
    W = torch.empty(dout, din, device=d, dtype=torch.bfloat16)
    amp.amp_cast(W32, amp.F32, dout, din, din, W, amp.BF16, din)       # FP32 master -> BF16
    shape = {"fwd": (T, dout), "dgrad": (T, din), "wgrad": (dout, din)}[p]
    out = torch.empty(*shape, device=d, dtype=torch.bfloat16)
    gemm_pass(p, X, W, dY, din, dout, out)
    wbits = W32.view(torch.int32).cpu().numpy().view(np.uint32)
    wq, _ = PU.cast(wbits, F.F32, F.BF16)
    assert np.array_equal(u16(W), wq)
    Wv = PU.values(wq, F.BF16)
    if p == "fwd":
        a, b = PU.values(u16(X), F.BF16), Wv.T
    elif p == "dgrad":
        a, b = PU.values(u16(dY), F.BF16), Wv
    else:
        a, b = PU.values(u16(dY), F.BF16).T, PU.values(u16(X), F.BF16)
    n = PU.check_full(u16(out), F.BF16, a, b, what=(layer, p))
    assert n == shape[0] * shape[1]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("layer", list(LAYERS))
def test_fp8_delayed_scaling_64_steps(layer):
    """X_t = 1.02^t * t3 (BF16) and W ~ N(0, 0.02) (FP32) cast to E4M3 and
    dY_t = 1e-3 * t3 (BF16) cast to E5M2, each with a transposed copy, using
    the scales of 1024-entry amax histories (margin 1); forward, dgrad and
    wgrad GEMMs on the FP8 codes with BF16 output."""
    din, dout = LAYERS[layer]
    gemm_steps = (0, 1, 32, 63) if layer == "qkv" else (0, 63)
    d = "cuda"
    gen = torch.Generator(device=d).manual_seed(4)
    W32 = torch.empty(dout, din, device=d).normal_(0.0, 0.02, generator=gen)
    W_bits = W32.view(torch.int32).cpu().numpy().view(np.uint32)
    W_amax = PU.amax(W_bits, F.F32)
    md = empty(16 * 3); hd = empty(4 * 3 * 1024)
    amp.amp_fp8_meta_init(md, hd, 3, 1024)
    om = [OR.FP8Meta() for _ in range(3)]
    r43 = amp.DelayedRecipe(448.0, 1.0, 1024, amp.AMAX_MAX)
    r52 = amp.DelayedRecipe(57344.0, 1.0, 1024, amp.AMAX_MAX)
    mp = lambda i, off: md.data_ptr() + 16 * i + off
    X8 = torch.empty(T, din, device=d, dtype=torch.uint8); X8t = torch.empty(din, T, device=d, dtype=torch.uint8)
    W8 = torch.empty(dout, din, device=d, dtype=torch.uint8); W8t = torch.empty(din, dout, device=d, dtype=torch.uint8)
    G8 = torch.empty(T, dout, device=d, dtype=torch.uint8); G8t = torch.empty(dout, T, device=d, dtype=torch.uint8)
    outs = {"fwd": torch.empty(T, dout, device=d, dtype=torch.bfloat16),
            "dgrad": torch.empty(T, din, device=d, dtype=torch.bfloat16),
            "wgrad": torch.empty(dout, din, device=d, dtype=torch.bfloat16)}
    rng = np.random.default_rng(0)
    x_scales = []
    for t in range(64):
        X = (synth.torch_student_t(gen, (T, din)) * (1.02 ** t)).to(torch.bfloat16)
        dY = (synth.torch_student_t(gen, (T, dout)) * 1e-3).to(torch.bfloat16)
        scales = [float(mm.scale) for mm in om]
        got = metas(md, 3)
        for i in range(3):
            assert got[i]["scale"] == np.float32(scales[i]), (t, i)
        amp.amp_cast(X, amp.BF16, T, din, din, X8, amp.E4M3, din, X8t, T, mp(0, 4), mp(0, 0))
        amp.amp_cast(W32, amp.F32, dout, din, din, W8, amp.E4M3, din, W8t, dout, mp(1, 4), mp(1, 0))
        amp.amp_cast(dY, amp.BF16, T, dout, dout, G8, amp.E5M2, dout, G8t, T, mp(2, 4), mp(2, 0))
        if t in gemm_steps:
            for p, o in outs.items():
                gemm_pass(p, X8, W8, G8, din, dout, o, at=amp.E4M3, wt=amp.E4M3, gt=amp.E5M2,
                          Wt=W8t, Xt=X8t, dYt=G8t, aX=mp(0, 8), aW=mp(1, 8), adY=mp(2, 8))
        # ---- oracle: amax of every full tensor, bit-exact
        xc, gc = u16(X), u16(dY)
        mid = metas(md, 3)
        want = (PU.amax(xc, F.BF16), W_amax, PU.amax(gc, F.BF16))
        for i in range(3):
            assert int(mid[i]["amax_cur"].view(np.uint32)) == want[i], (t, i)
            om[i].record(want[i])
        # ---- casts: sampled rows every step
        rows = rng.integers(0, T, 48)
        rows_d = torch.from_numpy(rows).to(d)
        for codes, buf, ofmt, sc in ((xc, X8, F.E4M3, scales[0]), (gc, G8, F.E5M2, scales[2])):
            wc, _ = PU.cast(codes[rows], F.BF16, ofmt, sc)
            assert np.array_equal(u8(buf[rows_d]), wc), t
        if t in gemm_steps:
            # whole tensors and their transposed copies
            xq, _ = PU.cast(xc, F.BF16, F.E4M3, scales[0])
            wq, _ = PU.cast(W_bits, F.F32, F.E4M3, scales[1])
            gq, _ = PU.cast(gc, F.BF16, F.E5M2, scales[2])
            for q, buf, bt in ((xq, X8, X8t), (wq, W8, W8t), (gq, G8, G8t)):
                assert np.array_equal(u8(buf), q), t
                assert np.array_equal(u8(bt), q.T), t
            inv = [float(np.float32(1.0) / np.float32(s)) for s in scales]
            al = lambda i, j: float(np.float32(np.float32(inv[i]) * np.float32(inv[j])))
            xv, wv, gv = PU.values(xq, F.E4M3), PU.values(wq, F.E4M3), PU.values(gq, F.E5M2)
            ops = {"fwd": (xv, wv.T, al(0, 1)), "dgrad": (gv, wv, al(2, 1)),
                   "wgrad": (gv.T, xv, al(2, 0))}
            for p, (a, b, alpha) in ops.items():
                o = outs[p]
                ii = rng.integers(0, a.shape[0], 4096)
                jj = rng.integers(0, b.shape[1], 4096)
                got_s = u16(o[torch.from_numpy(ii).to(d), torch.from_numpy(jj).to(d)])
                PU.check_entries(got_s, F.BF16, a[ii], b[:, jj].T, alpha, what=(layer, p, t))
                if t == 63:
                    PU.check_full(u16(o), F.BF16, a, b, alpha, what=(layer, p, t))
            del xv, wv, gv, ops
        x_scales.append(scales[0])
        print(f"fp8 {layer} step {t}: scales {scales[0]:.4g} {scales[1]:.4g} {scales[2]:.4g}",
              flush=True)
        amp.amp_delayed_scaling_update(md, hd, 2, r43)
        amp.amp_delayed_scaling_update(mp(2, 0), hd.data_ptr() + 4 * 1024 * 2, 1, r52)
        OR.update(om[0], 448.0); OR.update(om[1], 448.0); OR.update(om[2], 57344.0)
    # the sigma drift shrinks the activation scale step by step
    assert x_scales[-1] < x_scales[2]


def _transformed_amax(x_codes, seed):
    """The oracle's tensor amax of the RHT'd wgrad operand x^T (tokens along K),
    over column chunks of x (max |z| is order-free)."""
    signs = OH.sign_vector(seed)
    xt = np.ascontiguousarray(x_codes.T)
    res = PU.map_rows(lambda c: float(np.max(np.abs(OH.rht16(PU.values(c, F.BF16), signs)))), xt)
    return float(np.max(np.array(res)))


@pytest.mark.timeout(300)
def test_nvfp4_wgrad_quantize_then_gemm_full_size():
    O, I, TT = 20480, 5120, 16384
    d = "cuda"
    gen = torch.Generator(device=d).manual_seed(8)

    def operand(cols):
        x = torch.randn(TT, cols, generator=gen, device=d)
        mask = torch.rand(TT, cols, generator=gen, device=d) < 1e-3
        return torch.where(mask, torch.sign(x) * 50.0, x).to(torch.bfloat16)

    dY, X = operand(O), operand(I)
    rht_seed, sr_seed = 1234, 5678
    qg = empty(O * TT // 2); sg = empty(O * TT // 16); tg = empty(12)
    qx = empty(I * TT // 2); sx = empty(I * TT // 16); tx = empty(12)
    amp.amp_nvfp4_quantize(dY, amp.BF16, TT, O, O, 1, 0, 1, rht_seed, amp.ROUND_SR, sr_seed,
                           qg, sg, tg)
    amp.amp_nvfp4_quantize(X, amp.BF16, TT, I, I, 1, 0, 1, rht_seed, amp.ROUND_RNE, 0,
                           qx, sx, tx)
    ts = lambda t: t.view(torch.float32)       # [amax, enc, 1/enc]
    c = torch.empty(O, I, device=d, dtype=torch.bfloat16)
    amp.amp_gemm(amp.OP_N, amp.OP_T, O, I, TT, qg, amp.E2M1X2, TT // 2, ts(tg)[2:3], qx,
                 amp.E2M1X2, TT // 2, ts(tx)[2:3], c, amp.BF16, I,
                 amp.BlockScales(sg.data_ptr(), TT // 16, 0, 0),
                 amp.BlockScales(sx.data_ptr(), TT // 16, 0, 0))
    gc, xc = u16(dY), u16(X)
    A_g, A_x = _transformed_amax(gc, rht_seed), _transformed_amax(xc, rht_seed)
    enc_g, enc_x = ON.tensor_enc(A_g), ON.tensor_enc(A_x)
    g_ts, x_ts = ts(tg).cpu().numpy(), ts(tx).cpu().numpy()
    assert g_ts[1] == np.float32(enc_g) and x_ts[1] == np.float32(enc_x)
    rng = np.random.default_rng(9)
    ri = np.sort(rng.choice(O, 64, replace=False))
    rj = np.sort(rng.choice(I, 64, replace=False))
    qa, sa, _ = ON.quantize(PU.values(gc[:, ri], F.BF16), transpose=True, rht=True,
                            rht_seed=rht_seed, sr=True, sr_seed=sr_seed, tensor_amax=A_g,
                            row_ids=ri)
    qb, sb, _ = ON.quantize(PU.values(xc[:, rj], F.BF16), transpose=True, rht=True,
                            rht_seed=rht_seed, tensor_amax=A_x, row_ids=rj)
    assert np.array_equal(u8(qg).reshape(O, TT // 2)[ri], qa)
    assert np.array_equal(u8(sg).reshape(O, TT // 16)[ri], sa)
    assert np.array_equal(u8(qx).reshape(I, TT // 2)[rj], qb)
    assert np.array_equal(u8(sx).reshape(I, TT // 16)[rj], sb)
    A = ON.dequantize(qa, sa, enc_g)
    B = ON.dequantize(qb, sb, enc_x)
    ii, jj = np.meshgrid(np.arange(64), np.arange(64), indexing="ij")
    ii, jj = ii.ravel(), jj.ravel()
    got = u16(c[torch.from_numpy(ri[ii]).to(d), torch.from_numpy(rj[jj]).to(d)])
    PU.check_entries(got, F.BF16, A[ii], B[jj], what="nvfp4 wgrad")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("p", ["dgrad", "wgrad"])
def test_blockwise_ffn_up_backward_full_size_sampled(p):
    """Fine-grained FP8 dgrad (dX = dY W: dY in 1x128 tiles, W^T in 128x128
    blocks) and wgrad (dW = dY^T X: both transposed operands in 1x128 tiles
    along tokens) of the FFN up projection (8192 tokens, 4096 -> 28672):
    sampled operand rows bit-exact against the oracle's quantization of the
    same slices, 4096 sampled outputs against the oracle's GEMM."""
    I, O = 4096, 28672
    d = "cuda"
    gen = torch.Generator(device=d).manual_seed(22)
    x = torch.randn(T, I, generator=gen, device=d).to(torch.bfloat16)
    w = (torch.randn(O, I, generator=gen, device=d) * 0.02).to(torch.bfloat16)
    g = (torch.randn(T, O, generator=gen, device=d) * 1e-3).to(torch.bfloat16)
    rng = np.random.default_rng(23)
    if p == "dgrad":
        M, N, K = T, I, O
        qa = torch.empty(T, O, dtype=torch.uint8, device=d)
        sa = torch.empty(O // 128, T, dtype=torch.float32, device=d)
        amp.amp_quantize_blockwise(g, amp.BF16, T, O, O, amp.E4M3, 0, qa, O, sa, T)
        qb = torch.empty(I, O, dtype=torch.uint8, device=d)          # W^T in blocks
        sb = torch.empty(O // 128, I // 128, dtype=torch.float32, device=d)   # K-block-major
        amp.amp_quantize_blockwise(w, amp.BF16, O, I, I, amp.E4M3, 1, None, 0, None, 0,
                                   qb, O, sb, I // 128)
        b_block, ldsb = 1, I // 128
        a_src, a_tr, b_src, b_tr = g, False, w, True
        sa_h, sb_d = sa, sb
    else:
        M, N, K = O, I, T
        qa = torch.empty(O, T, dtype=torch.uint8, device=d)          # dY^T, tiles along tokens
        sa = torch.empty(T // 128, O, dtype=torch.float32, device=d)
        amp.amp_quantize_blockwise(g, amp.BF16, T, O, O, amp.E4M3, 0, None, 0, None, 0,
                                   qa, T, sa, O)
        qb = torch.empty(I, T, dtype=torch.uint8, device=d)          # X^T, tiles along tokens
        sb = torch.empty(T // 128, I, dtype=torch.float32, device=d)
        amp.amp_quantize_blockwise(x, amp.BF16, T, I, I, amp.E4M3, 0, None, 0, None, 0,
                                   qb, T, sb, I)
        b_block, ldsb = 0, I
        a_src, a_tr, b_src, b_tr = g, True, x, True
        sa_h, sb_d = sa, sb
    c = torch.empty(M, N, dtype=torch.bfloat16, device=d)
    amp.amp_gemm_blockwise(M, N, K, qa, amp.E4M3, K, sa_h, M, 0, qb, amp.E4M3, K, sb_d, ldsb,
                           b_block, c, amp.BF16, N)
    # oracle: quantize sampled A rows (their own 1xK tiles) and sampled B rows
    # (128-row blocks for W^T, single rows otherwise)
    src = u16(a_src)
    ra = np.sort(rng.choice(M, 48, replace=False))
    a_slice = src[:, ra] if a_tr else src[ra]
    aq, asc = OB.quantize(a_slice, F.BF16, F.E4M3, block=False, transpose=a_tr)
    assert np.array_equal(u8(qa)[ra], aq)
    assert np.array_equal(sa_h.cpu().numpy()[:, ra], asc.astype(np.float32))
    bsrc = u16(b_src)
    if b_block:
        blocks = np.sort(rng.choice(N // 128, 2, replace=False))
        rb = np.concatenate([np.arange(k * 128, k * 128 + 128) for k in blocks])
        bq_parts, bs_parts = [], []
        for k in blocks:
            q_k, s_k = OB.quantize(bsrc[:, k * 128:(k + 1) * 128], F.BF16, F.E4M3, block=True,
                                   transpose=True)
            bq_parts.append(q_k); bs_parts.append(s_k)
        bq = np.concatenate(bq_parts)
        bsc = np.concatenate(bs_parts, axis=1)
        assert np.array_equal(u8(qb)[rb], bq)
        assert np.array_equal(sb_d.cpu().numpy()[:, blocks], bsc.astype(np.float32))
    else:
        rb = np.sort(rng.choice(N, 48, replace=False))
        bq, bsc = OB.quantize(bsrc[:, rb], F.BF16, F.E4M3, block=False, transpose=True)
        assert np.array_equal(u8(qb)[rb], bq)
        assert np.array_equal(sb_d.cpu().numpy()[:, rb], bsc.astype(np.float32))
    cref, mag = OB.gemm(aq, asc, F.E4M3, False, bq, bsc, F.E4M3, bool(b_block))
    got = u16(c[torch.from_numpy(ra).to(d)][:, torch.from_numpy(rb).to(d)])
    from oracle import gemm as OG
    ok = OG.check_rounded(got, F.BF16, cref, mag)
    assert ok.all(), np.argwhere(~ok)[:5]
