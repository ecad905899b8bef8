"""MX block formats on the GPU: amp_mx_quantize bit-exact against oracle/mx.py
and the MX GEMM on CDNA4's block-scaled matrix cores against the float64
product of the dequantized operands."""
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
