"""Empty work through the C entry points.  A zero size is a successful no-op
that writes nothing, except where a call defines a result for it: the NVFP4
quantizer stores the tensor scales of an all-zero operand (amax 0, encode and
decode scales 1), the column sum of zero rows is zero, and an optimizer step
over an empty shard still commits the step (the Adam step count and the beta
powers advance, as on every rank that holds parameters)."""
import numpy as np
import pytest
import torch

import mixed_precision_numerics_amd as amp
from gpu_util import empty, f32_dev, host, scaler_state

pytestmark = pytest.mark.gpu

PAT = 0x5A


def untouched(*ts):
    return all(bool(np.all(host(t, np.uint8) == PAT)) for t in ts)


@pytest.mark.parametrize("rows,cols", [(0, 64), (64, 0), (0, 0)])
def test_empty_casts_and_quantizers_write_nothing(rows, cols):
    x, y, yt, s, st = (empty(1 << 16, PAT) for _ in range(5))
    am = empty(4, PAT)
    sc = f32_dev([2.0])
    meta = empty(amp.FP8_META_DTYPE.itemsize, PAT)
    recipe = amp.DelayedRecipe(448.0, 1.0, 16, amp.AMAX_MAX)
    amp.amp_cast(x, amp.BF16, rows, cols, cols, y, amp.E4M3, cols, yt, rows, sc, am)
    amp.amp_cast(x, amp.F32, rows, cols, cols, y, amp.F16, cols, None, 0, None, am)
    amp.amp_cast_ex(x, amp.BF16, rows, cols, cols, y, amp.E5M2, cols, yt, rows, sc, am, st)
    amp.amp_cast_current_scaling(x, amp.BF16, rows, cols, cols, y, amp.E4M3, cols, yt, rows,
                                 recipe, meta)
    amp.amp_quantize_blockwise(x, amp.BF16, rows, cols, cols, amp.E4M3, 0, y, cols, s, rows,
                               yt, rows, st, cols)
    amp.amp_mx_quantize(x, amp.BF16, rows, cols, cols, 0, amp.E4M3, y, s)
    assert untouched(x, y, yt, s, st, am, meta)


@pytest.mark.parametrize("rows,cols,transpose", [(0, 64, 0), (64, 0, 1), (0, 0, 0)])
def test_empty_nvfp4_operand_gets_unit_tensor_scales(rows, cols, transpose):
    x, q, sc = (empty(1 << 12, PAT) for _ in range(3))
    d_tensor = empty(12, PAT)
    amp.amp_nvfp4_quantize(x, amp.BF16, rows, cols, cols, transpose, 0, 1, 7, amp.ROUND_SR, 9,
                           q, sc, d_tensor)
    assert untouched(x, q, sc)
    assert host(d_tensor, np.float32).tolist() == [0.0, 1.0, 1.0]


def test_empty_gemms_write_nothing():
    a, b, c = (empty(1 << 16, PAT) for _ in range(3))
    for M, N in ((0, 256), (256, 0), (0, 0)):
        amp.amp_gemm(amp.OP_N, amp.OP_T, M, N, 64, a, amp.BF16, 64, None, b, amp.BF16, 64, None,
                     c, amp.F32, max(N, 1))
        amp.amp_gemm_blockwise(M, N, 128, a, amp.E4M3, 128, None, max(M, 1), 0, b, amp.E4M3, 128,
                               None, 1, 1, c, amp.BF16, max(N, 1))
    assert untouched(a, b, c)


def test_empty_gradient_passes_and_copy_write_nothing():
    g, acc = empty(1 << 12, PAT), empty(1 << 12, PAT)
    st = empty(amp.SCALER_STATE_DTYPE.itemsize)
    amp.amp_scaler_init(st, 1024.0)
    before = host(st, np.uint8).copy()
    ns = empty(amp.NORM_STATE_BYTES)
    amp.amp_grad_norm_init(ns)
    ns_before = host(ns, np.uint8).copy()
    amp.amp_check_overflow(g, amp.F16, 0, st)
    amp.amp_grad_accumulate(acc, g, amp.F16, 0, True)
    amp.amp_grad_norm_accumulate(g, amp.F16, 0, st, ns)
    amp.amp_stream_copy(g, acc, 0)
    assert untouched(g, acc)
    assert np.array_equal(host(st, np.uint8), before)
    assert np.array_equal(host(ns, np.uint8), ns_before)


def test_column_sum_of_zero_rows_is_zero():
    out = empty(2 * 40, PAT)
    amp.amp_colsum_f16(empty(16, PAT), 0, 40, out)
    assert np.all(host(out, np.uint16) == 0)


def test_empty_optimizer_shard_commits_the_step():
    st = empty(amp.SCALER_STATE_DTYPE.itemsize)
    amp.amp_scaler_init(st, 65536.0)
    th, m, v, g, w = (empty(1 << 10, PAT) for _ in range(5))
    hp = amp.AdamWHParams(1e-3, 0.9, 0.95, 1e-8, 0.1)
    amp.amp_optimizer_step(th, m, v, g, amp.F16, w, amp.F16, 0, hp, st)
    amp.amp_optimizer_step(th, m, v, g, amp.F16, w, amp.F16, 0, hp, st)
    s = scaler_state(st)
    assert int(s["adam_step"]) == 2 and int(s["found_inf"]) == 0
    assert float(s["beta1_pow"]) == 0.9 * 0.9 and float(s["beta2_pow"]) == 0.95 * 0.95
    assert float(s["scale"]) == 65536.0
    assert untouched(th, m, v, g, w)
