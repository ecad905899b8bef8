"""The no-allocation norm entry point against the one that takes a state
struct: the same sum of squares bit for bit and the same overflow flag, on two
calls in a row, the second with a smaller input (the shared device scratch
keeps the first call's partials, which the second must not read)."""
import numpy as np
import pytest
import torch

import mixed_precision_numerics_amd as amp
import synth
from gpu_util import dev, empty, host, scaler_state

pytestmark = pytest.mark.gpu


def _with_state(g, gt, n, S):
    st = empty(40)
    amp.amp_scaler_init(st, S)
    ns = empty(amp.NORM_STATE_BYTES)
    amp.amp_grad_norm_init(ns)
    amp.amp_grad_norm_accumulate(g, gt, n, st, ns)
    return host(ns, np.float64)[0], int(scaler_state(st)["found_inf"])


def _no_alloc(g, gt, n, S, sumsq):
    st = empty(40)
    amp.amp_scaler_init(st, S)
    sumsq.zero_()
    amp.amp_grad_norm_accumulate_noalloc(g, gt, n, st, sumsq)
    return host(sumsq, np.float64)[0], int(scaler_state(st)["found_inf"])


@pytest.mark.parametrize("gt", [amp.F16, amp.BF16, amp.F32])
def test_no_alloc_norm_matches_the_state_struct_entry_point(gt):
    sumsq = torch.zeros(1, dtype=torch.float64, device="cuda")
    big = (1 << 24) + 37                      # 1024 work-groups, ragged tail
    x = synth.normal_f32(31, big, 300.0)
    codes = {amp.F16: synth.to_f16_codes, amp.BF16: synth.to_bf16_codes,
             amp.F32: synth.f32_bits}[gt](x)
    g = dev(codes)
    for n in (big, 3 * 8192 + 5, 1000):       # each call smaller than the last
        want = _with_state(g, gt, n, 512.0)
        got = _no_alloc(g, gt, n, 512.0, sumsq)
        assert got[0] == want[0] and got[1] == want[1] == 0, (n, got, want)
        assert got[0] > 0
    # a non-finite gradient sets the flag on both paths
    bad = codes.copy()
    bad[777] = {amp.F16: 0x7C00, amp.BF16: 0x7F80, amp.F32: 0x7F800000}[gt]
    gb = dev(bad)
    for n in (big, 1000):
        want = _with_state(gb, gt, n, 512.0)
        got = _no_alloc(gb, gt, n, 512.0, sumsq)
        assert got == want and got[1] == 1, (n, got, want)


def test_no_alloc_norm_rejects_bad_arguments():
    st = empty(40)
    sumsq = torch.zeros(2, dtype=torch.float64, device="cuda")
    g = dev(np.zeros(64, np.uint16))
    with pytest.raises(amp.AmpError):
        amp.amp_grad_norm_accumulate_noalloc(g, amp.F16, 64, st, None)
    with pytest.raises(amp.AmpError):
        amp.amp_grad_norm_accumulate_noalloc(g, amp.F16, 64, st, sumsq.data_ptr() + 4)
    with pytest.raises(amp.AmpError):
        amp.amp_grad_norm_accumulate_noalloc(g, amp.E4M3, 64, st, sumsq)
