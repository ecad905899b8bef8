"""Pins for the oracle's cast + amax, delayed-scaling recipe and loss scaler."""
import json
import os
from fractions import Fraction

import numpy as np

from oracle import cast as C
from oracle import formats as F
from oracle import recipe as R
from oracle import scaler as S
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def test_amax_constant_and_order_free():
    x = np.full(1000, -3.25, dtype=np.float32)
    _, am = C.cast(synth.f32_bits(x), F.F32, F.E4M3, 1.0)
    assert F.from_f32_bits(am) == 3.25
    y = synth.normal_f32(5, 4096)
    perm = np.random.default_rng(0).permutation(y.size)
    _, a1 = C.cast(synth.f32_bits(y), F.F32, F.F16, 1.0)
    _, a2 = C.cast(synth.f32_bits(y[perm]), F.F32, F.F16, 1.0)
    assert a1 == a2 and F.from_f32_bits(a1) == np.max(np.abs(y.astype(np.float64)))


def test_amax_specials():
    x = np.array([1.0, -np.inf, 2.0], dtype=np.float32)
    assert int(C.amax_bits(synth.f32_bits(x))) == 0x7F800000
    x = np.array([1.0, np.nan, -np.inf], dtype=np.float32)
    assert int(C.amax_bits(synth.f32_bits(x))) == 0x7FC00000
    assert int(C.amax_bits(np.zeros(0, np.uint32))) == 0
    _, am = C.cast(synth.f32_bits(np.array([0.5], np.float32)), F.F32, F.F16, None,
                   amax_prior_bits=int(synth.f32_bits(np.array([4.0], np.float32))[0]))
    assert F.from_f32_bits(am) == 4.0          # max-accumulate into the prior value


def test_scaled_cast_brute_force():
    """y = nearest (ties even) representable value to fl32(x*scale), by brute
    force over every code, on small random tensors."""
    x = synth.student_t_f32(7, 64, scale=40.0)
    for fmt, scale, n in ((F.E4M3, 448.0 / 300.0, 64), (F.E5M2, 3.0, 64), (F.F16, 1024.0, 6)):
        x = x[:n]
        codes, _ = C.cast(synth.f32_bits(x), F.F32, fmt, scale)
        got = F.decode(codes, fmt)
        allc = np.arange(1 << fmt.nbits)
        allv = F.decode(allc, fmt)
        fin = np.isfinite(allv)
        allc, allv = allc[fin], allv[fin]
        for xi, gi in zip(x, got):
            t = float(np.float32(np.float32(xi) * np.float32(scale)))
            if not fmt.saturate and abs(t) >= fmt.max_finite + (fmt.max_finite - float(allv[np.argsort(allv)[-2]])) / 2:
                assert np.isinf(gi)
                continue
            t = min(max(t, -fmt.max_finite), fmt.max_finite)
            ft = Fraction(t)
            d = [(abs(Fraction(float(v)) - ft), int(c) & 1) for c, v in zip(allc, allv)]
            assert gi == allv[min(range(len(d)), key=d.__getitem__)]


def test_bf16_input_widening_is_exact():
    codes = synth.bf16_codes_normal(3, 1000)
    bits = C.widen_to_f32_bits(codes, F.BF16)
    assert np.array_equal(bits, codes.astype(np.uint32) << 16)


def test_delayed_scaling_geometric_sequence():
    """amax_t = 2^t  =>  the scale derived after step t is 448 * 2^-t."""
    m = R.FP8Meta(history_len=GOLD["amax_history_len"]["value"])
    for t in range(20):
        m.record(int(synth.f32_bits(np.array([2.0 ** t], np.float32))[0]))
        R.update(m, R.E4M3_MAX, GOLD["margin"]["value"])
        assert m.scale == 448.0 * 2.0 ** -t
        assert m.scale_inv == 2.0 ** t / 448.0 or abs(m.scale_inv * m.scale - 1) < 2 ** -23


def test_delayed_scaling_spike_leaves_window_after_len_updates():
    L = GOLD["amax_history_len"]["value"]
    m = R.FP8Meta(history_len=L)
    bits = lambda v: int(synth.f32_bits(np.array([v], np.float32))[0])
    m.record(bits(1000.0))
    R.update(m, R.E4M3_MAX)
    assert m.scale == float(F.f32(448.0 / 1000.0))
    for step in range(1, L + 1):
        m.record(bits(1.0))
        R.update(m, R.E4M3_MAX)
        if step < L:
            assert m.scale == float(F.f32(448.0 / 1000.0)), step
    assert m.scale == 448.0            # update L (0-based) no longer sees the spike


def test_delayed_scaling_most_recent_margin_and_keep():
    m = R.FP8Meta(history_len=16)
    bits = lambda v: int(synth.f32_bits(np.array([v], np.float32))[0])
    m.record(bits(100.0)); R.update(m, R.E5M2_MAX, 2.0, "most_recent")
    assert m.scale == float(F.f32(57344.0 / 200.0))
    m.record(bits(10.0)); R.update(m, R.E5M2_MAX, 2.0, "most_recent")
    assert m.scale == float(F.f32(57344.0 / 20.0))
    keep = m.scale
    R.update(m, R.E5M2_MAX, 2.0, "most_recent")      # amax 0 -> keep scale
    assert m.scale == keep
    m.record(0x7FC00000); R.update(m, R.E5M2_MAX, 2.0, "max")   # NaN -> keep
    assert m.scale == keep


def test_scaler_defaults_and_c1_sequence():
    st = S.ScalerState()
    assert st.scale == GOLD["gradscaler_init"]["value"]
    seq = []
    for t in range(10):
        seq.append(st.scale)
        S.update(st, found_inf=(t == 3))
        seq.append(st.growth_tracker)
    scales, trackers = seq[0::2], seq[1::2]
    assert scales == [65536.0] * 4 + [32768.0] * 6
    assert trackers == [1, 2, 3, 0, 1, 2, 3, 4, 5, 6]


def test_scaler_growth_at_exactly_interval_and_reset():
    n = GOLD["gradscaler_interval"]["value"]
    st = S.ScalerState(scale=1024.0)
    for i in range(n - 1):
        S.update(st, False)
    assert st.scale == 1024.0 and st.growth_tracker == n - 1
    S.update(st, False)
    assert st.scale == 1024.0 * GOLD["gradscaler_growth"]["value"] and st.growth_tracker == 0
    for i in range(n - 1):
        S.update(st, False)
    S.update(st, True)
    assert st.scale == 1024.0 and st.growth_tracker == 0
    for i in range(n - 1):
        S.update(st, False)
    assert st.scale == 1024.0


def test_scaler_collapse_no_floor():
    st = S.ScalerState()
    for _ in range(40):
        S.update(st, True)
    assert st.scale == 2.0 ** (16 - 40)


def test_current_scaling_closed_forms():
    """Current scaling uses this tensor's amax: 2^t -> 448 * 2^-t; the largest
    element then casts to exactly +-448 (E4M3 max); zero or NaN amax -> 1."""
    bits = lambda v: int(synth.f32_bits(np.array([v], np.float32))[0])
    for t in range(-10, 11):
        sc, inv = R.current_scale(bits(2.0 ** t), R.E4M3_MAX)
        assert sc == 448.0 * 2.0 ** -t
        assert inv == float(np.float32(1.0) / np.float32(sc))
    x = synth.normal_f32(7, 1000, 3.0)
    am = C.amax_bits(synth.f32_bits(np.abs(x)))
    sc, _ = R.current_scale(int(am), R.E4M3_MAX)
    codes, _ = C.cast(synth.f32_bits(x), F.F32, F.E4M3, sc)
    i = int(np.argmax(np.abs(x)))
    assert abs(F.decode(codes[i:i + 1], F.E4M3)[0]) == 448.0       # no saturation loss
    assert np.all(np.abs(F.decode(codes, F.E4M3)) <= 448.0)
    assert R.current_scale(0, R.E4M3_MAX) == (1.0, 1.0)
    assert R.current_scale(0x7FC00000, R.E5M2_MAX) == (1.0, 1.0)
    sc, _ = R.current_scale(bits(100.0), R.E5M2_MAX, 2.0)
    assert sc == float(F.f32(57344.0 / 200.0))


def test_saturation_count_closed_forms():
    """hwlabs "FP8이 어려운 이유": values past the range are clipped; the count
    is of |fl32(x*scale)| > max (448 for E4M3, 57344 for E5M2), inf included,
    NaN and the maximum itself excluded."""
    above = float(np.nextafter(np.float32(448.0), np.float32(1e9)))
    x = np.array([447.0, 448.0, above, 500.0, np.inf, -np.inf, np.nan, -1000.0, 0.0],
                 dtype=np.float32)
    assert C.saturated_count(synth.f32_bits(x), F.F32, F.E4M3) == 5
    # a power-of-two scale moves the threshold exactly: x * 2 > 448 <=> x > 224
    y = np.array([224.0, 224.5, -225.0, 100.0], dtype=np.float32)
    assert C.saturated_count(synth.f32_bits(y), F.F32, F.E4M3, 2.0) == 2
    assert C.saturated_count(synth.f32_bits(y), F.F32, F.E4M3, 1.0) == 0
    z = np.array([57344.0, 57345.0, 60000.0, -1e6, 448.0], dtype=np.float32)
    assert C.saturated_count(synth.f32_bits(z), F.F32, F.E5M2) == 3
    # 16-bit IEEE outputs overflow to inf instead of saturating
    assert C.saturated_count(synth.f32_bits(z), F.F32, F.F16) == 0
    # BF16 input widens exactly: 449.0 is not BF16-representable (448 < 450)
    b = synth.to_bf16_codes(np.array([449.0, 450.0], dtype=np.float32))
    assert C.saturated_count(b, F.BF16, F.E4M3) == 1


def test_found_inf_from_amax_matches_the_cast_outputs():
    """The flag derived from the recorded amax equals the check of the cast's
    own outputs (oracle.adamw.found_inf), over tensors around the FP16 and
    BF16 overflow thresholds, with and without a scale, with inf and NaN."""
    from oracle import adamw as OA
    rng = np.random.default_rng(7)
    cases = 0
    for peak in (1.0, 6.55e4, 65519.0, 65520.0, 7e4, 3.3e38, 3.4e38, np.inf, np.nan):
        for scale in (None, 0.5, 2.0):
            x = (rng.standard_normal(257) * 10).astype(np.float32)
            x[17] = peak
            for out in (F.F16, F.BF16):
                codes, am = C.cast(synth.f32_bits(x), F.F32, out, scale)
                want = OA.found_inf(codes, out)
                assert C.found_inf_from_amax([am], out, scale) == want, (peak, scale, out.name)
                cases += int(want)
            codes8, am8 = C.cast(synth.f32_bits(x), F.F32, F.E4M3, scale)
            assert C.found_inf_from_amax([am8], F.E4M3, scale) == (not np.isfinite(peak))
    assert cases > 10
    # closed forms at the FP16 threshold: 65519 rounds to 65504, 65520 to inf
    assert not C.found_inf_from_amax([int(synth.f32_bits(np.array([65519.0], np.float32))[0])], F.F16)
    assert C.found_inf_from_amax([int(synth.f32_bits(np.array([65520.0], np.float32))[0])], F.F16)
    assert C.found_inf_from_amax([0, 0x7FC00000], F.F16)

