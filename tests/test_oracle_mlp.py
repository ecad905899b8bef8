"""Pins for the tiny FP16 AMP training step oracle."""
import numpy as np

from oracle import adamw as A
from oracle import formats as F
from oracle import mlp as M
import synth


def _init(seed=0):
    return synth.mlp_init(seed).astype(np.float64)


def _batch(t):
    x, y = synth.mlp_batch(t)
    return x.astype(np.float64), y


def test_param_count():
    assert M.N_PARAMS == 1_071_114


def test_gelu_closed_forms():
    assert M.gelu(0.0) == 0.0
    assert abs(M.gelu(10.0) - 10.0) < 1e-12
    assert abs(M.gelu(-10.0)) < 1e-12
    z = np.linspace(-4, 4, 101)
    num = (M.gelu(z + 1e-6) - M.gelu(z - 1e-6)) / 2e-6
    assert np.max(np.abs(num - M.gelu_grad(z))) < 1e-6


def test_loss_and_grad_against_finite_differences():
    """Unscaled analytic gradient direction of the FP64 model (rounding off)
    agrees with the oracle's FP16 gradient to FP16 accuracy on large entries."""
    master = _init()
    p = M.split(master)
    x, y = _batch(0)
    fb = M.forward_backward({k: F.round_to(v, F.F16) for k, v in p.items()}, x, y, 1024.0)
    # the loss at init is close to log(10)
    assert abs(fb["loss"] - np.log(10)) < 0.2
    # db2 = S * mean(p - onehot) summed over batch: columns sum to ~0
    assert abs(fb["db2"].sum()) / 1024.0 < 1e-2


def test_loss_scaling_identity():
    """grad(S L) = S grad(L): with power-of-two scales large enough that no
    intermediate underflows, the FP16 gradients scale bitwise; at S = 1 the
    small activation gradients underflow (the failure loss scaling fixes)."""
    master = _init()
    p16 = {k: F.round_to(v, F.F16) for k, v in M.split(master).items()}
    x, y = _batch(1)
    g10 = M.forward_backward(p16, x, y, 2.0 ** 10)
    g16 = M.forward_backward(p16, x, y, 2.0 ** 14)
    for k in ("dlog", "dA", "dZ1"):           # elementwise chain: exact where normal
        normal = np.abs(g10[k]) >= F.F16.min_normal
        assert np.array_equal(g16[k][normal], g10[k][normal] * 16.0), k
        assert normal.mean() > 0.99
    # sums may see subnormal addends (rounding error <= 2^-25 each at the
    # smaller scale); the difference stays within that plus one output ulp
    half_sub = 2.0 ** -25
    bounds = {"dW2": np.abs(g10["dlog"] < F.F16.min_normal).T.astype(float) @ np.abs(g10["a"]) * half_sub,
              "db2": np.zeros(M.D_OUT),
              "dW1": (np.abs(g10["dZ1"]) < F.F16.min_normal).T.astype(float) @ np.abs(g10["x16"]) * half_sub,
              "db1": (np.abs(g10["dZ1"]) < F.F16.min_normal).sum(0) * half_sub}
    for k in ("dW2", "db2", "dW1", "db1"):
        diff = np.abs(g16[k] / 16.0 - g10[k])
        ulp = np.spacing(np.abs(g10[k]).astype(np.float16)).astype(np.float64)
        assert np.all(diff <= bounds[k] + ulp), k
        assert np.mean(diff == 0) > 0.99, k
    g1 = M.forward_backward(p16, x, y, 1.0)
    sub = np.abs(g1["dZ1"]) < F.F16.min_normal
    assert sub.mean() > 0.05             # many activation grads are subnormal/zero
    assert not np.array_equal(g16["dW1"], g1["dW1"] * 2.0 ** 14)


def test_ten_steps_scaler_sequence_and_skip():
    st = M.MLPState(master=_init())
    hp = A.AdamWHParams(lr=1e-3)
    recs = []
    for t in range(10):
        x, y = _batch(t)
        before = st.master.copy()
        r = M.train_step(st, x, y, hp, inject=(t == 3))
        recs.append(r)
        if t == 3:
            assert not r["applied"] and np.array_equal(st.master, before)
    assert [r["scale"] for r in recs] == [65536.0] * 4 + [32768.0] * 6
    assert [r["tracker"] for r in recs] == [1, 2, 3, 0, 1, 2, 3, 4, 5, 6]
    assert [r["applied"] for r in recs] == [True] * 3 + [False] + [True] * 6
    assert st.ctr.step == 9
    losses = [r["loss"] for r in recs]
    assert all(np.isfinite(losses)) and all(abs(l - np.log(10)) < 0.5 for l in losses)
