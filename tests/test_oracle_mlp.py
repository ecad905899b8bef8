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


def test_loss_at_init_is_near_log_classes():
    """At the default init the logits are small, so the mean cross-entropy is
    close to log(10) and the bias gradient of the last layer (columns of
    softmax - onehot) sums to about zero."""
    master = _init()
    p = M.split(master)
    x, y = _batch(0)
    fb = M.forward_backward({k: F.round_to(v, F.F16) for k, v in p.items()}, x, y, 1024.0)
    assert abs(fb["loss"] - np.log(10)) < 0.2
    assert abs(fb["db2"].sum()) / 1024.0 < 1e-2


def _ulp16(v):
    """Spacing of FP16 at |v| (the subnormal spacing below the normal range)."""
    a = np.maximum(np.abs(v), F.F16.min_normal)
    return 2.0 ** (np.floor(np.log2(a)) - 10)


def _close16(got, want, ulps=1.0):
    """got (an FP16 value) lies within ``ulps`` FP16 spacings of the float64 value."""
    return np.abs(got - want) <= ulps * _ulp16(want) + 1e-300


def test_forward_backward_against_float64_autograd_per_op():
    """Each op of the oracle step against PyTorch float64 autograd (a separate
    derivation of every gradient) fed the oracle's own FP16 inputs to that op:
    the oracle rounds once (twice for the FP32 accumulate + FP16 store) per op,
    so each output lies within an FP16 spacing of the exact float64 value.
    A wrong sign, a dropped bias or a dropped 1/B fails here."""
    import torch
    import torch.nn.functional as TF
    master = _init()
    p16 = {k: F.round_to(v, F.F16) for k, v in M.split(master).items()}
    x, y = _batch(2)
    S = 2.0 ** 12
    fb = M.forward_backward(p16, x, y, S)
    T = {k: torch.tensor(v) for k, v in p16.items()}
    yt = torch.tensor(y.astype(np.int64))

    def t(a, grad=False):
        return torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=grad)

    # forward, op by op
    assert np.array_equal(fb["x16"], F.round_to(x, F.F16))
    z1 = TF.linear(t(fb["x16"]), T["W1"], T["b1"]).numpy()
    assert _close16(fb["z1"], z1).all()
    a = TF.gelu(t(fb["z1"]), approximate="none").numpy()
    assert _close16(fb["a"], a).all()
    lg = TF.linear(t(fb["a"]), T["W2"], T["b2"]).numpy()
    assert _close16(fb["logits"], lg).all()
    loss = TF.cross_entropy(t(fb["logits"]), yt, reduction="mean")
    assert abs(fb["loss"] - float(loss)) < 1e-12

    # backward of S * loss through the logits
    lt = t(fb["logits"], grad=True)
    (S * TF.cross_entropy(lt, yt, reduction="mean")).backward()
    assert _close16(fb["dlog"], lt.grad.numpy()).all()

    # second linear: weight, bias and input gradients for the oracle's dlog
    at, w2, b2 = t(fb["a"], True), t(p16["W2"], True), t(p16["b2"], True)
    TF.linear(at, w2, b2).backward(t(fb["dlog"]))
    assert _close16(fb["dW2"], w2.grad.numpy()).all()
    assert _close16(fb["db2"], b2.grad.numpy()).all()
    assert _close16(fb["dA"], at.grad.numpy()).all()

    # GELU backward for the oracle's dA (the oracle rounds gelu' to FP32 first)
    zt = t(fb["z1"], True)
    TF.gelu(zt, approximate="none").backward(t(fb["dA"]))
    assert _close16(fb["dZ1"], zt.grad.numpy(), ulps=1.5).all()

    # first linear: weight and bias gradients for the oracle's dZ1
    xt, w1, b1 = t(fb["x16"], True), t(p16["W1"], True), t(p16["b1"], True)
    TF.linear(xt, w1, b1).backward(t(fb["dZ1"]))
    assert _close16(fb["dW1"], w1.grad.numpy()).all()
    assert _close16(fb["db1"], b1.grad.numpy()).all()


def _f64_loss(p, x16, y):
    """Float64 loss of the model with no rounding anywhere (numpy)."""
    z1 = x16 @ p["W1"].T + p["b1"]
    a = M.gelu(z1)
    lg = a @ p["W2"].T + p["b2"]
    lg = lg - lg.max(axis=1, keepdims=True)
    lse = np.log(np.exp(lg).sum(axis=1))
    return float(np.mean(lse - lg[np.arange(len(y)), y]))


def test_gradients_against_central_differences():
    """Central differences of the float64 loss at the FP16 weights against the
    oracle's unscaled FP16 gradients, on the largest entries of every
    parameter (where FP16 rounding of the chain is far below the check)."""
    master = _init()
    p16 = {k: F.round_to(v, F.F16) for k, v in M.split(master).items()}
    x, y = _batch(3)
    S = 2.0 ** 12
    fb = M.forward_backward(p16, x, y, S)
    x16 = fb["x16"]
    h = 1e-5
    for name, gname in (("W1", "dW1"), ("b1", "db1"), ("W2", "dW2"), ("b2", "db2")):
        g = fb[gname] / S
        flat = np.abs(g).ravel()
        picks = np.argsort(flat)[-4:]
        for i in picks:
            idx = np.unravel_index(i, g.shape)
            pp = {k: v.copy() for k, v in p16.items()}
            pp[name][idx] += h
            up = _f64_loss(pp, x16, y)
            pp[name][idx] -= 2 * h
            dn = _f64_loss(pp, x16, y)
            num = (up - dn) / (2 * h)
            assert abs(num - g[idx]) <= 0.02 * abs(num) + 1e-7, (name, idx, num, g[idx])


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
