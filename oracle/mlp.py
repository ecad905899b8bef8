"""The tiny FP16 AMP training step (oracle).

Test infrastructure only (see ``oracle/__init__``).

Page "혼합 정밀도 학습" (itwiki), section "FP16 학습 루프": the model
``Linear(512, 2048) -> GELU -> Linear(2048, 10)`` trained with AdamW(lr=1e-3),
GradScaler and cross-entropy; linear layers run in FP16 under autocast while
cross-entropy runs in FP32 (section "PyTorch 자동 혼합 정밀도(torch.amp)";
page marovi, "Operaciones que permanecen en FP32": softmax and cross-entropy
stay FP32).  The backward pass starts from ``S * loss``; the parameters stay
FP32 masters and the 16-bit copies are made just before use.

Readings (the page prints a loop, not arithmetic):
* Working copies, activations and gradients are FP16 (itwiki "FP32 마스터
  가중치": 2-byte weights and 2-byte gradients).
* Linear layers: ``Z = round16(fl32(fl32(X16 @ W16^T) + b16))`` -- FP32
  accumulation (reference: float64 sum rounded once to FP32), bias added in
  FP32, then one rounding to FP16.
* GELU is the exact erf form, evaluated in float64 and rounded to FP16;
  its derivative is rounded to FP32 before multiplying the FP16 gradient.
* Loss: mean cross-entropy over the batch from the FP16 logits, in float64.
* ``dlogits = round16(S * (softmax - onehot) / B)``; weight and bias gradients
  are FP32-accumulated then rounded to FP16.
* Gradient clipping from the page's loop is not part of this step (it is a
  separate, later row); the optimizer sees the unscaled FP16 gradients.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from math import erf, sqrt, pi

import numpy as np

from . import adamw as A
from . import formats as F
from . import scaler as SC

D_IN, D_H, D_OUT, BATCH = 512, 2048, 10, 64
SHAPES = (("W1", (D_H, D_IN)), ("b1", (D_H,)), ("W2", (D_OUT, D_H)), ("b2", (D_OUT,)))
N_PARAMS = sum(int(np.prod(s)) for _, s in SHAPES)

_verf = np.vectorize(erf)


def r16(x):
    return F.round_to(x, F.F16)


def gelu(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + _verf(z / sqrt(2.0)))


def gelu_grad(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * (1.0 + _verf(z / sqrt(2.0))) + z * np.exp(-0.5 * z * z) / sqrt(2.0 * pi)


def linear(x16, w16, b16):
    """round16(fl32(fl32(x @ w^T) + b))."""
    acc = F.f32(x16 @ w16.T)
    return r16(F.f32(acc + b16[None, :]))


def split(flat):
    out, o = {}, 0
    for name, shp in SHAPES:
        n = int(np.prod(shp))
        out[name] = flat[o:o + n].reshape(shp)
        o += n
    return out


def forward_backward(p16: dict, x, y, S: float):
    """One forward + backward pass.  ``p16``: FP16 working copies (float64
    values); ``x``: FP32 input values [B, 512]; ``y``: int labels [B]."""
    x16 = r16(x)
    z1 = linear(x16, p16["W1"], p16["b1"])
    a = r16(gelu(z1))
    logits = linear(a, p16["W2"], p16["b2"])
    lg = logits - logits.max(axis=1, keepdims=True)
    lse = np.log(np.exp(lg).sum(axis=1))
    B = x.shape[0]
    loss = float(np.mean(lse - lg[np.arange(B), y]))
    prob = np.exp(lg - lse[:, None])
    onehot = np.zeros_like(prob)
    onehot[np.arange(B), y] = 1.0
    dlog = r16(S * (prob - onehot) / B)
    dW2 = r16(F.f32(dlog.T @ a))
    db2 = r16(F.f32(dlog.sum(axis=0)))
    dA = r16(F.f32(dlog @ p16["W2"]))
    gp = F.f32(gelu_grad(z1))
    dZ1 = r16(F.f32(dA * gp))
    dW1 = r16(F.f32(dZ1.T @ x16))
    db1 = r16(F.f32(dZ1.sum(axis=0)))
    return dict(x16=x16, z1=z1, a=a, logits=logits, loss=loss, dlog=dlog,
                dW2=dW2, db2=db2, dA=dA, gp=gp, dZ1=dZ1, dW1=dW1, db1=db1)


def flat_grads(fb: dict) -> np.ndarray:
    return np.concatenate([fb["dW1"].ravel(), fb["db1"].ravel(),
                           fb["dW2"].ravel(), fb["db2"].ravel()])


@dataclass
class MLPState:
    master: np.ndarray
    m: np.ndarray = None
    v: np.ndarray = None
    ctr: A.AdamCounters = field(default_factory=A.AdamCounters)
    scaler: SC.ScalerState = field(default_factory=SC.ScalerState)

    def __post_init__(self):
        if self.m is None:
            self.m = np.zeros_like(self.master)
        if self.v is None:
            self.v = np.zeros_like(self.master)


def train_step(st: MLPState, x, y, hp: A.AdamWHParams, inject: bool = False):
    """One full AMP step; returns a record of what happened."""
    S = st.scaler.scale
    p16 = split(r16(st.master))
    fb = forward_backward(p16, x, y, S)
    if inject:
        fb["dW1"] = fb["dW1"].copy()
        fb["dW1"][0, 0] = np.inf
    g = flat_grads(fb)
    codes = F.encode(g, F.F16)
    th, m, v, w16, applied = A.apply(st.master, st.m, st.v, codes, F.F16, hp, st.ctr, S)
    st.master, st.m, st.v = th, m, v
    SC.update(st.scaler, not applied)
    return dict(loss=fb["loss"], scale=S, applied=applied,
                tracker=st.scaler.growth_tracker, fb=fb, w16=w16)
