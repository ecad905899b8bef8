"""The FP16 AMP training step of Linear(512,2048) -> GELU -> Linear(2048,10)
(batch 64, AdamW lr 1e-3, dynamic loss scale from 65536, +inf injected into
dW1[0,0] at step 3) run through the C ABI, checked against the oracle:
  * every op teacher-forced (the oracle op applied to the GPU's inputs);
  * the optimizer step and the loss-scale sequence bit-exact;
  * the 10-step loss trajectory against the free-running oracle."""
import numpy as np
import pytest
import torch

import mixed_precision_numerics_amd as amp
from oracle import adamw as OA
from oracle import formats as F
from oracle import gemm as OG
from oracle import mlp as OM
import synth
from gpu_util import host, scaler_state

pytestmark = pytest.mark.gpu

B, DI, DH, DO = 64, 512, 2048, 10
OFF = {"W1": 0, "b1": DH * DI, "W2": DH * DI + DH, "b2": DH * DI + DH + DO * DH}
N = OFF["b2"] + DO
HP = (1e-3, 0.9, 0.999, 1e-8, 0.01)


class GpuMLP:
    def __init__(self, master0):
        d = "cuda"
        self.master = torch.from_numpy(master0.copy()).to(d)
        self.m = torch.zeros(N, device=d)
        self.v = torch.zeros(N, device=d)
        self.w16 = torch.empty(N, device=d, dtype=torch.int16)
        self.g16 = torch.empty(N, device=d, dtype=torch.int16)
        self.st = torch.empty(40, device=d, dtype=torch.uint8)
        self.x16 = torch.empty(B * DI, device=d, dtype=torch.int16)
        self.z1acc = torch.empty(B * DH, device=d)
        self.z1 = torch.empty(B * DH, device=d, dtype=torch.int16)
        self.a = torch.empty(B * DH, device=d, dtype=torch.int16)
        self.lacc = torch.empty(B * DO, device=d)
        self.logits = torch.empty(B * DO, device=d, dtype=torch.int16)
        self.loss = torch.empty(1, device=d)
        self.dlog = torch.empty(B * DO, device=d, dtype=torch.int16)
        self.dA = torch.empty(B * DH, device=d, dtype=torch.int16)
        self.dz1 = torch.empty(B * DH, device=d, dtype=torch.int16)
        self.hp = amp.AdamWHParams(*HP)
        amp.amp_scaler_init(self.st, 65536.0)
        # the FP16 working copy is made from the FP32 masters before the first step
        amp.amp_cast(self.master, amp.F32, 1, N, N, self.w16, amp.F16, N)

    def p(self, t, name):
        return t.data_ptr() + 2 * OFF[name]

    def step(self, x, y, inject=False):
        d = "cuda"
        xd = torch.from_numpy(x).to(d)
        yd = torch.from_numpy(y).to(d)
        amp.amp_cast(xd, amp.F32, B, DI, DI, self.x16, amp.F16, DI)
        amp.amp_gemm(amp.OP_N, amp.OP_T, B, DH, DI, self.x16, amp.F16, DI, None,
                     self.p(self.w16, "W1"), amp.F16, DI, None, self.z1acc, amp.F32, DH)
        amp.amp_bias_gelu_f16(self.z1acc, B, DH, self.p(self.w16, "b1"), self.z1, self.a)
        amp.amp_gemm(amp.OP_N, amp.OP_T, B, DO, DH, self.a, amp.F16, DH, None,
                     self.p(self.w16, "W2"), amp.F16, DH, None, self.lacc, amp.F32, DO)
        amp.amp_bias_gelu_f16(self.lacc, B, DO, self.p(self.w16, "b2"), self.logits, None)
        amp.amp_softmax_xent_f16(self.logits, yd, B, DO, self.st, self.loss, self.dlog)
        amp.amp_gemm(amp.OP_T, amp.OP_N, DO, DH, B, self.dlog, amp.F16, DO, None, self.a,
                     amp.F16, DH, None, self.p(self.g16, "W2"), amp.F16, DH)
        amp.amp_colsum_f16(self.dlog, B, DO, self.p(self.g16, "b2"))
        amp.amp_gemm(amp.OP_N, amp.OP_N, B, DH, DO, self.dlog, amp.F16, DO, None,
                     self.p(self.w16, "W2"), amp.F16, DH, None, self.dA, amp.F16, DH)
        amp.amp_gelu_backward_f16(self.dA, self.z1, B * DH, self.dz1)
        amp.amp_gemm(amp.OP_T, amp.OP_N, DH, DI, B, self.dz1, amp.F16, DH, None, self.x16,
                     amp.F16, DI, None, self.p(self.g16, "W1"), amp.F16, DI)
        amp.amp_colsum_f16(self.dz1, B, DH, self.p(self.g16, "b1"))
        if inject:       # host-forced overflow in the gradient of W1[0, 0]
            self.g16[0] = 0x7C00
        snap = {k: host(getattr(self, k), np.uint16 if getattr(self, k).dtype == torch.int16
                        else np.float32).copy()
                for k in ("x16", "z1acc", "z1", "a", "lacc", "logits", "dlog", "dA", "dz1", "g16",
                          "w16", "loss")}
        snap.update(master=host(self.master, np.float32).copy(), m=host(self.m, np.float32).copy(),
                    v=host(self.v, np.float32).copy(), state=scaler_state(self.st).copy())
        amp.amp_optimizer_step(self.master, self.m, self.v, self.g16, amp.F16, self.w16, amp.F16,
                               N, self.hp, self.st)
        applied_state = scaler_state(self.st).copy()
        amp.amp_scaler_update(self.st)
        snap.update(master1=host(self.master, np.float32).copy(),
                    m1=host(self.m, np.float32).copy(), v1=host(self.v, np.float32).copy(),
                    w16_1=host(self.w16, np.uint16).copy(), found_inf=int(applied_state["found_inf"]),
                    state1=scaler_state(self.st).copy())
        return snap


def dec16(c):
    return F.decode(c, F.F16)


def within_one_ulp16(got_codes, want_values):
    want = F.encode(want_values, F.F16)
    return F.ulp_distance(got_codes, want, F.F16) <= 1


def gemm_ok(got_codes_or_f32, a, b, bias=None, f32=False):
    cref, bound = OG.reference(a, b)
    if bias is not None:
        cref = cref + bias[None, :]
        bound = bound + np.abs(bias)[None, :]
    if f32:
        return OG.check_f32(got_codes_or_f32.astype(np.float64), cref, bound)
    return OG.check_rounded(got_codes_or_f32, F.F16, cref, bound)


def test_mlp_amp_ten_steps():
    master0 = synth.mlp_init(0)
    gm = GpuMLP(master0)
    ost = OM.MLPState(master=master0.astype(np.float64))
    hp = OA.AdamWHParams(*HP)
    ctr = OA.AdamCounters()
    gpu_losses, ref_losses, scales, trackers, applied = [], [], [], [], []
    for t in range(10):
        x, y = synth.mlp_batch(t)
        s = gm.step(x, y, inject=(t == 3))
        S = float(s["state"]["scale"])
        # working copy is round16(master), bit for bit
        assert np.array_equal(s["w16"], F.encode(s["master"].astype(np.float64), F.F16))
        p16 = OM.split(dec16(s["w16"]))
        # ---- forward, teacher-forced
        assert np.array_equal(s["x16"], F.encode(x.astype(np.float64), F.F16).ravel())
        x16 = dec16(s["x16"]).reshape(B, DI)
        ok = gemm_ok(s["z1acc"].reshape(B, DH), x16, p16["W1"].T, f32=True)
        assert ok.all(), t
        z1 = dec16(s["z1"]).reshape(B, DH)
        assert np.array_equal(s["z1"].reshape(B, DH),
                              F.encode(F.f32(s["z1acc"].reshape(B, DH).astype(np.float64) + p16["b1"][None, :]), F.F16))
        assert within_one_ulp16(s["a"], OM.gelu(z1).ravel()).all()
        a = dec16(s["a"]).reshape(B, DH)
        assert gemm_ok(s["lacc"].reshape(B, DO), a, p16["W2"].T, f32=True).all()
        logits = dec16(s["logits"]).reshape(B, DO)
        fb = OM.forward_backward(p16, x.astype(np.float64), y, S)
        lg = logits - logits.max(axis=1, keepdims=True)
        lse = np.log(np.exp(lg).sum(axis=1))
        loss_tf = float(np.mean(lse - lg[np.arange(B), y]))
        assert abs(float(s["loss"][0]) - loss_tf) <= 1e-5 * abs(loss_tf)
        prob = np.exp(lg - lse[:, None])
        onehot = np.zeros_like(prob); onehot[np.arange(B), y] = 1.0
        assert within_one_ulp16(s["dlog"], (S * (prob - onehot) / B).ravel()).all()
        dlog = dec16(s["dlog"]).reshape(B, DO)
        # ---- backward GEMMs and glue, teacher-forced
        g = s["g16"]
        assert gemm_ok(g[OFF["W2"]:OFF["b2"]].reshape(DO, DH), dlog.T, a).all()
        assert gemm_ok(g[OFF["b2"]:].reshape(1, DO), np.ones((1, B)), dlog).all()
        assert gemm_ok(s["dA"].reshape(B, DH), dlog, p16["W2"]).all()
        dA = dec16(s["dA"]).reshape(B, DH)
        gp = F.f32(OM.gelu_grad(z1))
        assert within_one_ulp16(s["dz1"], F.f32(dA * gp).ravel()).all()
        dz1 = dec16(s["dz1"]).reshape(B, DH)
        okw1 = gemm_ok(g[:OFF["b1"]].reshape(DH, DI), dz1.T, x16)
        if t == 3:
            assert g[0] == 0x7C00          # the injected +inf
            okw1[0, 0] = True
        assert okw1.all()
        assert gemm_ok(g[OFF["b1"]:OFF["W2"]].reshape(1, DH), np.ones((1, B)), dz1).all()
        # ---- optimizer step: bit-exact given the GPU's gradients and state
        ctr_tf = OA.AdamCounters(int(s["state"]["adam_step"]), float(s["state"]["beta1_pow"]),
                                 float(s["state"]["beta2_pow"]))
        th1, m1, v1, w1, ok_step = OA.apply(s["master"].astype(np.float64),
                                            s["m"].astype(np.float64), s["v"].astype(np.float64),
                                            g, F.F16, hp, ctr_tf, S)
        assert bool(s["found_inf"]) == (not ok_step)
        assert np.array_equal(s["master1"].astype(np.float64), th1)
        assert np.array_equal(s["m1"].astype(np.float64), m1)
        assert np.array_equal(s["v1"].astype(np.float64), v1)
        if ok_step:
            assert np.array_equal(s["w16_1"], w1)
        # ---- free-running oracle alongside
        rec = OM.train_step(ost, x.astype(np.float64), y, hp, inject=(t == 3))
        gpu_losses.append(float(s["loss"][0])); ref_losses.append(rec["loss"])
        scales.append(S); trackers.append(int(s["state1"]["growth_tracker"]))
        applied.append(ok_step)
    assert scales == [65536.0] * 4 + [32768.0] * 6
    assert trackers == [1, 2, 3, 0, 1, 2, 3, 4, 5, 6]
    assert applied == [True] * 3 + [False] + [True] * 6
    rel = np.abs(np.array(gpu_losses) - np.array(ref_losses)) / np.abs(ref_losses)
    print("losses gpu", np.round(gpu_losses, 5), "max rel diff vs oracle", rel.max())
    assert rel.max() < 1e-3
