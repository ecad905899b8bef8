"""Seeded synthetic inputs shared by the oracle-side tests and the GPU side.

This module draws random numbers and stores them in the input formats of the
workloads (FP32, and 16-bit codes made with NumPy / PyTorch's own
conversions).  It holds none of the mixed-precision method's arithmetic: no
scaled casts, no amax, no recipe, no optimizer, no quantizer.  Both the oracle
and the HIP path consume the bytes it returns.

Workload shapes and laws (each documented where the workload is defined):
* mlp:      x ~ N(0,1) [64 x 512] FP32, labels U{0..9}, nn.Linear-default
            uniform init U(+-1/sqrt(fan_in)) for weights and biases.
* adam:     theta ~ N(0, 0.02) FP32, grads 1e-4 * N(0,1) * exp(2 Z) scaled by the
            live loss scale and stored FP16, 4 injected non-finite steps of 200.
* gemm:     activations ~ N(0,1) BF16, weights ~ N(0, 0.02) FP32,
            output gradients ~ N(0,1) BF16.
* fp8:      activations sigma_t * Student-t(3) BF16 with sigma_t = 1.02^t,
            output gradients 1e-3 * Student-t(3) BF16.
* nvfp4:    N(0,1) BF16 with 0.1 % of entries set to +-50.
"""
from __future__ import annotations

import numpy as np

__all__ = ["mlp_init", "mlp_batch",
    "rng", "normal_f32", "student_t_f32", "to_bf16_codes", "to_f16_codes",
    "f32_bits", "bf16_codes_normal", "outlier_bf16_codes", "edge_f32_values",
    "injection_schedule",
]


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_f32(seed: int, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    return (rng(seed).standard_normal(shape, dtype=np.float64) * std + mean).astype(np.float32)


def student_t_f32(seed: int, shape, nu: float = 3.0, scale: float = 1.0) -> np.ndarray:
    return (rng(seed).standard_t(nu, size=shape) * scale).astype(np.float32)


def to_bf16_codes(x_f32: np.ndarray) -> np.ndarray:
    """BF16 codes of FP32 data via PyTorch's CPU conversion (input making only)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def to_f16_codes(x_f32: np.ndarray) -> np.ndarray:
    """FP16 codes via NumPy's IEEE conversion (input making only)."""
    return np.asarray(x_f32, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_bits(x_f32: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x_f32, dtype=np.float32).view(np.uint32)


def bf16_codes_normal(seed: int, shape, std: float = 1.0) -> np.ndarray:
    return to_bf16_codes(normal_f32(seed, shape, std))


def outlier_bf16_codes(seed: int, shape, frac: float = 1e-3, mag: float = 50.0) -> np.ndarray:
    """N(0,1) with a seeded fraction of entries replaced by +-mag."""
    g = rng(seed)
    x = g.standard_normal(shape).astype(np.float32)
    n = x.size
    k = int(round(frac * n))
    idx = g.choice(n, size=k, replace=False)
    sgn = np.where(g.random(k) < 0.5, -1.0, 1.0).astype(np.float32)
    x.reshape(-1)[idx] = sgn * np.float32(mag)
    return to_bf16_codes(x)


def edge_f32_values() -> np.ndarray:
    """Special FP32 inputs: signed zeros, subnormals, format boundaries and
    rounding ties of the 16- and 8-bit formats, inf and NaN."""
    v = [0.0, -0.0, 1.0, -1.0, 2.0 ** -149, -2.0 ** -149, 2.0 ** -126,
         2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25, 2.0 ** -14, 65504.0, 65519.0,
         65520.0, -65520.0, 448.0, 464.0, 465.0, 480.0, 2.0 ** -9, 2.0 ** -10,
         1.5 * 2.0 ** -10, 57344.0, 61440.0, 1e30, -1e30, 3.4e38,
         1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -11, 1.0 + 2.0 ** -12,
         np.inf, -np.inf, np.nan, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0,
         7.0, 2.0 ** -6, 2.0 ** -7 * 1.5, 0.1, -0.1, 3.14159]
    return np.array(v, dtype=np.float32)


def injection_schedule(seed: int, n_steps: int = 200, n_inject: int = 4,
                       n_params: int = 1 << 31):
    """(step, index, value) triples for injected non-finite gradients: exactly
    ``n_inject`` steps drawn without replacement; the k-th writes
    (+inf, NaN, -inf, NaN)[k % 4] at one seeded index."""
    g = rng(seed)
    steps = np.sort(g.choice(n_steps, size=n_inject, replace=False))
    vals = [np.inf, np.nan, -np.inf, np.nan]
    return [(int(s), int(g.integers(0, n_params)), vals[k % 4])
            for k, s in enumerate(steps)]


MLP_SHAPES = (("W1", (2048, 512), 512), ("b1", (2048,), 512), ("W2", (10, 2048), 2048),
              ("b2", (10,), 2048))


def mlp_init(seed: int = 0) -> np.ndarray:
    """Flat FP32 parameters [W1, b1, W2, b2] of Linear(512,2048) + Linear(2048,10),
    each drawn U(-1/sqrt(fan_in), 1/sqrt(fan_in)) (the nn.Linear default)."""
    g = rng(seed)
    parts = []
    for _, shp, fan_in in MLP_SHAPES:
        bnd = 1.0 / np.sqrt(fan_in)
        parts.append(g.uniform(-bnd, bnd, size=shp).astype(np.float32).ravel())
    return np.concatenate(parts)


def mlp_batch(t: int, batch: int = 64, d_in: int = 512, classes: int = 10):
    """Batch t: x ~ N(0,1) FP32 [batch, d_in], labels uniform in 0..classes-1."""
    x = normal_f32(1000 + t, (batch, d_in))
    y = rng(2000 + t).integers(0, classes, size=batch).astype(np.int32)
    return x, y


# ---- device-side generators (PyTorch RNG on the GPU; input making only) ----

def torch_student_t(gen, shape, device="cuda"):
    """Student-t with 3 degrees of freedom: N0 / sqrt((N1^2 + N2^2 + N3^2) / 3)."""
    import torch
    z = torch.randn((4,) + tuple(shape), generator=gen, device=device)
    return z[0] / torch.sqrt((z[1] ** 2 + z[2] ** 2 + z[3] ** 2) / 3.0)


def adam_grads_f16(gen, n, loss_scale, device="cuda"):
    """FP16 gradients round16(S * 1e-4 * N(0,1) * exp(2 Z)) (PyTorch's RNE
    conversion; values beyond the FP16 range become inf, as a real overflow)."""
    import torch
    out = torch.empty(n, device=device, dtype=torch.float16)
    chunk = 1 << 26
    for o in range(0, n, chunk):
        k = min(chunk, n - o)
        z = torch.randn(k, generator=gen, device=device)
        g = torch.randn(k, generator=gen, device=device) * 1e-4 * torch.exp(2.0 * z)
        out[o:o + k] = (g * loss_scale).half()
    return out


def nvfp4_operand(seed, rows, k):
    """Synthetic NVFP4 operand: random E2M1 codes, E4M3 block scales in
    [2^-6, 2^6] and a tensor scale (for GEMM tests independent of a quantizer)."""
    g = rng(seed)
    q = g.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    e = g.integers(1, 13, size=(rows, k // 16))            # exponent field 1..12
    m = g.integers(0, 8, size=(rows, k // 16))
    sc = ((e << 3) | m).astype(np.uint8)
    enc = float(np.float32(g.uniform(1.0, 100.0)))
    return q, sc, enc
