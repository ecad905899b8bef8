"""Device-memory plumbing for the GPU tests (torch allocates, the library computes)."""
import numpy as np
import torch

import mixed_precision_numerics_amd as amp


def dev(arr: np.ndarray) -> torch.Tensor:
    """Copy a NumPy array's bytes to a new device buffer."""
    a = np.ascontiguousarray(arr)
    return torch.from_numpy(a.view(np.uint8).reshape(-1).copy()).to("cuda")


def empty(nbytes: int, fill: int = 0) -> torch.Tensor:
    t = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device="cuda")
    t.fill_(fill)
    return t


def host(t: torch.Tensor, dtype, shape=None) -> np.ndarray:
    torch.cuda.synchronize()
    a = t.detach().cpu().numpy().view(np.uint8).view(dtype)
    return a.reshape(shape) if shape is not None else a


def f32_dev(vals) -> torch.Tensor:
    return dev(np.asarray(vals, dtype=np.float32))


def scaler_state(t: torch.Tensor):
    return host(t, amp.SCALER_STATE_DTYPE)[0]


def metas(t: torch.Tensor, n: int):
    return host(t, amp.FP8_META_DTYPE)[:n]
