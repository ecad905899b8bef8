"""MI355X (gfx950) mixed-precision training hot path.

A thin ctypes binding of ``libamp.so`` (built from ``csrc/`` by
``mixed_precision_numerics_amd.build``).  Every function has the name and
argument order of the C entry point declared in ``include/amp.h``; this module
only marshals arguments (device pointers from torch tensors or ints, host
structs, the stream handle) and turns a negative status into ``AmpError``.
All arithmetic runs in the HIP kernels.  There is no CPU fallback: when the
library is missing or no gfx950 device is current, the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "F32", "F16", "BF16", "E4M3", "E5M2", "E2M1X2", "OP_N", "OP_T", "ROUND_RNE", "ROUND_SR",
    "AMAX_MAX", "AMAX_MOST_RECENT", "OPT_SKIP_CHECK", "GEMM_FP8_NATIVE", "AmpError", "AdamWHParams",
    "ScalerParams", "DelayedRecipe", "BlockScales", "SCALER_STATE_DTYPE", "FP8_META_DTYPE",
    "lib_path", "load", "amp_abi_version", "amp_status_string", "amp_last_hip_error",
    "amp_cast", "amp_gemm", "amp_gemm_ex", "amp_scaler_init", "amp_optimizer_step", "amp_check_overflow",
    "amp_scaler_update", "amp_fp8_meta_init", "amp_delayed_scaling_update",
    "amp_nvfp4_quantize", "amp_bias_gelu_f16", "amp_softmax_xent_f16", "amp_gelu_backward_f16",
    "amp_colsum_f16", "amp_grad_accumulate", "amp_grad_norm_init", "amp_grad_norm_accumulate",
    "amp_clip_coefficient", "amp_optimizer_step_ex", "NORM_STATE_BYTES", "NORM_PARTIALS",
    "amp_cast_current_scaling", "amp_mx_quantize", "GEMM_MX",
    "amp_quantize_blockwise", "amp_gemm_blockwise", "amp_cast_ex",
    "amp_found_inf_from_amax", "amp_stream_copy", "amp_grad_norm_accumulate_noalloc",
    "amp_fp8_mfma_probe",
]

F32, F16, BF16, E4M3, E5M2, E2M1X2 = 0, 1, 2, 3, 4, 5
NORM_PARTIALS = 1024                       # amp_grad_norm_state: sumsq + partials
NORM_STATE_BYTES = 8 * (1 + NORM_PARTIALS)
OP_N, OP_T = 0, 1
ROUND_RNE, ROUND_SR = 0, 1
AMAX_MAX, AMAX_MOST_RECENT = 0, 1
OPT_SKIP_CHECK = 1
GEMM_FP8_NATIVE = 1
GEMM_MX = 2

# Device-resident state layouts (mirror the C structs; for reading back).
SCALER_STATE_DTYPE = np.dtype([("scale", "<f4"), ("growth_tracker", "<i4"),
                               ("found_inf", "<i4"), ("pad", "<i4"), ("adam_step", "<i8"),
                               ("beta1_pow", "<f8"), ("beta2_pow", "<f8")])
FP8_META_DTYPE = np.dtype([("amax_cur", "<f4"), ("scale", "<f4"), ("scale_inv", "<f4"),
                           ("pos", "<i4")])
assert SCALER_STATE_DTYPE.itemsize == 40 and FP8_META_DTYPE.itemsize == 16


class AmpError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = load()
        msg = lib.amp_status_string(status).decode()
        if status == -3:
            msg += f" (hipError_t {lib.amp_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [{status}]")
        self.status = status


class AdamWHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double)]


class ScalerParams(ctypes.Structure):
    _fields_ = [("growth_factor", ctypes.c_float), ("backoff_factor", ctypes.c_float),
                ("growth_interval", ctypes.c_int32)]


class DelayedRecipe(ctypes.Structure):
    _fields_ = [("fp8_max", ctypes.c_float), ("margin", ctypes.c_float),
                ("history_len", ctypes.c_int32), ("algo", ctypes.c_int32)]


class BlockScales(ctypes.Structure):
    _fields_ = [("scales", ctypes.c_void_p), ("ld", ctypes.c_int64),
                ("block2d", ctypes.c_int32), ("pad_", ctypes.c_int32)]


_P, _I, _I64, _U64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64
_SIGS = {
    "amp_abi_version": ([], _I),
    "amp_status_string": ([_I], ctypes.c_char_p),
    "amp_last_hip_error": ([], _I),
    "amp_cast": ([_P, _I, _I64, _I64, _I64, _P, _I, _I64, _P, _I64, _P, _P, _P], _I),
    "amp_found_inf_from_amax": ([_P, ctypes.c_int32, _I, _P, _P, _P], _I),
    "amp_cast_ex": ([_P, _I, _I64, _I64, _I64, _P, _I, _I64, _P, _I64, _P, _P, _P, _P], _I),
    "amp_gemm": ([_I, _I, _I64, _I64, _I64, _P, _I, _I64, _P, _P, _I, _I64, _P, _P, _I, _I64,
                  _P, _P, _P], _I),
    "amp_gemm_ex": ([_I, _I, _I64, _I64, _I64, _P, _I, _I64, _P, _P, _I, _I64, _P, _P, _I, _I64,
                     _P, _P, _I, _P], _I),
    "amp_scaler_init": ([_P, ctypes.c_float, _P], _I),
    "amp_optimizer_step": ([_P, _P, _P, _P, _I, _P, _I, _I64, _P, _P, _I, _P], _I),
    "amp_check_overflow": ([_P, _I, _I64, _P, _P], _I),
    "amp_optimizer_step_ex": ([_P, _P, _P, _P, _I, _P, _I, _I64, _P, _P, _P, _I, _P], _I),
    "amp_stream_copy": ([_P, _P, _I64, _P], _I),
    "amp_fp8_mfma_probe": ([_I, _I, _P, _P, _P, _I64, _P], _I),
    "amp_grad_norm_accumulate_noalloc": ([_P, _I, _I64, _P, _P, _P], _I),
    "amp_grad_accumulate": ([_P, _P, _I, _I64, _I, _P], _I),
    "amp_mx_quantize": ([_P, _I, _I64, _I64, _I64, _I, _I, _P, _P, _P], _I),
    "amp_quantize_blockwise": ([_P, _I, _I64, _I64, _I64, _I, _I, _P, _I64, _P, _I64, _P, _I64,
                                _P, _I64, _P], _I),
    "amp_gemm_blockwise": ([_I64, _I64, _I64, _P, _I, _I64, _P, _I64, _I, _P, _I, _I64, _P, _I64,
                            _I, _P, _I, _I64, _P], _I),
    "amp_cast_current_scaling": ([_P, _I, _I64, _I64, _I64, _P, _I, _I64, _P, _I64, _P, _P, _P],
                                 _I),
    "amp_grad_norm_init": ([_P, _P], _I),
    "amp_grad_norm_accumulate": ([_P, _I, _I64, _P, _P, _P], _I),
    "amp_clip_coefficient": ([_P, ctypes.c_float, _P, _P, _P], _I),
    "amp_scaler_update": ([_P, _P, _P], _I),
    "amp_fp8_meta_init": ([_P, _P, ctypes.c_int32, ctypes.c_int32, _P], _I),
    "amp_delayed_scaling_update": ([_P, _P, ctypes.c_int32, _P, _P], _I),
    "amp_nvfp4_quantize": ([_P, _I, _I64, _I64, _I64, _I, _I, _I, _U64, _I, _U64, _P, _P, _P,
                            _P], _I),
    "amp_bias_gelu_f16": ([_P, _I64, _I64, _P, _P, _P, _P], _I),
    "amp_softmax_xent_f16": ([_P, _P, _I64, _I64, _P, _P, _P, _P], _I),
    "amp_gelu_backward_f16": ([_P, _P, _I64, _P, _P], _I),
    "amp_colsum_f16": ([_P, _I64, _I64, _P, _P], _I),
}

_lib = None


def lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libamp.so")


def load():
    """Load ``libamp.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        p = lib_path()
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing: build it with "
                               "`python -m mixed_precision_numerics_amd.build`")
        lib = ctypes.CDLL(p)
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, ctypes.Structure):
        return ctypes.addressof(x)
    raise TypeError(f"cannot take a device pointer from {type(x)!r}")


def _stream(s) -> int | None:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise AmpError(fn, status)


# bytes per element of the whole-byte types (E2M1X2 packs two per byte and is
# not size-checked here)
_EB = {F32: 4, F16: 2, BF16: 2, E4M3: 1, E5M2: 1}


def _mat(rows, cols, ld, dt) -> int:
    """Bytes a row-major [rows, cols] operand with row stride ``ld`` spans."""
    if rows <= 0 or cols <= 0 or dt not in _EB:
        return 0
    return ((rows - 1) * ld + cols) * _EB[dt]


def _vec(n, dt) -> int:
    return n * _EB[dt] if n > 0 and dt in _EB else 0


def _room(fn: str, what: str, t, nbytes: int) -> None:
    """Raise before the launch when a torch tensor's storage, from its data
    pointer on, holds fewer bytes than the call will touch.  The C entry
    points take bare pointers and cannot see allocation sizes; integer
    pointers stay the caller's responsibility."""
    if nbytes <= 0 or t is None or not hasattr(t, "untyped_storage"):
        return
    st = t.untyped_storage()
    have = st.nbytes() - (t.data_ptr() - st.data_ptr())
    if have < nbytes:
        raise ValueError(f"{fn}: {what} holds {have} bytes from its data pointer; "
                         f"the call spans {nbytes}")


def _room_cast(fn, x, xt, rows, cols, ldx, y, yt, ldy, y_t, ldy_t) -> None:
    _room(fn, "x", x, _mat(rows, cols, ldx, xt))
    _room(fn, "y", y, _mat(rows, cols, ldy, yt))
    _room(fn, "y_t", y_t, _mat(cols, rows, ldy_t, yt))


def _room_opt(fn, master, m, v, grads, gt, w16, wt, n) -> None:
    for what, t in (("master", master), ("m", m), ("v", v)):
        _room(fn, what, t, _vec(n, F32))
    _room(fn, "grads", grads, _vec(n, gt))
    _room(fn, "w16", w16, _vec(n, wt))


def _room_gemm(fn, opA, opB, M, N, K, A, at, lda, B, bt, ldb, C, ct, ldc) -> None:
    _room(fn, "A", A, _mat(M, K, lda, at) if opA == OP_N else _mat(K, M, lda, at))
    _room(fn, "B", B, _mat(K, N, ldb, bt) if opB == OP_N else _mat(N, K, ldb, bt))
    _room(fn, "C", C, _mat(M, N, ldc, ct))


def amp_abi_version() -> int:
    return load().amp_abi_version()


def amp_status_string(status: int) -> str:
    return load().amp_status_string(status).decode()


def amp_last_hip_error() -> int:
    return load().amp_last_hip_error()


def amp_cast(x, xt, rows, cols, ldx, y, yt, ldy, y_t=None, ldy_t=0, d_scale=None, d_amax=None,
             stream=None):
    _room_cast("amp_cast", x, xt, rows, cols, ldx, y, yt, ldy, y_t, ldy_t)
    _check("amp_cast", load().amp_cast(_ptr(x), xt, rows, cols, ldx, _ptr(y), yt, ldy,
                                       _ptr(y_t), ldy_t, _ptr(d_scale), _ptr(d_amax),
                                       _stream(stream)))


def amp_found_inf_from_amax(d_amax, n, yt, d_scale, d_state, stream=None):
    _check("amp_found_inf_from_amax", load().amp_found_inf_from_amax(
        _ptr(d_amax), n, yt, _ptr(d_scale), _ptr(d_state), _stream(stream)))


def amp_cast_ex(x, xt, rows, cols, ldx, y, yt, ldy, y_t=None, ldy_t=0, d_scale=None,
                d_amax=None, d_sat_count=None, stream=None):
    _room_cast("amp_cast_ex", x, xt, rows, cols, ldx, y, yt, ldy, y_t, ldy_t)
    _check("amp_cast_ex", load().amp_cast_ex(_ptr(x), xt, rows, cols, ldx, _ptr(y), yt, ldy,
                                             _ptr(y_t), ldy_t, _ptr(d_scale), _ptr(d_amax),
                                             _ptr(d_sat_count), _stream(stream)))


def amp_gemm(opA, opB, M, N, K, A, at, lda, d_alphaA, B, bt, ldb, d_alphaB, C, ct, ldc,
             bsA=None, bsB=None, stream=None):
    _room_gemm("amp_gemm", opA, opB, M, N, K, A, at, lda, B, bt, ldb, C, ct, ldc)
    _check("amp_gemm", load().amp_gemm(
        opA, opB, M, N, K, _ptr(A), at, lda, _ptr(d_alphaA), _ptr(B), bt, ldb, _ptr(d_alphaB),
        _ptr(C), ct, ldc, ctypes.byref(bsA) if bsA is not None else None,
        ctypes.byref(bsB) if bsB is not None else None, _stream(stream)))


def amp_gemm_ex(opA, opB, M, N, K, A, at, lda, d_alphaA, B, bt, ldb, d_alphaB, C, ct, ldc,
                bsA=None, bsB=None, flags=0, stream=None):
    _room_gemm("amp_gemm_ex", opA, opB, M, N, K, A, at, lda, B, bt, ldb, C, ct, ldc)
    _check("amp_gemm_ex", load().amp_gemm_ex(
        opA, opB, M, N, K, _ptr(A), at, lda, _ptr(d_alphaA), _ptr(B), bt, ldb, _ptr(d_alphaB),
        _ptr(C), ct, ldc, ctypes.byref(bsA) if bsA is not None else None,
        ctypes.byref(bsB) if bsB is not None else None, flags, _stream(stream)))


def amp_scaler_init(d_state, init_scale=65536.0, stream=None):
    _check("amp_scaler_init", load().amp_scaler_init(_ptr(d_state), init_scale, _stream(stream)))


def amp_optimizer_step(master, m, v, grads, gt, w16, wt, n, hp: AdamWHParams, d_state,
                       flags=0, stream=None):
    _room_opt("amp_optimizer_step", master, m, v, grads, gt, w16, wt, n)
    _check("amp_optimizer_step", load().amp_optimizer_step(
        _ptr(master), _ptr(m), _ptr(v), _ptr(grads), gt, _ptr(w16), wt, n, ctypes.byref(hp),
        _ptr(d_state), flags, _stream(stream)))


def amp_optimizer_step_ex(master, m, v, grads, gt, w16, wt, n, hp: AdamWHParams, d_state,
                          d_grad_mult=None, flags=0, stream=None):
    _room_opt("amp_optimizer_step_ex", master, m, v, grads, gt, w16, wt, n)
    _check("amp_optimizer_step_ex", load().amp_optimizer_step_ex(
        _ptr(master), _ptr(m), _ptr(v), _ptr(grads), gt, _ptr(w16), wt, n, ctypes.byref(hp),
        _ptr(d_state), _ptr(d_grad_mult), flags, _stream(stream)))


def amp_cast_current_scaling(x, xt, rows, cols, ldx, y, yt, ldy, y_t, ldy_t,
                             r: "DelayedRecipe", d_meta, stream=None):
    _room_cast("amp_cast_current_scaling", x, xt, rows, cols, ldx, y, yt, ldy, y_t, ldy_t)
    _check("amp_cast_current_scaling", load().amp_cast_current_scaling(
        _ptr(x), xt, rows, cols, ldx, _ptr(y), yt, ldy, _ptr(y_t), ldy_t, ctypes.byref(r),
        _ptr(d_meta), _stream(stream)))


def amp_quantize_blockwise(x, xt, rows, cols, ldx, yt, block, q, ldq, s, lds, qt=None, ldqt=0,
                           st=None, ldst=0, stream=None):
    f = "amp_quantize_blockwise"
    _room(f, "x", x, _mat(rows, cols, ldx, xt))
    _room(f, "q", q, _mat(rows, cols, ldq, yt))
    _room(f, "qt", qt, _mat(cols, rows, ldqt, yt))
    _check("amp_quantize_blockwise", load().amp_quantize_blockwise(
        _ptr(x), xt, rows, cols, ldx, yt, int(block), _ptr(q), ldq, _ptr(s), lds, _ptr(qt), ldqt,
        _ptr(st), ldst, _stream(stream)))


def amp_gemm_blockwise(M, N, K, A, at, lda, sA, ldsA, a_block, B, bt, ldb, sB, ldsB, b_block,
                       C, ct, ldc, stream=None):
    f = "amp_gemm_blockwise"
    _room(f, "A", A, _mat(M, K, lda, at))
    _room(f, "B", B, _mat(N, K, ldb, bt))
    _room(f, "C", C, _mat(M, N, ldc, ct))
    _check("amp_gemm_blockwise", load().amp_gemm_blockwise(
        M, N, K, _ptr(A), at, lda, _ptr(sA), ldsA, int(a_block), _ptr(B), bt, ldb, _ptr(sB),
        ldsB, int(b_block), _ptr(C), ct, ldc, _stream(stream)))


def amp_mx_quantize(x, xt, rows, cols, ldx, transpose, yt, q, scales, stream=None):
    R, K = (cols, rows) if transpose else (rows, cols)
    _room("amp_mx_quantize", "x", x, _mat(rows, cols, ldx, xt))
    if R > 0 and K > 0:
        _room("amp_mx_quantize", "q", q, R * K // 2 if yt == E2M1X2 else R * K)
        _room("amp_mx_quantize", "scales", scales, R * (K // 32))
    _check("amp_mx_quantize", load().amp_mx_quantize(_ptr(x), xt, rows, cols, ldx,
                                                     int(transpose), yt, _ptr(q), _ptr(scales),
                                                     _stream(stream)))


def amp_grad_accumulate(acc, grads, gt, n, first, stream=None):
    _room("amp_grad_accumulate", "acc", acc, _vec(n, F32))
    _room("amp_grad_accumulate", "grads", grads, _vec(n, gt))
    _check("amp_grad_accumulate", load().amp_grad_accumulate(_ptr(acc), _ptr(grads), gt, n,
                                                             int(bool(first)), _stream(stream)))


def amp_grad_norm_init(d_norm, stream=None):
    _check("amp_grad_norm_init", load().amp_grad_norm_init(_ptr(d_norm), _stream(stream)))


def amp_grad_norm_accumulate(grads, gt, n, d_state, d_norm, stream=None):
    _room("amp_grad_norm_accumulate", "grads", grads, _vec(n, gt))
    _check("amp_grad_norm_accumulate", load().amp_grad_norm_accumulate(
        _ptr(grads), gt, n, _ptr(d_state), _ptr(d_norm), _stream(stream)))


def amp_grad_norm_accumulate_noalloc(grads, gt, n, d_state, d_sumsq, stream=None):
    _room("amp_grad_norm_accumulate_noalloc", "grads", grads, _vec(n, gt))
    _check("amp_grad_norm_accumulate_noalloc", load().amp_grad_norm_accumulate_noalloc(
        _ptr(grads), gt, n, _ptr(d_state), _ptr(d_sumsq), _stream(stream)))


def amp_clip_coefficient(d_norm, max_norm, d_state, d_out, stream=None):
    _check("amp_clip_coefficient", load().amp_clip_coefficient(
        _ptr(d_norm), float(max_norm), _ptr(d_state), _ptr(d_out), _stream(stream)))


def amp_check_overflow(x, xt, n, d_state, stream=None):
    _room("amp_check_overflow", "x", x, _vec(n, xt))
    _check("amp_check_overflow", load().amp_check_overflow(_ptr(x), xt, n, _ptr(d_state),
                                                           _stream(stream)))


def amp_scaler_update(d_state, p: ScalerParams | None = None, stream=None):
    _check("amp_scaler_update", load().amp_scaler_update(
        _ptr(d_state), ctypes.byref(p) if p is not None else None, _stream(stream)))


def amp_fp8_meta_init(d_metas, d_history, n, history_len, stream=None):
    _check("amp_fp8_meta_init", load().amp_fp8_meta_init(_ptr(d_metas), _ptr(d_history), n,
                                                         history_len, _stream(stream)))


def amp_delayed_scaling_update(d_metas, d_history, n, r: DelayedRecipe, stream=None):
    _check("amp_delayed_scaling_update", load().amp_delayed_scaling_update(
        _ptr(d_metas), _ptr(d_history), n, ctypes.byref(r), _stream(stream)))


def amp_nvfp4_quantize(x, xt, rows, cols, ldx, transpose, block2d, rht, rht_seed, rnd, sr_seed,
                       q, scales, d_tensor, stream=None):
    R, K = (cols, rows) if transpose else (rows, cols)
    _room("amp_nvfp4_quantize", "x", x, _mat(rows, cols, ldx, xt))
    if R > 0 and K > 0:
        _room("amp_nvfp4_quantize", "q", q, R * (K // 2))
        _room("amp_nvfp4_quantize", "scales", scales,
              (R // 16) * (K // 16) if block2d else R * (K // 16))
    _check("amp_nvfp4_quantize", load().amp_nvfp4_quantize(
        _ptr(x), xt, rows, cols, ldx, int(transpose), int(block2d), int(rht), rht_seed, rnd,
        sr_seed, _ptr(q), _ptr(scales), _ptr(d_tensor), _stream(stream)))


def amp_bias_gelu_f16(acc, rows, cols, b16, z16, a16=None, stream=None):
    _check("amp_bias_gelu_f16", load().amp_bias_gelu_f16(_ptr(acc), rows, cols, _ptr(b16), _ptr(z16),
                                                         _ptr(a16), _stream(stream)))


def amp_softmax_xent_f16(logits16, labels, rows, cols, d_state, d_loss, dlogits16, stream=None):
    _check("amp_softmax_xent_f16", load().amp_softmax_xent_f16(
        _ptr(logits16), _ptr(labels), rows, cols, _ptr(d_state), _ptr(d_loss), _ptr(dlogits16),
        _stream(stream)))


def amp_gelu_backward_f16(dA16, z16, n, dz16, stream=None):
    _check("amp_gelu_backward_f16", load().amp_gelu_backward_f16(_ptr(dA16), _ptr(z16), n,
                                                                 _ptr(dz16), _stream(stream)))


def amp_colsum_f16(x16, rows, cols, out16, stream=None):
    _check("amp_colsum_f16", load().amp_colsum_f16(_ptr(x16), rows, cols, _ptr(out16),
                                                   _stream(stream)))


def amp_stream_copy(src, dst, nbytes, stream=None):
    _room("amp_stream_copy", "src", src, nbytes)
    _room("amp_stream_copy", "dst", dst, nbytes)
    _check("amp_stream_copy", load().amp_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def amp_fp8_mfma_probe(shape, at, a, b, c, tiles, stream=None):
    _check("amp_fp8_mfma_probe", load().amp_fp8_mfma_probe(shape, at, _ptr(a), _ptr(b), _ptr(c),
                                                           tiles, _stream(stream)))
