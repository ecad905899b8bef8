"""The C-ABI library loads and exports every function declared in include/amp.h
(no GPU needed: nothing is called except the version and status strings)."""
import ctypes
import os
import re

import pytest

import mixed_precision_numerics_amd as amp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "amp.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(amp_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("amp_cast", "amp_gemm", "amp_optimizer_step", "amp_scaler_update",
                     "amp_scaler_init", "amp_delayed_scaling_update", "amp_nvfp4_quantize",
                     "amp_check_overflow", "amp_fp8_meta_init"):
        assert required in names


@pytest.mark.skipif(not os.path.exists(amp.lib_path()), reason="libamp.so not built")
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(amp.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(amp._SIGS) == set(declared_functions())


@pytest.mark.skipif(not os.path.exists(amp.lib_path()), reason="libamp.so not built")
def test_version_and_status_strings():
    assert amp.amp_abi_version() == 1
    assert amp.amp_status_string(0) == "ok"
    assert amp.amp_status_string(-4).startswith("no gfx950")


@pytest.mark.skipif(not os.path.exists(amp.lib_path()), reason="libamp.so not built")
def test_invalid_arguments_rejected_before_any_device_work():
    lib = amp.load()
    # negative sizes, bad dtypes and bad enums fail validation without a device
    assert lib.amp_cast(None, 0, -1, 4, 4, None, 1, 4, None, 0, None, None, None) == -1
    assert lib.amp_cast(None, 7, 1, 4, 4, None, 1, 4, None, 0, None, None, None) == -2
    assert lib.amp_gemm(5, 0, 1, 1, 1, None, 2, 1, None, None, 2, 1, None, None, 2, 1,
                        None, None, None) == -1
    assert lib.amp_gemm(0, 1, 1, 1, 1, None, 2, 1, None, None, 1, 1, None, None, 2, 1,
                        None, None, None) == -2
    assert lib.amp_optimizer_step(None, None, None, None, 1, None, 1, -5, None, None, 0, None) == -1
    assert lib.amp_nvfp4_quantize(None, 2, 17, 32, 32, 0, 0, 0, 0, 0, 0, None, None, None, None) == -1
    # fine-grained FP8: bad block flag, non-FP8 output, missing scale buffer,
    # short scale stride, non-FP8 GEMM operand
    assert lib.amp_quantize_blockwise(None, 2, 4, 4, 4, 3, 2, None, 4, None, 4, None, 0, None, 0,
                                      None) == -1
    assert lib.amp_quantize_blockwise(None, 2, 4, 4, 4, 1, 0, None, 4, None, 4, None, 0, None, 0,
                                      None) == -2
    assert lib.amp_quantize_blockwise(8, 2, 4, 4, 4, 3, 0, 8, 4, None, 4, None, 0, None, 0,
                                      None) == -1
    assert lib.amp_quantize_blockwise(8, 2, 4, 4, 4, 3, 0, 8, 4, 8, 3, None, 0, None, 0,
                                      None) == -1
    assert lib.amp_gemm_blockwise(4, 4, 4, 8, 2, 4, 8, 4, 0, 8, 3, 4, 8, 4, 0, 8, 0, 4,
                                  None) == -2
    assert lib.amp_gemm_blockwise(4, 4, 4, 8, 3, 4, 8, 3, 0, 8, 3, 4, 8, 4, 0, 8, 0, 4,
                                  None) == -1
    # misaligned state / scalar pointers are argument errors, not faults
    assert lib.amp_scaler_init(12, 1024.0, None) == -1
    assert lib.amp_cast_ex(8, 2, 4, 4, 4, 8, 3, 4, None, 0, None, None, 12, None) == -1
    assert lib.amp_found_inf_from_amax(6, 1, 1, None, 8, None) == -1
    # empty work is a successful no-op
    assert lib.amp_cast(None, 0, 0, 4, 4, None, 1, 4, None, 0, None, None, None) == 0
    assert lib.amp_gemm_blockwise(0, 4, 4, None, 3, 4, None, 0, 0, None, 3, 4, None, 0, 0, None,
                                  0, 4, None) == 0


def test_binding_rejects_tensors_smaller_than_the_extents():
    """The binding compares each torch operand's storage with the bytes the
    call's sizes and strides span and raises before anything is launched
    (the C entry points see bare pointers and cannot)."""
    import torch
    bf, u8, f32 = torch.bfloat16, torch.uint8, torch.float32
    x = torch.zeros(8, 64, dtype=bf)
    with pytest.raises(ValueError, match="x holds"):
        amp.amp_cast(x, amp.BF16, 8, 448, 448, torch.zeros(8 * 448, dtype=u8), amp.E4M3, 448)
    with pytest.raises(ValueError, match="y_t holds"):
        amp.amp_cast(x, amp.BF16, 8, 64, 64, torch.zeros(512, dtype=u8), amp.E5M2, 64,
                     torch.zeros(511, dtype=u8), 8)
    # a view's span is counted from its own data pointer
    with pytest.raises(ValueError, match="y holds"):
        amp.amp_cast(x, amp.BF16, 8, 64, 64, torch.zeros(513, dtype=u8)[2:], amp.E4M3, 64)
    a, b = torch.zeros(64, 32, dtype=bf), torch.zeros(16, 32, dtype=bf)
    with pytest.raises(ValueError, match="B holds"):
        amp.amp_gemm(amp.OP_N, amp.OP_T, 64, 32, 32, a, amp.BF16, 32, None, b, amp.BF16, 32, None,
                     torch.zeros(64, 32, dtype=f32), amp.F32, 32)
    with pytest.raises(ValueError, match="C holds"):
        amp.amp_gemm(amp.OP_N, amp.OP_N, 64, 16, 32, a, amp.BF16, 32, None, b.view(32, 16),
                     amp.BF16, 16, None, torch.zeros(64, 15, dtype=f32), amp.F32, 16)
    p = torch.zeros(100, dtype=f32)
    with pytest.raises(ValueError, match="v holds"):
        amp.amp_optimizer_step(p, p, p[1:], torch.zeros(100, dtype=torch.float16), amp.F16, None,
                               amp.F16, 100, amp.AdamWHParams(1e-3, 0.9, 0.999, 1e-8, 0.0), None)
    with pytest.raises(ValueError, match="src holds"):
        amp.amp_stream_copy(torch.zeros(10, dtype=u8), torch.zeros(16, dtype=u8), 16)
    q = torch.zeros(64 * 32, dtype=u8)
    with pytest.raises(ValueError, match="qt holds"):
        amp.amp_quantize_blockwise(torch.zeros(64, 32, dtype=bf), amp.BF16, 64, 32, 32, amp.E4M3, 0,
                                   q, 32, torch.zeros(64), 64, q[1:], 64)
    with pytest.raises(ValueError, match="scales holds"):
        amp.amp_mx_quantize(torch.zeros(64, 64, dtype=bf), amp.BF16, 64, 64, 64, 1, amp.E4M3,
                            torch.zeros(64 * 64, dtype=u8), torch.zeros(127, dtype=u8))
    with pytest.raises(ValueError, match="q holds"):
        amp.amp_nvfp4_quantize(torch.zeros(32, 64, dtype=bf), amp.BF16, 32, 64, 64, 1, 0, 0, 0,
                               amp.ROUND_RNE, 0, torch.zeros(64 * 16 - 1, dtype=u8),
                               torch.zeros(64 * 2, dtype=u8), torch.zeros(3))
    with pytest.raises(ValueError, match="A holds"):
        amp.amp_gemm_blockwise(128, 128, 128, torch.zeros(128 * 127, dtype=u8), amp.E4M3, 128,
                               None, 128, 0, torch.zeros(128 * 128, dtype=u8), amp.E4M3, 128,
                               None, 1, 1, torch.zeros(128, 128), amp.F32, 128)
