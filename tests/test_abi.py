"""C-ABI checks that need no GPU: the library loads, exports every function
include/aqgemv.h declares, and rejects invalid calls with the documented
status before any HIP call (fake, never-dereferenced pointers are used).
"""
import ctypes
import os
import re

import pytest

import affine_quantized_gemv_amd as aqg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "aqgemv.h")
HAS_GPU_NODE = os.path.exists("/dev/kfd")

A16 = 0x10000            # fake, 16-byte aligned device addresses
B16 = 0x20000
C16 = 0x30000
D16 = 0x40000
E16 = 0x50000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(aqg_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return aqg.load()


def test_header_declares_expected_entry_points():
    names = declared_functions()
    expected = {"aqg_abi_version", "aqg_status_string", "aqg_workspace_bytes", "aqg_gemv_bf16",
                "aqg_swiglu_bf16", "aqg_unpack_codes"} | {"aqg_gemv_affine_q%d" % b for b in range(2, 9)}
    assert set(names) == expected


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings(lib):
    assert aqg.abi_version() == 1
    for s in range(6):
        assert aqg.status_string(s).startswith(
            ["AQG_OK", "AQG_ERR_INVALID_ARG", "AQG_ERR_UNSUPPORTED", "AQG_ERR_ALIGNMENT",
             "AQG_ERR_LAUNCH", "AQG_ERR_DEVICE"][s])
    assert aqg.status_string(99) == "unknown aqg status"
    assert aqg.workspace_bytes(4, 1, 100, 1024) == 0


def dense(lib, x=A16, W=B16, y=C16, M=1, N=16, K=64, out=0, ws=None, wsb=0):
    return lib.aqg_gemv_bf16(x, W, y, M, N, K, out, ws, wsb, None)


def affine(lib, bits=4, x=A16, Wq=B16, s=D16, b=E16, y=C16, M=1, N=16, K=64, out=0):
    return getattr(lib, "aqg_gemv_affine_q%d" % bits)(x, Wq, s, b, y, M, N, K, out, None, 0, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(W=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(y=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(M=0), aqg.AQG_ERR_INVALID_ARG),
    (dict(N=0), aqg.AQG_ERR_INVALID_ARG),
    (dict(K=0), aqg.AQG_ERR_INVALID_ARG),
    (dict(M=-1), aqg.AQG_ERR_INVALID_ARG),
    (dict(out=2), aqg.AQG_ERR_INVALID_ARG),
    (dict(M=33), aqg.AQG_ERR_UNSUPPORTED),
    (dict(K=12), aqg.AQG_ERR_UNSUPPORTED),
    (dict(x=A16 + 8), aqg.AQG_ERR_ALIGNMENT),
    (dict(W=B16 + 4), aqg.AQG_ERR_ALIGNMENT),
    (dict(y=C16 + 1), aqg.AQG_ERR_ALIGNMENT),
    (dict(y=C16 + 2, out=1), aqg.AQG_ERR_ALIGNMENT),
    (dict(y=A16), aqg.AQG_ERR_INVALID_ARG),          # output overlaps x
    (dict(y=B16 + 16), aqg.AQG_ERR_INVALID_ARG),     # output overlaps W
])
def test_dense_validation(lib, kwargs, status):
    assert dense(lib, **kwargs) == status


@pytest.mark.parametrize("kwargs,status", [
    (dict(Wq=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(s=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(b=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(K=96), aqg.AQG_ERR_UNSUPPORTED),            # groups other than 64 are refused
    (dict(K=32), aqg.AQG_ERR_UNSUPPORTED),
    (dict(M=40), aqg.AQG_ERR_UNSUPPORTED),
    (dict(Wq=B16 + 8), aqg.AQG_ERR_ALIGNMENT),
    (dict(s=D16 + 1), aqg.AQG_ERR_ALIGNMENT),
    (dict(s=D16 + 2), aqg.AQG_ERR_ALIGNMENT),         # scales and biases: 4-byte aligned
    (dict(b=E16 + 2), aqg.AQG_ERR_ALIGNMENT),
    (dict(y=D16), aqg.AQG_ERR_INVALID_ARG),           # output overlaps scales
])
def test_affine_validation(lib, kwargs, status):
    for bits in range(2, 9):
        assert affine(lib, bits=bits, **kwargs) == status


def test_swiglu_validation(lib):
    f = lib.aqg_swiglu_bf16
    assert f(A16, B16, None, C16, 1, 16, 64, 0, None, 0, None) == aqg.AQG_ERR_INVALID_ARG
    assert f(A16, B16, D16 + 8, C16, 1, 16, 64, 0, None, 0, None) == aqg.AQG_ERR_ALIGNMENT
    assert f(A16, B16, D16, C16, 33, 16, 64, 0, None, 0, None) == aqg.AQG_ERR_UNSUPPORTED
    assert f(A16, B16, D16, D16, 1, 16, 64, 0, None, 0, None) == aqg.AQG_ERR_INVALID_ARG


def test_unpack_validation(lib):
    f = lib.aqg_unpack_codes
    assert f(4, None, A16, 4, 64, None) == aqg.AQG_ERR_INVALID_ARG
    assert f(4, B16, None, 4, 64, None) == aqg.AQG_ERR_INVALID_ARG
    assert f(1, B16, A16, 4, 64, None) == aqg.AQG_ERR_UNSUPPORTED
    assert f(9, B16, A16, 4, 64, None) == aqg.AQG_ERR_UNSUPPORTED
    assert f(4, B16, A16, 4, 100, None) == aqg.AQG_ERR_UNSUPPORTED
    assert f(4, B16 + 4, A16, 4, 64, None) == aqg.AQG_ERR_ALIGNMENT
    assert f(4, B16, B16, 4, 64, None) == aqg.AQG_ERR_INVALID_ARG


@pytest.mark.skipif(HAS_GPU_NODE, reason="only meaningful where no GPU can be reached")
def test_valid_call_without_gpu_reports_device_error(lib):
    """Arguments pass validation, then the device check fails: nothing is launched."""
    assert dense(lib) == aqg.AQG_ERR_DEVICE
    assert affine(lib) == aqg.AQG_ERR_DEVICE
    assert lib.aqg_unpack_codes(4, B16, A16, 4, 64, None) == aqg.AQG_ERR_DEVICE


def test_python_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        aqg.gemv_bf16(x, torch.zeros(4, 64, dtype=torch.bfloat16))
