"""The allocation-free row argmax (aqg_gemv_argmax_noalloc) against the
argmax entry points with a caller's workspace, through the C ABI.

Its scratch is a static device array shared by every call on the GPU, left
with the previous call's contents: two calls in a row (the second with a
smaller input, on another kernel family), and a dense call that runs the
GEMV-then-reduce route through the same array, must each equal the
workspace entry point bit for bit.  A shape that needs more than the
array's size is refused with AQG_ERR_UNSUPPORTED.
"""
import ctypes

import numpy as np
import pytest
import torch

import affine_quantized_gemv_amd as aqg
import synth
from gpu_helpers import bf16_dev, u32_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aqg.load()
    yield


def _noalloc(bits, x, W, s, b, M, N, K):
    val = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    st = aqg.load().aqg_gemv_argmax_noalloc(bits, p(x), p(W), p(s), p(b), p(val), p(idx), M, N, K,
                                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, val, idx


def _affine(bits, M, N, K, tag):
    x = bf16_dev(synth.normal_bf16((M, K), 1.0, 62, "na/x/%s" % tag))
    aw = synth.affine_weight(62, "na/%s" % tag, bits, N, K)
    return x, u32_dev(aw.words), bf16_dev(aw.scales), bf16_dev(aw.biases)


def test_noalloc_matches_workspace_entry_two_calls_then_smaller():
    # call 1: the 4-bit LM head shape at M = 16 (matrix-core argmax epilogue)
    x, w, s, b = _affine(4, 16, 151936, 1024, "big")
    st, val, idx = _noalloc(4, x, w, s, b, 16, 151936, 1024)
    assert st == aqg.AQG_OK
    rv, ri = aqg.gemv_affine_argmax(x, w, s, b, 4)
    torch.cuda.synchronize()
    assert torch.equal(idx, ri) and torch.equal(val.view(torch.int32), rv.view(torch.int32))
    # call 2, smaller: 40000 rows at M = 2 (dot-product kernel's epilogue); the
    # array still holds call 1's partials
    x2, w2, s2, b2 = _affine(4, 2, 40000, 1024, "small")
    st, val2, idx2 = _noalloc(4, x2, w2, s2, b2, 2, 40000, 1024)
    assert st == aqg.AQG_OK
    rv2, ri2 = aqg.gemv_affine_argmax(x2, w2, s2, b2, 4)
    torch.cuda.synchronize()
    assert torch.equal(idx2, ri2) and torch.equal(val2.view(torch.int32), rv2.view(torch.int32))


def test_noalloc_dense_through_the_reduce_route():
    M, N, K = 8, 1536, 1536          # a kernel without the argmax epilogue: fp32 y in the array first
    x = bf16_dev(synth.normal_bf16((M, K), 1.0, 63, "na/dx"))
    W = bf16_dev(synth.dense_weight(63, "na/dw", N, K))
    for m in (M, 3):
        st, val, idx = _noalloc(0, x[:m], W, None, None, m, N, K)
        assert st == aqg.AQG_OK
        rv, ri = aqg.gemv_bf16_argmax(x[:m], W)
        torch.cuda.synchronize()
        assert torch.equal(idx, ri) and torch.equal(val.view(torch.int32), rv.view(torch.int32))


def test_noalloc_refuses_a_shape_beyond_the_array():
    M, N, K = 32, 100000, 1024       # 3-bit: no argmax epilogue, fp32 y alone is 12.8 MB
    need = aqg.workspace_bytes(aqg.AQG_KIND_ARGMAX_DENSE + 3, M, N, K)
    assert need > (8 << 20)
    d = torch.empty(16, dtype=torch.int32, device="cuda")
    p = ctypes.c_void_p(d.data_ptr())
    st = aqg.load().aqg_gemv_argmax_noalloc(3, p, p, p, p, p, p, M, N, K, None)
    assert st == aqg.AQG_ERR_UNSUPPORTED
