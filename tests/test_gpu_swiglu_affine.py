"""GPU parity of the fused SwiGLU over affine b-bit gate and up matrices.

aqg_swiglu_affine_q{b}: out = silu(x . Wg^T) * (x . Wu^T), both projections
affine group-quantized (each matrix with its own codes, scales and biases),
fp32 inside, against the oracle's unfused double chain (oracle.swiglu_affine)
with the propagated SwiGLU bound; bf16 outputs are exactly RNE of the same
call's fp32 outputs; zero gate or up matrices give exactly 0; rows do not
depend on M within a kernel family.  Shapes: the hidden-1536 MLP (4096 x
1536) and the ~0.8B decoder MLP (3584 x 1024), every width, M = 1..32.
"""
import functools

import numpy as np
import pytest
import torch

import affine_quantized_gemv_amd as aqg
import oracle
import synth
from gpu_helpers import assert_within, bf16_dev, run_guarded, u32_dev

pytestmark = pytest.mark.gpu

SHAPES = synth.SWIGLU_AFFINE_SHAPES
BITS = synth.SWIGLU_AFFINE_BITS
MS = [1, 2, 4, 8, 16, 32]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aqg.load()
    yield


@functools.lru_cache(maxsize=None)
def case(name, N, K, bits):
    x = synth.activations(synth.CFG_SWIGLU, K)
    g = synth.affine_weight(synth.CFG_SWIGLU, name + "/gate", bits, N, K)
    u = synth.affine_weight(synth.CFG_SWIGLU, name + "/up", bits, N, K)
    r = oracle.swiglu_affine(x, (g.words, g.scales, g.biases), (u.words, u.scales, u.biases), bits)
    dev = lambda w: (u32_dev(w.words), bf16_dev(w.scales), bf16_dev(w.biases))
    return x, g, u, bf16_dev(x), dev(g), dev(u), r


def _tol(r, M):
    return oracle.swiglu_tolerance(r["g"][:M], r["u"][:M], r["Ag"][:M], r["Au"][:M], r["out"][:M])


@pytest.mark.parametrize("M", MS)
@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s[0])
def test_swiglu_affine_against_unfused_oracle_chain(shape, bits, M):
    name, N, K = shape
    x, g, u, xd, gd, ud, r = case(name, N, K, bits)
    y = run_guarded(lambda out: aqg.swiglu_affine(xd[:M], gd, ud, bits, out=out), M, N)
    path = aqg.dispatch_path(aqg.AQG_KIND_SWIGLU_AFFINE + bits, M, N, K)[0]
    assert_within(y, r["out"][:M], _tol(r, M), "swiglu q%d %dx%dx%d (%s)" % (bits, M, N, K, path))


@pytest.mark.parametrize("M", [1, 5, 32])
def test_swiglu_affine_q7(M):
    x, g, u, xd, gd, ud, r = case("mlp_1024", 3584, 1024, 7)
    y = run_guarded(lambda out: aqg.swiglu_affine(xd[:M], gd, ud, 7, out=out), M, 3584)
    assert_within(y, r["out"][:M], _tol(r, M), "swiglu q7 M=%d" % M)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_swiglu_affine_zero_gate_or_up_gives_exact_zero(bits):
    """Zero codes and biases in Wg give g = 0 exactly (the exact code offset),
    silu(0) = 0; the same in Wu gives u = 0: out is exactly 0 either way."""
    name, N, K = SHAPES[1]
    x, g, u, xd, gd, ud, r = case(name, N, K, bits)
    zero = (torch.zeros_like(gd[0]), gd[1], torch.zeros_like(gd[2]))
    for M in (1, 8, 16):
        for a, b in ((zero, ud), (gd, zero)):
            y = aqg.swiglu_affine(xd[:M], a, b, bits, out_dtype=torch.float32)
            assert torch.count_nonzero(y).item() == 0, "M=%d" % M


def test_swiglu_affine_large_negative_gate_is_near_zero():
    """Codes 0 and bias -1 in every gate group with x = 1: g = -K, silu(g)
    underflows, out is 0 to within the bound's absolute floor."""
    N, K, bits = 300, 1024, 4
    x = np.full((4, K), 0x3F80, np.uint16)
    zw = np.zeros((N, K * bits // 32), np.uint32)
    ones = np.full((N, K // 64), 0x3F80, np.uint16)
    minus1 = np.full((N, K // 64), 0xBF80, np.uint16)
    gd = (u32_dev(zw), bf16_dev(ones), bf16_dev(minus1))
    ud = (u32_dev(zw), bf16_dev(ones), bf16_dev(ones))
    y = aqg.swiglu_affine(bf16_dev(x), gd, ud, bits, out_dtype=torch.float32).cpu().numpy()
    assert np.all(np.abs(y) <= 1e-6)


@pytest.mark.parametrize("bits", [2, 4, 5])
def test_swiglu_affine_rows_independent_of_m(bits):
    """Within one kernel family (and column count for the matrix-core ones)
    each output row is computed the same way whatever M is: every M's rows
    equal the rows of the largest M of its family bit for bit."""
    name, N, K = SHAPES[0]
    x, g, u, xd, gd, ud, r = case(name, N, K, bits)
    groups = {}
    for M in (1, 2, 3, 4, 5, 8, 9, 16, 17, 32):
        path, cols = aqg.dispatch_path(aqg.AQG_KIND_SWIGLU_AFFINE + bits, M, N, K)
        key = path if path in ("piece", "stream", "valu") else (path, cols)
        groups.setdefault(key, []).append(M)
    for key, ms in groups.items():
        big = max(ms)
        ref = aqg.swiglu_affine(xd[:big], gd, ud, bits, out_dtype=torch.float32).cpu().numpy()
        for M in ms:
            yM = aqg.swiglu_affine(xd[:M], gd, ud, bits, out_dtype=torch.float32).cpu().numpy()
            assert np.array_equal(yM, ref[:M]), "%s M=%d vs M=%d" % (key, M, big)
