"""GPU parity of the row argmax fused into the LM-head GEMVs.

aqg_gemv_bf16_argmax / aqg_gemv_affine_q{b}_argmax return, per row, the
largest fp32 output and its index (the lowest index on equal values) without
writing the logits.  Bars:
  * index: equal to the oracle's argmax of its fp64 outputs, except on rows
    whose oracle top-2 gap is within the two entries' summed tolerance (then
    either is a correct answer; counted and printed);
  * the (value, index) pair is exactly the argmax of the fp32 outputs that
    the plain GEMV of the same arguments writes (same kernel arithmetic), with
    ties broken towards the lowest index;
  * planted rows: a unique maximum with margin, and exact ties placed below
    and above it (the lowest index wins).
Both LM heads (dense 100000 x 1536 at M = 1..32, 4-bit 151936 x 1024 at
M = 1, 4, 16) run on kernels with the argmax epilogue; other shapes take the
GEMV-then-reduce route, also covered here.

Tie rule: nvfp4-megamoe-kernel commit log, "Router: full kernel stack",
Step 2 (lower index wins on equal scores).
"""
import functools

import numpy as np
import pytest
import torch

import affine_quantized_gemv_amd as aqg
import oracle
import synth
from gpu_helpers import bf16_dev, u32_dev

pytestmark = pytest.mark.gpu

FUSED = {"piece", "mfma_tile", "affine_mfma"}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aqg.load()
    yield


def _first_argmax(y32):
    """Row argmax of fp32 values, lowest index on ties, and the value."""
    idx = np.argmax(y32, axis=1)            # numpy returns the first maximum
    return y32[np.arange(y32.shape[0]), idx], idx


def _check(val, idx, y32, ref, A):
    v, i = val.cpu().numpy(), idx.cpu().numpy()
    ev, ei = _first_argmax(y32)
    assert np.array_equal(i, ei), "argmax differs from the GEMV's own fp32 outputs"
    assert np.array_equal(v.view(np.uint32), ev.view(np.uint32)), "max value differs from the GEMV's"
    ambiguous = 0
    ri = oracle.argmax(ref)
    tol = oracle.tolerance(A)
    for m in range(ref.shape[0]):
        if i[m] == ri[m]:
            continue
        gap = ref[m, ri[m]] - ref[m, i[m]]
        assert gap <= tol[m, ri[m]] + tol[m, i[m]], "row %d: %d vs oracle %d (gap %g)" % (m, i[m], ri[m], gap)
        ambiguous += 1
    return ambiguous


@functools.lru_cache(maxsize=None)
def dense_head():
    name, N, K = synth.DENSE_DECODE_SHAPES[7]
    x = synth.activations(synth.CFG_DENSE_DECODE, K)
    W = synth.dense_weight(synth.CFG_DENSE_DECODE, name, N, K)
    ref, A = oracle.gemv_bf16(x, W)
    return x, W, bf16_dev(x), bf16_dev(W), ref, A


@functools.lru_cache(maxsize=None)
def affine_head():
    name, N, K = synth.AFFINE4_SHAPES[3]
    x = synth.activations(synth.CFG_AFFINE4_08B, K)[:16]
    aw = synth.affine_weight(synth.CFG_AFFINE4_08B, name, 4, N, K)
    ref, A = oracle.gemv_affine(x, aw.words, aw.scales, aw.biases, 4)
    return x, aw, bf16_dev(x), u32_dev(aw.words), bf16_dev(aw.scales), bf16_dev(aw.biases), ref, A


@pytest.mark.parametrize("M", synth.DENSE_DECODE_M)
def test_dense_lm_head_argmax(M):
    x, W, xd, Wd, ref, A = dense_head()
    N, K = W.shape
    assert aqg.dispatch_path(0, M, N, K)[0] in FUSED
    val, idx = aqg.gemv_bf16_argmax(xd[:M], Wd)
    y32 = aqg.gemv_bf16(xd[:M], Wd, out_dtype=torch.float32).cpu().numpy()
    amb = _check(val, idx, y32, ref[:M], A[:M])
    print("dense lm_head M=%d: %d rows within tolerance of a tie" % (M, amb))


@pytest.mark.parametrize("M", synth.AFFINE4_M + [2, 8])
def test_affine4_lm_head_argmax(M):
    x, aw, xd, wq, sd, bd, ref, A = affine_head()
    N, K = aw.words.shape[0], x.shape[1]
    assert aqg.dispatch_path(4, M, N, K)[0] in FUSED
    val, idx = aqg.gemv_affine_argmax(xd[:M], wq, sd, bd, 4)
    y32 = aqg.gemv_affine(xd[:M], wq, sd, bd, 4, out_dtype=torch.float32).cpu().numpy()
    amb = _check(val, idx, y32, ref[:M], A[:M])
    print("q4 lm_head M=%d: %d rows within tolerance of a tie" % (M, amb))


@pytest.mark.parametrize("M", [1, 3, 16, 32])
def test_dense_planted_max_and_ties(M):
    """Row n* = 2 W[n0] (n0 the oracle argmax of x row 0, y[n0] > 0) is the
    unique maximum of row 0; copies of row n* at a lower and a higher index tie
    with it exactly, and the lowest of the three must win."""
    x, W, xd, Wd, ref, A = dense_head()
    n0 = int(oracle.argmax(ref[:1])[0])
    assert ref[0, n0] > 0
    N = W.shape[0]
    n_star, n_lo, n_hi = (n0 + 50021) % N, (n0 + 20011) % N, (n0 + 70001) % N
    n_lo, n_star, n_hi = sorted((n_lo, n_star, n_hi))
    W2 = W.copy()
    doubled = synth.to_bf16_bits(2.0 * oracle.bf16_to_f64(W[n0]))
    for n in (n_lo, n_star, n_hi):
        W2[n] = doubled
    Wd2 = bf16_dev(W2)
    y32 = aqg.gemv_bf16(xd[:M], Wd2, out_dtype=torch.float32).cpu().numpy()
    assert y32[0, n_lo] == y32[0, n_star] == y32[0, n_hi]
    val, idx = aqg.gemv_bf16_argmax(xd[:M], Wd2)
    assert int(idx[0]) == n_lo
    ev, ei = _first_argmax(y32)
    assert np.array_equal(idx.cpu().numpy(), ei)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_affine4_planted_max_and_ties(M):
    x, aw, xd, wq, sd, bd, ref, A = affine_head()
    N = aw.words.shape[0]
    n0 = int(oracle.argmax(ref[:1])[0])
    assert ref[0, n0] > 0
    rows = sorted(((n0 + 7919) % N, (n0 + 60013) % N, (n0 + 100003) % N))
    words, s, b = aw.words.copy(), aw.scales.copy(), aw.biases.copy()
    for n in rows:       # same codes, doubled scale and bias: y[n] = 2 y[n0] exactly
        words[n], s[n], b[n] = words[n0], s[n0] + 0x80, b[n0] + 0x80
    w2, s2, b2 = u32_dev(words), bf16_dev(s), bf16_dev(b)
    y32 = aqg.gemv_affine(xd[:M], w2, s2, b2, 4, out_dtype=torch.float32).cpu().numpy()
    assert y32[0, rows[0]] == y32[0, rows[1]] == y32[0, rows[2]]
    val, idx = aqg.gemv_affine_argmax(xd[:M], w2, s2, b2, 4)
    assert int(idx[0]) == rows[0]
    ev, ei = _first_argmax(y32)
    assert np.array_equal(idx.cpu().numpy(), ei)


# shapes whose kernel has no argmax epilogue (GEMV into the workspace, then a
# row reduction) and ragged fused ones
@pytest.mark.parametrize("bits,M,N,K", [(0, 8, 1536, 1536), (0, 20, 4096, 1536), (3, 4, 50000, 1024),
                                        (5, 16, 20000, 4096), (2, 12, 3000, 1024), (8, 32, 999, 4096),
                                        (0, 3, 40007, 1024), (4, 17, 40001, 1024), (2, 1, 33333, 2048),
                                        (8, 5, 700, 512), (2, 8, 14350, 4096), (8, 24, 14350, 4096),
                                        (4, 3, 3990, 4096)])
def test_argmax_other_shapes(bits, M, N, K):
    x = synth.normal_bf16((M, K), 1.0, 60, "am/x/%d" % K)
    xd = bf16_dev(x)
    if bits == 0:
        W = synth.dense_weight(60, "am/%d" % N, N, K)
        Wd = bf16_dev(W)
        ref, A = oracle.gemv_bf16(x, W)
        val, idx = aqg.gemv_bf16_argmax(xd, Wd)
        y32 = aqg.gemv_bf16(xd, Wd, out_dtype=torch.float32).cpu().numpy()
    else:
        aw = synth.affine_weight(60, "am/%d" % N, bits, N, K)
        args = (u32_dev(aw.words), bf16_dev(aw.scales), bf16_dev(aw.biases))
        ref, A = oracle.gemv_affine(x, aw.words, aw.scales, aw.biases, bits)
        val, idx = aqg.gemv_affine_argmax(xd, *args, bits)
        y32 = aqg.gemv_affine(xd, *args, bits, out_dtype=torch.float32).cpu().numpy()
    amb = _check(val, idx, y32, ref, A)
    print("q%d %dx%dx%d (%s): %d ambiguous" % (bits, M, N, K, aqg.dispatch_path(bits, M, N, K)[0], amb))


def test_argmax_repeatable_and_workspace_reuse():
    """Two calls with one workspace (left with the first call's partials) give
    identical results, also after a call of another shape in between."""
    x, aw, xd, wq, sd, bd, ref, A = affine_head()
    N, K = aw.words.shape[0], x.shape[1]
    ws = torch.empty(aqg.workspace_bytes(aqg.AQG_KIND_ARGMAX_DENSE + 4, 16, N, K), dtype=torch.uint8, device="cuda")
    a = aqg.gemv_affine_argmax(xd[:16], wq, sd, bd, 4, workspace=ws)
    aqg.gemv_affine_argmax(xd[:1], wq[:5000], sd[:5000], bd[:5000], 4, workspace=ws)
    b = aqg.gemv_affine_argmax(xd[:16], wq, sd, bd, 4, workspace=ws)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
