"""GPU parity of the affine prompt GEMM, aqg_gemm_affine_q{b} (any M).

Against the oracle's double-precision affine product (oracle.gemv_affine,
which takes any M) within |y - y_ref| <= 2e-3 sum|w||x| + 1e-6:

  * every element, every width 2..8, on shapes that span several tiles of
    both operands with ragged ends (M and N not multiples of the tile, N odd,
    one row of x, a single group-block of K) and that select each of the
    kernel's three splits of a workgroup (K / 64 odd, = 2 mod 4, = 0 mod 4);
  * sampled outputs (rows of x at the start, middle and end, rows of W
    spread over N including the last) at the full mixed-width and
    ~0.8B-decoder shapes for prompt chunks of 128, 512 and 640 rows;
  * bf16 outputs are exactly RNE of the same call's fp32 outputs, and no
    write lands outside y (canary words on both sides);
  * a row's result does not depend on the other rows of x (bit for bit,
    between M values that share a tiling), and one workspace serves calls of
    different M in a row;
  * small matrices whose tiles split their groups over several workgroups
    (partials in the workspace) and the same call with a workspace too small
    for the partials (run unsplit) are both within the bound.
Inputs: synth's mixed-width weight recipe (codes uniform in [0, 2^b - 1],
scales U(0.001, 0.02), biases U(-0.1, 0.1)) and x ~ N(0, 1), bf16.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import affine_quantized_gemv_amd as aqg
import oracle
import synth
from gpu_helpers import DEV, assert_within, bf16_dev, run_guarded, u32_dev

pytestmark = pytest.mark.gpu

CFG = synth.CFG_MIXED_WIDTH
BITS = synth.GEMM_BITS

# (M, N, K): K / 64 = 16 and 24 (four K chunks), 10 (two), 5 (one)
SMALL = [
    (33, 320, 1024),
    (64, 256, 640),
    (77, 515, 320),
    (300, 130, 1024),
    (1, 100, 1536),
    (129, 1000, 3584),
    (200, 64, 4096),
]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aqg.load()
    yield


@functools.lru_cache(maxsize=4)
def weight(name, bits, N, K):
    w = synth.affine_weight(CFG, "gemm/" + name, bits, N, K)
    return w, (u32_dev(w.words), bf16_dev(w.scales), bf16_dev(w.biases))


def call(xd, wd, bits, M):
    return lambda out: aqg.gemm_affine(xd[:M], wd[0], wd[1], wd[2], bits, out=out)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("M,N,K", SMALL)
def test_gemm_against_oracle(bits, M, N, K):
    print("gemm q%d M=%d N=%d K=%d" % (bits, M, N, K), file=sys.stderr, flush=True)
    w, wd = weight("small/%dx%d" % (N, K), bits, N, K)
    x = synth.prompt_activations(CFG, K, M)
    ref, A = oracle.gemv_affine(x, w.words, w.scales, w.biases, bits)
    y = run_guarded(call(bf16_dev(x), wd, bits, M), M, N)
    assert_within(y, ref, oracle.tolerance(A), "gemm q%d %dx%dx%d" % (bits, M, N, K))


FULL = [(name, N, K, M) for (name, N, K) in synth.GEMM_SHAPES for M in synth.GEMM_M] + \
       [("wide_14336", 14336, 4096, 640)]


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("name,N,K,M", FULL, ids=lambda v: str(v))
def test_gemm_full_size_sampled(bits, name, N, K, M):
    if M == 640 and bits not in (3, 4, 8):
        pytest.skip("the 640-row chunk runs for one odd, one even and the 8-bit width")
    print("gemm full q%d %s M=%d" % (bits, name, M), file=sys.stderr, flush=True)
    w, wd = weight(name, bits, N, K)
    x = synth.prompt_activations(CFG, K, M)
    out = torch.empty((M, N), dtype=torch.float32, device=DEV)
    aqg.gemm_affine(bf16_dev(x), wd[0], wd[1], wd[2], bits, out=out)
    y = out.cpu().numpy().astype(np.float64)
    ms = sorted({0, 1, 63, 64, M // 2, M - 1})
    ns = sorted(set(np.linspace(0, N - 1, 47).astype(int).tolist()) | {N - 1, 511, 512})
    ref, A = oracle.gemv_affine(x[ms], w.words[ns], w.scales[ns], w.biases[ns], bits)
    assert_within(y[np.ix_(ms, ns)], ref, oracle.tolerance(A), "gemm q%d %s M=%d (sampled)" % (bits, name, M))
    assert np.isfinite(y).all()


@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("M0,M1", [(33, 64), (100, 128), (1, 40)])
def test_gemm_rows_independent(bits, M0, M1):
    """M0 and M1 round up to the same multiple of 64, so both calls tile the
    same way: the first M0 rows agree bit for bit."""
    N, K = 515, 1024
    _, wd = weight("inv/%dx%d" % (N, K), bits, N, K)
    xd = bf16_dev(synth.prompt_activations(CFG, K, M1))
    y0 = torch.empty((M0, N), dtype=torch.float32, device=DEV)
    y1 = torch.empty((M1, N), dtype=torch.float32, device=DEV)
    aqg.gemm_affine(xd[:M0], wd[0], wd[1], wd[2], bits, out=y0)
    aqg.gemm_affine(xd, wd[0], wd[1], wd[2], bits, out=y1)
    assert torch.equal(y0, y1[:M0])


def test_gemm_workspace_reused_across_sizes():
    bits, N, K = 4, 320, 1024
    _, wd = weight("ws/%dx%d" % (N, K), bits, N, K)
    xd = bf16_dev(synth.prompt_activations(CFG, K, 300))
    need = aqg.workspace_bytes(aqg.AQG_KIND_GEMM_AFFINE + bits, 300, N, K)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    for M in (300, 33, 150):
        shared = torch.empty((M, N), dtype=torch.float32, device=DEV)
        fresh = torch.empty((M, N), dtype=torch.float32, device=DEV)
        aqg.gemm_affine(xd[:M], wd[0], wd[1], wd[2], bits, out=shared, workspace=ws)
        aqg.gemm_affine(xd[:M], wd[0], wd[1], wd[2], bits, out=fresh)
        assert torch.equal(shared, fresh), M


def test_gemm_split_and_unsplit_both_within_the_bound():
    """1024 x 3584 at M = 128: with the workspace the size query gives, each
    tile's groups are split over several workgroups (fp32 partial products,
    summed in a fixed order); with a workspace of only the operands' size the
    call is accepted and runs unsplit.  Every output of both within the bound
    of the oracle, and each repeatable bit for bit."""
    import test_abi
    bits, N, K, M = 4, 1024, 3584, 128
    w, wd = weight("split/%dx%d" % (N, K), bits, N, K)
    x = synth.prompt_activations(CFG, K, M)
    xd = bf16_dev(x)
    full = aqg.workspace_bytes(aqg.AQG_KIND_GEMM_AFFINE + bits, M, N, K)
    base = test_abi.gemm_ws_closed_form(bits, M, K)
    assert test_abi.gemm_split_closed_form(M, N, K) > 1 and full > base
    ref, A = oracle.gemv_affine(x, w.words, w.scales, w.biases, bits)
    fn = aqg.load().aqg_gemm_affine_q4
    for name, nbytes in (("split", full), ("unsplit", base)):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        runs = []
        for _ in range(2):
            out = torch.empty((M, N), dtype=torch.float32, device=DEV)
            st = fn(aqg._p(xd), aqg._p(wd[0]), aqg._p(wd[1]), aqg._p(wd[2]), aqg._p(out), M, N, K,
                    aqg.AQG_OUT_F32, aqg._p(ws), nbytes, None)
            torch.cuda.synchronize()
            assert st == 0, (name, st)
            runs.append(out.cpu().numpy().astype(np.float64))
        assert np.array_equal(runs[0], runs[1]), name
        assert_within(runs[0], ref, oracle.tolerance(A), "gemm q4 %s %dx%dx%d" % (name, M, N, K))
