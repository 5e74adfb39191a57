"""GPU exactness of the affine paths where the pages' format fixes the answer.

Every affine kernel computes the factored form of sum_k x (s q + bias):
s * (sum_k (C + q) x - D0) + bias * X, where C is the code offset that puts a
code into a bf16 mantissa and D0 = C * X as the kernel's own arithmetic
computes it.  These tests pin what must then hold exactly, on every kernel
family (each case names the family it covers, and the library's dispatch
query must agree):

  * rows with zero codes and zero biases (w = 0, nonzero scales) give exactly
    0, not a rounding residue of the offset;
  * zero codes give the closed form y = sum_g bias_g X_g (within the bound,
    which here is 2e-3 sum|bias||x| + 1e-6);
  * MLX-style groups (scale = range / (2^b - 1), bias = group minimum, so
    bias is about -s 2^(b-1)) stay within the bound;
  * one-hot activations with s = 1, bias = 0 read single codes exactly, and
    with s = 2, bias = -1 give 2q - 1 exactly (the streaming kernel of 3-, 5-,
    6- and 7-bit codes, which serves M <= 4 (6 and 7 bits: M <= 2) on
    matrices of more than 256 row tiles at K = 4096, and M = 1 at 4096 rows
    and more; the multi-tile kernel in the burst tests of test_gpu_parity).

Format: TensorFold PR #849, "qwen3_5 cuda: mixed-width MLX checkpoints, 2 to
8 bits in groups of 64" (MLX affine mode: value, scale and bias per group).
"""
import functools

import numpy as np
import pytest
import torch

import affine_quantized_gemv_amd as aqg
import oracle
import synth
from gpu_helpers import assert_within, bf16_dev, metrics, run_guarded, u32_dev

pytestmark = pytest.mark.gpu

# (family, bits, M, N, K): one case per kernel family and width class
CASES = [
    ("piece", 4, 1, 3000, 1024), ("piece", 2, 4, 3000, 1024), ("piece", 2, 8, 20000, 1024), ("piece", 8, 4, 3000, 1024),
    ("stream", 3, 1, 2304, 4096), ("stream", 5, 4, 4400, 4096), ("stream", 6, 2, 4400, 4096),
    ("stream", 7, 1, 2304, 4096),
    # rows whose group count is not a power of two: lane slots past the row's
    # last group (8 of 64 at K = 3584, 15 of 32 at K = 1088 with two rows a
    # tile, 1 of 64 at K = 4032) read past the row and must add nothing
    ("stream", 3, 1, 4500, 3584), ("stream", 5, 2, 4500, 1088), ("stream", 7, 4, 4500, 4032),
    ("valu", 3, 9, 300, 320), ("valu", 5, 32, 300, 320),
    ("affine_mfma", 4, 16, 40001, 1024), ("affine_mfma", 2, 12, 40001, 1024), ("affine_mfma", 8, 16, 40001, 3072),
    ("affine_mfma", 4, 4, 40001, 1024),
    ("affine_tile", 4, 16, 8000, 2048), ("affine_tile", 3, 8, 8000, 4096), ("affine_tile", 8, 16, 8000, 2048),
    ("affine_tile", 6, 32, 8000, 2048), ("affine_tile", 2, 16, 20000, 4096),
    ("affine_burst", 2, 8, 8001, 4096), ("affine_burst", 4, 3, 8000, 4096), ("affine_burst", 8, 32, 8000, 4096),
    ("affine_burst", 7, 4, 4100, 4096), ("affine_burst", 6, 1, 4000, 4096), ("affine_burst", 5, 2, 3500, 4096),
    ("affine_split", 4, 8, 1000, 1024), ("affine_split", 8, 16, 999, 4096), ("affine_split", 2, 32, 1000, 2048),
    ("affine_split", 3, 4, 1000, 1024), ("affine_split", 5, 16, 999, 1536), ("affine_split", 6, 1, 512, 1024),
    ("affine_split", 7, 32, 300, 3584),
]
IDS = ["%s-q%d-M%d-%dx%d" % c for c in CASES]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aqg.load()
    yield


def _gpu(x, words, s, b, bits, M, N):
    xd, wq, sd, bd = bf16_dev(x), u32_dev(words), bf16_dev(s), bf16_dev(b)
    return run_guarded(lambda out: aqg.gemv_affine(xd[:M], wq, sd, bd, bits, out=out), M, N)


def _check_family(family, bits, M, N, K):
    got, cols = aqg.dispatch_path(bits, M, N, K)
    assert got == family, "q%d %dx%dx%d runs on %s, not %s" % (bits, M, N, K, got, family)


@functools.lru_cache(maxsize=None)
def _x(M, K):
    return synth.normal_bf16((M, K), 1.0, 70, "ex/x/%d/%d" % (M, K))


@pytest.mark.parametrize("family,bits,M,N,K", CASES, ids=IDS)
def test_zero_weight_rows_give_exact_zero(family, bits, M, N, K):
    """Every third row has zero codes and zero biases but random nonzero
    scales: those outputs are exactly 0; the other rows are within the bound."""
    _check_family(family, bits, M, N, K)
    aw = synth.affine_weight(70, "zr/%s" % family, bits, N, K)
    zero = np.arange(N) % 3 == 1
    words = aw.words.copy()
    biases = aw.biases.copy()
    words[zero] = 0
    biases[zero] = 0
    x = _x(M, K)
    y = _gpu(x, words, aw.scales, biases, bits, M, N)
    assert np.all(y[:, zero] == 0.0), "w = 0 rows: max |y| = %g" % np.abs(y[:, zero]).max()
    ref, A = oracle.gemv_affine(x, words, aw.scales, biases, bits)
    assert_within(y, ref, oracle.tolerance(A), "%s q%d" % (family, bits))


@pytest.mark.parametrize("family,bits,M,N,K", CASES, ids=IDS)
def test_zero_codes_closed_form(family, bits, M, N, K):
    """q = 0 everywhere: y = sum_g bias_g X_g, the closed form (numpy, fp64
    group sums), within 2e-3 sum|bias||x| + 1e-6; the scales play no part."""
    _check_family(family, bits, M, N, K)
    aw = synth.affine_weight(71, "zc/%s" % family, bits, N, K)
    words = np.zeros_like(aw.words)
    x = _x(M, K)
    y = _gpu(x, words, aw.scales, aw.biases, bits, M, N)
    xd = oracle.bf16_to_f64(x)
    bd = oracle.bf16_to_f64(aw.biases)
    X = xd.reshape(M, K // 64, 64).sum(axis=2)
    absX = np.abs(xd).reshape(M, K // 64, 64).sum(axis=2)
    expect = X @ bd.T
    bound = 2e-3 * (absX @ np.abs(bd).T) + 1e-6
    assert_within(y, expect, bound, "closed form %s q%d" % (family, bits))
    # and the same scales doubled give the same bits: zero codes never see the scale
    y2 = _gpu(x, words, (aw.scales.astype(np.uint32) + 0x80).astype(np.uint16), aw.biases, bits, M, N)
    assert np.array_equal(y, y2)


def _mlx_like(bits, N, K, seed, name):
    """Weights ~ N(0, 0.02) quantized per group of 64 the MLX affine way:
    scale = (max - min) / (2^b - 1), bias = min, q = round((w - bias) / scale)."""
    g = synth.rng(seed, name)
    w = g.standard_normal((N, K // 64, 64)) * 0.02
    lo = w.min(axis=2)
    hi = w.max(axis=2)
    s = synth.to_bf16_bits((hi - lo) / ((1 << bits) - 1))
    b = synth.to_bf16_bits(lo)
    sd = oracle.bf16_to_f64(s)[:, :, None]
    bd = oracle.bf16_to_f64(b)[:, :, None]
    q = np.clip(np.rint((w - bd) / sd), 0, (1 << bits) - 1).astype(np.uint8)
    return oracle.pack(q.reshape(N, K), bits), s, b


@pytest.mark.parametrize("family,bits,M,N,K", CASES, ids=IDS)
def test_mlx_like_groups_within_bound(family, bits, M, N, K):
    """Realistic groups (bias near -scale * 2^(b-1), |w| small against the
    code offset's scale * C * |x|) stay within the GEMV bound."""
    _check_family(family, bits, M, N, K)
    words, s, b = _mlx_like(bits, N, K, 72, "mlx/%s/%d" % (family, bits))
    x = _x(M, K)
    y = _gpu(x, words, s, b, bits, M, N)
    ref, A = oracle.gemv_affine(x, words, s, b, bits)
    assert_within(y, ref, oracle.tolerance(A), "MLX-like %s q%d" % (family, bits))
    print(family, bits, metrics(y, ref, A))


@pytest.mark.parametrize("bits,M", [(3, 1), (3, 4), (5, 1), (5, 4), (6, 1), (6, 2), (7, 1), (7, 2)])
def test_stream_kernel_one_hot_exact(bits, M):
    """The streaming kernel (3, 5, 6, 7 bits, more than 256 row tiles of
    K = 4096; 6 and 7 bits at M = 3, 4 run on the multi-tile kernel) reads
    every code exactly: one-hot x with s = 1, bias = 0 gives
    q[n, col]; with s = 2, bias = -1 it gives 2q - 1.  The columns cover every
    position of a 64-code group (including the codes that straddle two
    words)."""
    N, K = 4400, 4096
    _check_family("stream", bits, M, N, K)
    words = synth.random_words((N, K * bits // 32), 73, "ohs/%d" % bits)
    codes = oracle.unpack(words, bits, K).astype(np.float64)
    G = K // 64
    ones = np.full((N, G), 0x3F80, np.uint16)
    zeros = np.zeros((N, G), np.uint16)
    twos = np.full((N, G), 0x4000, np.uint16)
    minus1 = np.full((N, G), 0xBF80, np.uint16)
    positions = np.arange(64)
    for c0 in range(0, 64, M):
        cols = np.array([((p * 7 + 5) % G) * 64 + p for p in positions[c0:c0 + M]])
        x = np.zeros((M, K), np.uint16)
        x[np.arange(M), cols] = 0x3F80
        y = _gpu(x, words, ones, zeros, bits, M, N)
        assert np.array_equal(y, codes[:, cols].T), "q%d cols %s" % (bits, cols)
        y = _gpu(x, words, twos, minus1, bits, M, N)
        assert np.array_equal(y, 2 * codes[:, cols].T - 1), "q%d cols %s (s=2, b=-1)" % (bits, cols)
