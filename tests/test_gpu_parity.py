"""GPU parity: the HIP library against the CPU oracle, element by element.

Bars (all through the C ABI, via the Python binding):
  * unpacked codes: bit-exact with the oracle's unpack;
  * fp32 outputs: |y - y_ref| <= 2e-3 * sum|w||x| + 1e-6 per element;
  * bf16 outputs: exactly RNE of the same call's fp32 outputs;
  * LM heads: row argmax equal to the oracle's (ambiguous only within tolerance);
  * exact cases (one-hot rows, small integers, closed forms): bit-exact;
  * rows are independent: y(M)[m] == y(1, x[m]) bit for bit within the path;
  * no write outside the output (canary guards), deterministic repeats.
Inputs follow the seeded synthetic recipe in synth.py.
"""
import functools

import numpy as np
import pytest
import torch

import affine_quantized_gemv_amd as aqg
import oracle
import synth
from gpu_helpers import (Guarded, assert_within, bf16_dev, check_argmax, metrics, run_guarded,
                         u32_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aqg.load()
    yield


# ------------------------------------------------------------ cached inputs

@functools.lru_cache(maxsize=None)
def dense_case(cfg, name, N, K):
    x = synth.activations(cfg, K)
    W = synth.dense_weight(cfg, name, N, K)
    return x, W, bf16_dev(x), bf16_dev(W)


@functools.lru_cache(maxsize=None)
def dense_ref(cfg, name, N, K):
    x, W, _, _ = dense_case(cfg, name, N, K)
    return oracle.gemv_bf16(x, W)   # at M = 32; smaller M are prefixes


@functools.lru_cache(maxsize=None)
def affine_case(cfg, name, bits, N, K):
    x = synth.activations(cfg, K)
    aw = synth.affine_weight(cfg, name, bits, N, K)
    return x, aw, bf16_dev(x), u32_dev(aw.words), bf16_dev(aw.scales), bf16_dev(aw.biases)


@functools.lru_cache(maxsize=None)
def affine_ref(cfg, name, bits, N, K, M):
    x, aw = affine_case(cfg, name, bits, N, K)[:2]
    return oracle.gemv_affine(x[:M], aw.words, aw.scales, aw.biases, bits)


def gemv_dense_gpu(xd, Wd, M):
    return lambda out: aqg.gemv_bf16(xd[:M], Wd, out=out)


def gemv_affine_gpu(xd, wq, sd, bd, bits, M):
    return lambda out: aqg.gemv_affine(xd[:M], wq, sd, bd, bits, out=out)


# ------------------------------------------------------------------ codes

@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("shape", synth.MIXED_SHAPES, ids=lambda s: s[0])
def test_unpack_codes_bit_exact_mixed_width(bits, shape):
    name, N, K = shape
    _, aw, _, wq, _, _ = affine_case(synth.CFG_MIXED_WIDTH, name, bits, N, K)
    got = aqg.unpack_codes(wq, bits, K).cpu().numpy()
    assert np.array_equal(got, oracle.unpack(aw.words, bits, K))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_unpack_codes_bit_exact_small_and_patterns(bits):
    K = 192
    codes = [synth.random_codes((37, K), bits, 50, "up/%d" % bits)]
    top = (1 << bits) - 1
    codes.append(np.full((1, K), top, np.uint8))
    codes.append(np.zeros((1, K), np.uint8))
    codes.append((np.arange(K) % (top + 1)).astype(np.uint8)[None, :])
    codes = np.vstack(codes)
    words = oracle.pack(codes, bits)
    got = aqg.unpack_codes(u32_dev(words), bits, K).cpu().numpy()
    assert np.array_equal(got, codes)


def test_unpack_codes_lm_head_4bit():
    name, N, K = synth.AFFINE4_SHAPES[3]
    _, aw, _, wq, _, _ = affine_case(synth.CFG_AFFINE4_08B, name, 4, N, K)
    assert np.array_equal(aqg.unpack_codes(wq, 4, K).cpu().numpy(), oracle.unpack(aw.words, 4, K))


# ------------------------------------------------------------------ dense

def test_dense_config1_m1():
    N = K = 1536
    x, W, xd, Wd = dense_case(synth.CFG_DENSE_1536, "W", N, K)
    y = run_guarded(gemv_dense_gpu(xd, Wd, 1), 1, N)
    ref, A = oracle.gemv_bf16(x[:1], W)
    assert_within(y, ref, oracle.tolerance(A), "dense 1536x1536 M=1")
    print(metrics(y, ref, A))


@pytest.mark.parametrize("M", synth.DENSE_DECODE_M)
@pytest.mark.parametrize("shape", synth.DENSE_DECODE_SHAPES[:7], ids=lambda s: s[0])
def test_dense_decode_projections(shape, M):
    name, N, K = shape
    x, W, xd, Wd = dense_case(synth.CFG_DENSE_DECODE, name, N, K)
    ref, A = dense_ref(synth.CFG_DENSE_DECODE, name, N, K)
    y = run_guarded(gemv_dense_gpu(xd, Wd, M), M, N)
    assert_within(y, ref[:M], oracle.tolerance(A[:M]), "%s M=%d" % (name, M))


@functools.lru_cache(maxsize=None)
def dense_lm_head():
    name, N, K = synth.DENSE_DECODE_SHAPES[7]
    x = synth.activations(synth.CFG_DENSE_DECODE, K)
    W = synth.dense_weight(synth.CFG_DENSE_DECODE, name, N, K)
    ref, A = oracle.gemv_bf16(x, W)
    # plant a unique argmax with margin for row 0: W[n*] = 2 W[n0] (exact in bf16)
    n0 = int(oracle.argmax(ref[:1])[0])
    n_star = (n0 + N // 2) % N
    if ref[0, n0] > 0:
        W = W.copy()
        W[n_star] = W[n0] + 0x80  # +1 in the exponent field doubles a bf16 (no zeros/denormals here)
        assert np.all((W[n0] & 0x7F80) != 0)
        ref2, A2 = oracle.gemv_bf16(x, W[n_star:n_star + 1])
        ref[:, n_star], A[:, n_star] = ref2[:, 0], A2[:, 0]
    return x, W, bf16_dev(x), bf16_dev(W), ref, A, n_star


@pytest.mark.parametrize("M", synth.DENSE_DECODE_M)
def test_dense_lm_head_values_and_argmax(M):
    x, W, xd, Wd, ref, A, n_star = dense_lm_head()
    N = W.shape[0]
    y = run_guarded(gemv_dense_gpu(xd, Wd, M), M, N)
    assert_within(y, ref[:M], oracle.tolerance(A[:M]), "lm_head M=%d" % M)
    amb = check_argmax(y, ref[:M], A[:M])
    print("lm_head M=%d: %d argmax rows within tolerance of a tie" % (M, amb))
    assert oracle.argmax(y)[0] == n_star


def test_dense_one_hot_exact():
    N, K = 513, 1536
    W = synth.dense_weight(70, "onehot", N, K)
    cols = (np.arange(32) * 47 + 5) % K
    x = np.zeros((32, K), np.uint16)
    x[np.arange(32), cols] = 0x3F80
    y = run_guarded(gemv_dense_gpu(bf16_dev(x), bf16_dev(W), 32), 32, N)
    assert np.array_equal(y, oracle.bf16_to_f64(W[:, cols]).T)


@pytest.mark.parametrize("K", [1536, 4096, 1000])
def test_dense_one_hot_every_piece_position_m8(K):
    """M = 8 (streaming path) one-hot rows over all 8 positions of a 16-byte
    piece, spread over the row (K = 1000: the row's last lane slot is ragged):
    y = W[n, k] exactly."""
    N = 333
    W = synth.dense_weight(70, "onehot8/%d" % K, N, K)
    npiece = K // 8
    cols = np.array([((r * 37 + 11) % npiece) * 8 + r for r in range(8)] + [K - 1 - r for r in range(8)])
    for c0 in range(0, len(cols), 8):
        c = cols[c0:c0 + 8]
        x = np.zeros((8, K), np.uint16)
        x[np.arange(8), c] = 0x3F80
        y = run_guarded(gemv_dense_gpu(bf16_dev(x), bf16_dev(W), 8), 8, N)
        assert np.array_equal(y, oracle.bf16_to_f64(W[:, c]).T), "cols %s" % c


@pytest.mark.parametrize("M,N,K", [(1, 1, 8), (3, 5, 64), (5, 77, 136), (17, 1000, 520), (31, 129, 2048),
                                   (2, 257, 8192), (32, 64, 4096)])
def test_dense_ragged_shapes(M, N, K):
    x = synth.normal_bf16((M, K), 1.0, 71, "rg/x/%d" % K)
    W = synth.normal_bf16((N, K), 0.02, 71, "rg/W/%d/%d" % (N, K))
    y = run_guarded(gemv_dense_gpu(bf16_dev(x), bf16_dev(W), M), M, N)
    ref, A = oracle.gemv_bf16(x, W)
    assert_within(y, ref, oracle.tolerance(A), "dense %dx%dx%d" % (M, N, K))


def test_dense_small_integers_exact():
    M, N, K = 3, 5, 128
    g = synth.rng(72, "ex")
    x = synth.to_bf16_bits(g.integers(-4, 5, size=(M, K)).astype(np.float64))
    W = synth.to_bf16_bits(g.integers(-8, 9, size=(N, K)).astype(np.float64) / 8)
    y = run_guarded(gemv_dense_gpu(bf16_dev(x), bf16_dev(W), M), M, N)
    ref, _ = oracle.gemv_bf16(x, W)
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("shape", [synth.DENSE_DECODE_SHAPES[4], synth.DENSE_DECODE_SHAPES[6],
                                   synth.DENSE_DECODE_SHAPES[7]], ids=lambda s: s[0])
def test_dense_rows_independent_of_m(shape):
    """Within one code path each output row is computed the same way whatever M
    is.  The vector ALU path (M <= 8; M <= 2 on N >= 4096 with K <= 2048 and
    on large N, M <= 4 on at most 128 row tiles with K <= 2048) matches
    one-row calls bit for bit; the matrix-core paths
    (above those M) match the first rows of the 32-row call bit for bit.
    Across paths only the tolerance applies (checked by the parity tests)."""
    name, N, K = shape
    x, W, xd, Wd = dense_case(synth.CFG_DENSE_DECODE, name, N, K)
    tiles = (N + 15) // 16
    valu_max = 2 if (N >= 32768 or (N >= 4096 and K <= 2048)) else (4 if (K <= 2048 and tiles <= 128) else 8)
    y1 = torch.cat([aqg.gemv_bf16(xd[m:m + 1], Wd, out_dtype=torch.float32) for m in range(8)]).cpu().numpy()
    y32 = aqg.gemv_bf16(xd[:32], Wd, out_dtype=torch.float32).cpu().numpy()
    for M in (2, 3, 4, 5, 8, 9, 13, 16, 17, 24, 31):
        yM = aqg.gemv_bf16(xd[:M], Wd, out_dtype=torch.float32).cpu().numpy()
        want = y1[:M] if M <= valu_max else y32[:M]
        assert np.array_equal(yM, want), "M=%d" % M


def test_dense_small_n_column_pairs_m5_to_8():
    """q/k/v/o 1536 x 1536 (96 row tiles) at M = 5..8: two 4-column
    workgroups per tile, the second with M - 4 = 1..3 columns.  Each M
    against the oracle and bit for bit equal to the first rows of the 8-row
    call (an output's chain does not depend on its column block)."""
    name, N, K = synth.DENSE_DECODE_SHAPES[0]
    x, W, xd, Wd = dense_case(synth.CFG_DENSE_DECODE, name, N, K)
    ref, A = dense_ref(synth.CFG_DENSE_DECODE, name, N, K)
    y8 = None
    for M in (8, 5, 6, 7):
        y = run_guarded(lambda out: aqg.gemv_bf16(xd[:M], Wd, out=out), M, N)
        assert_within(y, ref[:M], oracle.tolerance(A[:M]), "dense %dx%dx%d" % (M, N, K))
        if y8 is None:
            y8 = y
        else:
            assert np.array_equal(y, y8[:M]), "M=%d" % M


@pytest.mark.parametrize("bits,N,K", [(4, 1000, 3584), (8, 999, 4096), (2, 3000, 2048)])
def test_affine_split_deterministic(bits, N, K):
    """The split path's partial tiles are summed in a fixed order: repeated
    calls give the same bits (M = 5, 16 and 32)."""
    x, aw, xd, wq, sd, bd = affine_mma_case(bits, N, K)
    for M in (5, 16, 32):
        a = aqg.gemv_affine(xd[:M], wq, sd, bd, bits, out_dtype=torch.float32).cpu().numpy()
        b = aqg.gemv_affine(xd[:M], wq, sd, bd, bits, out_dtype=torch.float32).cpu().numpy()
        assert np.array_equal(a, b), "M=%d" % M


def test_swiglu_rows_independent_of_m():
    """2 x 4096 x 1536: the vector ALU path (M <= 2) matches one-row calls bit
    for bit, the matrix-core path (M = 3..32) the 32-row call."""
    x, Wg, Wu, xd, Wgd, Wud, r = swiglu_case()
    y1 = torch.cat([aqg.swiglu_bf16(xd[m:m + 1], Wgd, Wud, out_dtype=torch.float32)
                    for m in range(2)]).cpu().numpy()
    y32 = aqg.swiglu_bf16(xd[:32], Wgd, Wud, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(aqg.swiglu_bf16(xd[:2], Wgd, Wud, out_dtype=torch.float32).cpu().numpy(), y1)
    for M in (3, 4, 5, 8, 9, 16, 20):
        assert np.array_equal(aqg.swiglu_bf16(xd[:M], Wgd, Wud, out_dtype=torch.float32).cpu().numpy(),
                              y32[:M]), "M=%d" % M


def test_dense_deterministic():
    name, N, K = synth.DENSE_DECODE_SHAPES[6]
    _, _, xd, Wd = dense_case(synth.CFG_DENSE_DECODE, name, N, K)
    a = aqg.gemv_bf16(xd[:8], Wd, out_dtype=torch.float32).cpu().numpy()
    b = aqg.gemv_bf16(xd[:8], Wd, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ----------------------------------------------------------------- SwiGLU

@functools.lru_cache(maxsize=None)
def swiglu_case():
    N, K = synth.SWIGLU_SHAPE
    x = synth.activations(synth.CFG_SWIGLU, K)
    Wg = synth.dense_weight(synth.CFG_SWIGLU, "gate", N, K)
    Wu = synth.dense_weight(synth.CFG_SWIGLU, "up", N, K)
    r = oracle.swiglu_bf16(x, Wg, Wu)
    return x, Wg, Wu, bf16_dev(x), bf16_dev(Wg), bf16_dev(Wu), r


@pytest.mark.parametrize("M", synth.SWIGLU_M)
def test_swiglu_against_unfused_oracle_chain(M):
    x, Wg, Wu, xd, Wgd, Wud, r = swiglu_case()
    N = Wg.shape[0]
    y = run_guarded(lambda out: aqg.swiglu_bf16(xd[:M], Wgd, Wud, out=out), M, N)
    tol = oracle.swiglu_tolerance(r["g"][:M], r["u"][:M], r["Ag"][:M], r["Au"][:M], r["out"][:M])
    assert_within(y, r["out"][:M], tol, "swiglu M=%d" % M)


@pytest.mark.parametrize("M", [9, 16, 32])
@pytest.mark.parametrize("K", [576, 512])
def test_dense_large_n_ragged_matrix_core(K, M):
    """N = 40001 (>= 2048 row tiles of 16, last one ragged): the persistent
    matrix-core paths (K = 576: per-wavefront stream; K = 512: whole tiles
    through LDS), within tolerance, and M = 9..31 bit for bit equal to the
    first rows of the M = 32 call."""
    N = 40001
    x = synth.normal_bf16((32, K), 1.0, 79, "ln/x/%d" % K)
    W = synth.normal_bf16((N, K), 0.02, 79, "ln/W/%d" % K)
    xd, Wd = bf16_dev(x), bf16_dev(W)
    y = run_guarded(gemv_dense_gpu(xd, Wd, M), M, N)
    ref, A = oracle.gemv_bf16(x[:M], W)
    assert_within(y, ref, oracle.tolerance(A), "dense %dx%dx%d" % (M, N, K))
    y32 = aqg.gemv_bf16(xd[:32], Wd, out_dtype=torch.float32).cpu().numpy()
    yM = aqg.gemv_bf16(xd[:M], Wd, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(yM, y32[:M])


@pytest.mark.parametrize("N,K", [(32769, 1536), (33000, 1024), (32800, 2048), (40001, 512)])
def test_dense_tile_path_every_k(N, K):
    """Large-N dense calls with K = 512 .. 2048 (tile ring of 4, 3, 2, 2
    buffers) at M = 3, 5, 8, 9, 16, 17, 32: parity with the oracle, bf16 = RNE of
    fp32, no write outside the output, and every M bit for bit equal to the
    first rows of the M = 32 call.  N leaves a ragged last tile (or none)."""
    x = synth.normal_bf16((32, K), 1.0, 80, "tp/x/%d" % K)
    W = synth.normal_bf16((N, K), 0.02, 80, "tp/W/%d/%d" % (N, K))
    xd, Wd = bf16_dev(x), bf16_dev(W)
    ref, A = oracle.gemv_bf16(x, W)
    y32 = None
    for M in (32, 3, 5, 8, 9, 16, 17):
        y = run_guarded(gemv_dense_gpu(xd, Wd, M), M, N)
        assert_within(y, ref[:M], oracle.tolerance(A[:M]), "dense tile %dx%dx%d" % (M, N, K))
        if M == 32:
            y32 = y
        else:
            assert np.array_equal(y, y32[:M]), "M=%d" % M


@pytest.mark.parametrize("K", [1536, 1024])
def test_dense_tile_path_one_hot_exact(K):
    """One-hot rows of x at k positions in every wavefront's share of K and in
    every 1 KB piece of a row: y[m, n] = W[n, k_m] exactly, over a ragged last
    tile.  Pins the copy into LDS (piece, row and column placement) and the
    operand reads."""
    N, M = 32769, 32
    W = synth.normal_bf16((N, K), 0.02, 81, "tpoh/W/%d" % K)
    cols = np.array([(m * (K // 32) + 5 * (m % 8) + 3) % K for m in range(M)])
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), cols] = 0x3F80
    for Mc in (32, 7):
        y = run_guarded(gemv_dense_gpu(bf16_dev(x), bf16_dev(W), Mc), Mc, N)
        assert np.array_equal(y, oracle.bf16_to_f64(W[:, cols[:Mc]]).T), "M=%d" % Mc


@pytest.mark.parametrize("M", [12, 32])
def test_swiglu_large_n_matrix_core_stream(M):
    N, K = 33001, 256
    x = synth.normal_bf16((32, K), 1.0, 80, "sl/x")
    Wg = synth.normal_bf16((N, K), 0.02, 80, "sl/g")
    Wu = synth.normal_bf16((N, K), 0.02, 80, "sl/u")
    xd, Wgd, Wud = bf16_dev(x), bf16_dev(Wg), bf16_dev(Wu)
    y = run_guarded(lambda out: aqg.swiglu_bf16(xd[:M], Wgd, Wud, out=out), M, N)
    r = oracle.swiglu_bf16(x[:M], Wg, Wu)
    tol = oracle.swiglu_tolerance(r["g"], r["u"], r["Ag"], r["Au"], r["out"])
    assert_within(y, r["out"], tol, "swiglu %dx%dx%d" % (M, N, K))


def test_swiglu_zero_weights_give_exact_zero():
    N, K = 300, 1536
    x = bf16_dev(synth.activations(synth.CFG_SWIGLU, K)[:4])
    W = bf16_dev(synth.dense_weight(73, "sz", N, K))
    Z = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda:0")
    for a, b in ((Z, W), (W, Z)):
        y = aqg.swiglu_bf16(x, a, b, out_dtype=torch.float32).cpu().numpy()
        assert np.all(y == 0)


def test_swiglu_large_negative_gate_is_near_zero():
    K = 64
    x = np.full((1, K), 0x3F80, np.uint16)          # ones
    Wg = np.full((2, K), 0xC100, np.uint16)         # -8  -> g = -512
    Wu = np.full((2, K), 0x3F80, np.uint16)         # 1   -> u = 64
    y = aqg.swiglu_bf16(bf16_dev(x), bf16_dev(Wg), bf16_dev(Wu), out_dtype=torch.float32).cpu().numpy()
    assert np.all(np.abs(y) < 1e-30)


# ----------------------------------------------------------------- affine

@pytest.mark.parametrize("M", synth.AFFINE4_M)
@pytest.mark.parametrize("shape", synth.AFFINE4_SHAPES[:3], ids=lambda s: s[0])
def test_affine4_decoder_shapes(shape, M):
    name, N, K = shape
    x, aw, xd, wq, sd, bd = affine_case(synth.CFG_AFFINE4_08B, name, 4, N, K)
    ref, A = affine_ref(synth.CFG_AFFINE4_08B, name, 4, N, K, 16)
    y = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, 4, M), M, N)
    assert_within(y, ref[:M], oracle.tolerance(A[:M]), "q4 %s M=%d" % (name, M))


@pytest.mark.parametrize("M", synth.AFFINE4_M)
def test_affine4_lm_head_values_and_argmax(M):
    name, N, K = synth.AFFINE4_SHAPES[3]
    x, aw, xd, wq, sd, bd = affine_case(synth.CFG_AFFINE4_08B, name, 4, N, K)
    ref, A = affine_ref(synth.CFG_AFFINE4_08B, name, 4, N, K, 16)
    y = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, 4, M), M, N)
    assert_within(y, ref[:M], oracle.tolerance(A[:M]), "q4 lm_head M=%d" % M)
    amb = check_argmax(y, ref[:M], A[:M])
    print("q4 lm_head M=%d: %d argmax rows within tolerance of a tie" % (M, amb))


def test_affine4_lm_head_planted_argmax():
    """Same codes with doubled scale and bias in row n*: y[n*] = 2 y[n0] exactly in
    the oracle, a unique argmax with margin when y[n0] > 0."""
    name, N, K = synth.AFFINE4_SHAPES[3]
    x, aw, xd, wq, sd, bd = affine_case(synth.CFG_AFFINE4_08B, name, 4, N, K)
    ref, A = affine_ref(synth.CFG_AFFINE4_08B, name, 4, N, K, 16)
    n0 = int(oracle.argmax(ref[:1])[0])
    assert ref[0, n0] > 0
    n_star = (n0 + 7919) % N
    words, s, b = aw.words.copy(), aw.scales.copy(), aw.biases.copy()
    words[n_star], s[n_star], b[n_star] = words[n0], s[n0] + 0x80, b[n0] + 0x80
    y = aqg.gemv_affine(xd[:1], u32_dev(words), bf16_dev(s), bf16_dev(b), 4,
                        out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    assert int(oracle.argmax(y)[0]) == n_star


@pytest.mark.parametrize("M", synth.MIXED_M)
@pytest.mark.parametrize("bits", synth.MIXED_BITS)
@pytest.mark.parametrize("shape", synth.MIXED_SHAPES, ids=lambda s: s[0])
def test_affine_mixed_width(shape, bits, M):
    name, N, K = shape
    x, aw, xd, wq, sd, bd = affine_case(synth.CFG_MIXED_WIDTH, name, bits, N, K)
    ref, A = affine_ref(synth.CFG_MIXED_WIDTH, name, bits, N, K, 16)
    y = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, bits, M), M, N)
    assert_within(y, ref[:M], oracle.tolerance(A[:M]), "q%d %s M=%d" % (bits, name, M))


@pytest.mark.parametrize("M", [1, 5, 32])
def test_affine_q7(M):
    N, K = 700, 1024
    x, aw, xd, wq, sd, bd = affine_case(74, "q7", 7, N, K)
    ref, A = affine_ref(74, "q7", 7, N, K, 32)
    y = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, 7, M), M, N)
    assert_within(y, ref[:M], oracle.tolerance(A[:M]), "q7 M=%d" % M)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_affine_one_hot_reads_codes_exactly(bits):
    """s = 1, bias = 0, x rows one-hot: y[m, n] = q[n, col_m] exactly -- pins the
    in-GEMV unpack and the activation layout for 32 columns per call."""
    N, K = 300, 1024
    words = synth.random_words((N, K * bits // 32), 75, "oh/%d" % bits)
    codes = oracle.unpack(words, bits, K)
    cols = (np.arange(32) * 31 + bits) % K
    x = np.zeros((32, K), np.uint16)
    x[np.arange(32), cols] = 0x3F80
    ones = np.full((N, K // 64), 0x3F80, np.uint16)
    zeros = np.zeros((N, K // 64), np.uint16)
    for M in (1, 32):
        y = run_guarded(gemv_affine_gpu(bf16_dev(x), u32_dev(words), bf16_dev(ones), bf16_dev(zeros), bits, M),
                        M, N)
        assert np.array_equal(y, codes[:, cols[:M]].T.astype(np.float64))


@pytest.mark.parametrize("K", [1024, 3584])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_affine_one_hot_every_group_position_m8(bits, K):
    """M = 8 one-hot rows over all 64 positions of a group, each in a
    different group of the row (K = 3584 at b = 4: the row's last lane slot
    is ragged): y[m, n] = q[n, col_m] exactly.  Pins the in-GEMV unpack for
    every code position on the path the shape takes at M = 8 (the piece
    kernel for 2, 4 and 8 bits, the small-matrix matrix-core kernel for 3
    bits; the failure message names it)."""
    N = 211
    words = synth.random_words((N, K * bits // 32), 78, "oh8/%d/%d" % (bits, K))
    codes = oracle.unpack(words, bits, K)
    G = K // 64
    cols = np.array([((r * 5 + 3) % G) * 64 + r for r in range(64)])
    ones = np.full((N, G), 0x3F80, np.uint16)
    zeros = np.zeros((N, G), np.uint16)
    wq, sd, bd = u32_dev(words), bf16_dev(ones), bf16_dev(zeros)
    for c0 in range(0, 64, 8):
        c = cols[c0:c0 + 8]
        x = np.zeros((8, K), np.uint16)
        x[np.arange(8), c] = 0x3F80
        y = run_guarded(gemv_affine_gpu(bf16_dev(x), wq, sd, bd, bits, 8), 8, N)
        assert np.array_equal(y, codes[:, c].T.astype(np.float64)), \
            "%s cols %s" % (aqg.dispatch_path(bits, 8, N, K)[0], c)


@functools.lru_cache(maxsize=None)
def affine4_large_n_case():
    N, K = 40001, 1024
    x = synth.normal_bf16((32, K), 1.0, 81, "a4l/x")
    aw = synth.affine_weight(81, "a4l", 4, N, K)
    return x, aw, bf16_dev(x), u32_dev(aw.words), bf16_dev(aw.scales), bf16_dev(aw.biases)


@pytest.mark.parametrize("M", [3, 4, 8, 9, 16, 17, 32])
def test_affine4_large_n_matrix_core(M):
    """4-bit, N = 40001 (>= 2048 row tiles of 16, last one ragged), M = 3..32:
    the matrix-core path, within tolerance, and bit for bit equal to the first
    rows of the M = 32 call."""
    x, aw, xd, wq, sd, bd = affine4_large_n_case()
    N, K = aw.scales.shape[0], x.shape[1]
    y = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, 4, M), M, N)
    ref, A = oracle.gemv_affine(x[:M], aw.words, aw.scales, aw.biases, 4)
    assert_within(y, ref, oracle.tolerance(A), "q4 %dx%dx%d" % (M, N, K))
    y32 = aqg.gemv_affine(xd[:32], wq, sd, bd, 4, out_dtype=torch.float32).cpu().numpy()
    yM = aqg.gemv_affine(xd[:M], wq, sd, bd, 4, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(yM, y32[:M])


@functools.lru_cache(maxsize=None)
def affine4_multi_tile_case():
    N, K = 131072, 1024
    x = synth.normal_bf16((32, K), 1.0, 83, "a4m/x")
    aw = synth.affine_weight(83, "a4m", 4, N, K)
    return x, aw, bf16_dev(x), u32_dev(aw.words), bf16_dev(aw.scales), bf16_dev(aw.biases)


@pytest.mark.parametrize("M", [4, 12, 16, 32])
def test_affine4_matrix_core_several_tiles_per_wavefront(M):
    """4-bit, N = 131072 (8192 row tiles): each wavefront of the persistent
    matrix-core launch owns two to four tiles, so most k-blocks go through the
    pipelined steady-state loop.  Sampled tiles from the start, the middle and
    the end against the oracle, and y(M) equal to the first rows of y(32)."""
    x, aw, xd, wq, sd, bd = affine4_multi_tile_case()
    y = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, 4, M), M, aw.scales.shape[0])
    tiles = [0, 1, 2, 2047, 2048, 2049, 4095, 4096, 6143, 6144, 8190, 8191]
    rows = np.concatenate([np.arange(16 * t, 16 * t + 16) for t in tiles])
    ref, A = oracle.gemv_affine(x[:M], aw.words[rows], aw.scales[rows], aw.biases[rows], 4)
    assert_within(y[:, rows], ref, oracle.tolerance(A), "q4 %dx131072x1024 sampled tiles" % M)
    y32 = aqg.gemv_affine(xd[:32], wq, sd, bd, 4, out_dtype=torch.float32).cpu().numpy()
    yM = aqg.gemv_affine(xd[:M], wq, sd, bd, 4, out_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(yM, y32[:M])


def test_affine4_large_n_one_hot_every_group_position_m16():
    """Matrix-core path, s = 1, bias = 0, one-hot x: y = q exactly for all 64
    positions of a group (each in a different group), 16 columns per call."""
    N, K = 33000, 1024
    words = synth.random_words((N, K // 8), 82, "oh16")
    codes = oracle.unpack(words, 4, K)
    G = K // 64
    cols = np.array([((r * 7 + 1) % G) * 64 + r for r in range(64)])
    ones = np.full((N, G), 0x3F80, np.uint16)
    zeros = np.zeros((N, G), np.uint16)
    wq, sd, bd = u32_dev(words), bf16_dev(ones), bf16_dev(zeros)
    for c0 in range(0, 64, 16):
        c = cols[c0:c0 + 16]
        x = np.zeros((16, K), np.uint16)
        x[np.arange(16), c] = 0x3F80
        y = run_guarded(gemv_affine_gpu(bf16_dev(x), wq, sd, bd, 4, 16), 16, N)
        assert np.array_equal(y, codes[:, c].T.astype(np.float64)), "cols %s" % c


@pytest.mark.parametrize("N,K", [(5000, 1792), (6000, 512), (4500, 3584), (7000, 256), (5024, 1024)])
def test_affine4_matrix_core_k_split(N, K):
    """4-bit, 257..2047 row tiles: the matrix-core path splits K over a
    workgroup's wavefronts (chunks of unequal length when the 256-k blocks do
    not divide evenly) and sums the partial tiles in chunk order.  Ragged N;
    M = 9 and 16 against the oracle and bit for bit against each other, M = 32
    as well where its x^T fits, and M = 3 (dot-product path) within
    tolerance."""
    x = synth.normal_bf16((32, K), 1.0, 84, "a4k/x/%d/%d" % (N, K))
    aw = synth.affine_weight(84, "a4k/%d/%d" % (N, K), 4, N, K)
    xd, wq, sd, bd = bf16_dev(x), u32_dev(aw.words), bf16_dev(aw.scales), bf16_dev(aw.biases)
    ref, A = oracle.gemv_affine(x, aw.words, aw.scales, aw.biases, 4)
    y16 = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, 4, 16), 16, N)
    assert_within(y16, ref[:16], oracle.tolerance(A[:16]), "q4 16x%dx%d" % (N, K))
    y9 = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, 4, 9), 9, N)
    assert_within(y9, ref[:9], oracle.tolerance(A[:9]), "q4 9x%dx%d" % (N, K))
    assert np.array_equal(y9, y16[:9])
    y3 = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, 4, 3), 3, N)
    assert_within(y3, ref[:3], oracle.tolerance(A[:3]), "q4 3x%dx%d" % (N, K))
    if K <= 1024:
        y32 = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, 4, 32), 32, N)
        assert_within(y32, ref, oracle.tolerance(A), "q4 32x%dx%d" % (N, K))
        assert np.array_equal(y16, y32[:16])


def test_affine4_k_split_one_hot_every_group_position_m16():
    """K split (5000 x 1792: 7 blocks of 256 k in 4 chunks), s = 1, bias = 0,
    one-hot x: y = q exactly at every position of a group, whichever chunk
    holds it (the other chunks add exact zeros)."""
    N, K = 5000, 1792
    words = synth.random_words((N, K // 8), 85, "oh16k")
    codes = oracle.unpack(words, 4, K)
    G = K // 64
    cols = np.array([((r * 5 + 3) % G) * 64 + r for r in range(64)])
    ones = np.full((N, G), 0x3F80, np.uint16)
    zeros = np.zeros((N, G), np.uint16)
    wq, sd, bd = u32_dev(words), bf16_dev(ones), bf16_dev(zeros)
    for c0 in range(0, 64, 16):
        c = cols[c0:c0 + 16]
        x = np.zeros((16, K), np.uint16)
        x[np.arange(16), c] = 0x3F80
        y = run_guarded(gemv_affine_gpu(bf16_dev(x), wq, sd, bd, 4, 16), 16, N)
        assert np.array_equal(y, codes[:, c].T.astype(np.float64)), "cols %s" % c


@functools.lru_cache(maxsize=None)
def affine_mma_case(bits, N, K):
    x = synth.normal_bf16((32, K), 1.0, 86, "amw/x/%d/%d/%d" % (bits, N, K))
    aw = synth.affine_weight(86, "amw/%d/%d/%d" % (bits, N, K), bits, N, K)
    return x, aw, bf16_dev(x), u32_dev(aw.words), bf16_dev(aw.scales), bf16_dev(aw.biases)


@pytest.mark.parametrize("bits", [2, 8])
@pytest.mark.parametrize("N,K", [(40001, 1024), (5000, 1536), (4500, 4096), (6000, 512)])
def test_affine_matrix_core_2_and_8_bit(bits, N, K):
    """2- and 8-bit codes on the matrix core (8-bit codes as two nibble
    chains): N = 40001 streams whole tiles, the others split K.  M = 9, 16
    and 32 against the oracle; 9 and 16 bit for bit against each other, and
    32 as well where its x^T fits."""
    x, aw, xd, wq, sd, bd = affine_mma_case(bits, N, K)
    ref, A = oracle.gemv_affine(x, aw.words, aw.scales, aw.biases, bits)
    y16 = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, bits, 16), 16, N)
    assert_within(y16, ref[:16], oracle.tolerance(A[:16]), "q%d 16x%dx%d" % (bits, N, K))
    y9 = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, bits, 9), 9, N)
    assert_within(y9, ref[:9], oracle.tolerance(A[:9]), "q%d 9x%dx%d" % (bits, N, K))
    assert np.array_equal(y9, y16[:9])
    y32 = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, bits, 32), 32, N)
    assert_within(y32, ref, oracle.tolerance(A), "q%d 32x%dx%d" % (bits, N, K))
    if K <= 1024:
        assert np.array_equal(y16, y32[:16])


@pytest.mark.parametrize("bits,N,K", [(4, 1000, 1024), (4, 3001, 2048), (4, 700, 3584), (4, 3000, 4096),
                                      (4, 300, 512), (4, 129, 256), (2, 1000, 4096), (2, 3000, 2048),
                                      (2, 999, 1536), (8, 2000, 1024), (8, 999, 4096), (8, 1000, 2048),
                                      (4, 1000, 8192), (2, 500, 8192),
                                      (3, 1000, 1024), (5, 999, 1536), (6, 700, 3584), (7, 3000, 1024),
                                      (3, 4090, 1536), (5, 300, 128)])
def test_affine_split_path(bits, N, K):
    """Small matrices (at most 256 row tiles) on the matrix core with one
    workgroup per tile and K split over its wavefronts (8-bit K = 4096 and
    4-bit K = 8192: two k-blocks per wavefront), M = 5..16, and M = 17..32 with at most 128 tiles:
    M = 9..16 in two 8-column workgroups where the tiles are few, M = 17..32
    in two 16-column ones.  Ragged last tile; every M against the oracle
    (bf16 = RNE of fp32, no write outside the output) and bit for bit equal to
    the first rows of its bucket's widest call (16 or 32 rows), and the two
    buckets to each other where both take this path.  3, 5, 6 and 7 bits
    (per-lane code windows, 2 or 4 groups per wavefront) take it from M = 1
    and up to 256 row tiles at every M."""
    x, aw, xd, wq, sd, bd = affine_mma_case(bits, N, K)
    ref, A = oracle.gemv_affine(x, aw.words, aw.scales, aw.biases, bits)
    nat = bits in (3, 5, 6, 7)
    tops = {}
    for M in ((16, 1, 2, 4, 5, 8, 9, 32, 17) if nat else (16, 5, 8, 9, 32, 17)):
        path = aqg.dispatch_path(bits, M, N, K)[0]
        if nat and M == 1 and path != "affine_split":
            continue
        if nat or M <= 16 or (N + 15) // 16 <= 128:
            assert path == "affine_split", "M=%d" % M
        y = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, bits, M), M, N)
        assert_within(y, ref[:M], oracle.tolerance(A[:M]), "q%d split %dx%dx%d" % (bits, M, N, K))
        b = 16 if M <= 16 else 32
        if b not in tops:
            tops[b] = y
        else:
            assert np.array_equal(y, tops[b][:M]), "M=%d" % M
    if 32 in tops and aqg.dispatch_path(bits, 32, N, K)[0] == "affine_split":
        assert np.array_equal(tops[16], tops[32][:16])


@pytest.mark.parametrize("bits,K", [(2, 4096), (4, 1024), (4, 3584), (8, 1024), (8, 4096),
                                    (3, 1024), (5, 1536), (6, 3584), (7, 1024), (7, 2048)])
def test_affine_split_path_one_hot_exact(bits, K):
    """Split path (N = 1001: 63 row tiles), s = 1, bias = 0, one-hot x: y = q
    exactly with the ones at every position of a group, in every wavefront's
    k-blocks, for M = 16 (8-column workgroups) and 32 (16-column ones); then
    s = 2, bias = -1 on the same codes: y = 2 q - 1 exactly."""
    N = 1001
    for MC in (16, 32):
        assert aqg.dispatch_path(bits, MC, N, K)[0] == "affine_split"
    words = synth.random_words((N, K * bits // 32), 89, "soh/%d/%d" % (bits, K))
    codes = oracle.unpack(words, bits, K)
    G = K // 64
    cols = np.array([((r * 5 + 3) % G) * 64 + r for r in range(64)])
    wq = u32_dev(words)
    for sv, bv in ((0x3F80, 0x0000), (0x4000, 0xBF80)):
        sd = bf16_dev(np.full((N, G), sv, np.uint16))
        bd = bf16_dev(np.full((N, G), bv, np.uint16))
        want_s, want_b = oracle.bf16_to_f64(np.array([sv], np.uint16))[0], oracle.bf16_to_f64(np.array([bv], np.uint16))[0]
        for MC in (16, 32):
            for c0 in range(0, 64, MC):
                c = cols[c0:c0 + MC]
                x = np.zeros((MC, K), np.uint16)
                x[np.arange(MC), c] = 0x3F80
                y = run_guarded(gemv_affine_gpu(bf16_dev(x), wq, sd, bd, bits, MC), MC, N)
                assert np.array_equal(y, (want_s * codes[:, c] + want_b).T.astype(np.float64)), "M=%d cols %s" % (MC, c)


@pytest.mark.parametrize("bits,N,K", [(4, 4201, 2048), (4, 4113, 4096), (2, 4105, 4096), (2, 4300, 2048),
                                      (8, 4150, 1024), (8, 4111, 2048), (8, 4099, 4096), (3, 1000, 4096),
                                      (5, 1001, 4096), (6, 999, 2048), (6, 500, 4096), (7, 777, 4096)])
def test_affine_tile_path(bits, N, K):
    """Affine tiles copied into LDS (2/4-bit K = 2048, 4096; 8-bit K = 1024,
    2048, and 4096 up to 16 columns; 3, 5, 7 bits K = 4096 and 6 bits K =
    2048, 4096 with codes taken from bit windows): M = 5, 9, 16, 17, 32 against the oracle
    (bf16 = RNE of fp32, no write outside the output), ragged last tile, and
    every M of a path bit for bit equal to the first rows of its widest call."""
    x, aw, xd, wq, sd, bd = affine_mma_case(bits, N, K)
    ref, A = oracle.gemv_affine(x, aw.words, aw.scales, aw.biases, bits)
    Ms = (16, 5, 9) if (bits == 8 and K == 4096) else (32, 5, 9, 16, 17)
    by_path = {}
    for M in Ms:
        y = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, bits, M), M, N)
        path = aqg.dispatch_path(bits, M, N, K)[0]
        assert_within(y, ref[:M], oracle.tolerance(A[:M]), "q%d %s %dx%dx%d" % (bits, path, M, N, K))
        by_path.setdefault(path, {})[M] = y
    assert "affine_tile" in by_path or (bits, K) in ((2, 4096), (4, 4096), (8, 4096))
    # (2-, 4- and 8-bit K = 4096 run on the multi-tile kernel up to 16 columns)
    for runs in by_path.values():
        top = runs[max(runs)]
        for M, y in runs.items():
            assert np.array_equal(y, top[:M]), "M=%d" % M


@pytest.mark.parametrize("bits,N", [(4, 8000), (2, 8000), (5, 8000), (2, 20000), (4, 20000)])
def test_affine_tile_path_several_tiles_per_workgroup(bits, N):
    """Several row tiles per workgroup at K = 4096, M = 16: N = 8000 (500
    tiles: 1-2 per workgroup; 2 and 4 bits on the multi-tile kernel, 5 bits
    on the tile ring) and N = 20000 (1250 tiles: 4-5 per workgroup on the tile
    ring, more than the multi-tile kernel takes).  The tile ring's first
    tiles are issued in two parts (tile 0 before x is staged, the rest
    after), so the waits of the first steps depend on how many tiles a
    workgroup has; each count is checked against the oracle."""
    K = 4096
    x, aw, xd, wq, sd, bd = affine_mma_case(bits, N, K)
    xs = x[:16]
    ref, A = oracle.gemv_affine(xs, aw.words, aw.scales, aw.biases, bits)
    y = run_guarded(gemv_affine_gpu(xd[:16], wq, sd, bd, bits, 16), 16, N)
    assert_within(y, ref, oracle.tolerance(A), "q%d tile 16x%dx%d" % (bits, N, K))


def burst_ms(bits, N):
    """The M <= 16 the multi-tile kernel serves for this width and N."""
    return [M for M in (16, 1, 2, 3, 4, 5, 8, 9) if aqg.dispatch_path(bits, M, N, 4096)[0] == "affine_burst"]


@pytest.mark.parametrize("bits,N", [(b, N) for b in (2, 4, 5, 6, 7, 8) for N in (3990, 14350)
                                    if (b, N) != (5, 14350)])
def test_affine_burst_path(bits, N):
    """Multi-tile kernel at K = 4096 (all of a workgroup's 1-4 row tiles in
    flight, codes straight into the MFMA lanes, bias and code-offset terms as
    an MFMA pair on exact bf16 pieces): N = 3990 (250 tiles, one per
    workgroup) and 14350 (897 tiles, 3-4 per workgroup), both with a ragged
    last tile.  Every M it serves against the oracle (bf16 = RNE of fp32, no
    write outside the output) and bit for bit equal to the first rows of
    its widest call; 8 bits at M = 17 and 32 (two 16-column launches) as
    well, the first 16 rows equal to the M = 16 call."""
    K = 4096
    Ms = burst_ms(bits, N)
    assert Ms, "no M of q%d %dx%d on the multi-tile kernel" % (bits, N, K)
    x, aw, xd, wq, sd, bd = affine_mma_case(bits, N, K)
    ref, A = oracle.gemv_affine(x, aw.words, aw.scales, aw.biases, bits)
    runs = {}
    for M in Ms:
        y = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, bits, M), M, N)
        assert_within(y, ref[:M], oracle.tolerance(A[:M]), "q%d burst %dx%dx%d" % (bits, M, N, K))
        runs[M] = y
    top = runs[max(runs)]
    for M, y in runs.items():
        assert np.array_equal(y, top[:M]), "M=%d" % M
    if bits == 8 and N > 4096:
        for M in (32, 17):
            assert aqg.dispatch_path(bits, M, N, K)[0] == "affine_burst"
            y = run_guarded(gemv_affine_gpu(xd, wq, sd, bd, bits, M), M, N)
            assert_within(y, ref[:M], oracle.tolerance(A[:M]), "q%d burst %dx%dx%d" % (bits, M, N, K))
            if 16 in runs:
                assert np.array_equal(y[:16], runs[16]), "M=%d" % M


@pytest.mark.parametrize("bits", [2, 4, 5, 6, 7, 8])
def test_affine_burst_one_hot_exact(bits):
    """Multi-tile kernel (N = 3990, K = 4096), s = 1, bias = 0, one-hot x: y
    = q exactly with the ones at every position of a group and in every
    wavefront's groups, at the widest M it serves; then s = 2, bias = -1 on
    the same codes: y = 2 q - 1 exactly (the bias and offset MFMA pair
    reproduces bias * X and cancels the code offset exactly here).  8 bits
    also at M = 32 on N = 14350 (two 16-column launches)."""
    K = 4096
    G = K // 64
    cols = np.array([((r * 5 + 3) % G) * 64 + r for r in range(64)])
    for N in ((3990, 14350) if bits == 8 else (3990,)):
        MC = 32 if N > 3990 else max(burst_ms(bits, N))
        assert aqg.dispatch_path(bits, MC, N, K)[0] == "affine_burst"
        words = synth.random_words((N, K * bits // 32), 91, "roh/%d/%d" % (bits, N))
        codes = oracle.unpack(words, bits, K)
        wq = u32_dev(words)
        for sv, bv in ((0x3F80, 0x0000), (0x4000, 0xBF80)):
            sd = bf16_dev(np.full((N, G), sv, np.uint16))
            bd = bf16_dev(np.full((N, G), bv, np.uint16))
            want_s = oracle.bf16_to_f64(np.array([sv], np.uint16))[0]
            want_b = oracle.bf16_to_f64(np.array([bv], np.uint16))[0]
            for c0 in range(0, 64, MC):
                c = cols[c0:c0 + MC]
                x = np.zeros((len(c), K), np.uint16)
                x[np.arange(len(c)), c] = 0x3F80
                y = run_guarded(gemv_affine_gpu(bf16_dev(x), wq, sd, bd, bits, len(c)), len(c), N)
                want = (want_s * codes[:, c] + want_b).T.astype(np.float64)
                assert np.array_equal(y, want), "q%d N=%d M=%d cols %s" % (bits, N, len(c), c)


@pytest.mark.parametrize("bits,K", [(2, 4096), (4, 2048), (8, 1024), (8, 4096), (3, 4096), (5, 4096), (6, 2048),
                                    (7, 4096)])
def test_affine_tile_path_one_hot_exact(bits, K):
    """s = 1, bias = 0, one-hot x: y = q exactly, with the ones at every
    position of a group, in every wavefront's share of K (M = 16, tile path:
    more than 256 row tiles); then s = 2, bias = -1 on the same codes: y =
    2 q - 1 exactly."""
    N = 4117
    words = synth.random_words((N, K * bits // 32), 88, "toh/%d/%d" % (bits, K))
    codes = oracle.unpack(words, bits, K)
    G = K // 64
    cols = np.array([((r * 5 + 3) % G) * 64 + r for r in range(64)])
    wq = u32_dev(words)
    for sv, bv in ((0x3F80, 0x0000), (0x4000, 0xBF80)):
        sd = bf16_dev(np.full((N, G), sv, np.uint16))
        bd = bf16_dev(np.full((N, G), bv, np.uint16))
        want_s, want_b = oracle.bf16_to_f64(np.array([sv], np.uint16))[0], oracle.bf16_to_f64(np.array([bv], np.uint16))[0]
        for c0 in range(0, 64, 16):
            c = cols[c0:c0 + 16]
            x = np.zeros((16, K), np.uint16)
            x[np.arange(16), c] = 0x3F80
            y = run_guarded(gemv_affine_gpu(bf16_dev(x), wq, sd, bd, bits, 16), 16, N)
            assert np.array_equal(y, (want_s * codes[:, c] + want_b).T.astype(np.float64)), "cols %s" % c


@pytest.mark.parametrize("bits", [2, 8])
@pytest.mark.parametrize("N,K", [(33000, 1024), (5000, 1536)])
def test_affine_matrix_core_2_and_8_bit_one_hot_m16(bits, N, K):
    """s = 1, bias = 0, one-hot x: y = q exactly at all 64 positions of a
    group (each in a different group), on the matrix core, whole tiles and
    K split."""
    words = synth.random_words((N, K * bits // 32), 87, "ohw/%d/%d" % (bits, N))
    codes = oracle.unpack(words, bits, K)
    G = K // 64
    cols = np.array([((r * 7 + 1) % G) * 64 + r for r in range(64)])
    ones = np.full((N, G), 0x3F80, np.uint16)
    zeros = np.zeros((N, G), np.uint16)
    wq, sd, bd = u32_dev(words), bf16_dev(ones), bf16_dev(zeros)
    for c0 in range(0, 64, 16):
        c = cols[c0:c0 + 16]
        x = np.zeros((16, K), np.uint16)
        x[np.arange(16), c] = 0x3F80
        y = run_guarded(gemv_affine_gpu(bf16_dev(x), wq, sd, bd, bits, 16), 16, N)
        assert np.array_equal(y, codes[:, c].T.astype(np.float64)), "cols %s" % c


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_affine_small_integers_exact(bits):
    M, N, K = 3, 5, 192
    g = synth.rng(76, "ex/%d" % bits)
    x = synth.to_bf16_bits(g.integers(-4, 5, size=(M, K)).astype(np.float64))
    words = synth.random_words((N, K * bits // 32), 76, "exw/%d" % bits)
    s = synth.to_bf16_bits(2.0 ** -g.integers(0, 4, size=(N, K // 64)))
    b = synth.to_bf16_bits(g.integers(-3, 4, size=(N, K // 64)).astype(np.float64))
    y = run_guarded(gemv_affine_gpu(bf16_dev(x), u32_dev(words), bf16_dev(s), bf16_dev(b), bits, M), M, N)
    ref, _ = oracle.gemv_affine(x, words, s, b, bits)
    assert np.array_equal(y, ref)


def test_affine_closed_form_half():
    codes = np.full((1, 64), 5, np.uint8)
    words = oracle.pack(codes, 4)
    s = np.array([[0x3C00]], np.uint16)
    b = np.array([[0xBD00]], np.uint16)
    x = np.full((1, 64), 0x3F80, np.uint16)
    y = aqg.gemv_affine(bf16_dev(x), u32_dev(words), bf16_dev(s), bf16_dev(b), 4,
                        out_dtype=torch.float32).cpu().numpy()
    assert y[0, 0] == 0.5


@pytest.mark.parametrize("bits", [2, 3, 5, 6])
def test_affine_cross_width_widened_to_8bit(bits):
    """The same codes stored at width b and widened to 8 bits give the same y (within
    tolerance: the two widths sum their code pairs in different orders)."""
    M, N, K = 4, 1000, 4096
    x, aw, xd, wq, sd, bd = affine_case(synth.CFG_MIXED_WIDTH, "sq_4096", bits, N, K)
    w8 = oracle.pack(oracle.unpack(aw.words, bits, K), 8)
    yb = aqg.gemv_affine(xd[:M], wq, sd, bd, bits, out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    y8 = aqg.gemv_affine(xd[:M], u32_dev(w8), sd, bd, 8, out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    _, A = oracle.gemv_affine(x[:M], aw.words, aw.scales, aw.biases, bits)
    assert_within(yb, y8, 2 * oracle.tolerance(A), "q%d vs widened q8" % bits)


@pytest.mark.parametrize("M,N,K,bits", [(1, 1, 64, 4), (3, 7, 64, 3), (5, 77, 128, 5), (17, 1000, 576, 2),
                                        (31, 129, 3584, 6), (2, 3000, 8192, 4), (32, 100, 4096, 8)])
def test_affine_ragged_shapes(M, N, K, bits):
    x = synth.normal_bf16((M, K), 1.0, 77, "ar/x/%d" % K)
    aw = synth.affine_weight(77, "ar", bits, N, K)
    y = run_guarded(gemv_affine_gpu(bf16_dev(x), u32_dev(aw.words), bf16_dev(aw.scales), bf16_dev(aw.biases),
                                    bits, M), M, N)
    ref, A = oracle.gemv_affine(x, aw.words, aw.scales, aw.biases, bits)
    assert_within(y, ref, oracle.tolerance(A), "q%d %dx%dx%d" % (bits, M, N, K))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_affine_rows_independent_of_m(bits):
    """On 4096 x 4096, calls whose M the library serves with the same kernel
    and column bucket (its dispatch query) agree bit for bit on their common
    rows: the one-row call, and the widest M of each (path, columns) group.
    The streaming and piece kernels (M <= 4 here for 2, 4, 8 bits and M = 1
    for the others) compute each row on its own, so they also match one-row
    calls."""
    name, N, K = synth.MIXED_SHAPES[0]
    x, aw, xd, wq, sd, bd = affine_case(synth.CFG_MIXED_WIDTH, name, bits, N, K)
    Ms = (1, 2, 3, 4, 5, 8, 9, 12, 16, 17, 20, 32)
    groups = {}
    for M in Ms:
        groups.setdefault(aqg.dispatch_path(bits, M, N, K), []).append(M)
    y1 = aqg.gemv_affine(xd[:1], wq, sd, bd, bits, out_dtype=torch.float32).cpu().numpy()
    path1 = aqg.dispatch_path(bits, 1, N, K)[0]
    for key, group in groups.items():
        top = max(group)
        ytop = aqg.gemv_affine(xd[:top], wq, sd, bd, bits, out_dtype=torch.float32).cpu().numpy()
        for M in group:
            yM = aqg.gemv_affine(xd[:M], wq, sd, bd, bits, out_dtype=torch.float32).cpu().numpy()
            assert np.array_equal(yM, ytop[:M]), "%s M=%d vs %d" % (key, M, top)
        if key[0] in ("stream", "piece") and key[0] == path1:
            rows = np.concatenate([aqg.gemv_affine(xd[m:m + 1], wq, sd, bd, bits, out_dtype=torch.float32)
                                   .cpu().numpy() for m in range(top)])
            assert np.array_equal(ytop, rows), "%s M=%d vs one-row calls" % (key, top)
    assert len(groups) >= 2
