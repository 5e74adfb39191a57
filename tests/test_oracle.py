"""Pins for the CPU oracle (no GPU needed).

Each test ties the oracle to something other than itself: a library routine
(torch's bf16 rounding, numpy matmul / argmax), hand-derived worked vectors,
closed forms, exact rational brute force, or an independent formulation
(Python big-integer bit streams).  Together they are chosen so that a dropped
term, a wrong sign or index, or a transposed operand in the oracle fails at
least one of them (see test_oracle_mutants.py, which plants such mistakes).
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_worked.txt")


# ------------------------------------------------------------------ bf16

def test_bf16_decode_all_patterns_match_torch():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bf16_to_f64(h)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


@pytest.mark.slow
def test_f32_to_bf16_rne_exhaustive_matches_torch():
    """All 2^32 float32 bit patterns, against torch's CPU float->bfloat16 (RNE)."""
    step = 1 << 26
    base = np.arange(step, dtype=np.uint32)
    u = np.empty_like(base)
    for start in range(0, 1 << 32, step):
        np.add(base, np.uint32(start), out=u)
        f = u.view(np.float32)
        mine = oracle.f32_to_bf16(f)
        ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        fnan = np.isnan(f)
        # every mismatch must be a NaN input (payloads are not compared) ...
        assert not np.any((mine != ref) & ~fnan), hex(start)
        # ... and NaN stays NaN
        if fnan.any():
            mn = mine[fnan]
            assert np.all(((mn & 0x7F80) == 0x7F80) & ((mn & 0x007F) != 0))


def test_f32_to_bf16_ties_to_even_by_hand():
    # 1 + 2^-8 is exactly halfway between bf16 1.0 (0x3F80) and 1+2^-7 (0x3F81): even -> 0x3F80.
    # 1 + 3*2^-8 is halfway between 0x3F81 and 0x3F82: even -> 0x3F82.
    vals = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20], np.float32)
    assert list(oracle.f32_to_bf16(vals)) == [0x3F80, 0x3F82, 0xBF80, 0x3F81]


# ---------------------------------------------------------- pack / unpack

def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((int(parts[0]), parts[1], [int(w, 16) for w in parts[2:]]))
    return rows


def _codes_from_formula(formula: str, bits: int):
    k = np.arange(64)
    table = {"k%4": k % 4, "k%8": k % 8, "k%16": k % 16, "k%32": k % 32, "k%64": k % 64,
             "k%128": k % 128, "k%256": k % 256, "(7k+3)%16": (7 * k + 3) % 16}
    c = table[formula].astype(np.uint8)
    assert c.max() < (1 << bits)
    return c


@pytest.mark.parametrize("row", _golden_rows(), ids=lambda r: "b%d_%s" % (r[0], r[1]))
def test_pack_worked_vectors(row):
    bits, formula, expect = row
    codes = _codes_from_formula(formula, bits)[None, :]
    words = oracle.pack(codes, bits)
    assert words.shape == (1, 2 * bits)
    assert [int(w) for w in words[0, :len(expect)]] == expect
    assert brute.pack_row(codes[0], bits)[:len(expect)] == expect
    assert np.array_equal(oracle.unpack(words, bits, 64), codes)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_pack_unpack_roundtrip_random_and_patterns(bits):
    N, K = 7, 320
    rnd = synth.random_codes((N, K), bits, 99, "roundtrip/%d" % bits)
    top = (1 << bits) - 1
    pats = [np.zeros(K, np.uint8), np.full(K, top, np.uint8),
            (np.arange(K) % 2 * top).astype(np.uint8)]
    for i in range(bits):  # walking single bit
        pats.append(np.full(K, 1 << i, np.uint8))
    codes = np.vstack([rnd] + [p[None, :] for p in pats])
    words = oracle.pack(codes, bits)
    assert np.array_equal(oracle.unpack(words, bits, K), codes)
    # the big-integer formulation reads the same codes out of the same words
    for n in range(codes.shape[0]):
        assert brute.row_codes(words[n], bits, K) == [int(c) for c in codes[n]]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_unpack_of_random_words_matches_bigint_stream(bits):
    N, K = 5, 192
    words = synth.random_words((N, K * bits // 32), 98, "unpack/%d" % bits)
    codes = oracle.unpack(words, bits, K)
    for n in range(N):
        assert brute.row_codes(words[n], bits, K) == [int(c) for c in codes[n]]
    # and pack inverts it exactly (every bit of the stream belongs to a code)
    assert np.array_equal(oracle.pack(codes, bits), words)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_unpack_closed_form_for_word_aligned_widths(bits):
    """b in {2,4,8}: code k is field (k mod 32/b) of word k // (32/b)."""
    N, K = 3, 256
    words = synth.random_words((N, K * bits // 32), 97, "closed/%d" % bits)
    per = 32 // bits
    k = np.arange(K)
    expect = (words[:, k // per] >> (bits * (k % per)).astype(np.uint32)) & ((1 << bits) - 1)
    assert np.array_equal(oracle.unpack(words, bits, K), expect.astype(np.uint8))


@pytest.mark.parametrize("bits,straddlers", [
    (3, [10, 21, 42, 53]),
    (5, [6, 12, 19, 25, 38, 44, 51, 57]),
    (6, [5, 10, 21, 26, 37, 42, 53, 58]),
    (7, [4, 9, 13, 18, 22, 27, 36, 41, 45, 50, 54, 59]),
])
def test_straddling_codes_take_low_bits_from_lower_word(bits, straddlers):
    """Codes whose bits cross a 32-bit word boundary (listed by hand) read correctly
    when only that code is nonzero."""
    K = 64
    for k in range(K):
        starts, ends = (bits * k) >> 5, (bits * k + bits - 1) >> 5
        assert (starts != ends) == (k in straddlers)
    for k in straddlers:
        codes = np.zeros((1, K), np.uint8)
        codes[0, k] = (1 << bits) - 1
        words = oracle.pack(codes, bits)
        lo_word = (bits * k) >> 5
        nlow = 32 - ((bits * k) & 31)
        assert int(words[0, lo_word]) == ((1 << nlow) - 1) << (32 - nlow)
        assert int(words[0, lo_word + 1]) == (1 << (bits - nlow)) - 1
        assert np.array_equal(oracle.unpack(words, bits, K), codes)


# ------------------------------------------------------------------ GEMV

def _bf16(vals):
    return synth.to_bf16_bits(np.asarray(vals, np.float64))


def test_affine_closed_form_all_equal_codes_exact():
    """b=4, K=64, all codes 5, s=2^-7, bias=-2^-5, x=1: w = 5/128 - 4/128 = 2^-7,
    y = 64 * 2^-7 = 0.5 exactly."""
    codes = np.full((1, 64), 5, np.uint8)
    words = oracle.pack(codes, 4)
    s = np.array([[0x3C00]], np.uint16)   # 2^-7
    b = np.array([[0xBD00]], np.uint16)   # -2^-5
    assert oracle.bf16_to_f64(s)[0, 0] == 2 ** -7 and oracle.bf16_to_f64(b)[0, 0] == -2 ** -5
    x = np.full((1, 64), 0x3F80, np.uint16)
    y, A = oracle.gemv_affine(x, words, s, b, 4)
    assert y[0, 0] == 0.5 and A[0, 0] == 0.5


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_affine_zero_codes_give_bias_times_group_sums(bits):
    M, N, K = 3, 4, 256
    x = synth.normal_bf16((M, K), 1.0, 96, "zc/x")
    b = synth.uniform_bf16((N, K // 64), -0.1, 0.1, 96, "zc/b")
    s = synth.uniform_bf16((N, K // 64), 0.001, 0.02, 96, "zc/s")
    words = np.zeros((N, K * bits // 32), np.uint32)
    y, _ = oracle.gemv_affine(x, words, s, b, bits)
    X = oracle.bf16_to_f64(x).reshape(M, K // 64, 64).sum(axis=2)      # [M, G]
    expect = X @ oracle.bf16_to_f64(b).T                                # [M, N]
    assert np.allclose(y, expect, rtol=0, atol=1e-12)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_affine_unit_scale_zero_bias_is_integer_dot(bits):
    """s=1, bias=0 and integer x: y is the integer dot product codes . x (numpy int64)."""
    M, N, K = 4, 9, 384
    x_int = synth.rng(95, "int/x").integers(-8, 9, size=(M, K))
    x = _bf16(x_int)
    words = synth.random_words((N, K * bits // 32), 95, "int/w%d" % bits)
    codes = oracle.unpack(words, bits, K).astype(np.int64)
    s = np.full((N, K // 64), 0x3F80, np.uint16)
    b = np.zeros((N, K // 64), np.uint16)
    y, _ = oracle.gemv_affine(x, words, s, b, bits)
    assert np.array_equal(y, (x_int @ codes.T).astype(np.float64))


@pytest.mark.parametrize("bits", [2, 3, 5, 8])
def test_affine_one_hot_reads_single_codes(bits):
    M, N, K = 64, 3, 128
    words = synth.random_words((N, K * bits // 32), 94, "onehot/%d" % bits)
    codes = oracle.unpack(words, bits, K)
    x = np.zeros((M, K), np.uint16)
    cols = np.arange(M) * 2 + 1
    x[np.arange(M), cols] = 0x3F80
    s = np.full((N, K // 64), 0x3F80, np.uint16)
    b = np.zeros((N, K // 64), np.uint16)
    y, _ = oracle.gemv_affine(x, words, s, b, bits)
    assert np.array_equal(y, codes[:, cols].T.astype(np.float64))


def test_dense_matches_numpy_matmul_and_abs_sum():
    M, N, K = 5, 33, 1536
    x = synth.normal_bf16((M, K), 1.0, 93, "d/x")
    W = synth.normal_bf16((N, K), 0.02, 93, "d/W")
    y, A = oracle.gemv_bf16(x, W)
    xd, Wd = oracle.bf16_to_f64(x), oracle.bf16_to_f64(W)
    ref = xd @ Wd.T
    aref = np.abs(xd) @ np.abs(Wd).T
    # both sum exact products in double; only the summation order differs
    assert np.all(np.abs(y - ref) <= 4 * K * 2.0 ** -53 * aref)
    assert np.all(np.abs(A - aref) <= 4 * K * 2.0 ** -53 * aref)


def test_dense_one_hot_returns_weight_exactly():
    N, K = 6, 64
    W = synth.normal_bf16((N, K), 0.02, 92, "oh/W")
    x = np.zeros((K, K), np.uint16)
    x[np.arange(K), np.arange(K)] = 0x3F80
    y, _ = oracle.gemv_bf16(x, W)
    assert np.array_equal(y, oracle.bf16_to_f64(W).T)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_affine_matches_exact_brute_force_on_tiny_exact_inputs(bits):
    """Small-integer x, s in {1, 2^-n}, integer bias: every product and sum is exact,
    so the double oracle equals the rational brute force bit for bit."""
    M, N, K = 3, 5, 128
    g = synth.rng(91, "tiny/%d" % bits)
    x = _bf16(g.integers(-4, 5, size=(M, K)))
    words = synth.random_words((N, K * bits // 32), 91, "tiny/w%d" % bits)
    s = _bf16(2.0 ** -g.integers(0, 4, size=(N, K // 64)))
    b = _bf16(g.integers(-3, 4, size=(N, K // 64)))
    y, _ = oracle.gemv_affine(x, words, s, b, bits)
    ref = brute.gemv_affine_exact(x.tolist(), words.tolist(), s.tolist(), b.tolist(), bits)
    for m in range(M):
        for n in range(N):
            assert Fraction(y[m, n]) == ref[m][n]


@pytest.mark.parametrize("bits", [3, 4, 6])
def test_affine_random_tiny_within_double_rounding_of_exact(bits):
    M, N, K = 2, 4, 192
    x = synth.normal_bf16((M, K), 1.0, 90, "rt/x")
    aw = synth.affine_weight(90, "rt", bits, N, K)
    y, A = oracle.gemv_affine(x, aw.words, aw.scales, aw.biases, bits)
    ref = brute.gemv_affine_exact(x.tolist(), aw.words.tolist(), aw.scales.tolist(),
                                  aw.biases.tolist(), bits)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(y[m, n]) - ref[m][n]) <= Fraction(2 * K * 2.0 ** -53) * Fraction(A[m, n])


def test_dense_matches_exact_brute_force():
    M, N, K = 2, 3, 64
    x = synth.normal_bf16((M, K), 1.0, 89, "bd/x")
    W = synth.normal_bf16((N, K), 0.02, 89, "bd/W")
    y, A = oracle.gemv_bf16(x, W)
    ref = brute.gemv_dense_exact(x.tolist(), W.tolist())
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(y[m, n]) - ref[m][n]) <= Fraction(2 * K * 2.0 ** -53) * Fraction(A[m, n])


@pytest.mark.parametrize("bits", [2, 5, 8])
def test_cross_width_widened_codes_give_same_result(bits):
    """Codes of width b, stored widened as 8-bit codes, give the same y (exactly)."""
    M, N, K = 2, 6, 256
    x = synth.normal_bf16((M, K), 1.0, 88, "cw/x")
    aw = synth.affine_weight(88, "cw", bits, N, K)
    y, _ = oracle.gemv_affine(x, aw.words, aw.scales, aw.biases, bits)
    codes = oracle.unpack(aw.words, bits, K)
    y8, _ = oracle.gemv_affine(x, oracle.pack(codes, 8), aw.scales, aw.biases, 8)
    assert np.array_equal(y, y8)


def test_affine_scale_and_bias_are_per_group_and_per_row():
    """Changing one group's scale changes exactly the terms of that group of that row."""
    M, N, K, bits = 1, 3, 192, 4
    x = synth.normal_bf16((M, K), 1.0, 87, "pg/x")
    aw = synth.affine_weight(87, "pg", bits, N, K)
    y0, _ = oracle.gemv_affine(x, aw.words, aw.scales, aw.biases, bits)
    s2 = aw.scales.copy()
    s2[1, 2] = 0  # zero the scale of row 1, group 2 (k in [128, 192))
    y1, _ = oracle.gemv_affine(x, aw.words, s2, aw.biases, bits)
    codes = oracle.unpack(aw.words, bits, K).astype(np.float64)
    xd = oracle.bf16_to_f64(x)[0]
    s = oracle.bf16_to_f64(aw.scales)[1, 2]
    delta = s * np.dot(codes[1, 128:192], xd[128:192])
    assert y1[0, 0] == y0[0, 0] and y1[0, 2] == y0[0, 2]
    assert abs((y0[0, 1] - y1[0, 1]) - delta) <= 1e-12 * (1 + abs(delta))


# --------------------------------------------------------------- SwiGLU

def test_swiglu_matches_numpy_chain():
    M, N, K = 3, 40, 1536
    x = synth.normal_bf16((M, K), 1.0, 86, "sw/x")
    Wg = synth.normal_bf16((N, K), 0.02, 86, "sw/g")
    Wu = synth.normal_bf16((N, K), 0.02, 86, "sw/u")
    r = oracle.swiglu_bf16(x, Wg, Wu)
    xd = oracle.bf16_to_f64(x)
    g = xd @ oracle.bf16_to_f64(Wg).T
    u = xd @ oracle.bf16_to_f64(Wu).T
    ref = g * (1.0 / (1.0 + np.exp(-g))) * u
    assert np.allclose(r["g"], g, rtol=1e-12, atol=1e-12)
    assert np.allclose(r["u"], u, rtol=1e-12, atol=1e-12)
    assert np.allclose(r["out"], ref, rtol=1e-11, atol=1e-13)
    # swapping the roles of gate and up changes the result (silu is not symmetric)
    r2 = oracle.swiglu_bf16(x, Wu, Wg)
    assert not np.allclose(r2["out"], r["out"])


def test_swiglu_special_cases():
    M, N, K = 2, 8, 128
    x = synth.normal_bf16((M, K), 1.0, 85, "ss/x")
    W = synth.normal_bf16((N, K), 0.02, 85, "ss/W")
    Z = np.zeros((N, K), np.uint16)
    assert np.all(oracle.swiglu_bf16(x, Z, W)["out"] == 0)   # silu(0) = 0
    assert np.all(oracle.swiglu_bf16(x, W, Z)["out"] == 0)
    # large negative gate: silu(g) -> 0; large positive: silu(g) -> g
    ones = np.full((1, K), 0x3F80, np.uint16)
    big = np.full((1, K), synth.to_bf16_bits(np.array([1.0]))[0], np.uint16)
    r = oracle.swiglu_bf16(ones, (big ^ 0x8000)[None, :].reshape(1, K), big.reshape(1, K))
    assert r["g"][0, 0] == -K and abs(r["out"][0, 0]) < 1e-50
    r = oracle.swiglu_bf16(ones, big.reshape(1, K), big.reshape(1, K))
    assert abs(r["out"][0, 0] - K * K) <= 1e-9 * K * K


# ---------------------------------------------------------------- argmax

def test_argmax_lowest_index_wins_ties_and_matches_numpy():
    y = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0], [-1.0, -2.0, -0.5, -0.5]])
    assert list(oracle.argmax(y)) == [1, 0, 2]
    g = synth.rng(84, "am")
    z = np.round(g.standard_normal((50, 1000)) * 4) / 4  # many ties
    assert np.array_equal(oracle.argmax(z), np.argmax(z, axis=1))


def test_oracle_is_thread_count_independent():
    M, N, K = 2, 257, 1024
    x = synth.normal_bf16((M, K), 1.0, 83, "th/x")
    aw = synth.affine_weight(83, "th", 3, N, K)
    n0 = oracle.max_threads()
    try:
        oracle.set_threads(1)
        y1, _ = oracle.gemv_affine(x, aw.words, aw.scales, aw.biases, 3)
        oracle.set_threads(max(2, n0))
        y2, _ = oracle.gemv_affine(x, aw.words, aw.scales, aw.biases, 3)
    finally:
        oracle.set_threads(n0)
    assert np.array_equal(y1, y2)


# ------------------------------------------------- SwiGLU abs sums and bound

def test_swiglu_abs_sums_pinned():
    """Ag, Au (which size the SwiGLU tolerance) are sum_k |w x| of each stream:
    equal to numpy's |x| |W|^T, unchanged by flipping the sign of x or of W,
    never below |g|, |u|, and equal to g, u when every product is >= 0."""
    M, N, K = 3, 24, 512
    x = synth.normal_bf16((M, K), 1.0, 82, "sa/x")
    Wg = synth.normal_bf16((N, K), 0.02, 82, "sa/g")
    Wu = synth.normal_bf16((N, K), 0.02, 82, "sa/u")
    r = oracle.swiglu_bf16(x, Wg, Wu)
    ax = np.abs(oracle.bf16_to_f64(x))
    assert np.allclose(r["Ag"], ax @ np.abs(oracle.bf16_to_f64(Wg)).T, rtol=1e-12, atol=0)
    assert np.allclose(r["Au"], ax @ np.abs(oracle.bf16_to_f64(Wu)).T, rtol=1e-12, atol=0)
    assert not np.allclose(r["Ag"], r["Au"], rtol=1e-3)       # each stream has its own sum
    r2 = oracle.swiglu_bf16(x ^ 0x8000, Wg, Wu ^ 0x8000)
    assert np.array_equal(r2["Ag"], r["Ag"]) and np.array_equal(r2["Au"], r["Au"])
    assert np.all(r["Ag"] >= np.abs(r["g"])) and np.all(r["Au"] >= np.abs(r["u"]))
    pos = oracle.swiglu_bf16(x & 0x7FFF, Wg & 0x7FFF, Wu & 0x7FFF)
    assert np.array_equal(pos["Ag"], pos["g"]) and np.array_equal(pos["Au"], pos["u"])


def _silu(g):
    return g / (1.0 + np.exp(-g))


def test_silu_slope_constant_of_the_bound():
    """The bound's 1.1 covers max |silu'| (about 1.0998 near g = 2.4); 1.0 would not."""
    g = np.linspace(-40.0, 40.0, 800001)
    e = np.exp(-g)
    slope = (1.0 + e + g * e) / (1.0 + e) ** 2       # d/dg of g / (1 + e^-g)
    assert 1.09 < slope.max() <= 1.1
    h = 1e-6
    fd = (_silu(g + h) - _silu(g - h)) / (2 * h)      # the derivative itself, by differences
    assert np.abs(fd - slope).max() < 1e-6


def _epilogue_f32(g, u):
    """silu(g) * u evaluated in fp32 from fp32 inputs, as a kernel epilogue does."""
    g32 = np.asarray(g, np.float32)
    u32 = np.asarray(u, np.float32)
    with np.errstate(over="ignore"):
        return ((g32 / (np.float32(1.0) + np.exp(-g32))) * u32).astype(np.float64)


def _admissible_swiglu_grid():
    """(g, u, Ag, Au) with Ag >= |g| and Au >= |u| (the only constraints the
    abs sums obey), over signs, magnitudes and the slope maximum of silu."""
    gs = np.concatenate([np.linspace(-30, 30, 61), [0.0, 1e-3, 2.3994, -1.2785, 12.0, -12.0]])
    us = np.array([0.0, 1e-3, -0.01, 1.0, -3.0, 100.0, -250.0])
    ga = np.array([1.0, 10.0, 100.0, 1000.0])
    ua = np.array([1.0, 10.0, 1000.0])
    G, U, GA, UA = np.meshgrid(gs, us, ga, ua, indexing="ij")
    G, U = G.ravel(), U.ravel()
    Ag = np.maximum(np.abs(G) * GA.ravel(), 1e-3 * GA.ravel())
    Au = np.maximum(np.abs(U) * UA.ravel(), 1e-3 * UA.ravel())
    return G, U, Ag, Au


def _worst_perturbed_error(G, U, Ag, Au, tol_fn):
    """Largest |out' - out| / bound over perturbations |dg| <= tg, |du| <= tu
    (corners, edges, interior), out' evaluated in fp32 like the kernels."""
    out = _silu(G) * U
    bound = tol_fn(G, U, Ag, Au, out)
    tg = oracle.tolerance(Ag)
    tu = oracle.tolerance(Au)
    worst = 0.0
    for fg in (-1.0, -0.5, 0.0, 0.5, 1.0):
        for fu in (-1.0, 0.0, 1.0):
            got = _epilogue_f32(G + fg * tg, U + fu * tu)
            worst = max(worst, float(np.max(np.abs(got - out) / bound)))
    return worst


def test_swiglu_tolerance_covers_admissible_perturbations():
    """Sound: whenever g and u are each within their GEMV bounds, the fp32
    silu(g) * u stays within the propagated SwiGLU bound."""
    G, U, Ag, Au = _admissible_swiglu_grid()
    assert _worst_perturbed_error(G, U, Ag, Au, oracle.swiglu_tolerance) <= 1.0
    # on real GEMV outputs as well
    M, N, K = 4, 64, 1536
    x = synth.normal_bf16((M, K), 1.0, 81, "sb/x")
    r = oracle.swiglu_bf16(x, synth.normal_bf16((N, K), 0.02, 81, "sb/g"),
                           synth.normal_bf16((N, K), 0.02, 81, "sb/u"))
    assert _worst_perturbed_error(r["g"], r["u"], r["Ag"], r["Au"], oracle.swiglu_tolerance) <= 1.0


def test_swiglu_tolerance_tight_terms_are_needed():
    """The gate term (with its tu part and slope 1.1) and the up term are each
    needed: the grid has admissible perturbations that break the bound
    without them."""
    G, U, Ag, Au = _admissible_swiglu_grid()
    tol = oracle.tolerance

    def without_gate(g, u, ag, au, out):
        return oracle.swiglu_tolerance(g, u, ag, au, out) - 1.1 * tol(ag) * (np.abs(u) + tol(au))

    def slope_one(g, u, ag, au, out):
        return oracle.swiglu_tolerance(g, u, ag, au, out) - 0.1 * tol(ag) * (np.abs(u) + tol(au))

    def without_tu_in_gate(g, u, ag, au, out):
        return oracle.swiglu_tolerance(g, u, ag, au, out) - 1.1 * tol(ag) * tol(au)

    def without_up(g, u, ag, au, out):
        return oracle.swiglu_tolerance(g, u, ag, au, out) - np.abs(_silu(g)) * tol(au)

    for fn in (without_gate, slope_one, without_tu_in_gate, without_up):
        assert _worst_perturbed_error(G, U, Ag, Au, fn) > 1.0, fn.__name__


# ------------------------------------------------------ affine SwiGLU chain

def _exact_affine(bits, N, K, seed, name):
    """Codes with scale 2^-e and bias -c 2^-e: every w = (q - c) 2^-e is exact in bf16."""
    g = synth.rng(seed, name)
    codes = g.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    e = g.integers(6, 10, size=(N, K // 64))
    c = g.integers(0, 1 << bits, size=(N, K // 64))
    s = _bf16(2.0 ** -e)
    b = _bf16(-c * 2.0 ** -e)
    w = (codes.astype(np.float64) - np.repeat(c, 64, axis=1)) * 2.0 ** -np.repeat(e, 64, axis=1)
    return oracle.pack(codes, bits), s, b, _bf16(w)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_swiglu_affine_equals_dense_chain_on_exact_weights(bits):
    """Where every dequantized weight is exact in bf16, the affine SwiGLU is the
    dense SwiGLU (pinned against numpy) on those weights, bit for bit."""
    M, N, K = 3, 12, 256
    x = synth.normal_bf16((M, K), 1.0, 80, "sx/x")
    gq, gs, gb, Wg = _exact_affine(bits, N, K, 80, "sx/g%d" % bits)
    uq, us, ub, Wu = _exact_affine(bits, N, K, 80, "sx/u%d" % bits)
    r = oracle.swiglu_affine(x, (gq, gs, gb), (uq, us, ub), bits)
    d = oracle.swiglu_bf16(x, Wg, Wu)
    for k in ("out", "g", "u", "Ag", "Au"):
        assert np.array_equal(r[k], d[k]), k


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_swiglu_affine_streams_and_special_cases(bits):
    """g and u are the affine GEMVs of their own matrices (rational brute force on
    tiny exact inputs); zero codes and biases in either stream give out = 0."""
    M, N, K = 2, 3, 128
    g = synth.rng(79, "ss/%d" % bits)
    x = _bf16(g.integers(-4, 5, size=(M, K)))
    mats = []
    for t in ("g", "u"):
        words = synth.random_words((N, K * bits // 32), 79, "ss/%s%d" % (t, bits))
        s = _bf16(2.0 ** -g.integers(0, 4, size=(N, K // 64)))
        b = _bf16(g.integers(-3, 4, size=(N, K // 64)))
        mats.append((words, s, b))
    r = oracle.swiglu_affine(x, mats[0], mats[1], bits)
    for key, (words, s, b) in (("g", mats[0]), ("u", mats[1])):
        ref = brute.gemv_affine_exact(x.tolist(), words.tolist(), s.tolist(), b.tolist(), bits)
        for m in range(M):
            for n in range(N):
                assert Fraction(r[key][m, n]) == ref[m][n], key
    assert np.allclose(r["out"], _silu(r["g"]) * r["u"], rtol=1e-15, atol=0)
    zero = (np.zeros_like(mats[0][0]), mats[0][1], np.zeros_like(mats[0][2]))
    assert np.all(oracle.swiglu_affine(x, zero, mats[1], bits)["out"] == 0)
    assert np.all(oracle.swiglu_affine(x, mats[0], zero, bits)["out"] == 0)
