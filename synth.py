"""Seeded synthetic inputs for the tests and the benchmark.

This module draws random numbers and names workload shapes; it holds none of
the projection arithmetic (no packing, unpacking, dequantization or dot
products), so both the oracle side and the GPU side can take their inputs from
it without sharing any of the method.

Recipe (stated once here and in the design notes):
  * every tensor has its own stream:
    ``numpy.random.default_rng(SeedSequence([0, config_id, crc32(tensor_name)]))``;
  * "N(0, s)" is drawn in float64, cast to float32, then rounded to bf16 (RNE,
    by torch's CPU conversion); "U(a, b)" likewise;
  * activations x are drawn once at the largest M (32) and row-sliced, so a
    smaller M is a prefix of the same rows;
  * packed affine weights are drawn as uniform random uint32 words.  With a
    contiguous LSB-first bit stream and no padding bits, every bit of a word
    belongs to exactly one code, so uniform words are exactly codes drawn
    i.i.d. uniform on [0, 2^b - 1] and then packed.

bf16 tensors are carried as numpy uint16 bit patterns.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass

import numpy as np
import torch

SEED = 0
M_MAX = 32

# Config ids (also used as the second seed word).
CFG_DENSE_1536 = 0       # dense bf16 GEMV, M=1, K=N=1536
CFG_DENSE_DECODE = 1     # dense bf16 decode projections, hidden 1536
CFG_SWIGLU = 2           # fused up/gate SwiGLU, K=1536, N=4096
CFG_AFFINE4_08B = 3      # 4-bit group-64, ~0.8B-decoder shapes
CFG_MIXED_WIDTH = 4      # b-bit group-64, K=4096, N in {4096, 14336}

# (name, N, K) shape tables, M lists per config.
DENSE_DECODE_SHAPES = [
    ("q_proj", 1536, 1536), ("k_proj", 1536, 1536), ("v_proj", 1536, 1536),
    ("o_proj", 1536, 1536), ("up_proj", 4096, 1536), ("gate_proj", 4096, 1536),
    ("down_proj", 1536, 4096), ("lm_head", 100000, 1536),
]
DENSE_DECODE_M = [1, 2, 4, 8, 16, 32]
SWIGLU_SHAPE = (4096, 1536)
SWIGLU_M = [1, 2, 4, 8, 16, 32]
AFFINE4_SHAPES = [
    ("attn_1024", 1024, 1024), ("mlp_up_3584", 3584, 1024),
    ("mlp_down_3584", 1024, 3584), ("lm_head", 151936, 1024),
]
AFFINE4_M = [1, 4, 16]
MIXED_BITS = [2, 3, 4, 5, 6, 8]
MIXED_SHAPES = [("sq_4096", 4096, 4096), ("wide_14336", 14336, 4096)]
MIXED_M = [1, 8, 16]
# fused SwiGLU over affine gate and up matrices: the hidden-1536 MLP and the
# ~0.8B decoder MLP
SWIGLU_AFFINE_SHAPES = [("mlp_1536", 4096, 1536), ("mlp_1024", 3584, 1024)]
SWIGLU_AFFINE_BITS = [2, 3, 4, 5, 6, 8]
SWIGLU_AFFINE_M = [1, 4, 16, 32]
# affine prompt GEMM (M > 32): the mixed-width and ~0.8B-decoder weight
# shapes at prompt chunks of 128 rows (the prompt length of the pages'
# decode benchmark) and 512 rows
GEMM_BITS = [2, 3, 4, 5, 6, 7, 8]
GEMM_SHAPES = [("wide_14336", 14336, 4096), ("mlp_up_3584", 3584, 1024), ("mlp_down_3584", 1024, 3584)]
GEMM_M = [128, 512]
PROMPT_M_MAX = 1024


def rng(config_id: int, name: str) -> np.random.Generator:
    key = [SEED, int(config_id), zlib.crc32(name.encode())]
    return np.random.default_rng(np.random.SeedSequence(key))


def to_bf16_bits(a) -> np.ndarray:
    """float64/float32 array -> bf16 bit patterns (float32 cast, then RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(shape, std: float, config_id: int, name: str) -> np.ndarray:
    g = rng(config_id, name)
    out = np.empty(shape, np.uint16)
    flat = out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat.size, step):
        n = min(step, flat.size - i)
        flat[i:i + n] = to_bf16_bits(g.standard_normal(n) * std)
    return out


def uniform_bf16(shape, lo: float, hi: float, config_id: int, name: str) -> np.ndarray:
    g = rng(config_id, name)
    return to_bf16_bits(g.uniform(lo, hi, size=shape))


def random_words(shape, config_id: int, name: str) -> np.ndarray:
    g = rng(config_id, name)
    return g.integers(0, 1 << 32, size=shape, dtype=np.uint32)


def activations(config_id: int, K: int, M: int = M_MAX) -> np.ndarray:
    """x[M, K] ~ N(0, 1) in bf16; drawn at M_MAX rows and sliced."""
    return normal_bf16((M_MAX, K), 1.0, config_id, "x/K%d" % K)[:M].copy()


def prompt_activations(config_id: int, K: int, M: int) -> np.ndarray:
    """x[M, K] ~ N(0, 1) in bf16 for a prompt chunk; drawn at PROMPT_M_MAX
    rows and sliced, so a shorter chunk is a prefix of a longer one."""
    assert M <= PROMPT_M_MAX
    return normal_bf16((PROMPT_M_MAX, K), 1.0, config_id, "xprompt/K%d" % K)[:M].copy()


def dense_weight(config_id: int, name: str, N: int, K: int) -> np.ndarray:
    """W[N, K] ~ N(0, 0.02) in bf16."""
    return normal_bf16((N, K), 0.02, config_id, "W/%s/%dx%d" % (name, N, K))


@dataclass
class AffineWeight:
    bits: int
    words: np.ndarray    # uint32[N, K*bits/32]
    scales: np.ndarray   # bf16 bits [N, K/64]
    biases: np.ndarray   # bf16 bits [N, K/64]


def affine_weight(config_id: int, name: str, bits: int, N: int, K: int) -> AffineWeight:
    """Codes uniform on [0, 2^bits-1] (as uniform packed words), scale ~ U(0.001, 0.02),
    bias ~ U(-0.1, 0.1), one of each per group of 64 along K."""
    if K % 64:
        raise ValueError("K must be a multiple of 64")
    tag = "Q%d/%s/%dx%d" % (bits, name, N, K)
    return AffineWeight(
        bits=bits,
        words=random_words((N, K * bits // 32), config_id, tag + "/codes"),
        scales=uniform_bf16((N, K // 64), 0.001, 0.02, config_id, tag + "/scales"),
        biases=uniform_bf16((N, K // 64), -0.1, 0.1, config_id, tag + "/biases"),
    )


def small_int_bf16(shape, lo: int, hi: int, config_id: int, name: str) -> np.ndarray:
    """Small integers (exact in bf16), for cases where every sum is exact."""
    g = rng(config_id, name)
    return to_bf16_bits(g.integers(lo, hi + 1, size=shape).astype(np.float64))


def random_codes(shape, bits: int, config_id: int, name: str) -> np.ndarray:
    """Unpacked codes uniform on [0, 2^bits - 1] (for tests that pack explicitly)."""
    g = rng(config_id, name)
    return g.integers(0, 1 << bits, size=shape, dtype=np.uint8)
