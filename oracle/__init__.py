"""CPU oracle for the small-M decode projections (test infrastructure only).

This package is the plain, slow, double-precision definition of what the GPU
library computes.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the product path never does, and it shares no
code with the HIP library.

``oracle.c`` holds the arithmetic (C, fp64, OpenMP over output rows);
``brute.py`` is an independent pure-Python formulation used to cross-check it
on tiny shapes.  Functions here take and return numpy arrays; bf16 tensors are
carried as their uint16 bit patterns.

What each function follows (web pages, cited by title and section):
  * affine format -- TensorFold PR #849 "qwen3_5 cuda: mixed-width MLX
    checkpoints, 2 to 8 bits in groups of 64", "What this changes" and the
    module-width comment;
  * SwiGLU -- AstrAI decode_linear_benchmark.md, commit message (fused up/gate
    SwiGLU vs. the unfused chain);
  * argmax tie rule -- nvfp4-megamoe-kernel commit log, "Router: full kernel
    stack", Step 2 (lower index wins on equal scores);
  * tolerance metrics -- AstrAI decode_linear_benchmark.md, last paragraph
    (max abs error, relative L2 error, row-wise argmax parity).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

__all__ = [
    "build", "bf16_to_f64", "f32_to_bf16", "pack", "unpack", "gemv_bf16",
    "gemv_affine", "swiglu_bf16", "swiglu_affine", "argmax", "set_threads", "max_threads",
    "tolerance", "swiglu_tolerance",
]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def bind(path: str):
    """Load a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_bf16_vec.argtypes = [P, P, I64]
    lib.oracle_bf16_to_double_vec.argtypes = [P, P, I64]
    lib.oracle_pack.restype = ctypes.c_int
    lib.oracle_pack.argtypes = [ctypes.c_int, P, P, I64, I64]
    lib.oracle_unpack.restype = ctypes.c_int
    lib.oracle_unpack.argtypes = [ctypes.c_int, P, P, I64, I64]
    lib.oracle_gemv_bf16.argtypes = [P, P, P, P, I64, I64, I64]
    lib.oracle_gemv_affine.restype = ctypes.c_int
    lib.oracle_gemv_affine.argtypes = [ctypes.c_int, P, P, P, P, P, P, I64, I64, I64]
    lib.oracle_swiglu_bf16.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64]
    lib.oracle_swiglu_affine.restype = ctypes.c_int
    lib.oracle_swiglu_affine.argtypes = [ctypes.c_int, P, P, P, P, P, P, P, P, P, P, P, P, I64, I64, I64]
    lib.oracle_argmax.argtypes = [P, P, I64, I64]
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build(force=True)
        _lib = bind(_LIB_PATH)
        return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected dtype %s, got %s" % (np.dtype(dtype), a.dtype))
    return a


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def bf16_to_f64(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    _load().oracle_bf16_to_double_vec(_ptr(h), _ptr(out), h.size)
    return out


def f32_to_bf16(f) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 bit patterns."""
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    _load().oracle_f32_to_bf16_vec(_ptr(f), _ptr(out), f.size)
    return out


def pack(codes, bits: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    N, K = codes.shape
    if (K * bits) % 32:
        raise ValueError("K*bits must be a multiple of 32")
    words = np.empty((N, K * bits // 32), np.uint32)
    if _load().oracle_pack(bits, _ptr(codes), _ptr(words), N, K):
        raise ValueError("bad bits")
    return words


def unpack(words, bits: int, K: int) -> np.ndarray:
    words = _c(words, np.uint32)
    N = words.shape[0]
    if words.shape[1] * 32 != K * bits:
        raise ValueError("words shape does not match K and bits")
    codes = np.empty((N, K), np.uint8)
    if _load().oracle_unpack(bits, _ptr(words), _ptr(codes), N, K):
        raise ValueError("bad bits")
    return codes


def gemv_bf16(x, W):
    """Return (y, A): y = x W^T and A = |x| |W|^T elementwise-abs sums, fp64."""
    x = _c(x, np.uint16)
    W = _c(W, np.uint16)
    M, K = x.shape
    N = W.shape[0]
    assert W.shape[1] == K
    y = np.empty((M, N), np.float64)
    A = np.empty((M, N), np.float64)
    _load().oracle_gemv_bf16(_ptr(x), _ptr(W), _ptr(y), _ptr(A), M, N, K)
    return y, A


def gemv_affine(x, Wq, scales, biases, bits: int):
    x = _c(x, np.uint16)
    Wq = _c(Wq, np.uint32)
    scales = _c(scales, np.uint16)
    biases = _c(biases, np.uint16)
    M, K = x.shape
    N = Wq.shape[0]
    assert Wq.shape[1] * 32 == K * bits and scales.shape == (N, K // 64) == biases.shape
    y = np.empty((M, N), np.float64)
    A = np.empty((M, N), np.float64)
    if _load().oracle_gemv_affine(bits, _ptr(x), _ptr(Wq), _ptr(scales), _ptr(biases),
                                  _ptr(y), _ptr(A), M, N, K):
        raise ValueError("bad bits or K")
    return y, A


def swiglu_bf16(x, Wg, Wu):
    """Return dict(out, g, u, Ag, Au), all fp64 [M, N]."""
    x = _c(x, np.uint16)
    Wg = _c(Wg, np.uint16)
    Wu = _c(Wu, np.uint16)
    M, K = x.shape
    N = Wg.shape[0]
    assert Wg.shape == Wu.shape == (N, K)
    r = {k: np.empty((M, N), np.float64) for k in ("out", "g", "u", "Ag", "Au")}
    _load().oracle_swiglu_bf16(_ptr(x), _ptr(Wg), _ptr(Wu), _ptr(r["out"]), _ptr(r["g"]),
                               _ptr(r["u"]), _ptr(r["Ag"]), _ptr(r["Au"]), M, N, K)
    return r


def swiglu_affine(x, gate, up, bits: int):
    """Unfused SwiGLU over two affine b-bit matrices.

    gate, up: (words uint32[N, K*bits/32], scales bf16[N, K/64], biases
    bf16[N, K/64]) each.  Returns dict(out, g, u, Ag, Au), all fp64 [M, N].
    """
    x = _c(x, np.uint16)
    gw, gs, gb = (_c(gate[0], np.uint32), _c(gate[1], np.uint16), _c(gate[2], np.uint16))
    uw, us, ub = (_c(up[0], np.uint32), _c(up[1], np.uint16), _c(up[2], np.uint16))
    M, K = x.shape
    N = gw.shape[0]
    assert gw.shape == uw.shape == (N, K * bits // 32)
    assert gs.shape == gb.shape == us.shape == ub.shape == (N, K // 64)
    r = {k: np.empty((M, N), np.float64) for k in ("out", "g", "u", "Ag", "Au")}
    if _load().oracle_swiglu_affine(bits, _ptr(x), _ptr(gw), _ptr(gs), _ptr(gb), _ptr(uw), _ptr(us),
                                    _ptr(ub), _ptr(r["out"]), _ptr(r["g"]), _ptr(r["u"]),
                                    _ptr(r["Ag"]), _ptr(r["Au"]), M, N, K):
        raise ValueError("bad bits or K")
    return r


def argmax(y) -> np.ndarray:
    y = _c(y, np.float64)
    M, N = y.shape
    idx = np.empty(M, np.int64)
    _load().oracle_argmax(_ptr(y), _ptr(idx), M, N)
    return idx


def tolerance(A) -> np.ndarray:
    """Per-element bound on |y_gpu_fp32 - y_oracle|: 2e-3 * sum|w||x| + 1e-6."""
    return 2e-3 * np.asarray(A, np.float64) + 1e-6


def swiglu_tolerance(g, u, Ag, Au, out) -> np.ndarray:
    """Bound for the fused SwiGLU output, propagated from the GEMV bound.

    With tg, tu the GEMV bounds of g and u, |silu'| <= 1.1 and |silu| <= |g|:
      |d out| <= 1.1*tg*(|u| + tu) + |silu(g)|*tu + 8*2^-24*|out| + 1e-6,
    the last two terms covering fp32 exp and the final products.
    """
    tg = tolerance(Ag)
    tu = tolerance(Au)
    silu = g / (1.0 + np.exp(-g))
    return 1.1 * tg * (np.abs(u) + tu) + np.abs(silu) * tu + 8 * 2.0 ** -24 * np.abs(out) + 1e-6
