"""Pure-Python brute force for tiny shapes (test infrastructure only).

A second, independent formulation of the oracle, used to cross-check
``oracle.c``:

  * bf16 values are decoded with ``struct`` instead of a bit copy;
  * a packed row is read as ONE Python integer (word i contributes
    ``word << 32*i``), and code k is ``(row >> b*k) & (2**b - 1)`` -- no word
    index or straddle case at all;
  * sums are exact rational arithmetic (``fractions.Fraction``), so on inputs
    whose products and partial sums are exactly representable the C oracle
    must agree bit for bit, and otherwise within its own rounding.

The affine form w = scale*q + bias and the LSB-first stream layout follow the
readings of TensorFold PR #849 ("2 to 8 bits in groups of 64", "every code
keeping its value, scale and bias") stated in the oracle's C source.
"""
from __future__ import annotations

import struct
from fractions import Fraction


def bf16_value(h: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(h) & 0xFFFF) << 16))[0]


def row_codes(words_row, bits: int, K: int):
    stream = 0
    for i, w in enumerate(words_row):
        stream |= int(w) << (32 * i)
    mask = (1 << bits) - 1
    return [(stream >> (bits * k)) & mask for k in range(K)]


def pack_row(codes, bits: int):
    stream = 0
    for k, c in enumerate(codes):
        stream |= (int(c) & ((1 << bits) - 1)) << (bits * k)
    nwords = len(codes) * bits // 32
    return [(stream >> (32 * i)) & 0xFFFFFFFF for i in range(nwords)]


def gemv_dense_exact(x, W):
    """x: list of M rows of bf16 bit patterns; W: N rows.  Returns Fractions."""
    M, N = len(x), len(W)
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        xv = [Fraction(bf16_value(h)) for h in x[m]]
        for n in range(N):
            out[m][n] = sum((Fraction(bf16_value(w)) * xv[k] for k, w in enumerate(W[n])),
                            Fraction(0))
    return out


def gemv_affine_exact(x, Wq, scales, biases, bits: int):
    M, N = len(x), len(Wq)
    K = len(x[0])
    out = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        q = row_codes(Wq[n], bits, K)
        w = [Fraction(bf16_value(scales[n][k // 64])) * q[k] + Fraction(bf16_value(biases[n][k // 64]))
             for k in range(K)]
        for m in range(M):
            out[m][n] = sum((w[k] * Fraction(bf16_value(x[m][k])) for k in range(K)), Fraction(0))
    return out
