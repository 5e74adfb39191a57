"""Helpers for the GPU parity tests: host<->device transfer of bf16 bit
patterns, canary-guarded output buffers and the parity checks themselves.

With AQG_PARITY_LOG=FILE every tolerance check appends its diagnostics (max
abs error, relative L2 error, max err/bound) to FILE as a JSON line;
`bench.py --summarize-parity FILE` tabulates them."""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle

DEV = "cuda:0"
CANARY_BF16 = 0x7F81          # a signalling-NaN pattern no kernel writes
CANARY_F32 = 0x7F812345
PAD = 2048                    # guard elements on each side of an output


def bf16_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def u32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(DEV)


class Guarded:
    """An [M, N] output tensor with canary words before and after it."""

    def __init__(self, M: int, N: int, dtype):
        self.M, self.N, self.dtype = M, N, dtype
        if dtype == torch.bfloat16:
            self.raw = torch.full((2 * PAD + M * N,), CANARY_BF16, dtype=torch.int16, device=DEV)
            self.out = self.raw[PAD:PAD + M * N].view(torch.bfloat16).view(M, N)
        else:
            self.raw = torch.full((2 * PAD + M * N,), CANARY_F32, dtype=torch.int32, device=DEV)
            self.out = self.raw[PAD:PAD + M * N].view(torch.float32).view(M, N)

    def check(self):
        raw = self.raw.cpu().numpy()
        c = CANARY_BF16 if self.dtype == torch.bfloat16 else CANARY_F32
        assert np.all(raw[:PAD] == np.array(c).astype(raw.dtype)), "write before the output"
        assert np.all(raw[PAD + self.M * self.N:] == np.array(c).astype(raw.dtype)), "write after the output"

    def numpy(self) -> np.ndarray:
        if self.dtype == torch.bfloat16:
            return self.out.view(torch.int16).cpu().numpy().view(np.uint16)
        return self.out.cpu().numpy()


def run_guarded(fn, M: int, N: int):
    """Call fn(out=...) for fp32 and bf16 outputs; check canaries and that the
    bf16 result is exactly the RNE rounding of the fp32 result.  Returns the
    fp32 result as float64."""
    g32 = Guarded(M, N, torch.float32)
    fn(out=g32.out)
    g16 = Guarded(M, N, torch.bfloat16)
    fn(out=g16.out)
    torch.cuda.synchronize()
    g32.check()
    g16.check()
    y32 = g32.numpy()
    assert np.array_equal(g16.numpy(), oracle.f32_to_bf16(y32)), "bf16 output != RNE(fp32 output)"
    return y32.astype(np.float64)


def assert_within(y: np.ndarray, ref: np.ndarray, bound: np.ndarray, what: str = ""):
    err = np.abs(y - ref)
    log = os.environ.get("AQG_PARITY_LOG")
    if log and err.size:
        rec = {"what": what, "n": int(err.size), "max_abs": float(err.max()),
               "rel_l2": float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300)),
               "max_err_over_bound": float((err / bound).max())}
        with open(log, "a") as f:
            f.write(json.dumps(rec) + "\n")
    bad = ~(err <= bound)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d of %d outside tolerance; first at %s: gpu=%r ref=%r bound=%r" % (
            what, int(bad.sum()), bad.size, tuple(i), y[tuple(i)], ref[tuple(i)], bound[tuple(i)]))


def metrics(y: np.ndarray, ref: np.ndarray, A: np.ndarray) -> dict:
    """Max abs error, relative L2 error and max err/bound (diagnostics)."""
    err = np.abs(y - ref)
    return {
        "max_abs": float(err.max()),
        "rel_l2": float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300)),
        "max_err_over_bound": float((err / oracle.tolerance(A)).max()),
    }


def check_argmax(y: np.ndarray, ref: np.ndarray, A: np.ndarray):
    """GPU argmax (fp32 outputs, lowest index on ties) must equal the oracle's,
    unless the oracle's top-2 gap is within the two entries' summed tolerance
    (then either index is a correct answer).  Returns the number of such rows."""
    gi = oracle.argmax(y)
    ri = oracle.argmax(ref)
    tol = oracle.tolerance(A)
    ambiguous = 0
    for m in range(y.shape[0]):
        if gi[m] == ri[m]:
            continue
        gap = ref[m, ri[m]] - ref[m, gi[m]]
        assert gap <= tol[m, ri[m]] + tol[m, gi[m]], \
            "row %d: gpu argmax %d, oracle %d, gap %g" % (m, gi[m], ri[m], gap)
        ambiguous += 1
    return ambiguous
