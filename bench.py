#!/usr/bin/env python3
"""Benchmark of the small-M decode projections on one MI355X.

Metric: microseconds per call and achieved HBM GB/s (and fraction of the
8 TB/s peak) for decode GEMV at M = 1..32.

Workload of one step (the default line): the dense bf16 decode projections of
a hidden-1536 model -- q/k/v/out 1536x1536, MLP up/gate 4096x1536, down
1536x4096, LM head 100000x1536 -- each at M = 1, 2, 4, 8, 16, 32: 48 GEMV
calls.  Weights and activations are seeded synthetic data (W ~ N(0, 0.02),
x ~ N(0, 1), bf16) resident in HBM before timing starts.  Every weight has
enough distinct copies (>= 1 GiB per shape, cycled) that no call reads a
cache-resident matrix.

value = algorithmic bytes of one step (2NK + 2MK + 2MN per call) / step time,
with the step replayed as a HIP graph (launch overhead excluded; the eager
rate is reported beside it).  Per call (the step's calls and the other
configurations: fused SwiGLU dense and affine, affine 4-bit decoder shapes,
mixed-width 2..8-bit, the LM heads' fused argmax, multi-projection q/k/v):
  * us: mean device time over a captured batch of >= 40 cold calls (the
    per-dispatch distribution, p10 / p50 / p90 over >= 200 dispatches of
    each call, comes from a rocprofv3 kernel trace of this script:
    --summarize-profile);
  * hot_us: the same call repeated on one weight copy (cache-resident: not
    an HBM number);
  * curve_frac: the time a plain read of the same bytes takes on the
    measured ceiling t0 + bytes/BW (aqg_stream_read over 0.5 MB .. 1 GB),
    over the call's time.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       [--no-extra] [--no-ceiling] [--copy-probe MIB] [--counter-call LABEL]
       [--summarize-profile DB] [--summarize-counters DIR LABEL ...]
       [--summarize-parity FILE]
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/call and achieved HBM GB/s (% of peak) for decode GEMV at M=1..32"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD published peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak (no sparsity)
ROTATION_BYTES = 1 << 30        # distinct copies per weight: at least this many bytes


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--calls", type=int, default=40, help="calls per per-call timing batch")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-extra", action="store_true", help="skip the other configurations")
    p.add_argument("--no-ceiling", action="store_true", help="skip the stream-read ceiling curve")
    p.add_argument("--copy-probe", type=float, default=0.0,
                   help="only run a device copy of this many MiB (counter calibration) and exit")
    p.add_argument("--counter-call", metavar="LABEL", default=None,
                   help="only run the call with this label (as in the profile summary, e.g. "
                        "'dense lm_head M=32 100000x1536') 8 times, for counter runs")
    p.add_argument("--summarize-profile", metavar="DB", default=None,
                   help="print a markdown summary of a rocprofv3 database (rocpd) taken with "
                        "--kernel-trace --marker-trace --kernel-rename of this script, then exit")
    p.add_argument("--summarize-counters", nargs="+", metavar="ARG", default=None,
                   help="DIR LABEL [LABEL ...]: from DIR/pmc_<COUNTER>/<name>_counter_collection.csv "
                        "(rocprofv3 --pmc runs of --counter-call LABEL named by the label's slug, and "
                        "of --copy-probe 256 named 'copy'), write profiles/counters.json for the current "
                        "kernel sources and print a markdown table, then exit")
    p.add_argument("--summarize-parity", metavar="FILE", default=None,
                   help="print a markdown table of the parity diagnostics a GPU test run wrote "
                        "(AQG_PARITY_LOG=FILE), then exit")
    return p.parse_args()


# ------------------------------------------------------------------ inputs

class Weights:
    """R distinct device copies of one weight set (dense W, or affine words/scales/biases)."""

    def __init__(self, tensors, nbytes, copies=None):
        import torch
        self.R = copies if copies else max(2, math.ceil(ROTATION_BYTES / nbytes))
        self.copies = [tuple(t.unsqueeze(0).repeat((self.R,) + (1,) * t.dim()) for t in tensors)]
        self.tensors = [tuple(c[i] for c in self.copies[0]) for i in range(self.R)]
        self.next = 0
        torch.cuda.synchronize()

    def take(self):
        t = self.tensors[self.next]
        self.next = (self.next + 1) % self.R
        return t


def dev_bf16(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u32(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).cuda()


def affine_bytes(N, K, bits):
    return N * K * bits // 8 + 4 * N * (K // 64)


class Call:
    """One call of a given shape and M, cycling over weight copies.

    kind: dense, affine, swiglu (dense), swiglu_affine, argmax (dense or
    affine by bits), multi (dense or affine by bits; N is the sum)."""

    def __init__(self, cfg, name, kind, M, N, K, x, weights, bits=0, parts=None):
        import torch
        import affine_quantized_gemv_amd as aqg
        self.cfg, self.name, self.kind, self.M, self.N, self.K, self.bits = cfg, name, kind, M, N, K, bits
        self.parts = parts
        self.x = x[:M]
        self.w = weights
        wb = affine_bytes(N, K, bits) if bits else 2 * N * K
        if kind in ("swiglu", "swiglu_affine"):
            wb *= 2
        out_b = 0 if kind == "argmax" else 2 * M * N
        self.bytes = wb + 2 * M * K + out_b
        self.flops = 2 * M * N * K * (2 if kind in ("swiglu", "swiglu_affine") else 1)
        if kind == "argmax":
            self.val = torch.empty(M, dtype=torch.float32, device="cuda")
            self.idx = torch.empty(M, dtype=torch.int32, device="cuda")
            kindcode = aqg.AQG_KIND_ARGMAX_DENSE + bits
            self.ws = torch.empty(aqg.workspace_bytes(kindcode, M, N, K), dtype=torch.uint8, device="cuda")
        elif kind == "multi":
            self.out = [torch.empty((M, n), dtype=torch.bfloat16, device="cuda") for n in parts]
        elif kind == "gemm":
            self.out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            self.ws = torch.empty(aqg.workspace_bytes(aqg.AQG_KIND_GEMM_AFFINE + bits, M, N, K),
                                  dtype=torch.uint8, device="cuda")
        else:
            self.out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def __call__(self):
        import affine_quantized_gemv_amd as aqg
        w = self.w.take()
        k = self.kind
        if k == "dense":
            aqg.gemv_bf16(self.x, w[0], out=self.out)
        elif k == "affine":
            aqg.gemv_affine(self.x, w[0], w[1], w[2], self.bits, out=self.out)
        elif k == "swiglu":
            aqg.swiglu_bf16(self.x, w[0], w[1], out=self.out)
        elif k == "swiglu_affine":
            aqg.swiglu_affine(self.x, w[0:3], w[3:6], self.bits, out=self.out)
        elif k == "argmax":
            if self.bits:
                aqg.gemv_affine_argmax(self.x, w[0], w[1], w[2], self.bits, out=(self.val, self.idx),
                                       workspace=self.ws)
            else:
                aqg.gemv_bf16_argmax(self.x, w[0], out=(self.val, self.idx), workspace=self.ws)
        elif k == "gemm":
            aqg.gemm_affine(self.x, w[0], w[1], w[2], self.bits, out=self.out, workspace=self.ws)
        elif k == "multi":
            if self.bits:
                mats = [tuple(w[3 * i:3 * i + 3]) for i in range(len(self.parts))]
                aqg.gemv_affine_multi(self.x, mats, self.bits, out=self.out)
            else:
                aqg.gemv_bf16_multi(self.x, list(w), out=self.out)

    def describe(self):
        d = {"config": self.cfg, "name": self.name, "kind": self.kind, "M": self.M, "N": self.N, "K": self.K,
             "bytes": self.bytes}
        if self.bits:
            d["bits"] = self.bits
        if self.parts:
            d["parts"] = self.parts
        return d


def dense_decode_calls():
    import synth
    cfg = synth.CFG_DENSE_DECODE
    xs = {}
    weights = {}
    for name, N, K in synth.DENSE_DECODE_SHAPES:
        if K not in xs:
            xs[K] = dev_bf16(synth.activations(cfg, K))
        W = dev_bf16(synth.dense_weight(cfg, name, N, K))
        weights[name] = Weights([W], 2 * N * K)
    calls = []
    for M in synth.DENSE_DECODE_M:
        for name, N, K in synth.DENSE_DECODE_SHAPES:
            calls.append(Call("dense_decode", name, "dense", M, N, K, xs[K], weights[name]))
    return calls


def other_calls():
    """Generator of the other configurations (weights freed as it goes)."""
    import synth
    # dense 1536x1536, M = 1
    x = dev_bf16(synth.activations(synth.CFG_DENSE_1536, 1536))
    W = Weights([dev_bf16(synth.dense_weight(synth.CFG_DENSE_1536, "W", 1536, 1536))], 2 * 1536 * 1536)
    yield Call("dense_1536_m1", "W", "dense", 1, 1536, 1536, x, W)
    # fused SwiGLU, dense
    N, K = synth.SWIGLU_SHAPE
    x = dev_bf16(synth.activations(synth.CFG_SWIGLU, K))
    WW = Weights([dev_bf16(synth.dense_weight(synth.CFG_SWIGLU, "gate", N, K)),
                  dev_bf16(synth.dense_weight(synth.CFG_SWIGLU, "up", N, K))], 4 * N * K)
    for M in synth.SWIGLU_M:
        yield Call("swiglu", "gate_up", "swiglu", M, N, K, x, WW)
    del WW

    def affine_w(cfg, name, bits, N, K):
        aw = synth.affine_weight(cfg, name, bits, N, K)
        return [dev_u32(aw.words), dev_bf16(aw.scales), dev_bf16(aw.biases)]

    for name, N, K in synth.AFFINE4_SHAPES:
        x = dev_bf16(synth.activations(synth.CFG_AFFINE4_08B, K))
        w = Weights(affine_w(synth.CFG_AFFINE4_08B, name, 4, N, K), affine_bytes(N, K, 4))
        for M in synth.AFFINE4_M:
            yield Call("affine4_decoder", name, "affine", M, N, K, x, w, bits=4)
        del w
    for bits in synth.MIXED_BITS:
        for name, N, K in synth.MIXED_SHAPES:
            x = dev_bf16(synth.activations(synth.CFG_MIXED_WIDTH, K))
            w = Weights(affine_w(synth.CFG_MIXED_WIDTH, name, bits, N, K), affine_bytes(N, K, bits))
            for M in synth.MIXED_M:
                yield Call("mixed_width", name, "affine", M, N, K, x, w, bits=bits)
            del w
    # fused SwiGLU over affine gate and up matrices
    for name, N, K in synth.SWIGLU_AFFINE_SHAPES:
        x = dev_bf16(synth.activations(synth.CFG_SWIGLU, K))
        for bits in synth.SWIGLU_AFFINE_BITS:
            w = Weights(affine_w(synth.CFG_SWIGLU, name + "/gate", bits, N, K) +
                        affine_w(synth.CFG_SWIGLU, name + "/up", bits, N, K), 2 * affine_bytes(N, K, bits))
            for M in synth.SWIGLU_AFFINE_M:
                yield Call("swiglu_affine", name, "swiglu_affine", M, N, K, x, w, bits=bits)
            del w
    # LM heads with the fused row argmax (logits never written)
    name, N, K = synth.DENSE_DECODE_SHAPES[7]
    x = dev_bf16(synth.activations(synth.CFG_DENSE_DECODE, K))
    w = Weights([dev_bf16(synth.dense_weight(synth.CFG_DENSE_DECODE, name, N, K))], 2 * N * K)
    for M in synth.DENSE_DECODE_M:
        yield Call("lm_head_argmax", name, "argmax", M, N, K, x, w)
    del w
    name, N, K = synth.AFFINE4_SHAPES[3]
    x = dev_bf16(synth.activations(synth.CFG_AFFINE4_08B, K))
    w = Weights(affine_w(synth.CFG_AFFINE4_08B, name, 4, N, K), affine_bytes(N, K, 4))
    for M in synth.AFFINE4_M:
        yield Call("lm_head_argmax", name, "argmax", M, N, K, x, w, bits=4)
    del w
    # q/k/v of one x in one launch
    K = 1536
    x = dev_bf16(synth.activations(synth.CFG_DENSE_DECODE, K))
    ws = [dev_bf16(synth.dense_weight(synth.CFG_DENSE_DECODE, n, 1536, K)) for n in ("q_proj", "k_proj", "v_proj")]
    w = Weights(ws, 3 * 2 * 1536 * K)
    for M in synth.DENSE_DECODE_M:
        yield Call("multi_qkv", "q_k_v", "multi", M, 3 * 1536, K, x, w, parts=[1536] * 3)
    del w
    K = 1024
    x = dev_bf16(synth.activations(synth.CFG_AFFINE4_08B, K))
    ws = []
    for n in ("attn_q", "attn_k", "attn_v"):
        ws += affine_w(synth.CFG_AFFINE4_08B, n, 4, 1024, K)
    w = Weights(ws, 3 * affine_bytes(1024, K, 4))
    for M in synth.AFFINE4_M:
        yield Call("multi_qkv", "attn_q_k_v", "multi", M, 3 * 1024, K, x, w, bits=4, parts=[1024] * 3)
    del w
    # prompt chunks through the affine prompt GEMM (M > 32)
    for name, N, K in synth.GEMM_SHAPES:
        x = dev_bf16(synth.prompt_activations(synth.CFG_MIXED_WIDTH, K, max(synth.GEMM_M)))
        for bits in (synth.GEMM_BITS if name == "wide_14336" else [4]):
            w = Weights(affine_w(synth.CFG_MIXED_WIDTH, name, bits, N, K), affine_bytes(N, K, bits))
            for M in synth.GEMM_M:
                yield Call("prompt_gemm", name, "gemm", M, N, K, x, w, bits=bits)
            del w


def make_call(label):
    """The call a label names (see label_of), with seeded synthetic inputs of
    its shape and two weight copies: for counter runs, which need only the
    kernel's own behaviour, not the full set of configurations."""
    import synth
    parts = label.split()
    bits = 0
    if parts[0].startswith("q") and parts[0][1:].isdigit():
        bits = int(parts[0][1:])
        parts = parts[1:]
    kind, name = parts[0], parts[1]
    M = int(parts[2].split("=")[1])
    N, K = (int(v) for v in parts[3].split("x"))
    cfg = 9
    x = dev_bf16(synth.normal_bf16((max(32, M), K), 1.0, cfg, "cc/x/%d" % K))

    def affine_w(tag, n):
        aw = synth.affine_weight(cfg, tag, bits, n, K)
        return [dev_u32(aw.words), dev_bf16(aw.scales), dev_bf16(aw.biases)]

    def dense_w(tag, n):
        return [dev_bf16(synth.normal_bf16((n, K), 0.02, cfg, "cc/W/%s/%dx%d" % (tag, n, K)))]
    parts_n = None
    if kind == "multi":
        parts_n = [N // 3] * 3
        ts = []
        for i, n in enumerate(parts_n):
            ts += affine_w("m%d" % i, n) if bits else dense_w("m%d" % i, n)
    elif kind in ("swiglu", "swiglu_affine"):
        ts = (affine_w("g", N) + affine_w("u", N)) if bits else (dense_w("g", N) + dense_w("u", N))
    else:
        ts = affine_w(name, N) if bits else dense_w(name, N)
    w = Weights(ts, 1, copies=2)
    return Call("counters", name, kind, M, N, K, x, w, bits=bits, parts=parts_n)


# ------------------------------------------------------------------ timing

def warm_clocks(g, s, e0, e1, ms=25.0):
    """Replay graph g for about `ms` of device time, untimed: the GPU's clocks
    settle after the host-side setup between calls (idle gaps in which they
    drop), so the timed replays that follow see the steady state a decode loop
    runs in rather than the first milliseconds after an idle period."""
    g.replay()
    e0.record(s)
    g.replay()
    e1.record(s)
    e1.synchronize()
    per = max(e0.elapsed_time(e1), 1e-3)
    for _ in range(min(500, int(ms / per))):
        g.replay()


def time_call(call, n, reps=5):
    """Average device time (us) per call.  At least n calls, and at least one
    call per weight copy (>= 1 GiB of distinct weights), are captured into a HIP
    graph; after ~25 ms of untimed replays (clocks settled) the graph is
    replayed `reps` times between HIP events on the launch stream, so host
    launch overhead is excluded and no weight is cache-hot."""
    import torch
    n = max(n, call.w.R)
    call()
    call()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            call()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    warm_clocks(g, s, e0, e1)
    torch.cuda.synchronize()
    MARKERS.push(label_of(call))
    e0.record(s)
    for _ in range(reps):
        g.replay()
    e1.record(s)
    e1.synchronize()
    MARKERS.pop()
    return e0.elapsed_time(e1) * 1e3 / (n * reps)


def time_call_hot(call, n=40, reps=3):
    """Mean device time (us) of the call repeated on one weight copy: the
    weights stay in the caches (MALL / L2) -- not an HBM number."""
    R, nxt = call.w.R, call.w.next
    call.w.R, call.w.next = 1, 0
    try:
        import torch
        call()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                call()
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        warm_clocks(g, s, e0, e1)
        torch.cuda.synchronize()
        e0.record(s)
        for _ in range(reps):
            g.replay()
        e1.record(s)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (n * reps)
    finally:
        call.w.R, call.w.next = R, nxt


def ceiling_curve():
    """Device time of a plain read (aqg_stream_read) of 0.5 MB .. 1 GB, cold
    (>= 1 GiB of distinct buffers per size), fitted as t = t0 + bytes / BW."""
    import torch
    import affine_quantized_gemv_amd as aqg
    lib = aqg.load()
    sink = torch.empty(1 << 16, dtype=torch.float32, device="cuda")
    points = []
    size = 1 << 19
    while size <= (1 << 30):
        copies = max(2, (1 << 30) // size)
        buf = torch.empty(copies * size, dtype=torch.uint8, device="cuda")
        buf.fill_(1)
        n = max(40, copies)

        def run(i, st):
            p = ctypes.c_void_p(buf.data_ptr() + (i % copies) * size)
            rc = lib.aqg_stream_read(p, size, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(st))
            if rc != 0:
                raise RuntimeError("aqg_stream_read: %d" % rc)
        run(0, torch.cuda.current_stream().cuda_stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st = torch.cuda.current_stream().cuda_stream
            for i in range(n):
                run(i, st)
        g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        MARKERS.push("read %d" % size)
        e0.record()
        for _ in range(3):
            g.replay()
        e1.record()
        e1.synchronize()
        MARKERS.pop()
        us = e0.elapsed_time(e1) * 1e3 / (3 * n)
        points.append((size, us))
        del g, buf
        size *= 2
    # least squares t = t0 + bytes / BW
    xs = [p[0] for p in points]
    ys = [p[1] for p in points]
    mx, my = statistics.fmean(xs), statistics.fmean(ys)
    slope = sum((a - mx) * (b - my) for a, b in zip(xs, ys)) / sum((a - mx) ** 2 for a in xs)
    t0 = my - slope * mx
    bw = 1e-3 / slope            # bytes/us -> GB/s
    return {"t0_us": round(t0, 3), "bw_GBps": round(bw, 1), "frac_of_peak": round(bw / HBM_PEAK_GBPS, 4),
            "points": [{"bytes": b, "us": round(u, 3), "GBps": round(b / u / 1e3, 1)} for b, u in points],
            "method": "aqg_stream_read (16-byte buffer loads, whole lines, 8 workgroups of 4 wavefronts per "
                      "CU) over >= 1 GiB of distinct buffers per size, HIP graph replay; least-squares fit"}


def measure(call, args, curve):
    us = time_call(call, args.calls)
    rec = dict(call.describe(), us=round(us, 3), GBps=round(call.bytes / us / 1e3, 1),
               frac=round(call.bytes / us / 1e3 / HBM_PEAK_GBPS, 4))
    if call.kind == "gemm":
        # a prompt GEMM is a dense contraction: also its matrix-core rate
        rec["TFLOPs"] = round(call.flops / us / 1e6, 1)
        rec["mfma_frac"] = round(call.flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4)
    rec["hot_us"] = round(time_call_hot(call), 3)
    if curve:
        rec["curve_frac"] = round((curve["t0_us"] + call.bytes / (curve["bw_GBps"] * 1e3)) / us, 4)
    return rec


class Markers:
    """roctx ranges around each timed region, so that a profile taken with
    `rocprofv3 --kernel-trace --marker-trace --kernel-rename --stats` lists every
    call's dispatches under that call's label.  A no-op when the roctx library of
    the ROCm profiler SDK is not present."""

    def __init__(self):
        self.lib = None
        for name in ("librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so"):
            for d in ("", "/opt/rocm/lib/"):
                try:
                    self.lib = ctypes.CDLL(d + name)
                    break
                except OSError:
                    continue
            if self.lib is not None:
                break
        if self.lib is not None:
            self.lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
            self.lib.roctxRangePushA.restype = ctypes.c_int
            self.lib.roctxRangePop.restype = ctypes.c_int

    def push(self, label):
        if self.lib is not None:
            self.lib.roctxRangePushA(label.encode())

    def pop(self):
        if self.lib is not None:
            self.lib.roctxRangePop()


MARKERS = None


def label_of(call):
    b = "q%d " % call.bits if call.bits else ""
    return "%s%s %s M=%d %dx%d" % (b, call.kind, call.name, call.M, call.N, call.K)


def slug(label):
    return "".join(ch if ch.isalnum() else "_" for ch in label)


def kernel_sources_hash():
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "affine_quantized_gemv_amd", "csrc", "*"))):
        if f.endswith((".hip", ".h")):
            h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_for(label):
    """HBM bytes per launch from committed counter runs, if taken on the current kernels."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    if d.get("sources_sha256_16") != kernel_sources_hash():
        return None
    t = d.get("calls", {}).get(label)
    return None if t is None else t.get("hbm_bytes_per_launch")


def copy_probe(mib):
    import torch
    n = int(mib * (1 << 20)) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n, "launches": 5}))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(steps_bytes):
    """The fp64 oracle on the host cores: whole steps of the dense decode
    workload (as many as fit in about 10 s, at least one); the 1536x1536
    M = 1 GEMV on one thread; and the 4-bit decoder shapes at M = 1."""
    import oracle
    import synth
    cfg = synth.CFG_DENSE_DECODE
    xs, Ws = {}, {}
    for name, N, K in synth.DENSE_DECODE_SHAPES:
        xs.setdefault(K, synth.activations(cfg, K))
        Ws[name] = synth.dense_weight(cfg, name, N, K)
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    nsteps = 0
    while True:
        for M in synth.DENSE_DECODE_M:
            for name, N, K in synth.DENSE_DECODE_SHAPES:
                oracle.gemv_bf16(xs[K][:M], Ws[name])
        nsteps += 1
        el = time.perf_counter() - t0
        if el >= 10.0 or nsteps >= 50:    # about 10 s of host work
            break
    gbps = steps_bytes * nsteps / el / 1e9
    out = {"value": round(gbps, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": "%d full step(s) of the dense decode workload (48 GEMVs, M=1..32) through the "
                     "fp64 C oracle, OpenMP over output rows; %.1f s wall" % (nsteps, el),
           "ms_per_step": round(el * 1e3 / nsteps, 1), "cpu_model": cpu_model(),
           "affinity_cpus": len(os.sched_getaffinity(0))}
    # config 1 on one thread (median of 3)
    x1 = synth.activations(synth.CFG_DENSE_1536, 1536, 1)
    W1 = synth.dense_weight(synth.CFG_DENSE_1536, "W", 1536, 1536)
    try:
        oracle.set_threads(1)
        ts = []
        for _ in range(3):
            a = time.perf_counter()
            oracle.gemv_bf16(x1, W1)
            ts.append(time.perf_counter() - a)
    finally:
        oracle.set_threads(threads)
    us1 = statistics.median(ts) * 1e6
    out["dense_1536_m1_1thread"] = {"us": round(us1, 1), "GBps": round(4724736 / us1 / 1e3, 3)}
    # 4-bit decoder shapes at M = 1, all threads (median of 3; 1 run for the LM head)
    aff = []
    for name, N, K in synth.AFFINE4_SHAPES:
        x = synth.activations(synth.CFG_AFFINE4_08B, K, 1)
        aw = synth.affine_weight(synth.CFG_AFFINE4_08B, name, 4, N, K)
        ts = []
        for _ in range(1 if N > 100000 else 3):
            a = time.perf_counter()
            oracle.gemv_affine(x, aw.words, aw.scales, aw.biases, 4)
            ts.append(time.perf_counter() - a)
        us = statistics.median(ts) * 1e6
        b = affine_bytes(N, K, 4) + 2 * K + 2 * N
        aff.append({"name": name, "N": N, "K": K, "M": 1, "us": round(us, 1), "GBps": round(b / us / 1e3, 3)})
    out["affine4_decoder_m1"] = aff
    return out


def label_bytes(label):
    """Algorithmic bytes of the call a region label names (see label_of)."""
    parts = label.split()
    bits = 0
    if parts[0].startswith("q") and parts[0][1:].isdigit():
        bits = int(parts[0][1:])
        parts = parts[1:]
    kind = parts[0]
    M = int(parts[2].split("=")[1])
    N, K = (int(v) for v in parts[3].split("x"))
    wb = affine_bytes(N, K, bits) if bits else 2 * N * K
    if kind in ("swiglu", "swiglu_affine"):
        wb *= 2
    return wb + 2 * M * K + (0 if kind == "argmax" else 2 * M * N)


def summarize_counters(d, labels):
    """Per-call counter table from rocprofv3 --pmc runs (one run per counter
    set): HBM bytes (FETCH_SIZE, WRITE_SIZE in KiB per dispatch, each scaled by
    what the same counter reads for a 256 MiB device copy), VALU and MFMA
    instructions, wave occupancy, busy and wait cycles, LDS bank conflicts."""
    import csv

    def rows(ctr, name):
        out = []
        for path in glob.glob(os.path.join(d, "pmc_*", name + "_counter_collection.csv")):
            with open(path) as f:
                out += [r for r in csv.DictReader(f) if r["Counter_Name"] == ctr]
        return out

    scale = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        copy = [float(r["Counter_Value"]) for r in rows(ctr, "copy") if "copyBuffer" in r["Kernel_Name"]]
        if copy:
            scale[ctr] = 256 * (1 << 20) / (statistics.median(copy) * 1024.0)
    doc = {"sources_sha256_16": kernel_sources_hash(),
           "method": "rocprofv3 --pmc runs of bench.py --counter-call LABEL (8 launches), one counter set per "
                     "run; FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by bytes per counter unit of a "
                     "256 MiB device copy (__amd_rocclr_copyBuffer); other counters per dispatch, mean",
           "calibration": {k: round(v, 5) for k, v in scale.items()}, "calls": {}}
    table = ["| call | kernel | HBM B / algorithmic | VALU inst / KiB | SALU inst / KiB | MFMA inst / KiB | "
             "VALU issue / CU busy cycle | waves / CU | busy % waiting | LDS bank conflicts / KiB |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for label in labels:
        name = slug(label)
        # a call may run several kernels (the row argmax: the GEMV, then the
        # reduction of its partials): bytes are summed over them, the other
        # counters are those of the kernel that moves the most bytes
        per = {}
        for ctr in ("FETCH_SIZE", "WRITE_SIZE", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_WAVES", "SQ_WAVE_CYCLES",
                    "SQ_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE",
                    "SQ_INSTS_SALU", "SQ_BUSY_CU_CYCLES",
                    "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES"):
            by_kernel = {}
            for r in rows(ctr, name):
                if "aqg" in r["Kernel_Name"]:
                    by_kernel.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
            for kname, v in by_kernel.items():
                per.setdefault(kname, {})[ctr] = statistics.fmean(v)
        kern = None
        vals = {}
        if per:
            main = max(per, key=lambda k: per[k].get("FETCH_SIZE", 0.0))
            kern = main.replace("void aqg::detail::", "").replace("(aqg::ProjArgs)", "")
            if len(per) > 1:
                kern += " (+ %d more)" % (len(per) - 1)
            vals = dict(per[main])
            for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
                if all(ctr in v for v in per.values()):
                    vals[ctr] = sum(v[ctr] for v in per.values())
        alg = label_bytes(label)
        kib = alg / 1024.0
        rec = {"kernel": kern, "algorithmic_bytes_per_launch": alg, "raw": {k: round(v, 1) for k, v in vals.items()}}
        if "FETCH_SIZE" in vals and "WRITE_SIZE" in vals and scale:
            hbm = vals["FETCH_SIZE"] * 1024 * scale["FETCH_SIZE"] + vals["WRITE_SIZE"] * 1024 * scale["WRITE_SIZE"]
            rec["hbm_bytes_per_launch"] = int(round(hbm))
            rec["traffic_over_algorithmic"] = round(hbm / alg, 4)
        doc["calls"][label] = rec

        def f(v, fmt="%.1f"):
            return fmt % v if v is not None else "-"
        # SQ_WAVE_CYCLES counts in units of 4 cycles; GRBM_GUI_ACTIVE is the
        # sum over the 8 XCDs of each one's busy cycles
        waves_cu = 4 * vals["SQ_WAVE_CYCLES"] / max(vals["GRBM_GUI_ACTIVE"] / 8, 1) / 256 \
            if "SQ_WAVE_CYCLES" in vals and "GRBM_GUI_ACTIVE" in vals else None
        wait = 100 * vals["SQ_WAIT_INST_ANY"] / vals["SQ_WAVE_CYCLES"] \
            if "SQ_WAIT_INST_ANY" in vals and vals.get("SQ_WAVE_CYCLES") else None
        # VALU instructions over the CUs' busy cycles (SQ_BUSY_CU_CYCLES, summed
        # over CUs): 1.0 is every SIMD issuing a wave64 VALU instruction every
        # 4 cycles, the vector unit's full rate
        vissue = vals["SQ_INSTS_VALU"] / vals["SQ_BUSY_CU_CYCLES"] \
            if "SQ_INSTS_VALU" in vals and vals.get("SQ_BUSY_CU_CYCLES") else None
        table.append("| %s | `%s` | %s | %s | %s | %s | %s | %s | %s | %s |" % (
            label, kern, f(rec.get("traffic_over_algorithmic"), "%.4f"),
            f(vals["SQ_INSTS_VALU"] / kib if "SQ_INSTS_VALU" in vals else None),
            f(vals["SQ_INSTS_SALU"] / kib if "SQ_INSTS_SALU" in vals else None),
            f(vals["SQ_INSTS_MFMA"] / kib if "SQ_INSTS_MFMA" in vals else None, "%.2f"),
            f(vissue, "%.2f"),
            f(waves_cu), f(wait), f(vals["SQ_LDS_BANK_CONFLICT"] / kib if "SQ_LDS_BANK_CONFLICT" in vals else None)))
    with open(os.path.join(ROOT, "profiles", "counters.json"), "w") as fh:
        json.dump(doc, fh, indent=1)
    print("\n".join(table))


def summarize_profile(db):
    """Per-call kernel durations from a rocprofv3 database of a run of this
    script: dispatches inside each call's timing region are grouped under the
    call's label (by --kernel-rename), with the kernel symbol they ran."""
    import sqlite3
    c = sqlite3.connect(db)
    rows = list(c.execute(
        "select region, name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
        "from kernels group by region, name order by sum(duration) desc"))
    durs = {}
    for region, name, dur in c.execute("select region, name, duration from kernels"):
        durs.setdefault((region, name), []).append(dur)

    def short(name):
        return name.replace("void aqg::detail::", "").replace("(aqg::ProjArgs)", "")

    def q(v, f):
        v = sorted(v)
        return v[min(len(v) - 1, int(round(f * (len(v) - 1))))]

    out = ["| call | kernel | n | avg us | p10 | p50 | p90 | GB/s (avg) | % peak |",
           "|---|---|---|---|---|---|---|---|---|"]
    for region, name, n, avg, mn, mx, _ in rows:
        if not region or region.startswith(("timed steps", "read ")):
            continue
        try:
            b = label_bytes(region)
        except (ValueError, IndexError):
            continue
        d = durs[(region, name)]
        gbps = b / avg
        out.append("| %s | `%s` | %d | %.2f | %.2f | %.2f | %.2f | %.0f | %.1f |" % (
            region, short(name), n, avg / 1e3, q(d, 0.1) / 1e3, q(d, 0.5) / 1e3, q(d, 0.9) / 1e3, gbps,
            100 * gbps / HBM_PEAK_GBPS))
    out.append("")
    out.append("Whole timed steps (graph replay and eager), by kernel symbol:")
    out.append("")
    out.append("| region | kernel | n | avg us | total ms |")
    out.append("|---|---|---|---|---|")
    for region, name, n, avg, mn, mx, tot in rows:
        if region and region.startswith("timed steps"):
            out.append("| %s | `%s` | %d | %.2f | %.3f |" % (region, short(name), n, avg / 1e3, tot / 1e6))
    print("\n".join(out))
    return 0


def summarize_parity(path):
    """Max abs error, relative L2 error and max(err / bound) per parity check,
    from the lines a GPU test run appended to `path` (AQG_PARITY_LOG)."""
    recs = [json.loads(l) for l in open(path) if l.strip()]
    by = {}
    for r in recs:
        by.setdefault(r["what"], r)
    out = ["| check | outputs | max abs err | rel L2 err | max err / bound |", "|---|---|---|---|---|"]
    for what in sorted(by):
        r = by[what]
        out.append("| %s | %d | %.3g | %.3g | %.4f |" % (what, r["n"], r["max_abs"], r["rel_l2"], r["max_err_over_bound"]))
    worst = max(recs, key=lambda r: r["max_err_over_bound"])
    out.append("")
    out.append("%d checks; the largest err/bound is %.4f (%s)." % (len(by), worst["max_err_over_bound"], worst["what"]))
    print("\n".join(out))
    return 0


# -------------------------------------------------------------------- main

def main():
    args = parse()
    if args.summarize_profile:
        return summarize_profile(args.summarize_profile)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters[0], args.summarize_counters[1:])
    if args.summarize_parity:
        return summarize_parity(args.summarize_parity)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the projections run on a single MI355X and this "
              "build has no multi-GPU path (requested --gpus %d)." % args.gpus, file=sys.stderr)
        return 2
    import torch
    import affine_quantized_gemv_amd as aqg
    aqg.load()
    torch.cuda.set_device(0)
    global MARKERS
    MARKERS = Markers()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return 0
    if args.counter_call:
        try:
            calls = [make_call(args.counter_call)]
        except (ValueError, IndexError):
            print("not a call label: %r" % args.counter_call, file=sys.stderr)
            return 2
        for _ in range(8):
            calls[0]()
        torch.cuda.synchronize()
        print(json.dumps({"counter_call": args.counter_call, "launches": 8, "bytes_per_launch": calls[0].bytes}))
        return 0

    t_setup = time.perf_counter()
    curve = None if args.no_ceiling else ceiling_curve()
    calls = dense_decode_calls()
    step_bytes = sum(c.bytes for c in calls)
    for c in calls:   # first use: arch check cached, kernels loaded
        c()
    torch.cuda.synchronize()

    # per-call timings (cold: each call of a batch reads a different copy)
    per_call = [measure(c, args, curve) for c in calls]

    def step():
        for c in calls:
            c()

    # HIP-graph capture of NG steps (each with its own weight copies)
    NG = 4
    graphs = []
    for _ in range(NG):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        graphs.append(g)
    torch.cuda.synchronize()

    for i in range(args.warmup):
        graphs[i % NG].replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    MARKERS.push("timed steps (graph replay)")
    e0.record(s)
    for i in range(args.steps):
        graphs[i % NG].replay()
    e1.record(s)
    torch.cuda.synchronize()
    MARKERS.pop()
    wall = time.perf_counter() - t0
    ms_graph = e0.elapsed_time(e1) / args.steps

    # eager steps for reference, and the host time per eager call
    for _ in range(max(1, args.warmup // 2)):
        step()
    torch.cuda.synchronize()
    MARKERS.push("timed steps (eager)")
    h0 = time.perf_counter()
    e0.record(s)
    for _ in range(args.steps):
        step()
    h1 = time.perf_counter()
    e1.record(s)
    torch.cuda.synchronize()
    MARKERS.pop()
    ms_eager = e0.elapsed_time(e1) / args.steps
    host_us_per_call = (h1 - h0) * 1e6 / (args.steps * len(calls))

    # dominant kernel: the call with the largest device time per step
    dom_i = max(range(len(calls)), key=lambda i: per_call[i]["us"])
    dom = calls[dom_i]
    us_dom = time_call(dom, max(args.calls, 100))
    achieved = dom.bytes / us_dom / 1e3
    traffic = traffic_for(label_of(dom))
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": "%s M=%d (%dx%d)" % (dom.name, dom.M, dom.N, dom.K),
                "bytes_per_launch": dom.bytes, "us_per_launch": round(us_dom, 3)}
    if curve:
        roofline["curve_frac"] = round((curve["t0_us"] + dom.bytes / (curve["bw_GBps"] * 1e3)) / us_dom, 4)
    del graphs, calls

    extra = []
    if not args.no_extra:
        for c in other_calls():
            c()
            extra.append(measure(c, args, curve))
            del c
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(step_bytes)

    value = step_bytes / (ms_graph * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_graph, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dense bf16 decode projections, hidden 1536: q/k/v/out 1536x1536, "
                               "up/gate 4096x1536, down 1536x4096, LM head 100000x1536, "
                               "each at M=1,2,4,8,16,32 (48 GEMVs per step), cold weights",
                   "mode": "HIP graph replay of whole steps", "step_bytes": step_bytes,
                   "frac_of_peak": round(value / HBM_PEAK_GBPS, 4)},
        "eager": {"ms_per_step": round(ms_eager, 4),
                  "GBps": round(step_bytes / (ms_eager * 1e-3) / 1e9, 1),
                  "host_us_per_call": round(host_us_per_call, 2)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ceiling": curve,
        "calls": per_call,
        "other_configs": extra,
        "device": torch.cuda.get_device_name(0),
        "setup_s": round(time.perf_counter() - t_setup, 1),
        "timed_wall_s": round(wall, 3),
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
