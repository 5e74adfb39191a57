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
rate is reported beside it).  Per-call timings come from HIP events around
batches of back-to-back calls on the launch stream.  The other configurations
(fused SwiGLU, affine 4-bit decoder shapes, mixed-width 2..8-bit) are
reported under "other_configs" with the same per-call method.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       [--no-extra] [--copy-probe MIB] [--counter-call LABEL]
       [--summarize-profile DB] [--summarize-counters DIR LABEL]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/call and achieved HBM GB/s (% of peak) for decode GEMV at M=1..32"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD published peak
ROTATION_BYTES = 1 << 30        # distinct copies per weight: at least this many bytes


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--calls", type=int, default=40, help="calls per per-call timing batch")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-extra", action="store_true", help="skip the other configurations")
    p.add_argument("--copy-probe", type=float, default=0.0,
                   help="only run a device copy of this many MiB (counter calibration) and exit")
    p.add_argument("--counter-call", metavar="LABEL", default=None,
                   help="only run the dense decode call with this label (as in the profile "
                        "summary, e.g. 'dense lm_head M=32 100000x1536') 8 times, for counter runs")
    p.add_argument("--summarize-profile", metavar="DB", default=None,
                   help="print a markdown summary of a rocprofv3 database (rocpd) taken with "
                        "--kernel-trace --marker-trace --kernel-rename of this script, then exit")
    p.add_argument("--summarize-counters", nargs=2, metavar=("DIR", "LABEL"), default=None,
                   help="from DIR/pmc_FETCH_SIZE and DIR/pmc_WRITE_SIZE (rocprofv3 --pmc CSV runs of "
                        "--counter-call LABEL named 'call' and of --copy-probe 256 named 'copy'), write "
                        "profiles/traffic.json for the current kernel sources and print a summary, then exit")
    return p.parse_args()


# ------------------------------------------------------------------ inputs

class Weights:
    """R distinct device copies of one weight set (dense W, or affine words/scales/biases)."""

    def __init__(self, tensors, nbytes):
        import torch
        self.R = max(2, math.ceil(ROTATION_BYTES / nbytes))
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


class Call:
    """One projection call of a given shape and M, cycling over weight copies."""

    def __init__(self, cfg, name, kind, M, N, K, x, weights, bits=0, out=None):
        import torch
        self.cfg, self.name, self.kind, self.M, self.N, self.K, self.bits = cfg, name, kind, M, N, K, bits
        self.x = x[:M]
        self.w = weights
        self.out = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        if kind == "dense":
            self.bytes = 2 * N * K + 2 * M * K + 2 * M * N
        elif kind == "swiglu":
            self.bytes = 4 * N * K + 2 * M * K + 2 * M * N
        else:
            self.bytes = N * K * bits // 8 + 4 * N * (K // 64) + 2 * M * K + 2 * M * N

    def __call__(self):
        import affine_quantized_gemv_amd as aqg
        w = self.w.take()
        if self.kind == "dense":
            aqg.gemv_bf16(self.x, w[0], out=self.out)
        elif self.kind == "swiglu":
            aqg.swiglu_bf16(self.x, w[0], w[1], out=self.out)
        else:
            aqg.gemv_affine(self.x, w[0], w[1], w[2], self.bits, out=self.out)

    def describe(self):
        d = {"config": self.cfg, "name": self.name, "kind": self.kind, "M": self.M, "N": self.N, "K": self.K,
             "bytes": self.bytes}
        if self.bits:
            d["bits"] = self.bits
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
    import synth
    calls = []
    # dense 1536x1536, M = 1
    x = dev_bf16(synth.activations(synth.CFG_DENSE_1536, 1536))
    W = Weights([dev_bf16(synth.dense_weight(synth.CFG_DENSE_1536, "W", 1536, 1536))], 2 * 1536 * 1536)
    calls.append(Call("dense_1536_m1", "W", "dense", 1, 1536, 1536, x, W))
    # fused SwiGLU
    N, K = synth.SWIGLU_SHAPE
    x = dev_bf16(synth.activations(synth.CFG_SWIGLU, K))
    WW = Weights([dev_bf16(synth.dense_weight(synth.CFG_SWIGLU, "gate", N, K)),
                  dev_bf16(synth.dense_weight(synth.CFG_SWIGLU, "up", N, K))], 4 * N * K)
    for M in synth.SWIGLU_M:
        calls.append(Call("swiglu", "gate_up", "swiglu", M, N, K, x, WW))

    def affine(cfg, tag, name, bits, N, K, Ms):
        aw = synth.affine_weight(cfg, name, bits, N, K)
        x = dev_bf16(synth.activations(cfg, K))
        w = Weights([dev_u32(aw.words), dev_bf16(aw.scales), dev_bf16(aw.biases)],
                    N * K * bits // 8 + 4 * N * (K // 64))
        for M in Ms:
            calls.append(Call(tag, name, "affine", M, N, K, x, w, bits=bits))

    for name, N, K in synth.AFFINE4_SHAPES:
        affine(synth.CFG_AFFINE4_08B, "affine4_decoder", name, 4, N, K, synth.AFFINE4_M)
    for bits in synth.MIXED_BITS:
        for name, N, K in synth.MIXED_SHAPES:
            affine(synth.CFG_MIXED_WIDTH, "mixed_width", name, bits, N, K, synth.MIXED_M)
    return calls


# ------------------------------------------------------------------ timing

def time_call(call, n, reps=3):
    """Average device time (us) per call.  At least n calls, and at least one
    call per weight copy (>= 1 GiB of distinct weights), are captured into a HIP
    graph; the graph is replayed `reps` times between HIP events on the launch
    stream, so host launch overhead is excluded and no weight is cache-hot."""
    import torch
    n = max(n, call.w.R)
    call()
    call()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            call()
    g.replay()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    MARKERS.push(label_of(call))
    e0.record(s)
    for _ in range(reps):
        g.replay()
    e1.record(s)
    e1.synchronize()
    MARKERS.pop()
    return e0.elapsed_time(e1) * 1e3 / (n * reps)


class Markers:
    """roctx ranges around each timed region, so that a profile taken with
    `rocprofv3 --kernel-trace --marker-trace --kernel-rename --stats` lists every
    call's dispatches under that call's label.  A no-op when the roctx library of
    the ROCm profiler SDK is not present."""

    def __init__(self):
        import ctypes
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


def kernel_sources_hash():
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "affine_quantized_gemv_amd", "csrc", "*"))):
        if f.endswith((".hip", ".h")):
            h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel_key):
    """HBM bytes per launch from committed counter runs, if taken on the current kernels."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    if d.get("sources_sha256_16") != kernel_sources_hash():
        return None
    t = d.get("kernels", {}).get(kernel_key)
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


def cpu_baseline(steps_bytes):
    """The fp64 oracle on the host cores over whole steps of the same workload
    (as many whole steps as fit in about 10 s, at least one)."""
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
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d full step(s) of the dense decode workload (48 GEMVs, M=1..32) through the "
                      "fp64 C oracle, OpenMP over output rows; %.1f s wall" % (nsteps, el),
            "ms_per_step": round(el * 1e3 / nsteps, 1)}


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
    if kind == "dense":
        return 2 * N * K + 2 * M * K + 2 * M * N
    if kind == "swiglu":
        return 4 * N * K + 2 * M * K + 2 * M * N
    return N * K * bits // 8 + 4 * N * (K // 64) + 2 * M * K + 2 * M * N


def summarize_counters(d, label):
    """HBM bytes per launch of one call from two counter runs (FETCH_SIZE and
    WRITE_SIZE, KiB per dispatch), each scaled by the bytes/KiB that the same
    counter reads for a device copy of known size."""
    import csv
    import statistics

    def rows(ctr, name):
        path = os.path.join(d, "pmc_" + ctr, name + "_counter_collection.csv")
        with open(path) as f:
            return [r for r in csv.DictReader(f) if r["Counter_Name"] == ctr]

    out = {}
    kernel = None
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        copy = [float(r["Counter_Value"]) for r in rows(ctr, "copy") if "copyBuffer" in r["Kernel_Name"]]
        call = rows(ctr, "call")
        if not copy or not call:
            raise SystemExit("no %s rows in %s" % (ctr, d))
        kernel = call[0]["Kernel_Name"]
        kib_copy = statistics.median(copy)
        nbytes = 256 * (1 << 20)
        scale = nbytes / (kib_copy * 1024.0)
        raw = statistics.mean(float(r["Counter_Value"]) for r in call)
        out[ctr] = {"kib_copy": kib_copy, "scale": scale, "kib_raw": raw, "bytes": raw * 1024.0 * scale,
                    "dispatches": len(call)}
    parts = label.split()
    M = int(parts[2].split("=")[1])
    N, K = (int(v) for v in parts[3].split("x"))
    alg = label_bytes(label)
    total = out["FETCH_SIZE"]["bytes"] + out["WRITE_SIZE"]["bytes"]
    sym = kernel.replace("void aqg::detail::", "").replace("(aqg::ProjArgs)", "")
    doc = {
        "sources_sha256_16": kernel_sources_hash(),
        "method": "rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE (separate runs), KiB per dispatch, each "
                  "scaled by bytes/counter of a 256 MiB device copy (__amd_rocclr_copyBuffer) in the same kind of run",
        "calibration": {"copy_bytes": 256 * (1 << 20),
                        "fetch_kib_per_copy": round(out["FETCH_SIZE"]["kib_copy"], 1),
                        "write_kib_per_copy": round(out["WRITE_SIZE"]["kib_copy"], 1),
                        "fetch_scale": round(out["FETCH_SIZE"]["scale"], 5),
                        "write_scale": round(out["WRITE_SIZE"]["scale"], 5)},
        "kernels": {"dense_M%d_N%d_K%d" % (M, N, K): {
            "call": label, "kernel": sym, "dispatches": out["FETCH_SIZE"]["dispatches"],
            "fetch_kib_raw": round(out["FETCH_SIZE"]["kib_raw"], 1),
            "write_kib_raw": round(out["WRITE_SIZE"]["kib_raw"], 1),
            "hbm_read_bytes_per_launch": int(round(out["FETCH_SIZE"]["bytes"])),
            "hbm_write_bytes_per_launch": int(round(out["WRITE_SIZE"]["bytes"])),
            "hbm_bytes_per_launch": int(round(total)),
            "algorithmic_bytes_per_launch": alg,
            "traffic_over_algorithmic": round(total / alg, 4)}},
    }
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(doc, f, indent=1)
    print("| counter | raw KiB / dispatch | copy KiB | scale | bytes / launch |")
    print("|---|---|---|---|---|")
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        o = out[ctr]
        print("| %s | %.1f | %.1f | %.5f | %d |" % (ctr, o["kib_raw"], o["kib_copy"], o["scale"], round(o["bytes"])))
    print("\n%s (`%s`): %d HBM bytes per launch against %d algorithmic (ratio %.4f); sources hash %s"
          % (label, sym, round(total), alg, total / alg, doc["sources_sha256_16"]))


def summarize_profile(db):
    """Per-call kernel durations from a rocprofv3 database of a run of this
    script: dispatches inside each call's timing region are grouped under the
    call's label (by --kernel-rename), with the kernel symbol they ran."""
    import sqlite3
    c = sqlite3.connect(db)
    rows = list(c.execute(
        "select region, name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
        "from kernels group by region, name order by sum(duration) desc"))
    def short(name):
        return name.replace("void aqg::detail::", "").replace("(aqg::ProjArgs)", "")

    out = ["| call | kernel | n | avg us | min | max | GB/s | % peak |",
           "|---|---|---|---|---|---|---|---|"]
    for region, name, n, avg, mn, mx, _ in rows:
        if not region or region.startswith("timed steps"):
            continue
        b = label_bytes(region)
        gbps = b / avg
        out.append("| %s | `%s` | %d | %.2f | %.1f | %.1f | %.0f | %.1f |" % (
            region, short(name), n, avg / 1e3, mn / 1e3, mx / 1e3, gbps, 100 * gbps / HBM_PEAK_GBPS))
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


# -------------------------------------------------------------------- main

def main():
    args = parse()
    if args.summarize_profile:
        return summarize_profile(args.summarize_profile)
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters)
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
        calls = [c for c in dense_decode_calls() if label_of(c) == args.counter_call]
        if not calls:
            calls = [c for c in other_calls() if label_of(c) == args.counter_call]
        if not calls:
            print("no call is labelled %r" % args.counter_call, file=sys.stderr)
            return 2
        for _ in range(8):
            calls[0]()
        torch.cuda.synchronize()
        print(json.dumps({"counter_call": args.counter_call, "launches": 8, "bytes_per_launch": calls[0].bytes}))
        return 0

    t_setup = time.perf_counter()
    calls = dense_decode_calls()
    step_bytes = sum(c.bytes for c in calls)
    for c in calls:   # first use: arch check cached, kernels loaded
        c()
    torch.cuda.synchronize()

    # per-call timings (cold: each call of a batch reads a different copy)
    per_call = []
    for c in calls:
        us = time_call(c, args.calls)
        per_call.append(dict(c.describe(), us=round(us, 3), GBps=round(c.bytes / us / 1e3, 1),
                             frac=round(c.bytes / us / 1e3 / HBM_PEAK_GBPS, 4)))

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

    # eager steps for reference
    for _ in range(max(1, args.warmup // 2)):
        step()
    torch.cuda.synchronize()
    MARKERS.push("timed steps (eager)")
    e0.record(s)
    for _ in range(args.steps):
        step()
    e1.record(s)
    torch.cuda.synchronize()
    MARKERS.pop()
    ms_eager = e0.elapsed_time(e1) / args.steps

    # dominant kernel: the call with the largest device time per step
    dom_i = max(range(len(calls)), key=lambda i: per_call[i]["us"])
    dom = calls[dom_i]
    us_dom = time_call(dom, max(args.calls, 100))
    achieved = dom.bytes / us_dom / 1e3
    key = "dense_M%d_N%d_K%d" % (dom.M, dom.N, dom.K)
    traffic = traffic_for(key)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": "%s M=%d (%dx%d)" % (dom.name, dom.M, dom.N, dom.K),
                "bytes_per_launch": dom.bytes, "us_per_launch": round(us_dom, 3)}

    extra = []
    if not args.no_extra:
        for c in other_calls():
            c()
            us = time_call(c, args.calls)
            extra.append(dict(c.describe(), us=round(us, 3), GBps=round(c.bytes / us / 1e3, 1),
                              frac=round(c.bytes / us / 1e3 / HBM_PEAK_GBPS, 4)))
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
                  "GBps": round(step_bytes / (ms_eager * 1e-3) / 1e9, 1)},
        "roofline": roofline,
        "cpu_baseline": cpu,
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
