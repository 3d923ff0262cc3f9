#!/usr/bin/env python3
"""Benchmark of the chunkwise gated linear attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one forward pass of the whole hot path (every kernel the library launches for
the workload) over one batch of synthetic, seeded inputs that are already resident in HBM.
The step first runs untimed for a fixed SETTLE_S seconds of wall clock (the GPU's clocks
and the inputs' page-table entries reach their steady state: short runs otherwise time the
first launches about 10% slower), then W untimed warmup steps run; then exactly K steps are
timed between two device synchronisations.  A second pass of K steps, with HIP events
around each launch, gives the launch durations the roofline uses.  Two input sets alternate between steps so successive steps do not
re-read the same bytes from the 256 MB last-level cache.  Prints one JSON line.

Reported beside the throughput:
* ``roofline`` of the dominant kernel: the I/O floor (inputs and gates read once, fp32
  output and final state written once) over the mean launch duration of the timed region
  (one pair of HIP events on the launch stream around the K timed launches; the median and
  the minimum of a second, per-launch timed pass beside it), against the
  8 TB/s HBM peak.  Bytes moved beyond the floor (segment states, second reads) are ``extra_bytes``
  and not credited.  ``traffic`` is the measured HBM traffic of that kernel from rocprofv3
  counters (profiles/), or null when the counters were taken on other kernel source.
* ``tflops`` counts the flops as executed (a chunk of more than 64 tokens runs as 64-token
  chunks unless the tile-pair form is selected).
* ``cpu_baseline``: the fp64 oracle (the plain token recurrence) timed on this host's
  cores on the same workload, converted to the same unit.

``--workload`` takes the gated linear attention workloads (default: the B8 H16 L2048 D128
per-channel GLA), the delta-rule workloads (DeltaNet, Gated DeltaNet) and the mLSTM with
exponential input gate and normaliser; ``--backward`` and ``--decode`` time the backward pass
and the one-token step of a gated linear attention workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix peak
METRIC = "GLA fwd tokens/s and TFLOP/s (% bf16 MFMA peak), B8 H16 L2048 D128 bf16"
KERNEL_SRC = os.path.join(ROOT, "gated_linear_rnn_chunkwise_amd", "csrc", "gla_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


SETTLE_S = 0.25


def settle(torch, step, seconds: float = SETTLE_S) -> int:
    """Run ``step`` untimed, in batches of 16 launches, until ``seconds`` of wall clock have
    passed; returns the number of launches.  Nothing it runs is part of the timed region."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n


def algorithmic_flops(w, chunk=None) -> float:
    """Inter-chunk products (K^T V and Q S: 4 Dk Dv per head-token) plus the causal
    intra-chunk score and value products ((C+1)(Dk+Dv) per head-token on average) for chunks
    of ``chunk`` tokens (default: the workload's)."""
    c = w.chunk if chunk is None else chunk
    return float(w.B * w.H * w.L) * (4.0 * w.Dk * w.Dv + (c + 1) * (w.Dk + w.Dv))


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def timed_steps(torch, step, stream, K):
    """Exactly K steps between two device synchronisations: the wall clock gives the
    throughput and one pair of HIP events on the launch stream, around the same K launches,
    the mean launch duration of the roofline (any gap between launches counted in).  Then K
    more steps, each between its own pair of events, give the median and minimum launch
    (those event packets cost about 6 us per step, so they stay out of the timed region).
    Returns (ms per step, mean launch ms, per-launch ms)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return (t1 - t0) * 1e3 / K, e0.elapsed_time(e1) / K, [a.elapsed_time(b) for a, b in ev]

def quantiles(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2], xs[0]


def io_floor_bytes(w) -> float:
    """Bytes every implementation must move: q, k, v and the gates read once, the fp32
    output written once, the fp32 final state written once."""
    ib = 4 if w.dtype == "f32" else 2
    gate = {"channel": 4 * w.Dk, "head": 4, "head_const": 0, "none": 0}[w.gate] + (4 if w.input_gate else 0)
    per_ht = ib * (2 * w.Dk + w.Dv) + gate + 4 * w.Dv
    return float(w.B * w.H * w.L) * per_ht + (w.B * w.H * w.Dk * w.Dv * 4 if w.final_state else 0)


# Source files of each kernel family; the committed counters are valid while they hash the same.
KERNEL_SOURCES = {
    "gla": ("gla_kernels.hip", "gla_layout.h"),
    "delta": ("delta_kernels.hip", "gla_rows.h", "gla_delta.h"),
    "mlstm": ("mlstm_kernels.hip", "gla_rows.h", "gla_mlstm.h"),
}


def kernel_source_hash(family: str = "gla") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[family]:
        with open(os.path.join(os.path.dirname(KERNEL_SRC), name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, family: str = "gla"):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 counters, if
    they were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("kernel_source_sha256_16") != kernel_source_hash(family):
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(w, d, budget_s: float = 20.0) -> dict:
    """Time the fp64 oracle on a bounded sample of (batch, head) pairs of the workload."""
    import numpy as np

    import oracle

    BH = w.B * w.H
    # size the sample from a one-head probe so the timed part stays near budget_s
    def prep(nheads):
        sel = lambda t: None if t is None else t.reshape(-1, *t.shape[2:])[:nheads][None]
        la = d["log_alpha"]
        if w.gate == "head_const":
            la = torch_stack_heads(la, w.H, nheads)
            gate_in = la
        else:
            gate_in = sel(la)
        q, k, v = (oracle.oracle._f64(sel(d[x])) for x in "qkv")
        la64 = oracle.expand_gate(w.gate, gate_in, 1, nheads, w.L, w.Dk)
        li = oracle.oracle._f64(sel(d["log_ig"]))
        return q, k, v, la64, li

    def run(nheads, min_time=0.0):
        q, k, v, la64, li = prep(nheads)
        reps, t = 0, 0.0
        while True:
            t0 = time.perf_counter()
            oracle.recurrent(q, k, v, "channel", la64, li)
            t += time.perf_counter() - t0
            reps += 1
            if t >= min_time or reps >= 200:
                return t, reps

    threads = oracle.threads()
    probe_heads = min(BH, threads)
    t_probe, _ = run(probe_heads)  # one head per thread
    rounds = max(1, min(int(budget_s / max(t_probe, 1e-6)), math.ceil(BH / threads)))
    nheads = min(BH, rounds * threads)
    # the whole sample is repeated until about half the budget has run, so a workload the
    # host finishes quickly is still timed over seconds
    t, reps = run(nheads, min_time=0.5 * budget_s)
    head_tokens_per_s = reps * nheads * w.L / t
    tokens_per_s = head_tokens_per_s / w.H  # tokens = batch x sequence positions
    return {
        "value": tokens_per_s,
        "unit": "tokens/s",
        "cores": threads,
        "host_cpu": host_cpu_model(),
        "host_logical_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": "%d of %d (batch, head) pairs at full length %d, %d repetition(s), fp64 token recurrence, "
                  "%.2f s" % (nheads, BH, w.L, reps, t),
    }


def torch_stack_heads(la, H, nheads):
    import torch

    return torch.stack([la[i % H] for i in range(nheads)])


COPY_PROBE_BYTES = 256 << 20


def copy_probe(torch, steps):
    """A plain device-to-device copy of COPY_PROBE_BYTES per launch: reads and writes that
    many bytes of HBM.  Its FETCH_SIZE / WRITE_SIZE counter readings convert the counters'
    units into bytes for the kernels measured the same way."""
    dev = torch.device("cuda:0")
    n = COPY_PROBE_BYTES // 4
    src = [torch.rand(n, device=dev) for _ in range(2)]
    dst = torch.empty(n, device=dev)
    ms = []
    for i in range(max(steps, 1)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src[i & 1])
        e1.record()
        ms.append((e0, e1))
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ms)
    med = t[len(t) // 2]
    # a copy reads and writes COPY_PROBE_BYTES: the rate a plain device copy reaches on this HBM
    print(json.dumps({"copy_probe_bytes_per_launch": COPY_PROBE_BYTES, "launches": max(steps, 1),
                      "median_launch_ms": round(med, 5),
                      "copy_gbps_read_plus_write": round(2.0 * COPY_PROBE_BYTES / (med * 1e-3) / 1e9, 1)}), flush=True)


def decode_bench(args, torch, gla, gin, w, wname):
    """``--decode``: the recurrent step entry point (one token for every (batch, head), state
    updated in place) on the workload's head shape.  A step is one ``gla_step`` call; the
    roofline counts the state read and written once, the token's q, k, v and gates read and
    its fp32 output written."""
    import ctypes

    lib = gla.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, H, Dk, Dv = w.B, w.H, w.Dk, w.Dv
    sets = []
    for i in range(2):
        # one token of the workload's recipe (its L dimension dropped)
        d = gin.make_inputs(w.with_(L=1), seed=args.seed + i)
        sq = lambda t: None if t is None else (t if t.dim() == 1 else t.select(2, 0)).contiguous().to(dev)
        sets.append((sq(d["q"]), sq(d["k"]), sq(d["v"]), sq(d["log_alpha"]), sq(d["log_ig"])))
    state = [torch.zeros(B, H, Dk, Dv, dtype=torch.float32, device=dev) for _ in range(2)]
    out = torch.empty(B, H, Dv, dtype=torch.float32, device=dev)
    descs = [gla.make_step_desc(q, k, v, state[i], out, la, li) for i, (q, k, v, la, li) in enumerate(sets)]
    stream = torch.cuda.current_stream(dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def step(i):
        st = lib.gla_step(ctypes.byref(descs[i & 1]), sptr)
        if st != 0:
            raise gla.GlaError(st, "gla_step")

    settle(torch, step)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    # one event pair around the K back-to-back launches: a launch is a few microseconds, so
    # events around each launch would measure mostly themselves
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    mean_launch_ms = e0.elapsed_time(e1) / K
    ib = 4 if w.dtype == "f32" else 2
    gate = {"channel": 4 * Dk, "head": 4, "head_const": 0, "none": 0}[w.gate] + (4 if w.input_gate else 0)
    nbytes = float(B * H) * (2.0 * 4 * Dk * Dv + ib * (2 * Dk + Dv) + gate + 4 * Dv)
    achieved = nbytes / (mean_launch_ms * 1e-3) / 1e9
    rec = {
        "metric": "gla_step decode tokens/s (one token per sequence per step)",
        "value": B / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wname + "_decode", "B": B, "H": H, "Dk": Dk, "Dv": Dv, "gate": w.gate,
                   "input_gate": w.input_gate, "in_dtype": w.dtype, "state_dtype": "fp32"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "step kernel (K back-to-back launches between two events)",
                     "algorithmic_bytes_per_launch": nbytes, "mean_launch_ms": round(mean_launch_ms, 6)},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def backward_bench(args, torch, gla, gin, w, wname):
    """``--backward``: the gradients of one forward pass (``gla_bwd``) on the workload.  A
    step is one call; the roofline counts the bytes a fused backward must move: q, k, v, the
    gates and the fp32 output gradient read, the fp32 dq, dk, dv and gate gradients written,
    plus the final-state gradient read and the initial-state gradient written."""
    import ctypes

    lib = gla.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sets = []
    for i in range(2):
        d = gin.make_inputs(w, seed=args.seed + i)
        g = torch.Generator().manual_seed(args.seed + 100 + i)
        dout = torch.randn(w.B, w.H, w.L, w.Dv, generator=g)
        dfin = torch.randn(w.B, w.H, w.Dk, w.Dv, generator=g) * 0.1
        sets.append({k: (v.to(dev) if hasattr(v, "to") else v) for k, v in d.items() if v is not None})
        sets[-1]["dout"], sets[-1]["dfin"] = dout.to(dev), dfin.to(dev)
    f = dict(dtype=torch.float32, device=dev)
    B, H, L, Dk, Dv = w.B, w.H, w.L, w.Dk, w.Dv
    dq, dk, dv = torch.empty(B, H, L, Dk, **f), torch.empty(B, H, L, Dk, **f), torch.empty(B, H, L, Dv, **f)
    ds0 = torch.empty(B, H, Dk, Dv, **f)
    descs = []
    for st in sets:
        la, li = st.get("log_alpha"), st.get("log_ig")
        dla = torch.empty(la.shape, **f) if la is not None else None
        dli = torch.empty(li.shape, **f) if li is not None else None
        st["dla"], st["dli"] = dla, dli
        descs.append(gla.make_bwd_desc(st["q"], st["k"], st["v"], st["dout"], dq, dk, dv, la, li, None, st["dfin"],
                                       dla, dli, ds0))
    need = ctypes.c_size_t(0)
    rc = lib.gla_bwd_workspace_size(ctypes.byref(descs[0]), ctypes.byref(need))
    if rc != 0:
        raise gla.GlaError(rc, "gla_bwd_workspace_size")
    ws = torch.empty(need.value, dtype=torch.uint8, device=dev)
    for dsc in descs:
        dsc.workspace, dsc.workspace_bytes = ws.data_ptr(), need.value
    stream = torch.cuda.current_stream(dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def step(i):
        st = lib.gla_bwd(ctypes.byref(descs[i & 1]), sptr)
        if st != 0:
            raise gla.GlaError(st, "gla_bwd")

    settle(torch, step)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    mean_ms = e0.elapsed_time(e1) / K
    ib = 4 if w.dtype == "f32" else 2
    gate = {"channel": 4 * Dk, "head": 4, "head_const": 0, "none": 0}[w.gate] + (4 if w.input_gate else 0)
    per_ht = ib * (2 * Dk + Dv) + gate + 4 * Dv + 4 * (2 * Dk + Dv) + gate
    nbytes = float(B * H * L) * per_ht + 2.0 * B * H * Dk * Dv * 4
    achieved = nbytes / (mean_ms * 1e-3) / 1e9
    rec = {
        "metric": "GLA backward tokens/s (gradients of one forward pass)",
        "value": B * L / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wname + "_backward", "B": B, "H": H, "L": L, "Dk": Dk, "Dv": Dv, "gate": w.gate,
                   "input_gate": w.input_gate, "in_dtype": w.dtype,
                   "pass_operands": ("fp32" if w.dtype != "bf16" else
                                     "fp16 (scaled output gradient) and bf16; dv pass fp32 when Dk = 256"
                                     if w.gate == "channel" else "fp16 (scaled output gradient) and bf16")},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "whole backward (K calls between two events)",
                     "algorithmic_bytes_per_launch": nbytes, "mean_launch_ms": round(mean_ms, 5)},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def delta_flops(w) -> float:
    """Flops of the chunkwise delta rule per step (C = 64 as executed): per head-token,
    6 Dk Dv for the products with the state (Q S, W S, K^T U), (C+1)(2 Dk + 2 Dv) for the
    causal products inside a chunk (Q K^T, N K, N V, P U), (C-1) Dk for K K^T below the
    diagonal, and C^2 / 3 for the triangular inverse."""
    C = 64
    per = 6.0 * w.Dk * w.Dv + (C + 1) * (2 * w.Dk + 2 * w.Dv) + (C - 1) * w.Dk + C * C / 3.0
    return float(w.B * w.H * w.L) * per


def delta_io_floor_bytes(w) -> float:
    """q, k, v, beta and the gate read once, the fp32 output and final state written once."""
    ib = 4 if w.dtype == "f32" else 2
    gate = {"head": 4, "head_const": 0, "none": 0}[w.gate]
    per_ht = ib * (2 * w.Dk + w.Dv) + 4 + gate + 4 * w.Dv
    return float(w.B * w.H * w.L) * per_ht + (w.B * w.H * w.Dk * w.Dv * 4 if w.final_state else 0)


def mlstm_flops(w) -> float:
    """Algorithmic flops of the chunkwise mLSTM with normaliser per step (C = 64 as executed):
    per head-token 4 Dk Dv for the products with the state (q C', K^T V), (C+1)(Dk + Dv) for
    the causal products inside a chunk (Q K^T, P V) and 4 Dk for the normaliser (q . n',
    K^T weights).  The fp16 residual products the kernel adds for accuracy are not counted."""
    C = 64
    per = 4.0 * w.Dk * w.Dv + (C + 1) * (w.Dk + w.Dv) + 4.0 * w.Dk
    return float(w.B * w.H * w.L) * per


def mlstm_io_floor_bytes(w) -> float:
    """q, k, v and both gates read once, the fp32 output and the stabilised final state
    (C', n', m) written once."""
    ib = 4 if w.dtype == "f32" else 2
    per_ht = ib * (2 * w.Dk + w.Dv) + 8 + 4 * w.Dv
    return float(w.B * w.H * w.L) * per_ht + w.B * w.H * (w.Dk * w.Dv + w.Dk + 1) * 4


def rows_cpu_baseline(w, d, fn, what, budget_s: float = 20.0) -> dict:
    """An fp64 oracle on a bounded sample of whole (batch, head) slices: ``fn(d, n)`` runs it on
    the first ``n`` slices."""
    import oracle

    BH = w.B * w.H
    threads = oracle.threads()

    def run(n, min_time=0.0):
        reps, t = 0, 0.0
        while True:
            t0 = time.perf_counter()
            fn(d, n)
            t += time.perf_counter() - t0
            reps += 1
            if t >= min_time or reps >= 200:
                return t, reps

    probe = min(BH, threads)
    t_probe, _ = run(probe)
    rounds = max(1, min(int(budget_s / max(t_probe, 1e-6)), math.ceil(BH / threads)))
    n = min(BH, rounds * threads)
    t, reps = run(n, min_time=0.5 * budget_s)
    return {"value": reps * n * w.L / t / w.H, "unit": "tokens/s", "cores": threads, "host_cpu": host_cpu_model(),
            "host_logical_cpus": os.cpu_count(), "kind": "oracle",
            "sample": "%d of %d (batch, head) pairs at full length %d, %d repetition(s), fp64 %s, %.2f s"
                      % (n, BH, w.L, reps, what, t)}


def _first_slices(t, n):
    import oracle

    return None if t is None else oracle.oracle._f64(t.reshape(-1, *t.shape[2:])[:n][None])


def delta_oracle_sample(d, n):
    import oracle

    f = lambda key: _first_slices(d[key], n)
    oracle.delta_recurrent(f("q"), f("k"), f("v"), f("beta"), f("log_alpha"))


def mlstm_oracle_sample(d, n):
    import oracle

    f = lambda key: _first_slices(d[key], n)
    oracle.mlstm_recurrent(f("q"), f("k"), f("v"), f("log_f"), f("log_i"))


def rows_bench(args, torch, gla, gin, w, wname, rule):
    """A delta-rule or mLSTM workload: a step is one call of its entry point (one kernel
    launch) on resident inputs; roofline against the I/O floor."""
    import ctypes

    lib = gla.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("bench: generating inputs for", wname)
    host = [gin.make_inputs(w, seed=args.seed + i) for i in range(2)]
    sets = [{k: (v.to(dev) if hasattr(v, "to") else v) for k, v in h.items() if v is not None} for h in host]
    out = torch.empty((w.B, w.H, w.L, w.Dv), dtype=torch.float32, device=dev)
    fin = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)
    if rule == "delta":
        descs = [gla.make_delta_desc(s["q"], s["k"], s["v"], s["beta"], s.get("log_alpha"), None, out, fin, w.chunk)
                 for s in sets]
        entry, call = "gla_delta_fwd", lib.gla_delta_fwd
        io, flops = delta_io_floor_bytes(w), delta_flops(w)
        metric = "delta-rule fwd tokens/s (%s)" % ("Gated DeltaNet" if w.gate != "none" else "DeltaNet")
        flops_note = "flops of the chunkwise WY form as executed (C = 64)"
        kernel = "delta chunk kernel (the only launch of a step)"
        oracle_fn, oracle_what = delta_oracle_sample, "delta-rule recurrence"
    else:
        fin3 = (fin, torch.empty((w.B, w.H, w.Dk), dtype=torch.float32, device=dev),
                torch.empty((w.B, w.H), dtype=torch.float32, device=dev))
        descs = [gla.make_mlstm_desc(s["q"], s["k"], s["v"], s["log_f"], s["log_i"], None, out, fin3, w.chunk)
                 for s in sets]
        entry, call = "gla_mlstm_fwd", lib.gla_mlstm_fwd
        io, flops = mlstm_io_floor_bytes(w), mlstm_flops(w)
        metric = "mLSTM (exponential input gate, normaliser) fwd tokens/s"
        flops_note = "algorithmic flops of the chunkwise form (C = 64), residual products not counted"
        kernel = "mLSTM chunk kernel (the only launch of a step)"
        oracle_fn, oracle_what = mlstm_oracle_sample, "mLSTM recurrence"
    stream = torch.cuda.current_stream(dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def step(i):
        st = call(ctypes.byref(descs[i & 1]), sptr)
        if st != 0:
            raise gla.GlaError(st, entry)

    settle(torch, step)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    ms_per_step, mean_ms, launch_ms = timed_steps(torch, step, stream, K)
    med_ms, min_ms = quantiles(launch_ms)
    achieved = io / (mean_ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the fp64 oracle on host cores")
        cpu = rows_cpu_baseline(w, host[0], oracle_fn, oracle_what)
    rec = {
        "metric": metric,
        "value": w.B * w.L / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wname, "B": w.B, "H": w.H, "L": w.L, "Dk": w.Dk, "Dv": w.Dv, "chunk": w.chunk,
                   "rule": rule, "gate": w.gate, "in_dtype": w.dtype,
                   "matrix_operands": "fp16 from bf16" if w.dtype == "bf16" else "fp32", "accumulate": "fp32",
                   "out_dtype": "fp32", "workgroups": w.B * w.H * (w.Dv // 64)},
        "head_tokens_per_s": w.B * w.H * w.L / (ms_per_step * 1e-3),
        "tflops": round(flops / (mean_ms * 1e-3) / 1e12, 2),
        "tflops_counts": flops_note,
        "pct_bf16_mfma_peak": round(100.0 * flops / (mean_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(wname, rule),
                     "kernel": kernel,
                     "algorithmic_bytes_per_launch": io, "extra_bytes": 0.0,
                     "median_launch_ms": round(med_ms, 5), "min_launch_ms": round(min_ms, 5),
                     "mean_launch_ms": round(mean_ms, 5),
                     "frac_at_median_launch": round(io / (med_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "frac_at_min_launch": round(io / (min_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seg-chunks", type=int, default=0)
    ap.add_argument("--tile-pairs", action="store_true",
                    help="chunks > 64 tokens in the tile-pair (tiled large-chunk) form")
    ap.add_argument("--query-tiles", action="store_true",
                    help="the tile-pair form with one workgroup per query tile of a chunk against "
                         "materialised chunk-start states")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of known size (HBM counter calibration)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (gla_bwd) of the workload (scalar gates or none)")
    ap.add_argument("--decode", action="store_true",
                    help="time the recurrent step entry point (one token per sequence) on the workload's heads")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the forward pass here is single-GPU work (see the sharding "
              "design notes); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        copy_probe(torch, args.steps)
        return

    import gated_linear_rnn_chunkwise_amd as gla
    from gated_linear_rnn_chunkwise_amd import inputs as gin

    wname = args.workload or gin.HEADLINE
    if wname in gin.DELTA_WORKLOADS:
        rows_bench(args, torch, gla, gin, gin.DELTA_WORKLOADS[wname], wname, "delta")
        return
    if wname in gin.MLSTM_WORKLOADS:
        rows_bench(args, torch, gla, gin, gin.MLSTM_WORKLOADS[wname], wname, "mlstm")
        return
    w = gin.WORKLOADS[wname]
    if args.decode:
        decode_bench(args, torch, gla, gin, w, wname)
        return
    if args.backward:
        backward_bench(args, torch, gla, gin, w, wname)
        return
    lib = gla.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    log("bench: generating inputs for", wname)
    host = [gin.make_inputs(w, seed=args.seed + i) for i in range(2)]
    sets = []
    for h in host:
        sets.append({k: (v.to(dev) if hasattr(v, "to") else v) for k, v in h.items() if v is not None})
    out = torch.empty((w.B, w.H, w.L, w.Dv), dtype=torch.float32, device=dev)
    fin = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev) if w.final_state else None
    descs = []
    for s in sets:
        descs.append(gla.make_desc(s["q"], s["k"], s["v"], s.get("log_alpha"), s.get("log_ig"), None, out, fin,
                                   w.chunk, args.seg_chunks, tile_pairs=args.tile_pairs,
                                   query_tiles=args.query_tiles))
    plan = gla.plan(descs[0])
    ws = None
    if plan.workspace_bytes:
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
        for dsc in descs:
            dsc.workspace, dsc.workspace_bytes = ws.data_ptr(), plan.workspace_bytes
    stream = torch.cuda.current_stream(dev)
    sptr = __import__("ctypes").c_void_p(stream.cuda_stream)
    import ctypes

    def step(i):
        st = lib.gla_fwd_ex(ctypes.byref(descs[i & 1]), sptr)
        if st != 0:
            raise gla.GlaError(st, "gla_fwd_ex")

    settle(torch, step)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    ms_per_step, mean_launch_ms, launch_ms = timed_steps(torch, step, stream, K)

    med_launch_ms, min_launch_ms = quantiles(launch_ms)

    tokens = w.B * w.L
    value = tokens / (ms_per_step * 1e-3)
    # flops as executed: without tile pairs a chunk of more than 64 tokens is computed as
    # 64-token chunks (the state advances per tile), so its intra-chunk work is that of C = 64
    exec_chunk = w.chunk if plan.tile_pairs else min(w.chunk, 64)
    flops = algorithmic_flops(w, exec_chunk)
    io = io_floor_bytes(w)
    tflops = flops / (ms_per_step * 1e-3) / 1e12

    # Roofline against the I/O floor: q, k, v and the gates read once, the fp32 output and
    # final state written once.  With one segment the chunk-output kernel is the only launch
    # of a step, so the events around the call time exactly that kernel.  With several
    # segments the events time the whole step (segment-state, segment-scan and chunk-output
    # kernels); the bytes those extra kernels move beyond the floor (the segment-state
    # kernel's second read of k, v and gates, the boundary states written and read) are
    # reported as ``extra_bytes`` and not credited.
    ib = 4 if w.dtype == "f32" else 2
    gate = {"channel": 4 * w.Dk, "head": 4, "head_const": 0, "none": 0}[w.gate] + (4 if w.input_gate else 0)
    if plan.n_seg == 1:
        extra = 0.0
        scope = "chunk-output kernel (the only launch of a step)"
    else:
        # sub-segment states per slice: written by the state kernel and read by the scan, which
        # writes one state per segment boundary that the chunk-output kernel reads (once per
        # query tile with --query-tiles; the re-reads of earlier tiles are not counted)
        nss = plan.grid_state // max(1, w.B * w.H * plan.dv_tiles)
        qs = plan.tiles_per_chunk if plan.query_tiles else 1
        extra = float(w.B * w.H * w.L) * (plan.n_seg - 1) / plan.n_seg * (ib * (w.Dk + w.Dv) + gate) \
            + float(w.B * w.H) * (2 * nss + (1 + qs) * (plan.n_seg - 1)) * (w.Dk * w.Dv + w.Dk) * 4
        scope = "whole step (segment-state, segment-scan and chunk-output kernels)"
    achieved = io / (mean_launch_ms * 1e-3) / 1e9
    # the committed counters are those of the default form's single kernel
    default_form = plan.n_seg == 1 and not plan.tile_pairs and not plan.query_tiles
    traffic = measured_traffic(wname) if default_form else None
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": scope,
            "algorithmic_bytes_per_launch": io, "extra_bytes": extra,
            "median_launch_ms": round(med_launch_ms, 5), "min_launch_ms": round(min_launch_ms, 5),
            "mean_launch_ms": round(mean_launch_ms, 5),
            "frac_at_median_launch": round(io / (med_launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "frac_at_min_launch": round(io / (min_launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the fp64 oracle on host cores")
        cpu = cpu_baseline(w, host[0])

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wname, "B": w.B, "H": w.H, "L": w.L, "Dk": w.Dk, "Dv": w.Dv, "chunk": w.chunk,
                   "gate": w.gate, "input_gate": w.input_gate, "in_dtype": w.dtype,
                   "matrix_operands": "fp16 from bf16" if w.dtype == "bf16" else "fp32",
                   "accumulate": "fp32", "out_dtype": "fp32", "n_seg": plan.n_seg,
                   "tile_pairs": bool(plan.tile_pairs), "query_tiles": bool(plan.query_tiles),
                   "executed_chunk": exec_chunk,
                   "workgroups": plan.grid_out},
        "head_tokens_per_s": value * w.H,
        "tflops": round(tflops, 2),
        "tflops_counts": "flops executed: chunk %d%s" % (exec_chunk, "" if exec_chunk == w.chunk else
                                                       " (chunk %d runs as 64-token chunks)" % w.chunk),
        "pct_bf16_mfma_peak": round(100.0 * tflops / BF16_MFMA_PEAK_TFLOPS, 2),
        "io_floor_gbps": round(io / (ms_per_step * 1e-3) / 1e9, 1),
        "pct_hbm_peak_io_floor": round(100.0 * io / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
