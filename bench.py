#!/usr/bin/env python3
"""Throughput of causal grouped-query FlashAttention, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gpu_model]
                    [--no-cpu-baseline] [--graph]

One step is one pass of the whole path over one batch of synthetic inputs already resident in
HBM: the forward (o, lse), then the two backward passes (dq + delta, then dk, dv), i.e. exactly
what ne_attn_fwd_ex followed by ne_attn_bwd_ex enqueue.  With RoPE the forward and the dq pass
each start with the pre-pass that rotates k (forward) or q and k (dq pass) into the workspace;
their per-call durations include it.  Untimed warm-up runs at least W steps and at least
half a second, so that the GPU clock has settled; the K timed steps are then
bracketed by device synchronisations; `value` is algorithmic TFLOP/s (causal FLOPs counted as
half of dense; forward 2 GEMMs, backward 5) over the wall-clock time per step.

Per-kernel durations come from HIP events recorded on the stream the kernels are launched on,
around every launch of the timed steps.  The `roofline` object describes the kernel with the
largest average duration; `cpu_baseline` times the fp64 oracle on the host cores on a bounded
sample of the same workload.  Prints one JSON line.

    python bench.py --workload block_gpu_model

times instead the attention sub-block x + attn(rmsnorm(x)) of the GPU model, forward and
backward (ne_attn_block_fwd, ne_attn_block_bwd), in TFLOP/s of its products.

    python bench.py --workload decode_gpu_model | decode_long

(or `--workload prefill_gpu_model | prefill_long`, a chunk of queries against a cache, in
TFLOP/s of its causal work) times instead one decode step against a key/value cache (ne_attn_decode: split kernel then
merge kernel): `value` is GB/s of the cache positions actually attended (plus q, o, lse) per
wall-clock step, and `roofline` compares the same bytes over the HIP-event time of the step
with the HBM peak.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn fwd+bwd TFLOP/s & % MFMA peak, B16 Hq12/Hkv4 T512 D64 causal"
# MI355X dense matrix-core peaks (256 CUs, 2.4 GHz), TFLOP/s.
MFMA_PEAK = {"f32": 157.3, "bf16": 2516.6}
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="gpu_model")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum host time spent on the oracle sample")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="run three plain device-to-device copies of this many MiB before the "
                        "steps (reference dispatches of known size for HBM counter calibration)")
    p.add_argument("--fused-bwd", action="store_true",
                   help="time the single-pass backward (ne_attn_bwd_fused: dq by fp32 atomics) "
                        "instead of the two passes")
    p.add_argument("--graph", action="store_true",
                   help="replay the step from a captured HIP graph instead of eager launches")
    return p.parse_args()


def kernel_flops(w):
    """Algorithmic FLOPs of each kernel launch: forward = QK^T + PV; the dK/dV pass holds four
    of the backward's five GEMMs (S, dP, dV, dK); the dQ pass holds dQ = dS K (its recomputed
    S and dP are not algorithmic work)."""
    f = w.flops_fwd()
    return {"fwd": f, "bwd_dq": 0.5 * f, "bwd_dkdv": 2.0 * f, "bwd_fused": 2.5 * f}


def kernel_bytes(w):
    """Algorithmic HBM bytes of each launch (inputs read once, outputs written once)."""
    elt = 2 if w.dtype == "bf16" else 4
    nq = w.B * w.Hq * w.T * w.D
    nk = w.B * w.Hkv * w.T * w.D
    nl = w.B * w.Hq * w.T
    return {"fwd": elt * (2 * nq + 2 * nk) + 4 * nl,                 # q,k,v -> o, lse
            "bwd_dq": elt * (4 * nq + 2 * nk) + 4 * 2 * nl,          # q,k,v,o,dO,lse -> dq, delta
            "bwd_dkdv": elt * (2 * nq + 4 * nk) + 4 * 2 * nl,        # q,k,v,dO,lse,delta -> dk,dv
            "bwd_fused": elt * (4 * nq + 4 * nk) + 4 * nl}           # q,k,v,o,dO,lse -> dq,dk,dv


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "causal_gqa_flashattention_attn_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def calibration_copies(torch, dev, mib: int):
    """Three device-to-device copies of `mib` MiB, each between synchronisations, so that byte
    counters can be scaled by what they read for a copy of known size (the median copy: a
    counter can credit part of a dispatch's traffic to its neighbour)."""
    src = torch.ones(mib * (1 << 18), dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
        torch.cuda.synchronize()
    del src, dst


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on the current
    kernel sources; None otherwise."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload, {}).get(kernel)
    if not e or e.get("source_digest") != source_digest():
        return None
    return e.get("bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name (first entry of /proc/cpuinfo), for the baseline's record."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x, min_seconds: float):
    """The fp64 oracle, as it stands, on batch elements 0, 1, 2, ... of the same inputs (one
    oracle forward + backward call per element, cycling) until `min_seconds` have passed."""
    import oracle
    per_b = {n: x[n].reshape((w.B, 1) + x[n].shape[1:]) for n in ("q", "k", "v", "dO")}
    one = w.with_(B=1)
    done = 0
    t0 = time.perf_counter()
    while True:
        b = done % w.B
        q, k, v, dO = (per_b[n][b] for n in ("q", "k", "v", "dO"))
        oracle.attn_fwd(q, k, v, causal=w.causal, rope_base=w.rope_base)
        oracle.attn_bwd(q, k, v, dO, causal=w.causal, rope_base=w.rope_base)
        done += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or done >= 100000:
            break
    return {"value": one.flops_fwd_bwd() * done / el / 1e12, "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "cpu": cpu_model(), "kind": "oracle",
            "sample": f"{done} single-batch-element fwd+bwd calls of {w.name} "
                      f"(B=1 Hq{w.Hq} Hkv{w.Hkv} T{w.T} D{w.D}), {el:.1f} s, fp64"}


def cpu_baseline_decode(w, x, min_seconds: float):
    """The fp64 oracle's decode step on batch rows 0, 1, 2, ... of the same inputs (cycling)
    until `min_seconds` have passed; GB/s of cached keys and values read."""
    import oracle
    done, nbytes = 0, 0
    t0 = time.perf_counter()
    while True:
        b = done % w.B
        sl = slice(b, b + 1)
        oracle.attn_decode(x["q"][sl], x["k"][sl], x["v"][sl], x["lens"][sl])
        nbytes += dataclasses.replace(w, B=1).cache_bytes(x["lens"][sl])
        done += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or done >= 100000:
            break
    return {"value": nbytes / el / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"{done} single-row decode steps of {w.name} (B=1 Hq{w.Hq} Hkv{w.Hkv} "
                      f"Tc{w.Tc} D{w.D}, lengths of the batch rows cycled), {el:.1f} s, fp64"}


GRAPH_STEPS = 10  # steps captured in one graph by the single-launch benches (--graph)
# Untimed warm-up lasts at least this long (and at least --warmup steps): the shader clock of an
# idle MI355X ramps up over tens of milliseconds of sustained load, so a few warm-up steps time
# the ramp rather than the sustained rate (the GPU model's step measured 0.367 ms over 20 steps
# after 10 warm-up steps, 0.335 ms once the clock had settled).
WARM_S = 0.5


def warm_up(torch, run, n: int):
    """Runs `run` n times, then keeps running it until WARM_S seconds have passed; returns the
    seconds spent."""
    t0 = time.perf_counter()
    for _ in range(n):
        run()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < WARM_S:
        for _ in range(8):
            run()
        torch.cuda.synchronize()
    return time.perf_counter() - t0


def timed_steps(torch, np, dev, a, make_step):
    """Runs a.warmup then a.steps steps of a single-launch workload (decode, prefill); returns
    (wall-clock ms per step, mean HIP-event ms per step).  Eager: one call per step, an event
    after each.  With --graph: GRAPH_STEPS steps captured in one HIP graph, replayed
    a.steps / GRAPH_STEPS times, so the host's per-call launch cost (larger than a short
    kernel) is out of the timed region; events then bracket each replay."""
    step = make_step(torch.cuda.current_stream(dev))
    if not a.graph:
        warm_up(torch, step, a.warmup)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
        gc.disable()
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(a.steps):
            step()
            ev[i + 1].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        gc.enable()
        return ((t1 - t0) * 1e3 / a.steps,
                float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(a.steps)])))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        make_step(s)()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = make_step(torch.cuda.current_stream())
        for _ in range(GRAPH_STEPS):
            st()
    reps = max(1, a.steps // GRAPH_STEPS)
    warm_up(torch, g.replay, max(1, a.warmup // GRAPH_STEPS))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    gc.disable()
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(reps):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    n = reps * GRAPH_STEPS
    return ((t1 - t0) * 1e3 / n,
            float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])) / GRAPH_STEPS)


def main_decode(a):
    """Decode step (`--workload decode_*`): GB/s of the key/value cache read per step."""
    import numpy as np
    import torch

    import causal_gqa_flashattention_attn_amd as ne
    from workloads import DECODE_WORKLOADS, make_decode_inputs

    w = DECODE_WORKLOADS[a.workload]
    x = make_decode_inputs(w, a.seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(dt).contiguous() for n in ("q", "k", "v"))
    lens = torch.from_numpy(x["lens"]).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
    code = ne.NE_BF16 if w.dtype == "bf16" else ne.NE_F32
    ws = torch.empty(ne.ne_attn_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Tc, w.D, code),
                     dtype=torch.uint8, device=dev)
    L = ne.lib()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def make_step(stream):
        args = (P(q), P(k), P(v), P(lens), P(o), P(lse), P(ws), w.B, w.Hq, w.Hkv, w.Tc, w.D, code,
                ctypes.c_void_p(stream.cuda_stream))

        def step():
            rc = L.ne_attn_decode(*args)
            if rc != ne.NE_OK:
                raise ne.NeAttnError(rc, "ne_attn_decode")
        return step

    if a.copy_mib > 0:
        calibration_copies(torch, dev, a.copy_mib)
    ms_per_step, ev_ms = timed_steps(torch, np, dev, a, make_step)
    nbytes = w.cache_bytes(x["lens"])
    line = {
        "metric": f"attn decode GB/s (cache bytes read per step), B{w.B} Hq{w.Hq}/Hkv{w.Hkv} "
                  f"Tc{w.Tc} D{w.D} {w.dtype}",
        "value": round(nbytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Tc": w.Tc,
                   "D": w.D, "cached_positions": int(np.sum(x["lens"])), "seed": a.seed,
                   "launch": "hip_graph" if a.graph else "eager"},
        "roofline": {"bound": "hbm", "kernel": "decode step",
                     "achieved": round(nbytes / (ev_ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(nbytes / (ev_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("decode", w.name),
                     "algorithmic_bytes_per_launch": nbytes},
        "cpu_baseline": None if a.no_cpu_baseline else cpu_baseline_decode(w, x, a.cpu_seconds),
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_prefill(w, x, min_seconds: float):
    """The fp64 oracle's prefill on batch elements 0, 1, 2, ... (cycling) for `min_seconds`."""
    import oracle
    done = 0
    t0 = time.perf_counter()
    while True:
        b = done % w.B
        sl = slice(b, b + 1)
        oracle.attn_prefill(x["q"][sl], x["k"][sl], x["v"][sl])
        done += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or done >= 100000:
            break
    return {"value": dataclasses.replace(w, B=1).flops() * done / el / 1e12, "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "cpu": cpu_model(), "kind": "oracle",
            "sample": f"{done} single-batch-element prefill chunks of {w.name} (B=1 Hq{w.Hq} "
                      f"Hkv{w.Hkv} Tq{w.Tq} Tk{w.Tk} D{w.D}), {el:.1f} s, fp64"}


def main_prefill(a):
    """Chunked prefill (`--workload prefill_*`): TFLOP/s of the causal work of the chunk."""
    import numpy as np
    import torch

    import causal_gqa_flashattention_attn_amd as ne
    from workloads import PREFILL_WORKLOADS, make_prefill_inputs

    w = PREFILL_WORKLOADS[a.workload]
    x = make_prefill_inputs(w, a.seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(dt).contiguous() for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Tq), dtype=torch.float32, device=dev)
    code = ne.NE_BF16 if w.dtype == "bf16" else ne.NE_F32
    L = ne.lib()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def make_step(stream):
        args = (P(q), P(k), P(v), P(o), P(lse), w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.D, code,
                ctypes.c_void_p(stream.cuda_stream))

        def step():
            rc = L.ne_attn_prefill(*args)
            if rc != ne.NE_OK:
                raise ne.NeAttnError(rc, "ne_attn_prefill")
        return step

    if a.copy_mib > 0:
        calibration_copies(torch, dev, a.copy_mib)
    ms_per_step, ev_ms = timed_steps(torch, np, dev, a, make_step)
    fl = w.flops()
    peak = MFMA_PEAK[w.dtype]
    line = {
        "metric": f"attn prefill TFLOP/s (causal work of the chunk), B{w.B} Hq{w.Hq}/Hkv{w.Hkv} "
                  f"Tq{w.Tq} Tk{w.Tk} D{w.D} {w.dtype}",
        "value": round(fl / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Tq": w.Tq, "Tk": w.Tk,
                   "D": w.D, "seed": a.seed, "launch": "hip_graph" if a.graph else "eager"},
        "roofline": {"bound": "mfma", "kernel": "forward with a query offset",
                     "achieved": round(fl / (ev_ms * 1e-3) / 1e12, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(fl / (ev_ms * 1e-3) / 1e12 / peak, 4),
                     "traffic": measured_traffic("prefill", w.name),
                     "algorithmic_flops_per_launch": fl},
        "cpu_baseline": None if a.no_cpu_baseline else cpu_baseline_prefill(w, x, a.cpu_seconds),
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_block(w, x, min_seconds: float):
    """The sub-block oracle (numpy fp64 products + the C attention oracle) on single batch
    elements of the same inputs, forward + backward, until `min_seconds` have passed."""
    import dataclasses

    import oracle
    from oracle.block import block_bwd
    one = dataclasses.replace(w, B=1)
    done, t0 = 0, time.perf_counter()
    while True:
        b = done % w.B
        block_bwd(x["x"][b:b + 1], x["gamma"], x["w_qkv"], x["w_o"], x["dy"][b:b + 1], w.Hq,
                  w.Hkv, w.D, w.eps, w.rope_base)  # runs the forward too
        done += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {"value": one.flops() * done / el / 1e12, "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "cpu": cpu_model(), "kind": "oracle",
            "sample": f"{done} single-batch-element sub-block forward + backward calls of "
                      f"{w.name} (B=1 T{w.T} Hq{w.Hq} Hkv{w.Hkv} D{w.D}), {el:.1f} s, fp64"}


def main_block(a):
    """The attention sub-block x + attn(rmsnorm(x)), forward + backward (`--workload block_*`):
    TFLOP/s of its products (three projection GEMMs per pass pair and the attention)."""
    import numpy as np
    import torch

    import causal_gqa_flashattention_attn_amd as ne
    from workloads import BLOCK_WORKLOADS, make_block_inputs

    w = BLOCK_WORKLOADS[a.workload]
    x = make_block_inputs(w, a.seed)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = {n: torch.from_numpy(v).to(dev).contiguous() for n, v in x.items()}
    y = torch.empty_like(t["x"])
    dx, dgamma = torch.empty_like(t["x"]), torch.empty_like(t["gamma"])
    dwq, dwo = torch.empty_like(t["w_qkv"]), torch.empty_like(t["w_o"])
    ws = torch.empty(ne.ne_attn_block_workspace_bytes(w.B, w.T, w.Hq, w.Hkv, w.D, w.rope_base),
                     dtype=torch.uint8, device=dev)
    L = ne.lib()
    P = lambda v: ctypes.c_void_p(v.data_ptr())  # noqa: E731
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    dims = (w.B, w.T, w.Hq, w.Hkv, w.D, ctypes.c_float(w.eps), ctypes.c_float(w.rope_base), st)
    fa = (P(t["x"]), P(t["gamma"]), P(t["w_qkv"]), P(t["w_o"]), P(y), P(ws)) + dims
    ba = (P(t["x"]), P(t["gamma"]), P(t["w_qkv"]), P(t["w_o"]), P(t["dy"]), P(dx), P(dgamma),
          P(dwq), P(dwo), P(ws)) + dims
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]

    def step(e=None):
        if e is not None:
            e[0].record()
        rc = L.ne_attn_block_fwd(*fa)
        if rc != ne.NE_OK:
            raise ne.NeAttnError(rc, "ne_attn_block_fwd")
        if e is not None:
            e[1].record()
        rc = L.ne_attn_block_bwd(*ba)
        if rc != ne.NE_OK:
            raise ne.NeAttnError(rc, "ne_attn_block_bwd")
        if e is not None:
            e[2].record()

    warm_up(torch, step, a.warmup)
    gc.disable()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    ms = (t1 - t0) * 1e3 / a.steps
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    fl = w.flops()
    line = {
        "metric": f"attention sub-block fwd+bwd TFLOP/s (rmsnorm, QKV and output projections, "
                  f"causal GQA attention with RoPE), B{w.B} T{w.T} Hq{w.Hq}/Hkv{w.Hkv} D{w.D} f32",
        "value": round(fl / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "rope_base": w.rope_base, "eps": w.eps, "seed": a.seed},
        "kernels": {"block_fwd": {"avg_ms": fwd_ms}, "block_bwd": {"avg_ms": bwd_ms}},
        "roofline": {"bound": "mfma", "kernel": "sub-block forward + backward",
                     "achieved": round(fl / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 3),
                     "peak": MFMA_PEAK["f32"], "unit": "TFLOP/s",
                     "frac": round(fl / ((fwd_ms + bwd_ms) * 1e-3) / 1e12 / MFMA_PEAK["f32"], 4),
                     "traffic": None, "algorithmic_flops_per_launch": fl},
        "cpu_baseline": None if a.no_cpu_baseline else cpu_baseline_block(w, x, a.cpu_seconds),
    }
    print(json.dumps(line), flush=True)


def main():
    a = parse()
    if a.workload.startswith("block"):
        world = int(os.environ.get("WORLD_SIZE", "1"))
        if a.gpus != 1 or world != 1:
            print("bench.py measures one GPU only (run with --gpus 1)", file=sys.stderr)
            sys.exit(2)
        return main_block(a)
    if a.workload.startswith("prefill"):
        world = int(os.environ.get("WORLD_SIZE", "1"))
        if a.gpus != 1 or world != 1:
            print("bench.py measures one GPU only (run with --gpus 1)", file=sys.stderr)
            sys.exit(2)
        return main_prefill(a)
    if a.workload.startswith("decode"):
        world = int(os.environ.get("WORLD_SIZE", "1"))
        if a.gpus != 1 or world != 1:
            print("bench.py measures one GPU only (run with --gpus 1)", file=sys.stderr)
            sys.exit(2)
        return main_decode(a)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py measures one GPU only: this attention path has no multi-GPU mode "
                  "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import causal_gqa_flashattention_attn_amd as ne
    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[a.workload]
    x = make_inputs(w, a.seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v, dO = (torch.from_numpy(x[n]).to(dev).to(dt).contiguous() for n in ("q", "k", "v", "dO"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.T), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    c, rb = w.causal, w.rope_base
    ws = ne.workspace(q, k, rb)
    names = ("fwd", "bwd_fused") if a.fused_bwd else ("fwd", "bwd_dq", "bwd_dkdv")
    if a.fused_bwd and w.dtype != "f32":
        print("--fused-bwd: float32 only", file=sys.stderr)
        sys.exit(2)

    # Arguments are marshalled once: a step is three calls straight into the C entry points
    # (which validate their arguments themselves), so the host stays well ahead of the GPU.
    L = ne.lib()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def bind(stream):
        dims = (w.B, w.Hq, w.Hkv, w.T, w.D, int(c),
                ne.NE_BF16 if w.dtype == "bf16" else ne.NE_F32, ctypes.c_float(rb),
                ctypes.c_void_p(stream.cuda_stream))
        if a.fused_bwd:
            return ((L.ne_attn_fwd_ex, (P(q), P(k), P(v), P(o), P(lse), P(ws)) + dims),
                    (L.ne_attn_bwd_fused, (P(q), P(k), P(v), P(o), P(lse), P(dO), P(dq), P(dk),
                                           P(dv), P(ws)) + dims))
        return ((L.ne_attn_fwd_ex, (P(q), P(k), P(v), P(o), P(lse), P(ws)) + dims),
                (L.ne_attn_bwd_dq_ex, (P(q), P(k), P(v), P(o), P(lse), P(dO), P(dq), P(ws)) + dims),
                (L.ne_attn_bwd_dkdv_ex, (P(q), P(k), P(v), P(lse), P(dO), P(ws), P(dk), P(dv))
                 + dims))

    calls = bind(torch.cuda.current_stream(dev))

    def step(ev=None, calls_=None):
        for j, (fn, args) in enumerate(calls_ or calls):
            if ev is not None:
                ev[j].record()
            rc = fn(*args)
            if rc != ne.NE_OK:
                raise ne.NeAttnError(rc, fn.__name__)
        if ev is not None:
            ev[len(names)].record()

    if a.copy_mib > 0:
        calibration_copies(torch, dev, a.copy_mib)

    graph = None
    if a.graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step(calls_=bind(s))
        torch.cuda.current_stream().wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(calls_=bind(torch.cuda.current_stream()))

    warm_up(torch, graph.replay if graph is not None else step, a.warmup)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
              for _ in range(a.steps)]
    torch.cuda.synchronize()
    gc.disable()  # no collector pause while the host enqueues the timed steps
    t0 = time.perf_counter()
    for i in range(a.steps):
        if graph is not None:
            events[i][0].record()
            graph.replay()
            events[i][len(names)].record()
        else:
            step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()

    ms_per_step = (t1 - t0) * 1e3 / a.steps
    tflops = w.flops_fwd_bwd() / (ms_per_step * 1e-3) / 1e12
    fl = kernel_flops(w)
    by = kernel_bytes(w)
    kern = {}
    if graph is None:
        for j, n in enumerate(names):
            ms = float(np.mean([e[j].elapsed_time(e[j + 1]) for e in events]))
            kern[n] = {"avg_ms": ms, "tflops": fl[n] / (ms * 1e-3) / 1e12,
                       "gbs": by[n] / (ms * 1e-3) / 1e9}
        dom = max(kern, key=lambda n: kern[n]["avg_ms"])
        ach = kern[dom]["tflops"]
        traffic = measured_traffic(dom, w.name)
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 3),
                "peak": MFMA_PEAK[w.dtype], "unit": "TFLOP/s",
                "frac": round(ach / MFMA_PEAK[w.dtype], 4), "traffic": traffic,
                "algorithmic_flops_per_launch": fl[dom],
                "algorithmic_bytes_per_launch": by[dom]}
    else:
        roof = None

    metric = METRIC if w.name == "gpu_model" else (
        f"attn fwd+bwd TFLOP/s & % MFMA peak, B{w.B} Hq{w.Hq}/Hkv{w.Hkv} T{w.T} D{w.D} "
        f"{'causal' if w.causal else 'non-causal'} {w.dtype}" + (" RoPE" if w.rope_base else ""))
    line = {
        "metric": metric,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "T": w.T, "D": w.D,
                   "causal": w.causal, "rope_base": w.rope_base, "seed": a.seed,
                   "launch": "hip_graph" if graph is not None else "eager",
                   "backward": "single-pass, dq by fp32 atomics" if a.fused_bwd
                   else "two passes, atomics-free"},
        "pct_mfma_peak": round(100 * tflops / MFMA_PEAK[w.dtype], 2),
        # algorithmic HBM bytes of the step (inputs read and outputs written once per pass)
        "step_gbs": round(w.bytes_fwd_bwd() / (ms_per_step * 1e-3) / 1e9, 2),
        "kernels": {n: {kk: round(vv, 4) for kk, vv in d.items()} for n, d in kern.items()},
        "roofline": roof,
        "cpu_baseline": None if a.no_cpu_baseline else cpu_baseline(w, x, a.cpu_seconds),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
