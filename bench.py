#!/usr/bin/env python3
"""Benchmark of the E2-TTT chunk forward on one MI355X.

One step = one e2ttt_chunk_forward over the whole workload (all batch x head
units, all chunks: scan, forward at W_0, readout, backward, both scaled
aggregations, chunk-end states), inputs already resident in HBM.

Prints ONE JSON line:
  value         tokens/s = batch * seq_len / (time per step), N = 1 GPU
  roofline      dominant kernel: algorithmic flops per launch / its average
                launch duration (HIP events recorded at the start and end of
                every launch of that kernel by e2ttt_chunk_forward_timed, in
                a second timed pass of the same steps) against the published
                peak; traffic = HBM bytes per launch from the committed
                rocprofv3 counter summary when it matches the current code
  cpu_baseline  the fp64 oracle timed on this host's cores on a bounded
                sample of the same workload, scaled to tokens/s
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha256():
    """Hash of the HIP sources (kernels and host code): a committed traffic
    measurement only counts for the code it was taken on."""
    import hashlib
    h = hashlib.sha256()
    src = os.path.join(ROOT, "chunk_weight_update_amd", "csrc")
    for name in sorted(os.listdir(src)):
        if name.endswith((".hip", ".hpp", ".h")):
            with open(os.path.join(src, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (profiles/traffic_<kernel>_
    <workload>.txt, counters scaled by what they read for a copy kernel of
    known size), or None when there is none or it was taken on other code."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != source_sha256():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class HipEvents:
    """Raw hipEvent_t handles (needed to bracket launches inside the library)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.h.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        f = ctypes.c_float()
        rc = self.h.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(f.value)

    def destroy(self, evs):
        for e in evs:
            self.h.hipEventDestroy(ctypes.c_void_p(e))


def kernel_work(w, cls):
    """Algorithmic work of ALL launches of one kernel class in one step:
    (amount, unit).  Flops for the contractions, HBM bytes for the rest."""
    import chunk_weight_update_amd as cwu
    BH, L, d, h = w.B * w.H, w.L, w.d, w.h
    iob = 2 if w.io == 1 else 4
    if w.kind == 0:
        if cls == cwu.KERNEL_LINEAR_FWD:
            return 2.0 * 2 * L * d * d * BH, "flop"
        if cls == cwu.KERNEL_LINEAR_AGG:
            return 4.0 * L * d * d * BH, "flop"
    else:
        if cls == cwu.KERNEL_FWD13:
            return 8.0 * L * d * h * BH, "flop"
        if cls == cwu.KERNEL_FWD2:
            return 4.0 * L * d * h * BH, "flop"
        if cls == cwu.KERNEL_BWD:
            return 2.0 * L * d * h * BH, "flop"
        if cls == cwu.KERNEL_AGG:
            return 12.0 * L * d * h * BH, "flop"
        if cls == cwu.KERNEL_PHASE_A:   # forward of K and Q rows
            return 12.0 * L * d * h * BH, "flop"
        if cls == cwu.KERNEL_PHASE_B:   # backward (dZ) + both aggregations
            return 14.0 * L * d * h * BH, "flop"
        if cls == cwu.KERNEL_STATE:     # W0, M0 read; W_end, M_end written; bf16 shadow
            return 18.0 * 3 * d * h * BH * w.n_chunks, "byte"
        if cls == cwu.KERNEL_PREP:
            # K read + K^T written; W0 read + operand shadows written
            return 2.0 * BH * L * d * iob + BH * 3 * d * h * (4 + 4 * iob), "byte"
        if cls == cwu.KERNEL_PROLOGUE:  # scan + K^T staging + W0 shadow
            return (20.0 * BH * L + 2.0 * BH * L * d * iob
                    + BH * 3 * d * h * (4 + 4 * iob)), "byte"
    if cls == cwu.KERNEL_SCAN:
        return 20.0 * BH * L, "byte"  # eta, alpha, beta read; K^W, K^M written
    return 0.0, "byte"


def scan_microbench(reps=10):
    """The scalar-kernel scan alone at 2^26 token-heads (B64 x H16 x L65536,
    C = 2048: 32768 segments), through e2ttt_scalar_kernels, seeded synthetic
    scalars drawn as in the workloads.  The in-situ scan of the bench workload
    moves under 1 MB, so its rate says little about the kernel; this one is
    sized for HBM.  Algorithmic bytes: 20 per token-head."""
    import torch
    import chunk_weight_update_amd as cwu
    B, H, L, C = 64, 16, 65536, 2048
    g = torch.Generator(device="cuda").manual_seed(0)
    shp = (B, H, L)
    eta = 0.1 * torch.sigmoid(torch.randn(shp, generator=g, device="cuda"))
    alpha = 1.0 - 0.05 * torch.sigmoid(torch.randn(shp, generator=g, device="cuda"))
    beta = 0.9 * torch.sigmoid(torch.randn(shp, generator=g, device="cuda"))
    kw = torch.empty(shp, device="cuda")
    km = torch.empty(shp, device="cuda")
    cf = torch.empty((B, H, L // C, 3), device="cuda")
    prob = cwu.make_problem(cwu.LINEAR, B, H, L, 16, 0, C, cwu.F32, 0)
    for _ in range(2):
        cwu.scalar_kernels(prob, eta, alpha, beta, kw, km, cf)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        cwu.scalar_kernels(prob, eta, alpha, beta, kw, km, cf)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = 20.0 * B * H * L / (ms * 1e-3) / 1e9
    return {"label": "scan-only microbenchmark, 2^26 token-heads (not the bench workload)",
            "shape": {"batch": B, "heads": H, "seq_len": L, "chunk": C}, "ms": ms,
            "gbs": gbs, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS}


def decode_bench(w, reps=200):
    """The decode step (one token of every unit per call, e2ttt_decode_step)
    on the workload's B, H, d, h and io dtype, seeded synthetic inputs.
    Algorithmic bytes per step and unit: W0 read once, W and M read and
    written (5 P fp32), plus q, k, v, out.  Reported beside the main metric,
    not as it."""
    import torch
    import chunk_weight_update_amd as cwu
    B, H, d, h = w.B, w.H, w.d, w.h
    io = torch.bfloat16 if w.io == 1 else torch.float32
    P = d * d if w.kind == 0 else 3 * d * h
    g = torch.Generator(device="cuda").manual_seed(1)
    x = [torch.nn.functional.normalize(torch.randn((B, H, d), generator=g, device="cuda"),
                                       dim=-1).to(io) for _ in range(3)]
    eta = 0.1 * torch.sigmoid(torch.randn((B, H), generator=g, device="cuda"))
    alpha = 1.0 - 0.05 * torch.sigmoid(torch.randn((B, H), generator=g, device="cuda"))
    beta = 0.9 * torch.sigmoid(torch.randn((B, H), generator=g, device="cuda"))
    W0 = torch.randn((B, H, P), generator=g, device="cuda") * (1.0 / d) ** 0.5
    W, M = W0.clone(), torch.zeros_like(W0)
    out = torch.empty_like(x[0])
    prob = cwu.make_problem(w.kind, B, H, w.C, d, h, w.C, w.io, 0)
    ws = torch.empty(cwu.decode_workspace_bytes(prob), dtype=torch.uint8, device="cuda")
    for _ in range(20):
        cwu.decode_step(prob, *x, eta, alpha, beta, W0, W, M, out, False, ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        cwu.decode_step(prob, *x, eta, alpha, beta, W0, W, M, out, False, ws)
    e1.record()
    torch.cuda.synchronize()
    us_eager = e0.elapsed_time(e1) / reps * 1e3  # includes the host's per-call cost
    # Device time per step: 50 steps captured in a graph (the step makes no
    # allocation and no memset, so it captures), replayed.
    us = None
    try:
        steps = 50
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(steps):
                cwu.decode_step(prob, *x, eta, alpha, beta, W0, W, M, out, False, ws)
        graph.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(4):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / (4 * steps) * 1e3
    except Exception as exc:  # report the eager rate only
        log(f"bench: decode graph capture unavailable ({exc})")
    t = us if us is not None else us_eager
    nbytes = B * H * (20.0 * P + 4 * d * (2 if w.io == 1 else 4))
    gbs = nbytes / (t * 1e-6) / 1e9
    return {"label": "decode step, one token per (b,h) unit per call (not the main metric)",
            "shape": {"batch": B, "heads": H, "dim": d, "hidden": h},
            "us_per_step": t, "us_per_step_eager_calls": us_eager,
            "timing": "graph replay" if us is not None else "eager calls",
            "tokens_per_s": B * H / (t * 1e-6), "gbs": gbs, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS}


def backward_bench(with_oracle, reps=50):
    """The outer-loop backward (e2ttt_chunk_backward) on the linear workload's
    shape (d = 64, fp32; seeded synthetic inputs and upstream gradients),
    timed per call with events.  Algorithmic flops per token: the forward
    re-run (8 d^2) and the backward's matrix-vector and outer products (e, u, m,
    dq, three for dk, two for the state adjoint: 18 d^2).  At this size the
    call is latency-bound; the line reports its time beside the main metric,
    not as it.  With ``with_oracle``, the oracle's reverse mode is timed on the
    host for the same problem."""
    import numpy as np
    import torch
    import chunk_weight_update_amd as cwu
    from chunk_weight_update_amd.inputs import WORKLOADS, make_workload_inputs
    w = WORKLOADS["linear-d64-b1h1-l256-c64-fp32"]
    inp = make_workload_inputs(w, seed=0, m0_scale=0.01)
    rng = np.random.default_rng(1000)
    B, H, L, d = w.B, w.H, w.L, w.d
    up = [rng.standard_normal(s).astype(np.float32)
          for s in ((B, H, L, d), (B, H, d * d), (B, H, d * d))]
    names = ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")
    t = {n: torch.from_numpy(np.ascontiguousarray(inp[n], dtype=np.float32)).cuda() for n in names}
    dout, dW, dM = (torch.from_numpy(a).cuda() for a in up)
    g = {n: torch.empty_like(t[n]) for n in names}
    prob = cwu.make_problem(w.kind, B, H, L, d, 0, w.C, w.io, 0)
    ws = torch.empty(cwu.backward_workspace_bytes(prob), dtype=torch.uint8, device="cuda")

    def call():
        cwu.chunk_backward(prob, *[t[n] for n in names], dout, dW, dM,
                           *[g[n] for n in names], ws)
    for _ in range(10):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 26.0 * d * d * L * B * H
    out = {"label": "outer-loop backward of the chunk forward, linear learner "
                    "(not the main metric)",
           "config": w.describe(), "ms_per_call": ms, "tokens_per_s": B * L / (ms * 1e-3),
           "tflops_algorithmic": flops / (ms * 1e-3) / 1e12,
           "bound": "latency (16.8 MFLOP per call)"}
    if with_oracle:
        import oracle
        oracle.build(force=False)
        t0 = time.perf_counter()
        oracle.chunk_backward(w.kind, inp["q64"], inp["k64"], inp["v64"], inp["eta"],
                              inp["alpha"], inp["beta"], inp["W0"], inp["M0"], up[0], up[1],
                              up[2], w.C)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": B * L / dt, "unit": "tokens/s", "cores": 1,
                               "kind": "oracle", "sample": "the whole problem, one run "
                               "(fp64 reverse mode of the literal recurrence, one thread)"}
    return out


def backward_bench_swiglu(with_oracle, reps=10):
    """The outer-loop backward of the SwiGLU learner on the main workload's
    shape (B = 2, H = 4, L = 4096, C = 512, d = 128, h = 256) with fp32
    inputs (the backward's one supported io type), timed per call with events.
    Algorithmic flops per token: the forward re-run (26 d h) and the
    backward's products (64 d h: the learner's forward at the chunk-start
    weights for keys and queries, eight products with the chunk-end adjoints,
    the two W2 products of the error's adjoint, four for dk and dq, five
    token sums for the state adjoint).  With ``with_oracle``, the oracle's
    reverse mode is timed on the host on a sample: the first unit, first 1024
    tokens (two chunks)."""
    import numpy as np
    import torch
    import chunk_weight_update_amd as cwu
    from chunk_weight_update_amd.inputs import F32, SWIGLU, make_inputs
    B, H, L, d, h, C = 2, 4, 4096, 128, 256, 512
    P = 3 * d * h
    inp = make_inputs(SWIGLU, B, H, L, d, h, F32, seed=0, m0_scale=0.01)
    rng = np.random.default_rng(1000)
    up = [rng.standard_normal(s).astype(np.float32)
          for s in ((B, H, L, d), (B, H, P), (B, H, P))]
    names = ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")
    t = {n: torch.from_numpy(np.ascontiguousarray(inp[n], dtype=np.float32)).cuda() for n in names}
    dout, dW, dM = (torch.from_numpy(a).cuda() for a in up)
    g = {n: torch.empty_like(t[n]) for n in names}
    prob = cwu.make_problem(SWIGLU, B, H, L, d, h, C, F32, 0)
    ws = torch.empty(cwu.backward_workspace_bytes(prob), dtype=torch.uint8, device="cuda")

    def call():
        cwu.chunk_backward(prob, *[t[n] for n in names], dout, dW, dM,
                           *[g[n] for n in names], ws)
    for _ in range(3):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 90.0 * d * h * L * B * H
    # The same backward given the chunk-start states kept by the forward
    # (e2ttt_chunk_forward_states), which skips the forward re-run.
    nC = (L + C - 1) // C
    Wk = torch.empty((nC - 1, B, H, P), device="cuda")
    Mk = torch.empty((nC - 1, B, H, P), device="cuda")
    fws = torch.empty(cwu.workspace_bytes(prob), dtype=torch.uint8, device="cuda")
    o_, We_, Me_ = (torch.empty_like(t["q"]), torch.empty_like(t["W0"]), torch.empty_like(t["W0"]))
    cwu.chunk_forward_states(prob, *[t[n] for n in names], o_, We_, Me_, Wk, Mk, fws)

    def call_kept():
        cwu.chunk_backward(prob, *[t[n] for n in names], dout, dW, dM,
                           *[g[n] for n in names], ws, W_starts=Wk, M_starts=Mk)
    for _ in range(3):
        call_kept()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        call_kept()
    e1.record()
    torch.cuda.synchronize()
    ms_kept = e0.elapsed_time(e1) / reps
    out = {"label": "outer-loop backward of the chunk forward, SwiGLU learner, fp32 "
                    "(not the main metric)",
           "ms_per_call_with_kept_states": ms_kept,
           "config": {"workload": f"swiglu-d{d}h{h}-b{B}h{H}-l{L}-c{C}-fp32"},
           "ms_per_call": ms, "tokens_per_s": B * H * L / (ms * 1e-3),
           "tflops_algorithmic": flops / (ms * 1e-3) / 1e12,
           "frac_of_fp32_vector_peak": flops / (ms * 1e-3) / 157.3e12}
    if with_oracle:
        import oracle
        oracle.build(force=False)
        n = 1024
        sl = (slice(0, 1), slice(0, 1), slice(0, n))
        t0 = time.perf_counter()
        oracle.chunk_backward(SWIGLU, inp["q64"][sl], inp["k64"][sl], inp["v64"][sl],
                              inp["eta"][sl], inp["alpha"][sl], inp["beta"][sl],
                              inp["W0"][:1, :1], inp["M0"][:1, :1], up[0][sl], up[1][:1, :1],
                              up[2][:1, :1], C, hidden=h)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": n / dt, "unit": "tokens/s", "cores": 1,
                               "kind": "oracle", "sample": f"unit 0, tokens 0..{n - 1} "
                               "(fp64 reverse mode of the literal recurrence, one thread)"}
    return out


def algorithmic_flops(w):
    if w.kind == 0:
        return 8.0 * w.d * w.d * w.L * w.B * w.H
    return 26.0 * w.d * w.h * w.L * w.B * w.H


def cpu_baseline(w, inp, budget_s):
    """Time the fp64 oracle on a bounded sample: the first n (b, h) units of
    the workload over the full sequence, n chosen so that it runs for about
    budget_s; scaled to workload tokens/s."""
    import numpy as np

    import oracle
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    oracle.set_threads(cores)
    oracle.build(force=False)
    BH = w.B * w.H

    def run_units(n):
        sl = lambda a: a.reshape((BH,) + a.shape[2:])[:n][None]
        t0 = time.perf_counter()
        oracle.chunk_forward(w.kind, sl(inp["q64"]), sl(inp["k64"]), sl(inp["v64"]),
                             sl(inp["eta"]), sl(inp["alpha"]), sl(inp["beta"]), sl(inp["W0"]),
                             sl(inp["M0"]), w.C, w.h)
        return time.perf_counter() - t0

    t1 = run_units(1)
    n = int(max(1, min(BH, budget_s / max(t1, 1e-6))))
    tn = run_units(n) if n > 1 else t1
    t_full = tn * BH / n
    return {"value": w.B * w.L / t_full, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {BH} (batch, head) units x all {w.L} tokens "
                      f"({tn:.1f} s fp64, literal token-wise recurrence), scaled to the "
                      f"whole workload"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--flags", type=int, default=0, help="e2ttt_problem.flags")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="skip the per-kernel event pass (for profiler runs)")
    ap.add_argument("--no-scan-microbench", action="store_true",
                    help="skip the 2^26-token scan microbenchmark")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, run a plain device-to-device copy of this "
                         "many MiB 5 times (the known-size reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the (batch, head) units would shard across GPUs with no communication); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import chunk_weight_update_amd as cwu
    from chunk_weight_update_amd.inputs import BENCH_WORKLOAD, WORKLOADS, make_workload_inputs

    w = WORKLOADS[args.workload or BENCH_WORKLOAD]
    torch.cuda.set_device(0)
    log(f"bench: workload {w.name}")
    inp = make_workload_inputs(w, seed=0)
    dev = "cuda:0"
    t = {}
    for n in ("q", "k", "v"):
        a = np.ascontiguousarray(inp[n])
        t[n] = (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if w.io == 1
                else torch.from_numpy(a)).to(dev)
    for n in ("eta", "alpha", "beta", "W0", "M0"):
        t[n] = torch.from_numpy(inp[n]).to(dev)
    prob = cwu.make_problem(w.kind, w.B, w.H, w.L, w.d, w.h, w.C, w.io, 0, args.flags)
    run = cwu.ChunkForward(prob, device=dev)
    call_args = (t["q"], t["k"], t["v"], t["eta"], t["alpha"], t["beta"], t["W0"], t["M0"])

    for _ in range(args.warmup):
        run(*call_args)
    torch.cuda.synchronize()
    log(f"bench: warmup {args.warmup} done")

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        run(*call_args)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tokens = w.B * w.L
    value = tokens / (ms * 1e-3)
    log(f"bench: {args.steps} steps, {ms:.4f} ms/step, {value:.4g} tokens/s")

    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"bench: copy calibration, 5 x {nbytes} bytes device to device")
        del src, dst

    if args.no_kernel_timing:
        print(json.dumps({"metric": "TTT-layer fwd tokens/sec on 1 MI355X; MFMA util % of bf16 peak",
                          "value": value, "unit": "tokens/s", "ms_per_step": ms,
                          "config": w.describe()}), flush=True)
        return
    # Second timed pass: per-kernel-class launch durations with HIP events.
    ev = HipEvents()
    classes = ([cwu.KERNEL_SCAN, cwu.KERNEL_LINEAR_FWD, cwu.KERNEL_LINEAR_AGG] if w.kind == 0
               else [cwu.KERNEL_SCAN, cwu.KERNEL_PREP, cwu.KERNEL_FWD13, cwu.KERNEL_FWD2,
                     cwu.KERNEL_BWD, cwu.KERNEL_AGG, cwu.KERNEL_PHASE_A, cwu.KERNEL_PHASE_B,
                     cwu.KERNEL_STATE, cwu.KERNEL_PROLOGUE])
    per_step_launches = 2 * max(w.n_chunks, 2) + 2
    kernels = {}
    steps_k = max(1, min(args.steps, 10))
    for cls in classes:
        evs = ev.create(2 * per_step_launches * steps_k)
        per = []
        for s in range(steps_k):
            chunk = evs[2 * per_step_launches * s: 2 * per_step_launches * (s + 1)]
            _, nrec = cwu.chunk_forward_timed(prob, *call_args, run.out, run.W_end, run.M_end,
                                              run.workspace, cls, chunk)
            per.append((chunk, nrec))
        torch.cuda.synchronize()
        durs = []
        for chunk, nrec in per:
            durs += [ev.elapsed_ms(chunk[2 * j], chunk[2 * j + 1]) for j in range(nrec)]
        ev.destroy(evs)
        if not durs:
            continue
        launches_per_step = len(durs) / steps_k
        avg_ms = sum(durs) / len(durs)
        work, unit = kernel_work(w, cls)
        per_launch = work / launches_per_step
        rate = per_launch / (avg_ms * 1e-3)
        kernels[cwu.KERNEL_NAMES[cls]] = {
            "launches_per_step": launches_per_step, "avg_launch_ms": avg_ms,
            "ms_per_step": avg_ms * launches_per_step,
            ("tflops" if unit == "flop" else "gbs"): rate / (1e12 if unit == "flop" else 1e9),
            "work_per_launch": per_launch, "work_unit": unit}
        log(f"bench: kernel {cwu.KERNEL_NAMES[cls]}: {launches_per_step:g} launches/step, "
            f"avg {avg_ms * 1e3:.1f} us, {kernels[cwu.KERNEL_NAMES[cls]]}")

    peak_mfma = PEAK_BF16_TFLOPS if w.io == 1 else PEAK_FP32_TFLOPS
    dom_name = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dom_name]
    traffic = measured_traffic(dom_name, w.name)
    if dk["work_unit"] == "flop":
        roof = {"kernel": dom_name, "bound": "mfma", "achieved": dk["tflops"],
                "peak": peak_mfma, "unit": "TFLOP/s", "frac": dk["tflops"] / peak_mfma,
                "traffic": traffic}
    else:
        roof = {"kernel": dom_name, "bound": "hbm", "achieved": dk["gbs"], "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": dk["gbs"] / PEAK_HBM_GBS, "traffic": traffic}
    flops = algorithmic_flops(w)
    line = {
        "metric": "TTT-layer fwd tokens/sec on 1 MI355X; MFMA util % of bf16 peak",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.io == 1 else "fp32", "data": "synthetic",
        "config": w.describe() | {"flags": args.flags},
        "mfma_util_pct_of_bf16_peak": 100.0 * flops / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "tflops_algorithmic": flops / (ms * 1e-3) / 1e12,
        "roofline": roof,
        "kernels": kernels,
    }
    if not args.no_scan_microbench:
        line["decode"] = decode_bench(w)
        log(f"bench: decode step {line['decode']}")
        line["scan_microbench"] = scan_microbench()
        log(f"bench: scan microbenchmark {line['scan_microbench']}")
        line["backward"] = backward_bench(not args.no_cpu_baseline)
        line["backward_swiglu"] = backward_bench_swiglu(not args.no_cpu_baseline)
        log(f"bench: linear backward {line['backward']}")
    if not args.no_cpu_baseline:
        log("bench: timing the fp64 oracle on the host cores")
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
