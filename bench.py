#!/usr/bin/env python3
"""Benchmark of the E2-TTT chunk forward on one MI355X.

One step = one e2ttt_chunk_forward over the whole workload (all batch x head
units, all chunks: scan, forward at W_0, readout, backward, both scaled
aggregations, chunk-end states), inputs already resident in HBM.  The
default workload is the largest layer of the set: one head, SwiGLU fast
weight d = 768 / h = 1536 (3.5M state entries), 57,344 tokens in chunks of
8,192, bf16 q/k/v, fp32 states.

Prints ONE JSON line:
  value         tokens/s = batch * seq_len / (time per step), N = 1 GPU,
                over K back-to-back steps; per_call_ms gives the median,
                p10 and p90 of the single calls (an event between calls)
  roofline      dominant kernel: algorithmic flops per launch / its average
                launch duration (HIP events recorded at the start and end of
                every launch of that kernel by e2ttt_chunk_forward_timed, in
                a second pass of the same steps) against the published
                peak; traffic = HBM bytes per launch from the committed
                rocprofv3 counter summary when it matches the current code
  cpu_baseline  the fp64 oracle timed on this host's cores on a bounded
                sample of the same workload (the first chunk of the first
                units), scaled to tokens/s
  parity        rel_fro of out, W_end, M_end against that oracle sample
  system        CPU model, ROCm version, device name and compute units
  other_configs the other workloads' timings (shorter runs)
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


def decode_bench(B, H, d, h, C, io, n_tok=64):
    """The decode step (e2ttt_decode_step, one token of every unit per call,
    the state update amortised over the chunk) on seeded synthetic inputs:
    the per-token cost from a graph of n_tok calls inside a chunk (replayed,
    so the host's per-call cost is excluded), the chunk-end call (buffered
    tokens aggregated into the state) separately, and the amortised time per
    token = per-token + (chunk end - per-token) / C.  Algorithmic bytes per
    token and unit: the chunk-start weights read once (4 P) plus q, k, v,
    out."""
    import torch
    import chunk_weight_update_amd as cwu
    dt = torch.bfloat16 if io == 1 else torch.float32
    kind = cwu.SWIGLU
    P = 3 * d * h
    g = torch.Generator(device="cuda").manual_seed(1)
    x = [torch.nn.functional.normalize(torch.randn((B, H, d), generator=g, device="cuda"),
                                       dim=-1).to(dt) for _ in range(3)]
    eta = 0.1 * torch.sigmoid(torch.randn((B, H), generator=g, device="cuda"))
    alpha = 1.0 - 0.05 * torch.sigmoid(torch.randn((B, H), generator=g, device="cuda"))
    beta = 0.9 * torch.sigmoid(torch.randn((B, H), generator=g, device="cuda"))
    W = torch.randn((B, H, P), generator=g, device="cuda") * (1.0 / d) ** 0.5
    M = torch.zeros_like(W)
    out = torch.empty_like(x[0])
    prob = cwu.make_problem(kind, B, H, C, d, h, C, io, 0)
    ws = torch.empty(cwu.decode_workspace_bytes(prob), dtype=torch.uint8, device="cuda")

    def step(pos, end):
        cwu.decode_step(prob, *x, eta, alpha, beta, W, M, out, pos, end, ws)
    for p_ in range(8):
        step(p_, False)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for p_ in range(n_tok):
            step(p_, False)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(4):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us_tok = e0.elapsed_time(e1) / (4 * n_tok) * 1e3
    W0 = W.clone()
    reps = 3
    times = []
    for _ in range(reps):
        W.copy_(W0)
        M.zero_()
        torch.cuda.synchronize()
        e0.record()
        step(C - 1, True)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    us_end = sorted(times)[reps // 2]
    us_amort = us_tok + max(us_end - us_tok, 0.0) / C
    nbytes = B * H * (4.0 * P + 4 * d * (2 if io == 1 else 4))
    return {"shape": {"batch": B, "heads": H, "dim": d, "hidden": h, "chunk": C,
                      "io": "bf16" if io == 1 else "fp32"},
            "us_per_token_in_chunk": us_tok, "us_chunk_end_call": us_end,
            "us_per_token_amortised": us_amort, "tokens_per_s": B * H / (us_amort * 1e-6),
            "gbs_per_token": nbytes / (us_tok * 1e-6) / 1e9,
            "frac_of_hbm_peak": nbytes / (us_tok * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "timing": f"graph of {n_tok} in-chunk calls; chunk-end call eager (median of {reps})"}


def heads_bench(reps=20):
    """e2ttt_scalar_heads on the 1.3B-shaped layer (batch 8, 4096 tokens,
    model dim 2048, 16 TTT heads, bf16 input and head weights; seeded
    synthetic).  Algorithmic bytes: x and the head weights read once, the
    three scalars written (12 B per token-head).  HBM-bound."""
    import torch
    import chunk_weight_update_amd as cwu
    B, L, D, H = 8, 4096, 2048, 16
    g = torch.Generator(device="cuda").manual_seed(2)
    x = torch.randn((B, L, D), generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn((3 * H, D), generator=g, device="cuda") / D ** 0.5).to(torch.bfloat16)
    bias = 0.5 * torch.randn((3 * H,), generator=g, device="cuda")
    out = [torch.empty((B, H, L), device="cuda") for _ in range(3)]
    prob = cwu.make_problem(cwu.SWIGLU, B, H, L, 128, 256, 2048, cwu.BF16)
    for _ in range(3):
        cwu.scalar_heads(prob, x, D, w, bias, 0.01, 0.1, *out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        cwu.scalar_heads(prob, x, D, w, bias, 0.01, 0.1, *out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = 2.0 * B * L * D + 2.0 * 3 * H * D + 12.0 * B * H * L
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"label": "per-token scalar heads, batch 8 x 4096 tokens, model dim 2048, 16 heads, "
                     "bf16 (not the main metric)", "us": ms * 1e3, "gbs": gbs,
            "frac_of_hbm_peak": gbs / PEAK_HBM_GBS, "bound": "hbm"}


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
           "frac_of_fp32_matrix_peak": flops / (ms * 1e-3) / (PEAK_FP32_TFLOPS * 1e12)}
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


def system_info():
    """Host CPU model, usable threads, ROCm version, device name and CU count."""
    import torch
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rocm = None
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            with open(path) as f:
                rocm = f.read().strip()
                break
        except OSError:
            continue
    prop = torch.cuda.get_device_properties(0)
    # The achievable HBM ceiling: a plain 1 GiB device-to-device copy (read +
    # write bytes over time), median of 5.
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    times = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    copy_gbs = 2 * (1 << 30) / (percentile(times, 50) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"cpu_model": cpu, "cpu_threads_usable": len(os.sched_getaffinity(0)),
            "hbm_copy_gbs_measured": copy_gbs,
            "rocm_version": rocm, "hip_runtime": torch.version.hip, "torch": torch.__version__,
            "device_name": prop.name, "gcn_arch": getattr(prop, "gcnArchName", None),
            "compute_units": prop.multi_processor_count,
            "peaks": {"bf16_mfma_tflops": PEAK_BF16_TFLOPS, "fp32_mfma_tflops": PEAK_FP32_TFLOPS,
                      "hbm_gbs": PEAK_HBM_GBS}}


def device_inputs(w, inp, dev="cuda:0"):
    import numpy as np
    import torch
    t = {}
    for n in ("q", "k", "v"):
        a = np.ascontiguousarray(inp[n])
        t[n] = (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if w.io == 1
                else torch.from_numpy(a)).to(dev)
    for n in ("eta", "alpha", "beta", "W0", "M0"):
        t[n] = torch.from_numpy(inp[n]).to(dev)
    return t


def percentile(xs, p):
    xs = sorted(xs)
    if not xs:
        return None
    k = (len(xs) - 1) * p / 100.0
    lo, hi = int(k), min(int(k) + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


def kernel_pass(w, prob, run, call_args, steps):
    """Per-kernel-class launch durations: e2ttt_chunk_forward_timed records
    HIP events at the start and end of every launch of one class."""
    import chunk_weight_update_amd as cwu
    import torch
    ev = HipEvents()
    classes = ([cwu.KERNEL_SCAN, cwu.KERNEL_LINEAR_FWD, cwu.KERNEL_LINEAR_AGG] if w.kind == 0
               else [cwu.KERNEL_SCAN, cwu.KERNEL_PREP, cwu.KERNEL_FWD13, cwu.KERNEL_FWD2,
                     cwu.KERNEL_BWD, cwu.KERNEL_AGG, cwu.KERNEL_PHASE_A, cwu.KERNEL_PHASE_B,
                     cwu.KERNEL_STATE, cwu.KERNEL_PROLOGUE])
    per_step_launches = 2 * max(w.n_chunks, 2) + 2
    kernels = {}
    steps_k = max(1, min(steps, 10))
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
    return kernels


def roofline_of(w, kernels):
    peak_mfma = PEAK_BF16_TFLOPS if w.io == 1 else PEAK_FP32_TFLOPS
    dom_name = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dom_name]
    traffic = measured_traffic(dom_name, w.name)
    if dk["work_unit"] == "flop":
        return {"kernel": dom_name, "bound": "mfma", "achieved": dk["tflops"],
                "peak": peak_mfma, "unit": "TFLOP/s", "frac": dk["tflops"] / peak_mfma,
                "traffic": traffic}
    return {"kernel": dom_name, "bound": "hbm", "achieved": dk["gbs"], "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": dk["gbs"] / PEAK_HBM_GBS, "traffic": traffic}


def run_workload(w, steps, warmup, flags=0, kernel_timing=True, inp=None):
    """Time `steps` back-to-back e2ttt_chunk_forward calls of workload `w`
    (inputs resident in HBM), with an event between consecutive calls, so
    both the whole timed region and every single call are measured."""
    import chunk_weight_update_amd as cwu
    import torch
    from chunk_weight_update_amd.inputs import make_workload_inputs
    if inp is None:
        inp = make_workload_inputs(w, seed=0)
    t = device_inputs(w, inp)
    prob = cwu.make_problem(w.kind, w.B, w.H, w.L, w.d, w.h, w.C, w.io, 0, flags)
    run = cwu.ChunkForward(prob, device="cuda:0")
    call_args = (t["q"], t["k"], t["v"], t["eta"], t["alpha"], t["beta"], t["W0"], t["M0"])
    for _ in range(warmup):
        run(*call_args)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(steps):
        run(*call_args)
        evs[i + 1].record()
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / steps
    per_call = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    res = {"config": w.describe() | {"flags": flags}, "ms_per_step": ms,
           "value": w.B * w.L / (ms * 1e-3),
           "per_call_ms": {"median": percentile(per_call, 50), "p10": percentile(per_call, 10),
                           "p90": percentile(per_call, 90), "n": steps},
           "tflops_algorithmic": algorithmic_flops(w) / (ms * 1e-3) / 1e12}
    res["mfma_util_pct_of_bf16_peak"] = 100.0 * res["tflops_algorithmic"] / PEAK_BF16_TFLOPS
    if kernel_timing:
        res["kernels"] = kernel_pass(w, prob, run, call_args, steps)
        res["roofline"] = roofline_of(w, res["kernels"])
    res["_run"] = (run, t, prob)
    return res


def oracle_sample(w, inp, budget_s):
    """The fp64 oracle on the first chunk of the first n (b, h) units (n
    chosen so that it runs for about budget_s): timed for the CPU baseline,
    and kept as the reference for the parity figures of the bench line."""
    import oracle
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    oracle.set_threads(cores)
    oracle.build(force=False)
    BH = w.B * w.H
    C = min(w.C, w.L)

    def sl(a, n):
        a = a.reshape((BH,) + a.shape[2:])[:n][None]
        return a[..., :C, :] if a.ndim == 4 else (a[..., :C] if a.shape[-1] == w.L else a)

    def run_units(n):
        t0 = time.perf_counter()
        ref = oracle.chunk_forward(w.kind, sl(inp["q64"], n), sl(inp["k64"], n),
                                   sl(inp["v64"], n), sl(inp["eta"], n), sl(inp["alpha"], n),
                                   sl(inp["beta"], n), sl(inp["W0"], n), sl(inp["M0"], n),
                                   w.C, w.h)
        return time.perf_counter() - t0, ref

    t1, ref = run_units(1)
    n = int(max(1, min(BH, budget_s / max(t1, 1e-6))))
    tn, ref = run_units(n) if n > 1 else (t1, ref)
    # A sample well under the budget is repeated (up to 3 runs, median).
    times = [tn]
    while len(times) < 3 and sum(times) + tn <= budget_s:
        times.append(run_units(n)[0])
    times.sort()
    return {"n_units": n, "tokens": C, "seconds": times[len(times) // 2], "runs": len(times),
            "cores": cores, "ref": ref, "slice": sl}


def parity_on_sample(w, res, smp, inp):
    """rel_fro of the timed call's first-chunk outputs, and of a first-chunk
    call's end states, against the oracle sample (the first chunk of the
    first n units: the whole chunk from W_0)."""
    import numpy as np
    import torch
    import chunk_weight_update_amd as cwu
    run, t, prob = res["_run"]
    n, C, sl = smp["n_units"], smp["tokens"], smp["slice"]
    ro, rW, rM = smp["ref"]
    BH = w.B * w.H

    def f64(x):
        return x.detach().float().cpu().numpy().astype(np.float64)

    def rel(x, r):
        return float(np.linalg.norm((x - r).ravel()) / np.linalg.norm(r.ravel()))
    out_timed = f64(run.out).reshape((BH, w.L, w.d))[:n, :C][None]
    sub = {k: sl(inp[k], n) for k in ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")}
    ts = device_inputs(w, sub)
    p1 = cwu.make_problem(w.kind, 1, n, C, w.d, w.h, w.C, w.io, 0)
    r1 = cwu.ChunkForward(p1, device="cuda:0")
    o1, W1, M1 = r1(ts["q"], ts["k"], ts["v"], ts["eta"], ts["alpha"], ts["beta"], ts["W0"],
                    ts["M0"])
    torch.cuda.synchronize()
    return {"sample": f"first chunk ({C} tokens) of {n} of {BH} (batch, head) units, from W_0",
            "out_timed_call": rel(out_timed, ro), "out": rel(f64(o1), ro),
            "W_end": rel(f64(W1), rW), "M_end": rel(f64(M1), rM),
            "tolerance": {"out": 1e-2, "W_end": 5e-3, "M_end": 5e-3} if w.io == 1
            else {"out": 1e-5, "W_end": 1e-5, "M_end": 1e-5}}


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
                    help="skip the side measurements (scan microbenchmark, decode, backward)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the other workloads' short timings")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, run a plain device-to-device copy of this "
                         "many MiB 5 times (the known-size reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the (batch, head) units would shard across GPUs with no communication); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from chunk_weight_update_amd.inputs import BENCH_WORKLOAD, WORKLOADS, make_workload_inputs

    w = WORKLOADS[args.workload or BENCH_WORKLOAD]
    torch.cuda.set_device(0)
    log(f"bench: workload {w.name}")
    inp = make_workload_inputs(w, seed=0)
    res = run_workload(w, args.steps, args.warmup, args.flags,
                       kernel_timing=not args.no_kernel_timing, inp=inp)
    log(f"bench: {args.steps} steps, {res['ms_per_step']:.4f} ms/step, "
        f"{res['value']:.4g} tokens/s, per call {res['per_call_ms']}")

    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"bench: copy calibration, 5 x {nbytes} bytes device to device")
        del src, dst

    metric = "TTT-layer fwd tokens/sec on 1 MI355X; MFMA util % of bf16 peak"
    if args.no_kernel_timing:
        print(json.dumps({"metric": metric, "value": res["value"], "unit": "tokens/s",
                          "ms_per_step": res["ms_per_step"], "config": res["config"]}),
              flush=True)
        return
    for k, v in res["kernels"].items():
        log(f"bench: kernel {k}: {v}")
    line = {
        "metric": metric, "value": res["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.io == 1 else "fp32", "data": "synthetic",
        "config": res["config"],
        "per_call_ms": res["per_call_ms"],
        "mfma_util_pct_of_bf16_peak": res["mfma_util_pct_of_bf16_peak"],
        "tflops_algorithmic": res["tflops_algorithmic"],
        "roofline": res["roofline"],
        "kernels": res["kernels"],
        "system": system_info(),
    }
    if not args.no_cpu_baseline:
        log("bench: fp64 oracle on a sample of the workload (host cores)")
        smp = oracle_sample(w, inp, args.cpu_seconds)
        line["parity"] = parity_on_sample(w, res, smp, inp)
        log(f"bench: parity on the sample {line['parity']}")
        line["cpu_baseline"] = {
            # token-heads per second on the sample -> tokens per second of
            # the workload (each token carries H heads)
            "value": smp["n_units"] * smp["tokens"] / smp["seconds"] / w.H,
            "unit": "tokens/s", "cores": smp["cores"], "kind": "oracle",
            "sample": f"first chunk ({smp['tokens']} tokens) of {smp['n_units']} of "
                      f"{w.B * w.H} (batch, head) units from W_0, {smp['seconds']:.1f} s fp64 "
                      f"(median of {smp['runs']} runs) "
                      f"(literal token-wise recurrence), scaled to the whole workload's "
                      f"tokens/s"}
    else:
        line["cpu_baseline"] = None
    del res["_run"]
    if not args.no_other_configs and args.workload is None:
        others = {}
        for name in ("linear-d64-b1h1-l256-c64-fp32", "swiglu-d128h256-b2h4-l4096-c512-bf16",
                     "swiglu-d128h256-b8h16-l4096-c2048-bf16",
                     "swiglu-d128h256-b1h16-l32768-c2048-bf16"):
            wo = WORKLOADS[name]
            inp_o = make_workload_inputs(wo, seed=0)
            ro = run_workload(wo, 50, 5, inp=inp_o)  # 50 timed calls for the smaller workloads
            others[name] = {k: ro[k] for k in ("ms_per_step", "value", "per_call_ms",
                                                "tflops_algorithmic",
                                                "mfma_util_pct_of_bf16_peak", "roofline")}
            others[name]["config"] = wo.describe()
            if not args.no_cpu_baseline:  # a short oracle sample: parity and CPU baseline
                smp = oracle_sample(wo, inp_o, 3.0)
                others[name]["parity"] = parity_on_sample(wo, ro, smp, inp_o)
                others[name]["cpu_baseline"] = {
                    "value": smp["n_units"] * smp["tokens"] / smp["seconds"] / wo.H,
                    "unit": "tokens/s", "cores": smp["cores"], "kind": "oracle",
                    "sample": f"first chunk ({smp['tokens']} tokens) of {smp['n_units']} of "
                              f"{wo.B * wo.H} units from W_0, {smp['seconds']:.2f} s fp64"}
            del ro["_run"]
            del inp_o
            log(f"bench: other workload {name}: {others[name]}")
            torch.cuda.empty_cache()
        line["other_configs"] = others
    if not args.no_scan_microbench:
        line["decode"] = {
            "label": "decode step, one token per (b,h) unit per call, state update once per "
                     "chunk (not the main metric)",
            "shapes": ([decode_bench(w.B, w.H, w.d, w.h, w.C, w.io)] if w.kind == 1 else []) + [
                       decode_bench(2, 4, 128, 256, 512, 1),
                       decode_bench(8, 16, 128, 256, 2048, 1)]}
        log(f"bench: decode step {line['decode']}")
        torch.cuda.empty_cache()
        line["scan_microbench"] = scan_microbench()
        log(f"bench: scan microbenchmark {line['scan_microbench']}")
        line["scalar_heads"] = heads_bench()
        log(f"bench: scalar heads {line['scalar_heads']}")
        line["backward"] = backward_bench(not args.no_cpu_baseline)
        line["backward_swiglu"] = backward_bench_swiglu(not args.no_cpu_baseline)
        log(f"bench: linear backward {line['backward']}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
