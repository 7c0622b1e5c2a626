"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
HIP library through its C ABI binding, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import chunk_weight_update_amd as cwu
from chunk_weight_update_amd.inputs import BF16, F32, LINEAR


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def rel_fro(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def to_device(inp, io, device="cuda"):
    import torch
    t = {}
    for n in ("q", "k", "v"):
        a = inp[n]
        if io == BF16:
            t[n] = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(device)
        else:
            t[n] = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    for n in ("eta", "alpha", "beta", "W0", "M0"):
        t[n] = torch.from_numpy(np.ascontiguousarray(inp[n], dtype=np.float32)).to(device)
    return t


def problem_for(kind, B, H, L, d, h, C, io, decay_mode=0, flags=0):
    return cwu.make_problem(kind, B, H, L, d, h if kind != LINEAR else 0, C, io,
                            decay_mode, flags)


def run_gpu(prob, t, stream=None):
    """One e2ttt_chunk_forward; returns (out, W_end, M_end) as float64 numpy."""
    import torch
    runner = cwu.ChunkForward(prob)
    out, W, M = runner(t["q"], t["k"], t["v"], t["eta"], t["alpha"], t["beta"], t["W0"],
                       t["M0"], stream=stream)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy().astype(np.float64), W.cpu().numpy().astype(np.float64),
            M.cpu().numpy().astype(np.float64))


def run_oracle(kind, inp, C, h, decay_mode=0, averaged=False, qk_norm=False, row_norm=False,
               lact=False, io=F32):
    """The oracle's chunk forward on a test's inputs.  With the q/k prologue
    and bf16 io the prologue's outputs are rounded to bf16, as the forward
    stores them for its bf16 products (input rounding is not charged to the
    GPU path)."""
    import oracle
    return oracle.chunk_forward(kind, inp["q64"], inp["k64"], inp["v64"], inp["eta"],
                                inp["alpha"], inp["beta"], inp["W0"], inp["M0"], C, h,
                                decay_mode=decay_mode, averaged=averaged, qk_norm=qk_norm,
                                row_norm=row_norm, lact=lact,
                                qk_round_bf16=bool(qk_norm) and io == BF16)
