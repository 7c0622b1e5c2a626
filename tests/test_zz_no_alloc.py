"""e2ttt_chunk_forward_noalloc (the built-in per-GPU scratch instead of a
caller workspace) against e2ttt_chunk_forward on the same inputs.  Both run
the same kernels with the same plan, and every sum runs in a fixed order, so
the results must be bit-identical.  Two calls in a row, the second on a
smaller problem, so that the second one starts from the first one's leftovers
in the shared scratch.  Collected last: a failure here hides no other test."""
import numpy as np
import pytest

import chunk_weight_update_amd as cwu
from chunk_weight_update_amd.inputs import BF16, F32, LINEAR, SWIGLU, make_inputs
from gpu_util import log, problem_for, to_device

pytestmark = pytest.mark.gpu

CASES = [
    # (kind, B, H, L, d, h, C, io, flags): the first needs ~38 MiB of scratch
    (SWIGLU, 2, 4, 4096, 128, 256, 512, BF16, 0),
    (SWIGLU, 1, 2, 1000, 128, 256, 256, BF16, 0),   # smaller, ragged last chunk
    (LINEAR, 1, 3, 300, 64, 0, 64, F32, 0),
    # the 256-tile path (scaled keys, split aggregation): ~56 MiB, then ~28 MiB
    (SWIGLU, 1, 2, 700, 256, 512, 256, BF16, 0),
    (SWIGLU, 1, 1, 512, 256, 512, 256, BF16, 0),
]


def run_both(case, seed):
    import torch
    kind, B, H, L, d, h, C, io, flags = case
    log(f"noalloc case {case} seed {seed}")
    inp = make_inputs(kind, B, H, L, d, h, io, seed=seed, m0_scale=0.01)
    t = to_device(inp, io)
    prob = problem_for(kind, B, H, L, d, h, C, io, 0, flags)
    assert cwu.workspace_bytes(prob) <= cwu.NOALLOC_SCRATCH_BYTES
    args = [t[n] for n in ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")]
    out_a, W_a, M_a = torch.empty_like(t["q"]), torch.empty_like(t["W0"]), torch.empty_like(t["W0"])
    cwu.chunk_forward_noalloc(prob, *args, out_a, W_a, M_a)
    torch.cuda.synchronize()
    ws = torch.empty(max(cwu.workspace_bytes(prob), 256), dtype=torch.uint8, device="cuda")
    out_b, W_b, M_b = torch.empty_like(t["q"]), torch.empty_like(t["W0"]), torch.empty_like(t["W0"])
    cwu.chunk_forward(prob, *args, out_b, W_b, M_b, ws)
    torch.cuda.synchronize()
    for x, y, name in ((out_a, out_b, "out"), (W_a, W_b, "W_end"), (M_a, M_b, "M_end")):
        xa = x.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
        ya = y.view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
        assert np.array_equal(xa, ya), f"{name} differs"
        assert torch.isfinite(x.float()).all()
    log("  bit-identical to e2ttt_chunk_forward")


def test_noalloc_matches_workspace_entry_point_two_calls():
    run_both(CASES[0], seed=0)
    run_both(CASES[1], seed=1)   # smaller, after the larger one


def test_noalloc_linear_and_repeat():
    run_both(CASES[2], seed=2)
    run_both(CASES[1], seed=3)


def test_noalloc_256_tile_path_two_calls():
    run_both(CASES[3], seed=4)
    run_both(CASES[4], seed=5)   # smaller, after the larger one


def test_noalloc_rejects_problems_beyond_the_scratch():
    import torch
    prob = problem_for(SWIGLU, 8, 16, 4096, 128, 256, 2048, BF16)
    assert cwu.workspace_bytes(prob) > cwu.NOALLOC_SCRATCH_BYTES
    W = torch.zeros((8, 16, 3 * 128 * 256), device="cuda")
    st = cwu.chunk_forward_noalloc(prob, W, W, W, W, W, W, W, W, W, W, W, check=False)
    assert st == cwu.EWORKSPACE
