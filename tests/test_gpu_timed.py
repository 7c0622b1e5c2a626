"""The instrumented entry point e2ttt_chunk_forward_timed, which the
benchmark uses for its per-kernel durations, enqueues exactly the work of
e2ttt_chunk_forward: for every kernel class its outputs are bit-identical to
the plain call's, and it records one event pair per launch of that class
(the expected launch counts of each path checked), with non-negative
elapsed times."""
import numpy as np
import pytest

import chunk_weight_update_amd as cwu
from chunk_weight_update_amd.inputs import BF16, F32, LINEAR, SWIGLU, make_inputs
from gpu_util import log, problem_for, to_device

pytestmark = pytest.mark.gpu


def _hip_events():
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from bench import HipEvents
    return HipEvents()


# (kind, B, H, L, d, h, C, io, {class: launches per call})
CASES = [
    # 256-tile path: scan, prep (scaled keys + shadow), then 5 launches per chunk
    (SWIGLU, 1, 2, 600, 256, 512, 256, BF16,
     {cwu.KERNEL_SCAN: 1, cwu.KERNEL_PREP: 2, cwu.KERNEL_FWD13: 3, cwu.KERNEL_FWD2: 3,
      cwu.KERNEL_BWD: 3, cwu.KERNEL_AGG: 3, cwu.KERNEL_STATE: 3}),
    # fused d = 128 path with the token-split phase B
    (SWIGLU, 2, 2, 1024, 128, 256, 512, BF16,
     {cwu.KERNEL_PROLOGUE: 1, cwu.KERNEL_PHASE_A: 2, cwu.KERNEL_PHASE_B: 2,
      cwu.KERNEL_STATE: 2}),
    # linear learner, fp32
    (LINEAR, 1, 1, 256, 64, 0, 64, F32,
     {cwu.KERNEL_SCAN: 1, cwu.KERNEL_LINEAR_FWD: 4, cwu.KERNEL_LINEAR_AGG: 4}),
]


@pytest.mark.parametrize("kind,B,H,L,d,h,C,io,launches", CASES)
def test_timed_entry_matches_plain_call(kind, B, H, L, d, h, C, io, launches):
    import torch
    log(f"timed entry kind={kind} B={B} H={H} L={L} d={d} h={h} C={C} io={io}")
    inp = make_inputs(kind, B, H, L, d, h, io, seed=31, regime="nearunit", m0_scale=1e-6)
    t = to_device(inp, io)
    prob = problem_for(kind, B, H, L, d, h, C, io)
    args = [t[n] for n in ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")]
    ws = torch.empty(cwu.workspace_bytes(prob), dtype=torch.uint8, device="cuda")
    out0, W0, M0 = torch.empty_like(t["q"]), torch.empty_like(t["W0"]), torch.empty_like(t["M0"])
    cwu.chunk_forward(prob, *args, out0, W0, M0, ws)
    torch.cuda.synchronize()
    ev = _hip_events()
    for cls in range(cwu.KERNEL_NUM_CLASSES):
        out, W, M = torch.empty_like(out0), torch.empty_like(W0), torch.empty_like(M0)
        events = ev.create(2 * 16)
        _, nrec = cwu.chunk_forward_timed(prob, *args, out, W, M, ws, cls, events)
        torch.cuda.synchronize()
        assert nrec == launches.get(cls, 0), (cwu.KERNEL_NAMES[cls], nrec)
        for j in range(nrec):
            assert ev.elapsed_ms(events[2 * j], events[2 * j + 1]) >= 0.0
        ev.destroy(events)
        assert torch.equal(out.view(torch.int16) if io == BF16 else out,
                           out0.view(torch.int16) if io == BF16 else out0)
        assert torch.equal(W, W0) and torch.equal(M, M0)
