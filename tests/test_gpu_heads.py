"""GPU parity of the per-token scalar heads (e2ttt_scalar_heads) against the
oracle, and of heads -> chunk forward end to end.

The heads' products accumulate in fp32 (bf16 inputs multiply exactly), so
each scalar is compared elementwise at 1e-5 relative: the fp32 sum of D
terms of size ~1/sqrt(D) errs by ~sqrt(D) 2^-24 / sqrt(D) ~ 1e-7 in the
pre-activation, and the gate's derivative is at most 1/4."""
import numpy as np
import pytest

import chunk_weight_update_amd as cwu
import oracle
from chunk_weight_update_amd.inputs import BF16, F32, SWIGLU, make_head_inputs, make_inputs
from gpu_util import log, problem_for, rel_fro, run_gpu, to_device

pytestmark = pytest.mark.gpu


def heads_on_gpu(B, L, D, H, io, inp, eb, ab):
    import torch
    if io == BF16:
        x = torch.from_numpy(inp["x"].view(np.int16)).view(torch.bfloat16).cuda()
        w = torch.from_numpy(inp["w"].view(np.int16)).view(torch.bfloat16).cuda()
    else:
        x = torch.from_numpy(inp["x"]).cuda()
        w = torch.from_numpy(inp["w"]).cuda()
    bias = torch.from_numpy(inp["bias"]).cuda()
    out = [torch.empty((B, H, L), device="cuda") for _ in range(3)]
    prob = cwu.make_problem(SWIGLU, B, H, L, 128, 256, 512, io)
    cwu.scalar_heads(prob, x, D, w, bias, eb, ab, *out)
    torch.cuda.synchronize()
    return [o.cpu().numpy().astype(np.float64) for o in out]


@pytest.mark.parametrize("B,L,D,H,io", [
    (8, 4096, 2048, 16, BF16),   # the 1.3B-shaped layer: hidden 2048, 16 heads
    (1, 8192, 768, 1, BF16),     # one head, model dim 768
    (2, 1000, 512, 4, F32),      # tokens not a multiple of the 128-row tile
    (1, 77, 64, 64, BF16),       # the most heads, the smallest model dim
    (3, 129, 192, 5, F32),
])
def test_scalar_heads_match_oracle(B, L, D, H, io):
    log(f"heads B={B} L={L} D={D} H={H} io={io}")
    inp = make_head_inputs(B, L, D, H, io, seed=B * 7 + H)
    eb, ab = 0.01, 0.1
    got = heads_on_gpu(B, L, D, H, io, inp, eb, ab)
    ref = oracle.scalar_heads(inp["x64"], inp["w64"], inp["bias"], H, eb, ab)
    for g, r, name in zip(got, ref, ("eta", "alpha", "beta")):
        err = float(np.max(np.abs(g - r) / np.abs(r)))
        log(f"  {name}: max rel err {err:.2e}")
        assert err <= 1e-5, (name, err)


def test_heads_then_chunk_forward_end_to_end():
    """The B2 x H4, L 4096, C 512 layer (d = 128, h = 256, model dim 512):
    eta, alpha, beta from the heads on the GPU, then the chunk forward; the
    reference is the oracle's heads followed by the oracle's forward, at the
    bf16 bar."""
    import torch
    B, H, L, d, h, C, D = 2, 4, 4096, 128, 256, 512, 512
    hin = make_head_inputs(B, L, D, H, BF16, seed=3)
    eb, ab = 0.01, 0.1
    eta, alpha, beta = (torch.from_numpy(a.astype(np.float32)).cuda()
                        for a in heads_on_gpu(B, L, D, H, BF16, hin, eb, ab))
    inp = make_inputs(SWIGLU, B, H, L, d, h, BF16, seed=4)
    t = to_device(inp, BF16)
    t["eta"], t["alpha"], t["beta"] = eta, alpha, beta
    out, W, M = run_gpu(problem_for(SWIGLU, B, H, L, d, h, C, BF16), t)
    re, ra, rb = oracle.scalar_heads(hin["x64"], hin["w64"], hin["bias"], H, eb, ab)
    ro, rW, rM = oracle.chunk_forward(SWIGLU, inp["q64"], inp["k64"], inp["v64"], re, ra, rb,
                                      inp["W0"], inp["M0"], C, h)
    e = (rel_fro(out, ro), rel_fro(W, rW), rel_fro(M, rM))
    log(f"  heads + forward rel_fro out={e[0]:.3e} W={e[1]:.3e} M={e[2]:.3e}")
    assert e[0] <= 1e-2 and e[1] <= 5e-3 and e[2] <= 5e-3, e
