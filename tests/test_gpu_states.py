"""The state-keeping forward and the backward that takes its states
(e2ttt_chunk_forward_states, e2ttt_chunk_backward_states).

The kept state of chunk r must be bit-identical to W_end, M_end of the same
forward run on the first r*C tokens (the chunk-to-chunk carry of §3.2), and
the backward given the states of an fp32 forward must be bit-identical to the
backward that recomputes them (it re-runs the same fp32 kernels).  With bf16 io
the kept states are the bf16 forward's, so the gradients are those of that
forward: checked against the oracle at the bf16 bars."""
import numpy as np
import pytest

from chunk_weight_update_amd.inputs import BF16, F32, LINEAR, MLP, SWIGLU, make_inputs
from gpu_util import log, problem_for, rel_fro, to_device

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")


def _forward_states(prob, t):
    import torch
    import chunk_weight_update_amd as cwu
    B, H, L, d = prob.batch, prob.heads, prob.seq_len, prob.dim
    P = d * d if prob.kind == LINEAR else (2 if prob.kind == MLP else 3) * d * prob.hidden
    nC = (L + prob.chunk - 1) // prob.chunk
    io = torch.bfloat16 if prob.io_dtype == BF16 else torch.float32
    out = torch.empty((B, H, L, d), dtype=io, device="cuda")
    We = torch.empty((B, H, P), device="cuda")
    Me = torch.empty((B, H, P), device="cuda")
    Ws = torch.full((max(nC - 1, 1), B, H, P), float("nan"), device="cuda")
    Ms = torch.full((max(nC - 1, 1), B, H, P), float("nan"), device="cuda")
    ws = torch.empty(max(cwu.workspace_bytes(prob), 256), dtype=torch.uint8, device="cuda")
    cwu.chunk_forward_states(prob, *[t[n] for n in NAMES], out, We, Me, Ws, Ms, ws)
    torch.cuda.synchronize()
    return out, We, Me, Ws, Ms


@pytest.mark.parametrize("kind,B,H,L,d,h,C,io", [
    (SWIGLU, 2, 4, 1100, 128, 256, 256, BF16),   # fused path, ragged last chunk
    (SWIGLU, 1, 2, 700, 128, 256, 256, F32),     # generic fp32 path
    (LINEAR, 1, 3, 300, 64, 0, 64, F32),         # linear path
    (MLP, 1, 2, 700, 128, 256, 256, F32),        # MLP learner, its [W1 | W2] states
    (MLP, 1, 1, 700, 256, 512, 256, BF16),       # MLP learner on the 256-tile path
])
def test_kept_states_equal_prefix_runs(kind, B, H, L, d, h, C, io):
    import torch
    import chunk_weight_update_amd as cwu
    log(f"kept states case kind={kind} B={B} H={H} L={L} d={d} h={h} C={C} io={io}")
    inp = make_inputs(kind, B, H, L, d, h, io, seed=9, m0_scale=0.01)
    t = to_device(inp, io)
    prob = problem_for(kind, B, H, L, d, h, C, io)
    out, We, Me, Ws, Ms = _forward_states(prob, t)
    ref = cwu.ChunkForward(prob)(*[t[n] for n in NAMES])
    torch.cuda.synchronize()
    assert torch.equal(out, ref[0]) and torch.equal(We, ref[1]) and torch.equal(Me, ref[2])
    nC = (L + C - 1) // C
    for r in range(1, nC):
        Lr = r * C
        tp = {n: (t[n][:, :, :Lr].contiguous() if n not in ("W0", "M0") else t[n]) for n in NAMES}
        pr = problem_for(kind, B, H, Lr, d, h, C, io)
        _, Wp, Mp = cwu.ChunkForward(pr)(*[tp[n] for n in NAMES])
        torch.cuda.synchronize()
        assert torch.equal(Ws[r - 1], Wp), r
        assert torch.equal(Ms[r - 1], Mp), r


def _backward(prob, t, dout, dW, dM, Ws=None, Ms=None):
    import torch
    import chunk_weight_update_amd as cwu
    g = {n: torch.full_like(t[n], float("nan")) for n in NAMES}
    ws = torch.empty(max(cwu.backward_workspace_bytes(prob), 256), dtype=torch.uint8,
                     device="cuda")
    cwu.chunk_backward(prob, *[t[n] for n in NAMES], dout, dW, dM, *[g[n] for n in NAMES], ws,
                       W_starts=Ws, M_starts=Ms)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("kind,B,H,L,d,h,C", [
    (SWIGLU, 1, 2, 300, 128, 256, 128),
    (LINEAR, 2, 1, 200, 64, 0, 64),
    (MLP, 1, 2, 300, 128, 256, 128),     # kept [W1 | W2] states, expanded inside
])
def test_backward_with_kept_states_matches_recompute(kind, B, H, L, d, h, C):
    import torch
    log(f"backward with kept states kind={kind} B={B} H={H} L={L} C={C}")
    inp = make_inputs(kind, B, H, L, d, h, F32, seed=10, m0_scale=0.01)
    t = to_device(inp, F32)
    prob = problem_for(kind, B, H, L, d, h, C, F32)
    _, _, _, Ws, Ms = _forward_states(prob, t)
    P = d * d if kind == LINEAR else (2 if kind == MLP else 3) * d * h
    gen = torch.Generator(device="cuda").manual_seed(3)
    dout = torch.randn(B, H, L, d, device="cuda", generator=gen)
    dW = torch.randn(B, H, P, device="cuda", generator=gen)
    dM = torch.randn(B, H, P, device="cuda", generator=gen)
    a = _backward(prob, t, dout, dW, dM)
    b = _backward(prob, t, dout, dW, dM, Ws, Ms)
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n


def test_backward_with_kept_bf16_states_matches_oracle():
    import torch
    import oracle
    from chunk_weight_update_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits
    B, H, L, d, h, C = 1, 2, 600, 128, 256, 256
    log(f"bf16 kept-state backward B={B} H={H} L={L} C={C}")
    inp = make_inputs(SWIGLU, B, H, L, d, h, BF16, seed=11, m0_scale=0.01)
    t = to_device(inp, BF16)
    prob = problem_for(SWIGLU, B, H, L, d, h, C, BF16)
    _, _, _, Ws, Ms = _forward_states(prob, t)
    P = 3 * d * h
    rng = np.random.default_rng(12)
    do_bits = f32_to_bf16_bits(rng.standard_normal((B, H, L, d)).astype(np.float32))
    dW = rng.standard_normal((B, H, P)).astype(np.float32)
    dM = rng.standard_normal((B, H, P)).astype(np.float32)
    dout = torch.from_numpy(do_bits.view(np.int16)).cuda().view(torch.bfloat16)
    g = _backward(prob, t, dout, torch.from_numpy(dW).cuda(), torch.from_numpy(dM).cuda(), Ws, Ms)
    ref = oracle.chunk_backward(SWIGLU, inp["q64"], inp["k64"], inp["v64"], inp["eta"],
                                inp["alpha"], inp["beta"], inp["W0"], inp["M0"],
                                bf16_bits_to_f32(do_bits).astype(np.float64), dW, dM, C,
                                hidden=h)
    errs = {n: rel_fro(g[n].float().cpu().numpy(), ref[n]) for n in NAMES}
    log("  rel_fro " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n in NAMES:
        assert errs[n] <= 1e-2, (n, errs[n])
