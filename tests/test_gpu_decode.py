"""Decode step (one token per call, the state update amortised over the
chunk) against the oracle.

Running e2ttt_decode_step over every token of a sequence, position t mod C
within the chunk, with chunk_end on every C-th token and on the last, must
give the chunk forward's outputs and end states: the oracle's literal
recurrence (readout and gradients at the chunk-start weights, token-wise
momentum/decay update) is the reference.  The chunk-end update is fp32, so
the states meet 1e-5 for both io types."""
import numpy as np
import pytest

from chunk_weight_update_amd.inputs import BF16, F32, LINEAR, MLP, SWIGLU, make_inputs
from gpu_util import log, problem_for, rel_fro, run_oracle, to_device

pytestmark = pytest.mark.gpu

TOL = {F32: (1e-5, 1e-5, 1e-5), BF16: (1e-2, 1e-5, 1e-5)}


def run_decode(prob, t, L, C, check_mid_chunk=False):
    import torch
    import chunk_weight_update_amd as cwu
    W = t["W0"].clone()
    M = t["M0"].clone()
    outs = torch.empty_like(t["q"])
    out_t = torch.empty_like(t["q"][:, :, 0])
    ws = torch.empty(cwu.decode_workspace_bytes(prob), dtype=torch.uint8, device="cuda")
    for s in range(L):
        col = lambda x: x[:, :, s].clone()  # fresh, aligned (a [1,1] slice is a view)
        end = (s + 1) % C == 0 or s == L - 1
        before = (W.clone(), M.clone()) if check_mid_chunk and not end else None
        cwu.decode_step(prob, col(t["q"]), col(t["k"]), col(t["v"]), col(t["eta"]),
                        col(t["alpha"]), col(t["beta"]), W, M, out_t, s % C, end, ws)
        outs[:, :, s] = out_t
        if before is not None:  # between chunk ends the state is the chunk start's
            torch.cuda.synchronize()
            assert torch.equal(before[0], W) and torch.equal(before[1], M)
    torch.cuda.synchronize()
    return (outs.float().cpu().numpy().astype(np.float64), W.cpu().numpy().astype(np.float64),
            M.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("kind,B,H,L,d,h,C,io,regime", [
    (LINEAR, 1, 2, 40, 64, 0, 16, F32, "default"),          # ragged last chunk
    (LINEAR, 2, 1, 33, 32, 0, 8, BF16, "default"),
    (SWIGLU, 1, 2, 48, 128, 256, 16, F32, "nearunit"),
    (SWIGLU, 2, 2, 40, 128, 256, 16, BF16, "nearunit"),     # ragged
    (SWIGLU, 1, 1, 24, 256, 512, 8, BF16, "default"),
    (SWIGLU, 1, 2, 300, 128, 256, 128, BF16, "nearunit"),   # chunks past one 128-slot tile
])
def test_decode_matches_oracle(kind, B, H, L, d, h, C, io, regime):
    log(f"decode kind={kind} B={B} H={H} L={L} d={d} h={h} C={C} io={io} {regime}")
    inp = make_inputs(kind, B, H, L, d, h, io, seed=9, regime=regime,
                      m0_scale=1e-6 if regime == "nearunit" else 0.01)
    prob = problem_for(kind, B, H, L, d, h, C, io)
    out, W, M = run_decode(prob, to_device(inp, io), L, C, check_mid_chunk=True)
    ro, rW, rM = run_oracle(kind, inp, C, h)
    e = (rel_fro(out, ro), rel_fro(W, rW), rel_fro(M, rM))
    log(f"  rel_fro out={e[0]:.3e} W={e[1]:.3e} M={e[2]:.3e}")
    t = TOL[io]
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(W)) and np.all(np.isfinite(M))
    assert e[0] <= t[0] and e[1] <= t[1] and e[2] <= t[2], e


def test_decode_with_qk_prologue():
    """Raw q, k with the SiLU + L2 prologue flag, token by token."""
    import chunk_weight_update_amd as cwu
    from test_gpu_parity import raw_projections
    kind, B, H, L, d, h, C, io = SWIGLU, 1, 2, 24, 128, 256, 8, BF16
    log("decode with the q/k prologue")
    inp = raw_projections(make_inputs(kind, B, H, L, d, h, io, seed=13, regime="nearunit",
                                      m0_scale=1e-6), io, 13)
    prob = problem_for(kind, B, H, L, d, h, C, io, 0, cwu.FLAG_QK_SILU_L2)
    out, W, M = run_decode(prob, to_device(inp, io), L, C)
    import oracle
    ro, rW, rM = oracle.chunk_forward(kind, inp["q64"], inp["k64"], inp["v64"], inp["eta"],
                                      inp["alpha"], inp["beta"], inp["W0"], inp["M0"], C, h,
                                      qk_norm=True, qk_round_bf16=io == BF16)
    e = (rel_fro(out, ro), rel_fro(W, rW), rel_fro(M, rM))
    log(f"  rel_fro out={e[0]:.3e} W={e[1]:.3e} M={e[2]:.3e}")
    assert e[0] <= 1e-2 and e[1] <= 5e-3 and e[2] <= 5e-3, e


@pytest.mark.parametrize("kind,B,H,L,d,h,C,io,regime", [
    (LINEAR, 1, 2, 40, 64, 0, 16, F32, "default"),
    (SWIGLU, 2, 2, 40, 128, 256, 16, BF16, "nearunit"),     # ragged
])
def test_decode_with_row_normalisation(kind, B, H, L, d, h, C, io, regime):
    """Chunk-boundary row normalisation at every call with chunk_end set,
    against the oracle's chunk forward with the same option."""
    import chunk_weight_update_amd as cwu
    import oracle
    log(f"decode with row normalisation kind={kind} B={B} H={H} L={L} C={C} io={io}")
    inp = make_inputs(kind, B, H, L, d, h, io, seed=15, regime=regime,
                      m0_scale=1e-6 if regime == "nearunit" else 0.01)
    prob = problem_for(kind, B, H, L, d, h, C, io, 0, cwu.FLAG_POST_CHUNK_ROW_L2)
    out, W, M = run_decode(prob, to_device(inp, io), L, C)
    ro, rW, rM = oracle.chunk_forward(kind, inp["q64"], inp["k64"], inp["v64"], inp["eta"],
                                      inp["alpha"], inp["beta"], inp["W0"], inp["M0"], C, h,
                                      row_norm=True)
    e = (rel_fro(out, ro), rel_fro(W, rW), rel_fro(M, rM))
    log(f"  rel_fro out={e[0]:.3e} W={e[1]:.3e} M={e[2]:.3e}")
    t = TOL[io]
    assert e[0] <= t[0] and e[1] <= t[1] and e[2] <= t[2], e


@pytest.mark.parametrize("variant", ["averaged", "lact"])
@pytest.mark.parametrize("kind,B,H,L,d,h,C,io,regime", [
    (LINEAR, 1, 2, 40, 64, 0, 16, F32, "default"),          # ragged last chunk
    (SWIGLU, 2, 2, 40, 128, 256, 16, BF16, "nearunit"),     # ragged
    (SWIGLU, 1, 1, 24, 256, 512, 8, F32, "nearunit"),
])
def test_decode_variants(variant, kind, B, H, L, d, h, C, io, regime):
    """The chunk-averaged variant and the LaCT rule change only the chunk-end
    kernels and coefficients (means over the buffered tokens, the last chunk
    ragged); token by token against the oracle's chunk forward with the same
    option."""
    import chunk_weight_update_amd as cwu
    flag = cwu.FLAG_CHUNK_AVERAGED_DECAY if variant == "averaged" else cwu.FLAG_LACT_RULE
    log(f"decode {variant} kind={kind} B={B} H={H} L={L} d={d} C={C} io={io}")
    inp = make_inputs(kind, B, H, L, d, h, io, seed=17, regime=regime,
                      m0_scale=1e-6 if regime == "nearunit" else 0.01)
    prob = problem_for(kind, B, H, L, d, h, C, io, 0, flag)
    out, W, M = run_decode(prob, to_device(inp, io), L, C, check_mid_chunk=True)
    ro, rW, rM = run_oracle(kind, inp, C, h, averaged=variant == "averaged",
                            lact=variant == "lact")
    e = (rel_fro(out, ro), rel_fro(W, rW), rel_fro(M, rM))
    log(f"  rel_fro out={e[0]:.3e} W={e[1]:.3e} M={e[2]:.3e}")
    t = TOL[io]
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(W)) and np.all(np.isfinite(M))
    assert e[0] <= t[0] and e[1] <= t[1] and e[2] <= t[2], e


@pytest.mark.parametrize("kind,B,H,L,d,h,C,io,flags", [
    (MLP, 1, 2, 48, 128, 256, 16, F32, 0),
    (MLP, 2, 2, 40, 128, 256, 16, BF16, 0),       # ragged last chunk
    (MLP, 1, 1, 24, 256, 512, 8, F32, 8),         # with row normalisation
    (MLP, 1, 2, 40, 128, 256, 16, F32, 32),       # the LaCT rule
])
def test_decode_mlp_learner(kind, B, H, L, d, h, C, io, flags):
    """The MLP learner f(x) = W2 silu(W1 x), token by token: its [W1 | W2]
    state read in place by the per-token kernels (a3 = 1, dA3 = 0) and
    updated at each chunk end through the [W1 | W3 = 0 | W2] layout of the
    aggregation; against the oracle's MLP chunk forward."""
    import chunk_weight_update_amd as cwu
    log(f"decode MLP B={B} H={H} L={L} d={d} h={h} C={C} io={io} flags={flags}")
    inp = make_inputs(kind, B, H, L, d, h, io, seed=19, regime="nearunit", m0_scale=1e-6)
    prob = problem_for(kind, B, H, L, d, h, C, io, 0, flags)
    out, W, M = run_decode(prob, to_device(inp, io), L, C, check_mid_chunk=True)
    ro, rW, rM = run_oracle(kind, inp, C, h, row_norm=bool(flags & cwu.FLAG_POST_CHUNK_ROW_L2),
                            lact=bool(flags & cwu.FLAG_LACT_RULE))
    e = (rel_fro(out, ro), rel_fro(W, rW), rel_fro(M, rM))
    log(f"  rel_fro out={e[0]:.3e} W={e[1]:.3e} M={e[2]:.3e}")
    t = TOL[io]
    assert W.shape[-1] == 2 * d * h
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(W)) and np.all(np.isfinite(M))
    assert e[0] <= t[0] and e[1] <= t[1] and e[2] <= t[2], e
