"""Outer-loop backward of the SwiGLU learner's chunk forward (fp32) against
the oracle's reverse mode (the literal token recurrence differentiated token
by token, pinned in test_oracle_backward.py by finite differences and by
autograd of an independent closed form).

Inputs: the workloads' recipe (unit-norm q, k, v; per-token eta, alpha, beta
of the default or near-unit regime; W0 ~ N(0, 1/fan_in), M0 ~ N(0, 0.01/fan_in)),
plus upstream gradients dout, dW_end, dM_end ~ N(0, 1) from a second seeded
generator.  The bar is the fp32 one: every output within 1e-5 relative
Frobenius error of the fp64 oracle."""
import numpy as np
import pytest

from chunk_weight_update_amd.inputs import F32, MLP, SWIGLU, make_inputs
from gpu_util import log, problem_for, rel_fro
from test_gpu_backward import NAMES, TOL, run_backward

pytestmark = pytest.mark.gpu


def _upstream(B, H, L, d, h, seed, with_state=True):
    rng = np.random.default_rng(seed + 2000)
    P = 3 * d * h
    dout = rng.standard_normal((B, H, L, d)).astype(np.float32)
    dW = rng.standard_normal((B, H, P)).astype(np.float32) if with_state else None
    dM = rng.standard_normal((B, H, P)).astype(np.float32) if with_state else None
    return dout, dW, dM


def check(B, H, L, d, h, C, mode=0, regime="default", seed=0, with_state=True, kind=SWIGLU,
          flags=0, tol=None):
    import oracle
    log(f"backward case kind={kind} B={B} H={H} L={L} d={d} h={h} C={C} mode={mode} "
        f"regime={regime} seed={seed} state_grads={with_state} flags={flags}")
    inp = make_inputs(kind, B, H, L, d, h, F32, seed=seed, regime=regime, m0_scale=0.01)
    P = oracle.state_size(kind, d, h)
    rng = np.random.default_rng(seed + 2000)
    dout = rng.standard_normal((B, H, L, d)).astype(np.float32)
    dW = rng.standard_normal((B, H, P)).astype(np.float32) if with_state else None
    dM = rng.standard_normal((B, H, P)).astype(np.float32) if with_state else None
    prob = problem_for(kind, B, H, L, d, h, C, F32, decay_mode=mode, flags=flags)
    got = run_backward(prob, inp, dout, dW, dM)
    ref = oracle.chunk_backward(kind, inp["q64"], inp["k64"], inp["v64"], inp["eta"],
                                inp["alpha"], inp["beta"], inp["W0"], inp["M0"], dout, dW, dM,
                                C, decay_mode=mode, hidden=h, qk_norm=bool(flags & 4),
                                averaged=bool(flags & 2), row_norm=bool(flags & 8),
                                lact=bool(flags & 32))
    errs = {n: rel_fro(got[n], ref[n]) for n in NAMES}
    log("  rel_fro " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n in NAMES:
        assert np.all(np.isfinite(got[n])), n
        assert errs[n] <= (tol or {}).get(n, TOL), (n, errs[n])


@pytest.mark.parametrize("B,H,L,C,mode,regime", [
    (1, 2, 300, 128, 0, "default"),     # ragged last chunk, two units
    (1, 1, 256, 256, 1, "default"),     # alpha taken as gamma, one chunk
    (2, 1, 200, 64, 0, "nearunit"),     # chunk below the 128-row tile
    (1, 1, 5, 1, 0, "default"),         # chunks of one token
])
def test_swiglu_backward_matches_oracle(B, H, L, C, mode, regime):
    check(B, H, L, 128, 256, C, mode, regime)


def test_swiglu_backward_large_state():
    """The large-state learner's shape (d = 768, h = 1536) on a short sequence
    (the oracle's reverse mode stores the state before every token)."""
    check(1, 1, 20, 768, 1536, 8, seed=2)


@pytest.mark.parametrize("kind,L,d,h,C", [(SWIGLU, 300, 128, 256, 128), (0, 200, 64, 0, 64)])
def test_backward_through_qk_prologue(kind, L, d, h, C):
    """E2TTT_FLAG_QK_SILU_L2: dq, dk taken back through SiLU + L2 per token."""
    check(1, 2, L, d, h, C, seed=7, kind=kind, flags=4)


@pytest.mark.parametrize("kind,L,d,h,C,mode", [(SWIGLU, 300, 128, 256, 128, 0),
                                               (0, 1000, 64, 0, 512, 1)])
def test_backward_chunk_averaged(kind, L, d, h, C, mode):
    """E2TTT_FLAG_CHUNK_AVERAGED_DECAY: the adjoints of the chunk means of beta
    and gamma, shared out over the chunk's tokens."""
    check(1, 2, L, d, h, C, mode=mode, seed=8, kind=kind, flags=2)


@pytest.mark.parametrize("kind,L,d,h,C,flags", [(SWIGLU, 300, 128, 256, 128, 8),
                                                (0, 200, 64, 0, 64, 8),
                                                (SWIGLU, 100, 128, 256, 128, 8),   # one chunk
                                                (SWIGLU, 260, 128, 256, 128, 14)])  # all three
def test_backward_row_normalisation(kind, L, d, h, C, flags):
    """E2TTT_FLAG_POST_CHUNK_ROW_L2: the adjoint goes back through every
    chunk's normalisation, the last one included (alone and with the
    averaged variant and the q/k prologue)."""
    check(1, 2, L, d, h, C, seed=9, kind=kind, flags=flags)


def test_swiglu_backward_without_state_gradients():
    check(1, 1, 160, 128, 256, 64, seed=4, with_state=False)


def test_swiglu_backward_is_deterministic():
    B, H, L, d, h, C = 1, 2, 192, 128, 256, 128
    inp = make_inputs(SWIGLU, B, H, L, d, h, F32, seed=6, m0_scale=0.01)
    dout, dW, dM = _upstream(B, H, L, d, h, 6)
    prob = problem_for(SWIGLU, B, H, L, d, h, C, F32)
    a = run_backward(prob, inp, dout, dW, dM)
    b = run_backward(prob, inp, dout, dW, dM)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n


# --------------------------------------------------------------------------
# bf16 io: q, k, v, dout in and dq, dk, dv out as bf16 (the state tensors and
# per-token scalars stay fp32).  The library widens the inputs and computes in
# fp32, so the fp32 outputs keep the fp32 bar; the bf16 outputs carry one
# rounding each (at most 2^-9 relative) and take the bf16 output bar.

BF16_OUT_TOL = 1e-2
BF16_OUT = ("q", "k", "v")


def check_bf16(kind, B, H, L, d, h, C, mode=0, regime="default", seed=0):
    import torch
    import oracle
    import chunk_weight_update_amd as cwu
    from chunk_weight_update_amd.inputs import BF16, bf16_bits_to_f32, f32_to_bf16_bits
    log(f"bf16-io backward case kind={kind} B={B} H={H} L={L} d={d} h={h} C={C} mode={mode} "
        f"regime={regime} seed={seed}")
    inp = make_inputs(kind, B, H, L, d, h, BF16, seed=seed, regime=regime, m0_scale=0.01)
    P = oracle.state_size(kind, d, h)
    rng = np.random.default_rng(seed + 3000)
    do_bits = f32_to_bf16_bits(rng.standard_normal((B, H, L, d)).astype(np.float32))
    dout64 = bf16_bits_to_f32(do_bits).astype(np.float64)
    dW = rng.standard_normal((B, H, P)).astype(np.float32)
    dM = rng.standard_normal((B, H, P)).astype(np.float32)
    prob = problem_for(kind, B, H, L, d, h, C, BF16, decay_mode=mode)
    dev = "cuda"

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
    t = {n: bf(inp[n]) for n in ("q", "k", "v")}
    for n in ("eta", "alpha", "beta", "W0", "M0"):
        t[n] = torch.from_numpy(np.ascontiguousarray(inp[n], dtype=np.float32)).to(dev)
    g = {n: torch.full_like(t[n], float("nan")) for n in NAMES}
    ws = torch.empty(max(cwu.backward_workspace_bytes(prob), 256), dtype=torch.uint8, device=dev)
    cwu.chunk_backward(prob, *[t[n] for n in NAMES], bf(do_bits), torch.from_numpy(dW).to(dev),
                       torch.from_numpy(dM).to(dev), *[g[n] for n in NAMES], ws)
    torch.cuda.synchronize()
    got = {n: g[n].float().cpu().numpy().astype(np.float64) for n in NAMES}
    ref = oracle.chunk_backward(kind, inp["q64"], inp["k64"], inp["v64"], inp["eta"],
                                inp["alpha"], inp["beta"], inp["W0"], inp["M0"], dout64, dW, dM,
                                C, decay_mode=mode, hidden=h)
    errs = {n: rel_fro(got[n], ref[n]) for n in NAMES}
    log("  rel_fro " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n in NAMES:
        assert np.all(np.isfinite(got[n])), n
        assert errs[n] <= (BF16_OUT_TOL if n in BF16_OUT else TOL), (n, errs[n])


@pytest.mark.parametrize("kind,B,H,L,d,h,C,mode", [
    (SWIGLU, 1, 2, 300, 128, 256, 128, 0),   # the bf16 workloads' learner, ragged last chunk
    (0, 2, 2, 200, 64, 0, 64, 1),            # linear learner, alpha taken as gamma
    (MLP, 1, 2, 300, 128, 256, 128, 0),      # MLP learner
])
def test_backward_bf16_io_matches_oracle(kind, B, H, L, d, h, C, mode):
    check_bf16(kind, B, H, L, d, h, C, mode)


def test_swiglu_backward_bench_shape_sampled_units():
    """The bench's backward shape (B2 x H4, L4096, C512, d128/h256, fp32) in
    its launch configuration; units are independent, so the oracle's reverse
    mode is run on two sampled (batch, head) units and compared unit by unit."""
    import oracle
    B, H, L, d, h, C = 2, 4, 4096, 128, 256, 512
    log(f"bench-shape backward B={B} H={H} L={L} C={C}, oracle on units (0,0) and (1,3)")
    inp = make_inputs(SWIGLU, B, H, L, d, h, F32, seed=0, m0_scale=0.01)
    dout, dW, dM = _upstream(B, H, L, d, h, 0)
    prob = problem_for(SWIGLU, B, H, L, d, h, C, F32)
    got = run_backward(prob, inp, dout, dW, dM)
    for (bi, hi) in ((0, 0), (1, 3)):
        sl = (slice(bi, bi + 1), slice(hi, hi + 1))
        ref = oracle.chunk_backward(oracle.SWIGLU, inp["q64"][sl], inp["k64"][sl],
                                    inp["v64"][sl], inp["eta"][sl], inp["alpha"][sl],
                                    inp["beta"][sl], inp["W0"][sl], inp["M0"][sl], dout[sl],
                                    dW[sl], dM[sl], C, hidden=h)
        errs = {n: rel_fro(got[n][sl], ref[n]) for n in NAMES}
        log(f"  unit ({bi},{hi}) rel_fro " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
        for n in NAMES:
            assert errs[n] <= TOL, (bi, hi, n, errs[n])


@pytest.mark.parametrize("kind,L,d,h,C,mode,flags", [
    (SWIGLU, 300, 128, 256, 128, 0, 32),     # ragged last chunk
    (0, 1000, 64, 0, 512, 1, 32),            # linear learner, alpha taken as gamma
    (0, 200, 64, 0, 64, 0, 32 | 4),          # with the q/k prologue
])
def test_backward_lact_rule(kind, L, d, h, C, mode, flags):
    """E2TTT_FLAG_LACT_RULE: K^W = K^M = eta, so deta takes both kernels'
    adjoints directly, and the adjoints of the chunk means of beta and gamma
    are shared out over the chunk's tokens; everything else is the default
    rule's backward."""
    check(1, 2, L, d, h, C, mode, seed=11, kind=kind, flags=flags)


def test_backward_lact_rule_with_row_normalisation():
    """The LaCT rule with chunk-boundary normalisation.  Under the LaCT rule
    a token's dalpha (and the decay part of dbeta's companion, dgamma) is one
    dot product, <dW_C, W_s> / n; with the normalisation, dW_C (the adjoint
    of the chunk end before it) is orthogonal to every row of W_C, which is
    nearly parallel to W_s, so that dot cancels to a few parts in 10^3 of
    its terms and the fp32 rounding of W_s alone (6e-8 relative) leaves
    ~2e-5 relative error in it.  alpha and beta are held to 1e-4 here,
    every other gradient to the fp32 bar."""
    check(1, 2, 200, 128, 256, 64, 0, seed=11, kind=SWIGLU, flags=32 | 8,
          tol={"alpha": 1e-4, "beta": 1e-4})


# --------------------------------------------------------------------------
# The MLP learner f(x) = W2 silu(W1 x): the SwiGLU backward with the gate held
# at one, on an internal [W1 | 0 | W2] copy of the states and adjoints; the
# caller's states and gradients are [W1 | W2].

@pytest.mark.parametrize("B,H,L,C,mode,regime,flags", [
    (1, 2, 300, 128, 0, "default", 0),    # ragged last chunk, two units
    (1, 1, 256, 256, 1, "default", 0),    # alpha taken as gamma, one chunk
    (2, 1, 200, 64, 0, "default", 0),     # chunk below the 128-row tile
    (1, 1, 5, 1, 0, "default", 0),        # chunks of one token
    (1, 2, 300, 128, 0, "default", 4),    # q/k prologue
    (1, 2, 300, 128, 1, "default", 2),    # chunk-averaged variant
    (1, 2, 260, 128, 0, "default", 8),    # chunk-boundary row normalisation
    (1, 2, 300, 128, 0, "default", 32),   # LaCT rule
])
def test_mlp_backward_matches_oracle(B, H, L, C, mode, regime, flags):
    check(B, H, L, 128, 256, C, mode, regime, seed=13, kind=MLP, flags=flags)


def test_mlp_backward_without_state_gradients():
    check(1, 1, 160, 128, 256, 64, seed=14, with_state=False, kind=MLP)


def test_mlp_backward_large_state():
    """The MLP learner at the large-state shape (d = 768, h = 1536), short sequence."""
    check(1, 1, 20, 768, 1536, 8, seed=15, kind=MLP)


def test_mlp_backward_near_unit_retention():
    """The MLP learner under near-unit retention (beta ~ 0.995, eta ~ 0.005):
    over 200 tokens the momentum piles up and the gradients reach ~1e10 in
    norm, so the problem itself is ill-conditioned.  Its condition is measured
    here on the oracle: one fp32-sized relative perturbation (6e-8) of M0 moves
    the fp64 gradients by s ~ 2e-6 relative, about 30 times the perturbation.
    An fp32 evaluation rounds every intermediate state of the chain, so its
    error is a sum of many such responses: the bar is the larger of the fp32
    bar and 10 s per gradient (the case is checked to be this badly
    conditioned: some s above 1e-6), with q, whose gradient needs no reverse
    chain, at the fp32 bar."""
    import oracle
    B, H, L, d, h, C, seed = 2, 1, 200, 128, 256, 64, 13
    inp = make_inputs(MLP, B, H, L, d, h, F32, seed=seed, regime="nearunit", m0_scale=0.01)
    P = oracle.state_size(MLP, d, h)
    rng = np.random.default_rng(seed + 2000)
    dout = rng.standard_normal((B, H, L, d)).astype(np.float32)
    dW = rng.standard_normal((B, H, P)).astype(np.float32)
    dM = rng.standard_normal((B, H, P)).astype(np.float32)

    def ref(M0):
        return oracle.chunk_backward(MLP, inp["q64"], inp["k64"], inp["v64"], inp["eta"],
                                     inp["alpha"], inp["beta"], inp["W0"], M0, dout, dW, dM, C,
                                     hidden=h)
    r0 = ref(inp["M0"])
    pert = np.random.default_rng(99).standard_normal(inp["M0"].shape)
    r1 = ref(np.asarray(inp["M0"], dtype=np.float64) * (1 + 6e-8 * pert))
    sens = {n: rel_fro(r1[n], r0[n]) for n in NAMES}
    log("  oracle sensitivity " + " ".join(f"{n}={e:.1e}" for n, e in sens.items()))
    got = run_backward(problem_for(MLP, B, H, L, d, h, C, F32), inp, dout, dW, dM)
    errs = {n: rel_fro(got[n], r0[n]) for n in NAMES}
    log("  rel_fro " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    assert max(sens.values()) > 1e-6, sens
    for n in NAMES:
        assert np.all(np.isfinite(got[n])), n
        bar = TOL if n == "q" else max(TOL, 10 * sens[n])
        assert errs[n] <= bar, (n, errs[n], bar)
