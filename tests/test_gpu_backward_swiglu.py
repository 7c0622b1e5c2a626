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

from chunk_weight_update_amd.inputs import F32, SWIGLU, make_inputs
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


def check(B, H, L, d, h, C, mode=0, regime="default", seed=0, with_state=True):
    import oracle
    log(f"swiglu backward case B={B} H={H} L={L} d={d} h={h} C={C} mode={mode} "
        f"regime={regime} seed={seed} state_grads={with_state}")
    inp = make_inputs(SWIGLU, B, H, L, d, h, F32, seed=seed, regime=regime, m0_scale=0.01)
    dout, dW, dM = _upstream(B, H, L, d, h, seed, with_state)
    prob = problem_for(SWIGLU, B, H, L, d, h, C, F32, decay_mode=mode)
    got = run_backward(prob, inp, dout, dW, dM)
    ref = oracle.chunk_backward(oracle.SWIGLU, inp["q64"], inp["k64"], inp["v64"], inp["eta"],
                                inp["alpha"], inp["beta"], inp["W0"], inp["M0"], dout, dW, dM,
                                C, decay_mode=mode, hidden=h)
    errs = {n: rel_fro(got[n], ref[n]) for n in NAMES}
    log("  rel_fro " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n in NAMES:
        assert np.all(np.isfinite(got[n])), n
        assert errs[n] <= TOL, (n, errs[n])


@pytest.mark.parametrize("B,H,L,C,mode,regime", [
    (1, 2, 300, 128, 0, "default"),     # ragged last chunk, two units
    (1, 1, 256, 256, 1, "default"),     # alpha taken as gamma, one chunk
    (2, 1, 200, 64, 0, "nearunit"),     # chunk below the 128-row tile
    (1, 1, 5, 1, 0, "default"),         # chunks of one token
])
def test_swiglu_backward_matches_oracle(B, H, L, C, mode, regime):
    check(B, H, L, 128, 256, C, mode, regime)


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
