"""Outer-loop backward of the linear learner's chunk forward against the
oracle's reverse mode (the literal token recurrence differentiated token by
token, pinned in test_oracle_backward.py).

Inputs: the workloads' recipe (unit-norm q, k, v; per-token eta, alpha, beta
of the default or near-unit regime; W0 ~ N(0, 1/d), M0 ~ N(0, 0.01/d)), plus
upstream gradients dout, dW_end, dM_end ~ N(0, 1) from a second seeded
generator.  The bar is the fp32 one: every output within 1e-5 relative
Frobenius error of the fp64 oracle."""
import numpy as np
import pytest

from chunk_weight_update_amd.inputs import F32, LINEAR, make_inputs
from gpu_util import log, problem_for, rel_fro

pytestmark = pytest.mark.gpu

TOL = 1e-5
NAMES = ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")


def _upstream(B, H, L, d, seed, with_state=True):
    rng = np.random.default_rng(seed + 1000)
    dout = rng.standard_normal((B, H, L, d)).astype(np.float32)
    dW = rng.standard_normal((B, H, d * d)).astype(np.float32) if with_state else None
    dM = rng.standard_normal((B, H, d * d)).astype(np.float32) if with_state else None
    return dout, dW, dM


def run_backward(prob, inp, dout, dW, dM):
    import torch
    import chunk_weight_update_amd as cwu
    dev = "cuda"
    t = {n: torch.from_numpy(np.ascontiguousarray(inp[n], dtype=np.float32)).to(dev)
         for n in NAMES}
    do = torch.from_numpy(dout).to(dev)
    dWt = torch.from_numpy(dW).to(dev) if dW is not None else None
    dMt = torch.from_numpy(dM).to(dev) if dM is not None else None
    g = {n: torch.full_like(t[n], float("nan")) for n in NAMES}
    ws = torch.empty(max(cwu.backward_workspace_bytes(prob), 256), dtype=torch.uint8, device=dev)
    cwu.chunk_backward(prob, t["q"], t["k"], t["v"], t["eta"], t["alpha"], t["beta"], t["W0"],
                       t["M0"], do, dWt, dMt, g["q"], g["k"], g["v"], g["eta"], g["alpha"],
                       g["beta"], g["W0"], g["M0"], ws)
    torch.cuda.synchronize()
    return {n: g[n].cpu().numpy().astype(np.float64) for n in NAMES}


def run_oracle_backward(inp, dout, dW, dM, C, mode):
    import oracle
    return oracle.chunk_backward(oracle.LINEAR, inp["q64"], inp["k64"], inp["v64"],
                                 inp["eta"], inp["alpha"], inp["beta"], inp["W0"], inp["M0"],
                                 dout, dW, dM, C, decay_mode=mode)


def check(B, H, L, d, C, mode=0, regime="default", seed=0, with_state=True):
    log(f"backward case B={B} H={H} L={L} d={d} C={C} mode={mode} regime={regime} "
        f"seed={seed} state_grads={with_state}")
    inp = make_inputs(LINEAR, B, H, L, d, 0, F32, seed=seed, regime=regime, m0_scale=0.01)
    dout, dW, dM = _upstream(B, H, L, d, seed, with_state)
    prob = problem_for(LINEAR, B, H, L, d, 0, C, F32, decay_mode=mode)
    got = run_backward(prob, inp, dout, dW, dM)
    ref = run_oracle_backward(inp, dout, dW, dM, C, mode)
    errs = {n: rel_fro(got[n], ref[n]) for n in NAMES}
    log("  rel_fro " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n in NAMES:
        assert np.all(np.isfinite(got[n])), n
        assert errs[n] <= TOL, (n, errs[n])
    return got


@pytest.mark.parametrize("B,H,L,d,C,mode,regime", [
    (1, 1, 256, 64, 64, 0, "default"),      # the linear workload's shape
    (2, 3, 200, 64, 64, 0, "default"),      # ragged last chunk, several units
    (1, 2, 150, 32, 48, 1, "default"),      # alpha taken as gamma; chunk not a tile multiple
    (1, 1, 1024, 64, 512, 0, "nearunit"),   # long segments: several tokens per lane
    (1, 1, 4096, 16, 2048, 0, "nearunit"),  # 32 tokens per lane in the scalar scan
    (1, 1, 10, 48, 1, 0, "default"),        # chunk of one token
])
def test_linear_backward_matches_oracle(B, H, L, d, C, mode, regime):
    check(B, H, L, d, C, mode, regime)


def test_linear_backward_without_state_gradients():
    check(1, 2, 130, 64, 64, seed=3, with_state=False)


def test_linear_backward_is_deterministic():
    import chunk_weight_update_amd as cwu  # noqa: F401
    B, H, L, d, C = 1, 2, 192, 64, 64
    inp = make_inputs(LINEAR, B, H, L, d, 0, F32, seed=5, m0_scale=0.01)
    dout, dW, dM = _upstream(B, H, L, d, 5)
    prob = problem_for(LINEAR, B, H, L, d, 0, C, F32)
    a = run_backward(prob, inp, dout, dW, dM)
    b = run_backward(prob, inp, dout, dW, dM)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n


def test_linear_backward_empty_sequence_passes_state_gradients():
    import torch
    import chunk_weight_update_amd as cwu
    B, H, d = 1, 2, 64
    prob = problem_for(LINEAR, B, H, 0, d, 0, 64, F32)
    W0 = torch.randn(B, H, d * d, device="cuda")
    M0 = torch.randn(B, H, d * d, device="cuda")
    dW = torch.randn(B, H, d * d, device="cuda")
    dM = torch.randn(B, H, d * d, device="cuda")
    gW = torch.full_like(W0, float("nan"))
    gM = torch.full_like(W0, float("nan"))
    cwu.chunk_backward(prob, None, None, None, None, None, None, W0, M0, None, dW, dM, None,
                       None, None, None, None, None, gW, gM, None, 0)
    cwu.chunk_backward(prob, None, None, None, None, None, None, W0, M0, None, dW, None, None,
                       None, None, None, None, None, gW, gM, None, 0)
    torch.cuda.synchronize()
    assert torch.equal(gW, dW)
    assert torch.count_nonzero(gM).item() == 0
