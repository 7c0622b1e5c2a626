"""GPU parity of the LaCT rule (E2TTT_FLAG_LACT_RULE) against the oracle.

The rule reuses every kernel of the chunk forward; only the scalar kernels
differ (K^W = K^M = eta, chunk coefficients from the means of beta and
gamma).  Tolerances as for the default rule: fp32 io 1e-5; bf16 io 1e-2 on
out, 5e-3 on W_end and M_end; scalar kernels 1e-6 elementwise."""
import numpy as np
import pytest

import chunk_weight_update_amd as cwu
import oracle
from chunk_weight_update_amd.inputs import BF16, F32, LINEAR, SWIGLU, WORKLOADS, make_inputs
from gpu_util import log
from test_gpu_parity import check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,H,L,C,mode", [
    (2, 4, 4096, 512, 0),
    (1, 2, 1000, 300, 0),          # short last chunk
    (1, 1, 8192 * 2 + 17, 8192, 1),
])
def test_scalar_kernels_lact(B, H, L, C, mode):
    import torch
    log(f"scan lact B={B} H={H} L={L} C={C} mode={mode}")
    inp = make_inputs(LINEAR, B, H, L, 16, 0, F32, seed=6)
    prob = cwu.make_problem(LINEAR, B, H, L, 16, 0, C, F32, mode, cwu.FLAG_LACT_RULE)
    dev = {n: torch.from_numpy(inp[n]).cuda() for n in ("eta", "alpha", "beta")}
    nC = -(-L // C)
    kw = torch.empty(B, H, L, device="cuda")
    km = torch.empty(B, H, L, device="cuda")
    cf = torch.empty(B, H, nC, 3, device="cuda")
    cwu.scalar_kernels(prob, dev["eta"], dev["alpha"], dev["beta"], kw, km, cf)
    torch.cuda.synchronize()
    kw, km, cf = (x.cpu().numpy().astype(np.float64) for x in (kw, km, cf))
    for r in range(nC):
        sl = slice(r * C, min((r + 1) * C, L))
        n = sl.stop - sl.start
        okw, okm, ocf = oracle.scalar_kernels(inp["eta"][..., sl].reshape(-1, n),
                                              inp["alpha"][..., sl].reshape(-1, n),
                                              inp["beta"][..., sl].reshape(-1, n), mode,
                                              lact=True)
        for got, ref in ((kw[..., sl].reshape(-1, n), okw), (km[..., sl].reshape(-1, n), okm),
                         (cf[:, :, r, :].reshape(-1, 3), ocf)):
            err = np.abs(got - ref)
            assert np.all(err <= 1e-6 * np.abs(ref) + 2e-38), float(np.max(err / (np.abs(ref) + 1e-300)))


@pytest.mark.parametrize("kind,B,H,L,d,h,C,io,regime,mode", [
    (LINEAR, 1, 2, 600, 64, 0, 128, F32, "default", 0),      # ragged last chunk
    (LINEAR, 2, 1, 256, 32, 0, 64, BF16, "default", 1),
    (SWIGLU, 1, 2, 600, 128, 256, 256, F32, "nearunit", 0),  # generic fp32 path
    (SWIGLU, 1, 2, 600, 128, 256, 256, F32, "default", 0),
    (SWIGLU, 2, 2, 512, 128, 256, 256, BF16, "nearunit", 0), # fused path, split phase B
    (SWIGLU, 1, 1, 700, 256, 512, 256, BF16, "nearunit", 0), # 256-tile generic path
])
def test_lact_forward(kind, B, H, L, d, h, C, io, regime, mode):
    check(kind, B, H, L, d, h, C, io, seed=8, regime=regime, m0_scale=0.01, decay_mode=mode,
          flags=cwu.FLAG_LACT_RULE)


def test_lact_with_prologue_and_row_normalisation():
    check(SWIGLU, 1, 2, 512, 128, 256, 128, BF16, seed=9, regime="nearunit", m0_scale=0.01,
          flags=cwu.FLAG_LACT_RULE | cwu.FLAG_QK_SILU_L2 | cwu.FLAG_POST_CHUNK_ROW_L2,
          raw_qk=True)


def test_lact_bench_shape_whole_trajectory():
    """The B2 x H4, L 4096, C 512 bf16 layer with the default scalars, all
    eight chunks in one call: under the LaCT rule the state decays once per
    chunk and stays O(1), so the whole trajectory is compared."""
    w = WORKLOADS["swiglu-d128h256-b2h4-l4096-c512-bf16"]
    check(w.kind, w.B, w.H, w.L, w.d, w.h, w.C, w.io, seed=0, regime="default",
          flags=cwu.FLAG_LACT_RULE)
