"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (relative Frobenius norm over the whole tensor):
  fp32 io   : out, W_end, M_end <= 1e-5
  bf16 io   : out <= 1e-2, W_end and M_end <= 5e-3
Scalar kernels (fp64 scan, fp32 output): elementwise <= 1e-6 relative.
"""
import numpy as np
import pytest

import oracle
from chunk_weight_update_amd.inputs import BF16, F32, LINEAR, SWIGLU, make_inputs
from gpu_util import log, problem_for, rel_fro, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu

TOL = {F32: (1e-5, 1e-5, 1e-5), BF16: (1e-2, 5e-3, 5e-3)}


def raw_projections(inp, io, seed):
    """Replace q, k by raw projection-like vectors (2 * N(0,1), not
    normalised), rounded to the io dtype exactly as the workload inputs are."""
    import torch
    rng = np.random.default_rng(1000 + seed)
    out = dict(inp)
    for n in ("q", "k"):
        x = (2.0 * rng.standard_normal(inp[n + "64"].shape)).astype(np.float32)
        if io == BF16:  # the io representation is the bf16 bit pattern
            xb = torch.from_numpy(x).to(torch.bfloat16)
            out[n] = xb.view(torch.int16).numpy().view(np.uint16)
            out[n + "64"] = xb.to(torch.float32).numpy().astype(np.float64)
        else:
            out[n] = x
            out[n + "64"] = x.astype(np.float64)
    return out


def check(kind, B, H, L, d, h, C, io, seed=0, regime="default", m0_scale=0.0, decay_mode=0,
          flags=0, tol=None, raw_qk=False):
    log(f"case kind={kind} B={B} H={H} L={L} d={d} h={h} C={C} io={io} seed={seed} "
        f"regime={regime} m0={m0_scale} mode={decay_mode} flags={flags} raw_qk={raw_qk}")
    inp = make_inputs(kind, B, H, L, d, h, io, seed=seed, regime=regime, m0_scale=m0_scale)
    if raw_qk:
        inp = raw_projections(inp, io, seed)
    prob = problem_for(kind, B, H, L, d, h, C, io, decay_mode, flags)
    out, W, M = run_gpu(prob, to_device(inp, io))
    ro, rW, rM = run_oracle(kind, inp, C, h, decay_mode, averaged=bool(flags & 2),
                            qk_norm=bool(flags & 4), row_norm=bool(flags & 8),
                            lact=bool(flags & 32), io=io)
    e = (rel_fro(out, ro), rel_fro(W, rW), rel_fro(M, rM))
    log(f"  rel_fro out={e[0]:.3e} W={e[1]:.3e} M={e[2]:.3e}")
    t = tol or TOL[io]
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(W)) and np.all(np.isfinite(M))
    assert e[0] <= t[0] and e[1] <= t[1] and e[2] <= t[2], e
    return e


# --- scalar kernels ---------------------------------------------------------

@pytest.mark.parametrize("B,H,L,C,regime,mode", [
    (1, 1, 256, 64, "default", 0),
    (2, 4, 4096, 512, "default", 0),
    (1, 2, 1000, 300, "nearunit", 0),     # short last chunk
    (1, 1, 8192 * 2 + 17, 8192, "default", 0),
    (2, 3, 777, 1, "default", 0),         # C = 1
    (1, 2, 640, 128, "default", 1),       # alpha taken as gamma
])
def test_scalar_kernels_match_oracle(B, H, L, C, regime, mode):
    import torch
    import chunk_weight_update_amd as cwu
    log(f"scan B={B} H={H} L={L} C={C} {regime} mode={mode}")
    inp = make_inputs(LINEAR, B, H, L, 16, 0, F32, seed=3, regime=regime)
    prob = cwu.make_problem(LINEAR, B, H, L, 16, 0, C, F32, mode)
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
                                              inp["beta"][..., sl].reshape(-1, n), mode)
        for got, ref in ((kw[..., sl].reshape(-1, n), okw), (km[..., sl].reshape(-1, n), okm),
                         (cf[:, :, r, :].reshape(-1, 3), ocf)):
            err = np.abs(got - ref)
            assert np.all(err <= 1e-6 * np.abs(ref) + 2e-38), float(np.max(err / (np.abs(ref) + 1e-300)))


@pytest.mark.parametrize("L,C,mode", [(3 * 12288 - 5, 12288, 0), (4096 + 1000, 2048, 1)])
def test_scalar_kernels_signs_and_zeros(L, C, mode):
    """Negative and zero factors: beta in [-1, 1] with exact zeros, and
    eta*alpha up to 4 so that gamma = 1 - eta*alpha changes sign (mode 0), or
    alpha itself in [-1, 1] (mode 1).  Exercises negative factors and exact
    zeros across several rounds of the scan."""
    import torch
    import chunk_weight_update_amd as cwu
    log(f"scan signs L={L} C={C} mode={mode}")
    rng = np.random.default_rng(11)
    eta = rng.uniform(0.0, 2.0, (1, 2, L)).astype(np.float32)
    alpha = (rng.uniform(0.0, 2.0, (1, 2, L)) if mode == 0
             else rng.uniform(-1.0, 1.0, (1, 2, L))).astype(np.float32)
    beta = rng.uniform(-1.0, 1.0, (1, 2, L)).astype(np.float32)
    beta[0, 0, ::997] = 0.0
    prob = cwu.make_problem(LINEAR, 1, 2, L, 16, 0, C, F32, mode)
    dev = [torch.from_numpy(x).cuda() for x in (eta, alpha, beta)]
    nC = -(-L // C)
    kw = torch.empty(1, 2, L, device="cuda")
    km = torch.empty(1, 2, L, device="cuda")
    cf = torch.empty(1, 2, nC, 3, device="cuda")
    cwu.scalar_kernels(prob, *dev, kw, km, cf)
    torch.cuda.synchronize()
    kw, km, cf = (x.cpu().numpy().astype(np.float64) for x in (kw, km, cf))
    for r in range(nC):
        sl = slice(r * C, min((r + 1) * C, L))
        n = sl.stop - sl.start
        okw, okm, ocf = oracle.scalar_kernels(eta[..., sl].reshape(-1, n),
                                              alpha[..., sl].reshape(-1, n),
                                              beta[..., sl].reshape(-1, n), mode)
        for got, ref in ((kw[..., sl].reshape(-1, n), okw), (km[..., sl].reshape(-1, n), okm),
                         (cf[:, :, r, :].reshape(-1, 3), ocf)):
            err = np.abs(got - ref)
            assert np.all(err <= 1e-6 * np.abs(ref) + 2e-38), float(np.max(err / (np.abs(ref) + 1e-300)))


@pytest.mark.parametrize("B,H,L,C,regime,mode", [
    (2, 4, 4096, 512, "default", 0),
    (1, 2, 1000, 300, "nearunit", 0),     # short last chunk
    (1, 1, 8192 * 2 + 17, 8192, "default", 0),
    (1, 2, 640, 128, "default", 1),
])
def test_scalar_kernels_chunk_averaged(B, H, L, C, regime, mode):
    """The chunk-averaged variant: beta and gamma replaced by their chunk
    means (segment reduction in the scan) before the kernels are formed."""
    import torch
    import chunk_weight_update_amd as cwu
    log(f"scan averaged B={B} H={H} L={L} C={C} {regime} mode={mode}")
    inp = make_inputs(LINEAR, B, H, L, 16, 0, F32, seed=5, regime=regime)
    prob = cwu.make_problem(LINEAR, B, H, L, 16, 0, C, F32, mode, cwu.FLAG_CHUNK_AVERAGED_DECAY)
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
                                              averaged=True)
        for got, ref in ((kw[..., sl].reshape(-1, n), okw), (km[..., sl].reshape(-1, n), okm),
                         (cf[:, :, r, :].reshape(-1, 3), ocf)):
            err = np.abs(got - ref)
            assert np.all(err <= 1e-6 * np.abs(ref) + 2e-38), float(np.max(err / (np.abs(ref) + 1e-300)))


@pytest.mark.parametrize("kind,B,H,L,d,h,C,io,regime", [
    (LINEAR, 1, 2, 600, 64, 0, 128, F32, "default"),          # ragged last chunk
    (SWIGLU, 1, 2, 600, 128, 256, 256, F32, "nearunit"),      # generic fp32 path
    (SWIGLU, 2, 2, 512, 128, 256, 256, BF16, "nearunit"),     # fused path, split phase B
    (SWIGLU, 1, 1, 700, 256, 512, 256, BF16, "nearunit"),     # 256-tile generic path
])
def test_chunk_averaged_forward(kind, B, H, L, d, h, C, io, regime):
    import chunk_weight_update_amd as cwu
    check(kind, B, H, L, d, h, C, io, seed=8, regime=regime,
          m0_scale=M0.get(regime, 0.0), flags=cwu.FLAG_CHUNK_AVERAGED_DECAY)


@pytest.mark.parametrize("kind,B,H,L,d,h,C,io,regime,flags", [
    (LINEAR, 1, 2, 600, 64, 0, 128, F32, "default", 0),        # ragged last chunk
    (SWIGLU, 1, 2, 600, 128, 256, 256, F32, "nearunit", 0),    # generic fp32 path
    (SWIGLU, 2, 2, 512, 128, 256, 128, BF16, "nearunit", 0),   # fused path, 4 chunks
    (SWIGLU, 4, 9, 1024, 128, 256, 512, BF16, "nearunit", 0),  # fused path, unsplit phase B
    (SWIGLU, 1, 1, 700, 256, 512, 256, BF16, "nearunit", 0),   # 256-tile generic path
    (SWIGLU, 2, 2, 512, 128, 256, 128, BF16, "nearunit", 1),   # with hi/lo weight operands
    (SWIGLU, 2, 2, 512, 128, 256, 128, BF16, "nearunit", 6),   # with chunk averaging, q/k prologue
    (LINEAR, 1, 2, 300, 32, 0, 64, F32, "default", 6),         # the same on the linear learner
    (SWIGLU, 1, 1, 512, 256, 512, 256, BF16, "nearunit", 6),   # the same on the 256-tile path
])
def test_post_chunk_row_normalisation_forward(kind, B, H, L, d, h, C, io, regime, flags):
    """Rows of the fast weights divided by their L2 norm after every chunk
    (App. B.1); the next chunk's readout, descent directions and operand
    shadows use the normalised weights."""
    import chunk_weight_update_amd as cwu
    check(kind, B, H, L, d, h, C, io, seed=12, regime=regime,
          m0_scale=M0.get(regime, 0.0), flags=cwu.FLAG_POST_CHUNK_ROW_L2 | flags)


@pytest.mark.parametrize("kind,B,H,L,d,h,C,io,regime", [
    (LINEAR, 1, 2, 600, 64, 0, 128, F32, "default"),
    (SWIGLU, 1, 2, 600, 128, 256, 256, F32, "nearunit"),
    (SWIGLU, 2, 2, 512, 128, 256, 256, BF16, "nearunit"),     # fused path
    (SWIGLU, 1, 1, 512, 256, 512, 256, BF16, "nearunit"),     # 256-tile generic path
])
def test_qk_prologue_forward(kind, B, H, L, d, h, C, io, regime):
    """q, k passed raw (scaled N(0,1), not normalised); the library applies
    SiLU and L2 normalisation per token, as the oracle does."""
    import chunk_weight_update_amd as cwu
    check(kind, B, H, L, d, h, C, io, seed=12, regime=regime, raw_qk=True,
          m0_scale=M0.get(regime, 0.0), flags=cwu.FLAG_QK_SILU_L2)


# --- linear learner ---------------------------------------------------------

def test_linear_d64_l256_c64_fp32():
    check(LINEAR, 1, 1, 256, 64, 0, 64, F32)


@pytest.mark.parametrize("B,H,L,d,C,io,m0", [
    (2, 3, 300, 32, 48, F32, 0.1),    # several chunks, short last chunk
    (1, 2, 1000, 128, 256, F32, 0.1),
    (1, 1, 129, 16, 200, F32, 0.0),   # one short chunk
    (2, 2, 512, 64, 64, BF16, 0.1),
])
def test_linear_shapes(B, H, L, d, C, io, m0):
    # bf16 io rounds the readout to bf16; the fp32 states keep the fp32 bar.
    check(LINEAR, B, H, L, d, 0, C, io, seed=1, m0_scale=m0,
          tol=(1e-5, 1e-5, 1e-5) if io == F32 else (1e-2, 1e-5, 1e-5))


# --- SwiGLU learner, small shapes -------------------------------------------

# M0 scale per regime: with near-unit momentum and decay a large M0 is added
# to W at every token and the cubic learner diverges (|W| grows by ~1e9 in
# 300 tokens), which makes any relative comparison ill-conditioned; the
# default regime forgets M0 within a few tokens.
M0 = {"nearunit": 1e-6, "default": 0.01}


@pytest.mark.parametrize("regime", ["nearunit", "default"])
@pytest.mark.parametrize("L,C", [(128, 128), (300, 128), (640, 256), (200, 100)])
def test_swiglu_fp32_small(regime, L, C):
    check(SWIGLU, 1, 2, L, 128, 128, C, F32, seed=2, regime=regime, m0_scale=M0[regime])


@pytest.mark.parametrize("L,C,d,h", [(512, 256, 128, 256), (300, 128, 128, 128),
                                     (1024, 512, 256, 384), (700, 256, 128, 256)])
def test_swiglu_bf16_small_nearunit(L, C, d, h):
    check(SWIGLU, 2, 2, L, d, h, C, BF16, seed=4, regime="nearunit", m0_scale=M0["nearunit"])


def test_swiglu_bf16_compensated_small():
    """hi/lo operand shadows on a token-split phase B (the split-sum state
    epilogue writes both shadow halves)."""
    import chunk_weight_update_amd as cwu
    check(SWIGLU, 2, 2, 512, 128, 256, 256, BF16, seed=6, regime="nearunit",
          m0_scale=M0["nearunit"], flags=cwu.FLAG_COMPENSATED_WEIGHTS)


def test_swiglu_bf16_many_units_unsplit():
    """Enough (unit, hidden block) workgroups that phase B is not
    token-split: the fused state epilogue inside phase B."""
    check(SWIGLU, 4, 32, 256, 128, 128, 128, BF16, seed=7, regime="nearunit",
          m0_scale=M0["nearunit"])


def test_swiglu_bf16_register_resident_phase_a():
    """64 units: several 32-row tiles per phase A workgroup (the variant with
    register-resident weights, h = 256), two chunks, the second ragged."""
    check(SWIGLU, 2, 32, 200, 128, 256, 128, BF16, seed=8, regime="nearunit",
          m0_scale=M0["nearunit"])


@pytest.mark.parametrize("L,C", [(700, 256), (512, 512), (600, 200)])
def test_swiglu_bf16_d256_tiled_aggregation(L, C):
    """d = 256, h = 512 bf16: the 256x256-tile aggregation with a token
    split and the split-sum state epilogue (generic path)."""
    check(SWIGLU, 1, 2, L, 256, 512, C, BF16, seed=9, regime="nearunit",
          m0_scale=M0["nearunit"])


def test_swiglu_bf16_d256_tiled_aggregation_compensated():
    """The split-sum state epilogue writing hi/lo operand shadows (compensated
    weights): the 256-tile aggregation with the 128-tile forward products."""
    import chunk_weight_update_amd as cwu
    check(SWIGLU, 2, 1, 700, 256, 512, 256, BF16, seed=10, regime="nearunit",
          m0_scale=M0["nearunit"], flags=cwu.FLAG_COMPENSATED_WEIGHTS)


def test_swiglu_alpha_is_gamma_fp32():
    check(SWIGLU, 1, 2, 384, 128, 128, 128, F32, seed=5, regime="nearunit",
          m0_scale=M0["nearunit"], decay_mode=1)


def test_swiglu_empty_sequence_copies_state():
    import torch
    import chunk_weight_update_amd as cwu
    inp = make_inputs(SWIGLU, 1, 2, 0, 128, 128, BF16, seed=0, m0_scale=0.1)
    t = to_device(inp, BF16)
    prob = problem_for(SWIGLU, 1, 2, 0, 128, 128, 128, BF16)
    out, W, M = run_gpu(prob, t)
    assert out.size == 0
    assert np.array_equal(W, inp["W0"].astype(np.float64))
    assert np.array_equal(M, inp["M0"].astype(np.float64))


@pytest.mark.parametrize("d,h", [
    (512, 768),    # readout tiles of 128 features, backward tiles of 192 units
    (768, 1024),   # readout tiles of 192 features, backward tiles of 128 units
    (1024, 256),   # both at 128, the largest d
])
def test_swiglu_bf16_256_path_tile_widths(d, h):
    """The 256-tile path's readout and backward take 192-wide tiles where 192
    divides d (readout) or h (backward), else 128-wide: every combination,
    two chunks with a ragged last one (Cp = 256)."""
    check(SWIGLU, 1, 1, 450, d, h, 256, BF16, seed=12, regime="nearunit",
          m0_scale=M0["nearunit"])
