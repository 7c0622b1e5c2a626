"""A seeded sweep of forward shapes on the 256-tile path (bf16, d and h
multiples of 256) against the oracle: both gated learners, batch and heads,
ragged sequence lengths, chunk lengths whose padded size is or is not a
multiple of 256 (the latter take the 128-tile forward with the same split
aggregation), decay mode and flags drawn once from a fixed seed; near-unit
scalars (the carried state stays in fp32's normal range).

Every case is held to the bf16 bars (1e-2 on out, 5e-3 on W_end and M_end)
unless the problem itself moves by more than the bar when its q, k and v
carry one bf16 rounding (relative noise of RMS 2^-8/sqrt(3), the size of a
round-to-nearest error at 8 significant bits, on the oracle's inputs): no
bf16 operand path can then be expected inside the bar, and the case is held
to that measured sensitivity instead (logged).  In this draw that happens
for the MLP learner with alpha read as the retention itself (mode 1, so
under the near-unit scalars gamma = 0.1 sigma(z), about 5% kept per token),
the q/k prologue and row normalisation (sensitivity 8.6e-3 on W_end, 8.5e-3
on M_end), and, barely, for M_end of a SwiGLU case with the prologue and
row normalisation (5.1e-3)."""
import numpy as np
import pytest

from chunk_weight_update_amd.inputs import BF16, MLP, SWIGLU, make_inputs
from gpu_util import log, rel_fro, run_oracle
from test_gpu_parity import M0, TOL, check

pytestmark = pytest.mark.gpu


def _cases(n=8, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = SWIGLU if i % 2 == 0 else MLP
        d = int(rng.choice([256, 512]))
        h = int(rng.choice([256, 512, 768]))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        L = int(rng.integers(200, 1300))
        C = int(rng.integers(96, 700))
        mode = int(rng.integers(0, 2))
        flags = int(rng.choice([0, 2, 4, 8, 32, 10, 12]))
        out.append((kind, B, H, L, d, h, C, mode, flags, 300 + i))
    return out


def bf16_sensitivity(kind, B, H, L, d, h, C, mode, flags, seed):
    """rel_fro change of (out, W_end, M_end) of the oracle when q, k, v get
    relative noise of the size of one bf16 rounding (fixed seed)."""
    inp = make_inputs(kind, B, H, L, d, h, BF16, seed=seed, regime="nearunit",
                      m0_scale=M0["nearunit"])
    kw = dict(decay_mode=mode, averaged=bool(flags & 2), qk_norm=bool(flags & 4),
              row_norm=bool(flags & 8), lact=bool(flags & 32), io=BF16)
    ref = run_oracle(kind, inp, C, h, **kw)
    rng = np.random.default_rng(7)
    noisy = dict(inp)
    for n in ("q64", "k64", "v64"):
        noisy[n] = inp[n] * (1.0 + 2.0 ** -8 / np.sqrt(3.0) * rng.standard_normal(inp[n].shape))
    per = run_oracle(kind, noisy, C, h, **kw)
    return tuple(rel_fro(p, r) for p, r in zip(per, ref))


@pytest.mark.parametrize("kind,B,H,L,d,h,C,mode,flags,seed", _cases())
def test_forward_shape_sweep_256(kind, B, H, L, d, h, C, mode, flags, seed):
    s = bf16_sensitivity(kind, B, H, L, d, h, C, mode, flags, seed)
    tol = tuple(max(t, si) for t, si in zip(TOL[BF16], s))
    log(f"  bf16 sensitivity out={s[0]:.2e} W={s[1]:.2e} M={s[2]:.2e}; bars {tol}")
    check(kind, B, H, L, d, h, C, BF16, seed=seed, regime="nearunit", m0_scale=M0["nearunit"],
          decay_mode=mode, flags=flags, tol=tol)
