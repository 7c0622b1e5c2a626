"""GPU parity of the MLP learner (f(x) = W2 silu(W1 x), E2-TTT_MLP) against
the oracle.  The learner runs on the SwiGLU kernels of the generic path with
the gate branch held at one; tolerances as for every learner: fp32 io 1e-5;
bf16 io 1e-2 on out, 5e-3 on W_end and M_end.

Under the default scalars each chunk rebuilds the state from the previous
one's gradients, so with plain bf16 weights the relative error compounds
from chunk to chunk (about 5e-3 after three chunks); plain-weight cases with
those scalars span at most two chunks, and a three-chunk trajectory runs
with the weights as hi/lo pairs."""
import pytest

import chunk_weight_update_amd as cwu
from chunk_weight_update_amd.inputs import BF16, F32, MLP
from test_gpu_parity import check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,H,L,d,h,C,io,regime,m0", [
    (1, 2, 600, 128, 256, 256, F32, "default", 0.01),    # generic fp32 path, ragged
    (1, 2, 600, 128, 256, 256, F32, "nearunit", 1e-6),
    (2, 4, 1024, 128, 256, 512, BF16, "default", 0.01),  # 128-tile bf16 path
    (2, 2, 512, 128, 256, 128, BF16, "nearunit", 1e-6),
    (1, 1, 500, 256, 512, 256, BF16, "default", 0.01),   # 256-tile path, split aggregation
    (1, 1, 700, 256, 512, 256, BF16, "nearunit", 1e-6),
])
def test_mlp_forward(B, H, L, d, h, C, io, regime, m0):
    check(MLP, B, H, L, d, h, C, io, seed=8, regime=regime, m0_scale=m0)


def test_mlp_three_collapsing_chunks_with_compensated_weights():
    """Three chunks under the default scalars rebuild the state each chunk
    from gradients of the previous one, so relative errors compound (plain
    bf16 weights: 5.1e-3 on W_end after three chunks of this case); with the
    weights as hi/lo pairs the whole trajectory meets the bar."""
    check(MLP, 2, 4, 1536, 128, 256, 512, BF16, seed=8, regime="default", m0_scale=0.01,
          flags=cwu.FLAG_COMPENSATED_WEIGHTS)


def test_mlp_d768_first_chunk():
    """The large layer's shape (d = 768, h = 1536, C = 8192), one chunk from
    W_0 under the default scalars."""
    check(MLP, 1, 1, 8192, 768, 1536, 8192, BF16, seed=0, regime="default", m0_scale=0.01)


@pytest.mark.parametrize("flags", [cwu.FLAG_LACT_RULE, cwu.FLAG_CHUNK_AVERAGED_DECAY,
                                   cwu.FLAG_POST_CHUNK_ROW_L2, cwu.FLAG_COMPENSATED_WEIGHTS])
def test_mlp_with_flags(flags):
    check(MLP, 1, 2, 640, 128, 256, 256, BF16, seed=9, regime="nearunit", m0_scale=1e-6,
          flags=flags)


def test_mlp_qk_prologue_and_row_normalisation_fp32():
    """The q/k prologue with row normalisation on fp32 io.  (With bf16 io
    this synthetic input -- raw projections 2 N(0,1), whose SiLU shares one
    large positive mean direction over all tokens -- amplifies the bf16
    rounding of the normalised q, k in the MLP's aggregates to ~1e-2; the
    fp32 path shows the arithmetic itself is the oracle's.)"""
    check(MLP, 1, 2, 640, 128, 256, 256, F32, seed=9, regime="nearunit", m0_scale=1e-6,
          flags=cwu.FLAG_QK_SILU_L2 | cwu.FLAG_POST_CHUNK_ROW_L2, raw_qk=True)
