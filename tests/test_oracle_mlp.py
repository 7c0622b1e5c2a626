"""Pins of the oracle's MLP learner (CPU only).

E2-TTT_MLP ("Rethinking Expressivity and Efficiency in Test-Time Training",
§5, App. B.3 Table 11, App. B.5) uses a fast-weight network smaller than the
three-matrix SwiGLU; the page names no activation.  Reading: f(x) =
W2 silu(W1 x), state [W1 (h x d) | W2 (d x h)].  Pinned like the SwiGLU
learner: the recurrence against the paper's closed form (§3.2 kernels in
ratio-sum form, per-token gradients from torch autograd), descent directions
against autograd and finite differences, C = 1 against online descent; and
one chunk against the independently pinned SwiGLU learner given an extra
constant input feature that its gate reads (so the gate is identically 1)."""
import numpy as np
import pytest
import torch

import oracle
from closed_form_np import autograd_descent, closed_form_forward, learner_forward



@pytest.fixture(autouse=True)
def _float64_default():
    """torch's default dtype is float64 inside this module's tests only (set
    at import it would leak into every module collected after this one)."""
    prev = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(prev)
MLP = oracle.MLP


def _problem(rng, L, d, h, m0=True, beta_lo=0.2):
    q = rng.standard_normal((1, 1, L, d))
    k = rng.standard_normal((1, 1, L, d))
    v = rng.standard_normal((1, 1, L, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    eta = 0.3 * rng.random((1, 1, L)) + 0.05
    alpha = rng.random((1, 1, L))
    beta = beta_lo + (1 - beta_lo) * rng.random((1, 1, L))
    W0 = rng.standard_normal((1, 1, 2 * d * h)) * 0.5
    M0 = rng.standard_normal((1, 1, 2 * d * h)) * 0.1 if m0 else np.zeros((1, 1, 2 * d * h))
    return q, k, v, eta, alpha, beta, W0, M0


@pytest.mark.parametrize("d,h", [(3, 5), (4, 6)])
@pytest.mark.parametrize("C,L", [(1, 3), (2, 6), (3, 3), (7, 21), (5, 12)])
def test_mlp_recurrence_matches_paper_closed_form(d, h, C, L):
    rng = np.random.default_rng(20 + C + L)
    q, k, v, eta, alpha, beta, W0, M0 = _problem(rng, L, d, h)
    out, W, M = oracle.chunk_forward(MLP, q, k, v, eta, alpha, beta, W0, M0, C, h)
    co, cW, cM = closed_form_forward(2, q[0, 0], k[0, 0], v[0, 0], eta[0, 0], alpha[0, 0],
                                     beta[0, 0], W0[0, 0], M0[0, 0], C, d, h)
    assert np.max(np.abs(out[0, 0] - co)) <= 1e-10
    assert np.max(np.abs(W[0, 0] - cW)) <= 1e-10
    assert np.max(np.abs(M[0, 0] - cM)) <= 1e-10


def test_mlp_descent_matches_autograd_and_finite_differences():
    rng = np.random.default_rng(21)
    d, h = 4, 6
    W = rng.standard_normal(2 * d * h) * 0.5
    k, v = rng.standard_normal(d), rng.standard_normal(d)
    G = oracle.token_descent(MLP, W, k, v, d, h)
    assert np.max(np.abs(G - autograd_descent(2, W, k, v, d, h))) <= 1e-12

    def loss(Wx):
        y = oracle.fast_forward(MLP, Wx, k, d, h)
        return 0.5 * np.sum((y - v) ** 2)
    eps = 1e-6
    fd = np.array([(loss(W + eps * e) - loss(W - eps * e)) / (2 * eps)
                   for e in np.eye(W.size)])
    assert np.max(np.abs(G + fd)) <= 1e-7


def test_mlp_chunk_of_one_is_online_descent():
    rng = np.random.default_rng(22)
    d, h, L = 3, 4, 10
    q, k, v, eta, alpha, beta, W0, M0 = _problem(rng, L, d, h)
    out, Wend, Mend = oracle.chunk_forward(MLP, q, k, v, eta, alpha, beta, W0, M0, 1, h)
    W, M = W0[0, 0].copy(), M0[0, 0].copy()
    for t in range(L):
        o = learner_forward(2, torch.tensor(W), torch.tensor(q[0, 0, t]), d, h).numpy()
        assert np.max(np.abs(o - out[0, 0, t])) <= 1e-12
        G = autograd_descent(2, W, k[0, 0, t], v[0, 0, t], d, h)
        M = beta[0, 0, t] * M + eta[0, 0, t] * G
        W = (1.0 - eta[0, 0, t] * alpha[0, 0, t]) * W + M
    assert np.max(np.abs(Wend[0, 0] - W)) <= 1e-12 and np.max(np.abs(Mend[0, 0] - M)) <= 1e-12


def test_mlp_equals_gated_swiglu_with_a_constant_gate_input():
    """SwiGLU on inputs x' = [x, 1] (d + 1 features) with W1' = [W1, 0],
    W3' = [0, 1] (every gate reads only the constant: a3 = 1) and W2' =
    [W2; 0], values v' = [v, 0]: within one chunk (all gradients at W_0) its
    readout and its W1', W2' updates restricted to the MLP's entries are the
    MLP's."""
    rng = np.random.default_rng(23)
    d, h, C = 3, 5, 6
    q, k, v, eta, alpha, beta, W0, M0 = _problem(rng, C, d, h)
    out, W, M = oracle.chunk_forward(MLP, q, k, v, eta, alpha, beta, W0, M0, C, h)
    pad1 = lambda x: np.concatenate([x, np.ones(x.shape[:-1] + (1,))], axis=-1)
    pad0 = lambda x: np.concatenate([x, np.zeros(x.shape[:-1] + (1,))], axis=-1)

    def lift(S):
        W1 = S[: h * d].reshape(h, d)
        W2 = S[h * d:].reshape(d, h)
        W1p = np.concatenate([W1, np.zeros((h, 1))], axis=1)
        W3p = np.zeros((h, d + 1))
        W2p = np.concatenate([W2, np.zeros((1, h))], axis=0)
        return np.concatenate([W1p.ravel(), W3p.ravel(), W2p.ravel()])
    W0s = lift(W0[0, 0])
    W0s[h * (d + 1): 2 * h * (d + 1)].reshape(h, d + 1)[:, d] = 1.0
    M0s = lift(M0[0, 0])
    os_, Ws, Ms = oracle.chunk_forward(oracle.SWIGLU, pad1(q), pad1(k), pad0(v), eta, alpha, beta,
                                       W0s[None, None], M0s[None, None], C, h)
    assert np.max(np.abs(os_[0, 0, :, :d] - out[0, 0])) <= 1e-13

    def restrict(S):
        W1p = S[: h * (d + 1)].reshape(h, d + 1)[:, :d]
        W2p = S[2 * h * (d + 1):].reshape(d + 1, h)[:d]
        return np.concatenate([W1p.ravel(), W2p.ravel()])
    assert np.max(np.abs(restrict(Ws[0, 0]) - W[0, 0])) <= 1e-13
    assert np.max(np.abs(restrict(Ms[0, 0]) - M[0, 0])) <= 1e-13


def test_mlp_row_normalisation_and_variants_run():
    rng = np.random.default_rng(24)
    d, h, C, L = 3, 4, 4, 10
    args = _problem(rng, L, d, h)
    _, W, _ = oracle.chunk_forward(MLP, *args, C, h, row_norm=True)
    W1 = W[0, 0, : h * d].reshape(h, d)
    W2 = W[0, 0, h * d:].reshape(d, h)
    assert np.allclose(np.linalg.norm(W1, axis=1), 1.0) and np.allclose(np.linalg.norm(W2, axis=1), 1.0)
    for kw in ({"averaged": True}, {"lact": True}, {"qk_norm": True}):
        o, W, M = oracle.chunk_forward(MLP, *args, C, h, **kw)
        assert np.all(np.isfinite(W)) and np.all(np.isfinite(o))
