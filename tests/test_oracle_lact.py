"""Pins of the oracle's LaCT rule (CPU only).

"Rethinking Expressivity and Efficiency in Test-Time Training", §3.2 ("Two
scalar kernels with distinct temporal weighting") contrasts E2-TTT with the
LaCT rule (Eq. 5, lost in extraction): LaCT weights each token's gradient by
eta_t alone, without the momentum suffix product or the decay ratio sum, and
collapses the momentum factor to a chunk average; §1 describes it as one
fast-weight update per chunk from the gradient of a summed loss.  The reading
under test (the oracle's header states it):

    M_C = mean(beta) M_0 + sum_t eta_t G_t,   W_C = mean(gamma) W_0 + M_C

Pinned against facts that do not reuse the oracle's code:
  - a chunk of one token is one step of the token-wise recurrence, so the
    rule must coincide with E2-TTT at C = 1 (E2-TTT at C = 1 is itself pinned
    to online descent with momentum in test_oracle.py);
  - with beta = 0 and gamma = 1 each chunk is the plain step on the gradient
    of the eta-weighted summed loss, from torch autograd;
  - the linear learner's aggregate is a library matmul;
  - the rule has no position-dependent weighting: permuting the tokens of a
    chunk leaves the state unchanged (E2-TTT's does change: the test fails
    for a rule that kept the suffix-product weighting).
"""
import numpy as np
import pytest
import torch

import oracle
from closed_form_np import learner_forward



@pytest.fixture(autouse=True)
def _float64_default():
    """torch's default dtype is float64 inside this module's tests only (set
    at import it would leak into every module collected after this one)."""
    prev = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(prev)


def _problem(rng, kind, L, d, h, m0=True):
    q = rng.standard_normal((1, 1, L, d))
    k = rng.standard_normal((1, 1, L, d))
    v = rng.standard_normal((1, 1, L, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    eta = 0.3 * rng.random((1, 1, L)) + 0.05
    alpha = rng.random((1, 1, L))
    beta = 0.2 + 0.8 * rng.random((1, 1, L))
    P = d * d if kind == oracle.LINEAR else 3 * d * h
    W0 = rng.standard_normal((1, 1, P)) * 0.5
    M0 = rng.standard_normal((1, 1, P)) * 0.1 if m0 else np.zeros((1, 1, P))
    return q, k, v, eta, alpha, beta, W0, M0


CASES = [(oracle.LINEAR, 3, 0), (oracle.LINEAR, 5, 0), (oracle.SWIGLU, 3, 4),
         (oracle.SWIGLU, 4, 6)]


@pytest.mark.parametrize("kind,d,h", CASES)
@pytest.mark.parametrize("mode", [oracle.GAMMA_1_MINUS_ETA_ALPHA, oracle.ALPHA_IS_GAMMA])
def test_lact_chunk_of_one_is_the_token_recurrence(kind, d, h, mode):
    rng = np.random.default_rng(11)
    args = _problem(rng, kind, 9, d, h)
    e2 = oracle.chunk_forward(kind, *args, 1, h, decay_mode=mode)
    la = oracle.chunk_forward(kind, *args, 1, h, decay_mode=mode, lact=True)
    for x, y in zip(e2, la):
        assert np.max(np.abs(x - y)) <= 1e-14


@pytest.mark.parametrize("kind,d,h", CASES)
@pytest.mark.parametrize("C,L", [(4, 8), (5, 13), (16, 16)])
def test_lact_without_momentum_and_decay_is_summed_loss_step(kind, d, h, C, L):
    """beta = 0, alpha = 0 (gamma = 1): per chunk, W_C = W_0 - grad of
    sum_t eta_t 0.5||f_W(k_t) - v_t||^2 at W_0 and M_C = W_C - W_0."""
    rng = np.random.default_rng(12)
    q, k, v, eta, alpha, beta, W0, M0 = _problem(rng, kind, L, d, h)
    alpha[:] = 0.0
    beta[:] = 0.0
    out, Wend, Mend = oracle.chunk_forward(kind, q, k, v, eta, alpha, beta, W0, M0, C, h,
                                           lact=True)
    W = W0[0, 0].copy()
    M = M0[0, 0].copy()
    for t0 in range(0, L, C):
        Wt = torch.tensor(W, requires_grad=True)
        total = 0.0
        for t in range(t0, min(t0 + C, L)):
            o = learner_forward(kind, torch.tensor(W), torch.tensor(q[0, 0, t]), d, h)
            assert np.max(np.abs(o.numpy() - out[0, 0, t])) <= 1e-12
            y = learner_forward(kind, Wt, torch.tensor(k[0, 0, t]), d, h)
            total = total + eta[0, 0, t] * 0.5 * ((y - torch.tensor(v[0, 0, t])) ** 2).sum()
        (g,) = torch.autograd.grad(total, Wt)
        M = -g.numpy()
        W = W + M
    assert np.max(np.abs(Wend[0, 0] - W)) <= 1e-12
    assert np.max(np.abs(Mend[0, 0] - M)) <= 1e-12


@pytest.mark.parametrize("C,L", [(4, 12), (6, 17)])
def test_lact_linear_learner_is_a_matmul_aggregate(C, L):
    """Linear learner, general scalars: per chunk the rule is
    mean(gamma) W_0 + mean(beta) M_0 + (V - K W_0^T)^T diag(eta) K."""
    rng = np.random.default_rng(13)
    d = 5
    q, k, v, eta, alpha, beta, W0, M0 = _problem(rng, oracle.LINEAR, L, d, 0)
    _, Wend, Mend = oracle.chunk_forward(oracle.LINEAR, q, k, v, eta, alpha, beta, W0, M0, C,
                                         0, lact=True)
    W = W0[0, 0].reshape(d, d).copy()
    M = M0[0, 0].reshape(d, d).copy()
    for t0 in range(0, L, C):
        sl = slice(t0, min(t0 + C, L))
        K, V, e = k[0, 0, sl], v[0, 0, sl], eta[0, 0, sl]
        gam = 1.0 - e * alpha[0, 0, sl]
        A = (V - K @ W.T).T @ (e[:, None] * K)
        M = beta[0, 0, sl].mean() * M + A
        W = gam.mean() * W + M
    assert np.max(np.abs(Wend[0, 0] - W.ravel())) <= 1e-12
    assert np.max(np.abs(Mend[0, 0] - M.ravel())) <= 1e-12


@pytest.mark.parametrize("kind,d,h", [(oracle.LINEAR, 4, 0), (oracle.SWIGLU, 3, 5)])
def test_lact_ignores_token_order_within_a_chunk(kind, d, h):
    rng = np.random.default_rng(14)
    C, L = 6, 18
    q, k, v, eta, alpha, beta, W0, M0 = _problem(rng, kind, L, d, h)
    perm = np.concatenate([t0 + rng.permutation(C) for t0 in range(0, L, C)])
    args = (q, k, v, eta, alpha, beta)
    pargs = tuple(a[:, :, perm] for a in args)
    o1, W1, M1 = oracle.chunk_forward(kind, *args, W0, M0, C, h, lact=True)
    o2, W2, M2 = oracle.chunk_forward(kind, *pargs, W0, M0, C, h, lact=True)
    assert np.max(np.abs(W1 - W2)) <= 1e-12 and np.max(np.abs(M1 - M2)) <= 1e-12
    assert np.max(np.abs(o1[:, :, perm] - o2)) <= 1e-12
    # E2-TTT weights tokens by position, so its state does depend on the order.
    _, E1, _ = oracle.chunk_forward(kind, *args, W0, M0, C, h)
    _, E2, _ = oracle.chunk_forward(kind, *pargs, W0, M0, C, h)
    assert np.max(np.abs(E1 - E2)) > 1e-6


def test_lact_scalar_kernels_give_the_forward_state():
    """The impulse-response kernels of the rule, put through the linear
    learner's aggregate (a library matmul), give the forward's state."""
    rng = np.random.default_rng(15)
    d, C = 4, 7
    q, k, v, eta, alpha, beta, W0, M0 = _problem(rng, oracle.LINEAR, C, d, 0)
    kw, km, coef = oracle.scalar_kernels(eta[0], alpha[0], beta[0], lact=True)
    _, Wend, Mend = oracle.chunk_forward(oracle.LINEAR, q, k, v, eta, alpha, beta, W0, M0, C, 0,
                                         lact=True)
    W = W0[0, 0].reshape(d, d)
    M = M0[0, 0].reshape(d, d)
    E = v[0, 0] - k[0, 0] @ W.T
    cW, cM, cWM = coef[0]
    assert np.max(np.abs(Wend[0, 0] - (cW * W + cWM * M + E.T @ (kw[0][:, None] * k[0, 0])).ravel())) <= 1e-12
    assert np.max(np.abs(Mend[0, 0] - (cM * M + E.T @ (km[0][:, None] * k[0, 0])).ravel())) <= 1e-12


def test_lact_and_averaged_are_exclusive_and_have_no_reverse_mode():
    rng = np.random.default_rng(16)
    args = _problem(rng, oracle.LINEAR, 4, 3, 0)
    with pytest.raises(ValueError):
        oracle.chunk_forward(oracle.LINEAR, *args, 2, 0, averaged=True, lact=True)
