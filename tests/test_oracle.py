"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test ties the oracle to a fact fixed by E2-TTT ("Rethinking
Expressivity and Efficiency in Test-Time Training") or by mathematics:
  - the kernel formulas of §3.2 in their ratio-sum form (closed_form_np.py)
    reproduce the literal recurrence (the abstract and §3.2 claim the
    chunk-end weight and momentum of the token recurrence exactly);
  - per-token descent directions equal torch autograd and finite differences;
  - with no momentum (beta = 0) and no decay (gamma = 1) the chunk update is
    a plain summed-gradient step at W_0 (the LaCT-style update of §3.2);
  - gamma = 0 makes W_t = M_t (App. A.3, aggressive-decay limit);
  - C = 1 is token-wise online descent with momentum (App. B.3: in the
    limit of one-token chunks the update is the token-wise one);
  - constant scalars give geometric-series kernels (App. A.3 regimes);
  - readout with the chunk-start weights (Eq. 6);
  - linearity of the linear learner in (W_0, M_0, v);
  - cross-chunk induction: a run split at a chunk boundary resumes exactly
    (§3.2);
  - a worked example by hand (tests/golden/).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from closed_form_np import (autograd_descent, closed_form_forward,
                            learner_forward, paper_kernels)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_problem(rng, kind, L, d, h, beta_lo=0.2, m0=True):
    q = rng.standard_normal((1, 1, L, d))
    k = rng.standard_normal((1, 1, L, d))
    v = rng.standard_normal((1, 1, L, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    eta = 0.3 * rng.random((1, 1, L)) + 0.05
    alpha = rng.random((1, 1, L))
    beta = beta_lo + (1 - beta_lo) * rng.random((1, 1, L))
    P = d * d if kind == oracle.LINEAR else 3 * d * h
    W0 = rng.standard_normal((1, 1, P)) * 0.5
    M0 = rng.standard_normal((1, 1, P)) * 0.1 if m0 else np.zeros((1, 1, P))
    return q, k, v, eta, alpha, beta, W0, M0


def _rel(a, b):
    return np.linalg.norm(np.ravel(a - b)) / max(np.linalg.norm(np.ravel(b)), 1e-300)


@pytest.mark.parametrize("kind,d,h", [(oracle.LINEAR, 3, 0), (oracle.LINEAR, 4, 0),
                                      (oracle.SWIGLU, 3, 5), (oracle.SWIGLU, 4, 6)])
@pytest.mark.parametrize("C,nchunks", [(1, 3), (2, 3), (3, 1), (7, 3), (16, 1), (5, 2.4)])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_recurrence_matches_paper_closed_form(kind, d, h, C, nchunks, seed):
    rng = np.random.default_rng(100 + seed)
    L = int(round(C * nchunks))  # 5 * 2.4 = 12: a short last chunk
    q, k, v, eta, alpha, beta, W0, M0 = _rand_problem(rng, kind, L, d, h)
    out, Wend, Mend = oracle.chunk_forward(kind, q, k, v, eta, alpha, beta, W0, M0, C, h)
    out2, W2, M2 = closed_form_forward(kind, q[0, 0], k[0, 0], v[0, 0], eta[0, 0],
                                       alpha[0, 0], beta[0, 0], W0[0, 0], M0[0, 0], C, d, h)
    assert _rel(Wend[0, 0], W2) <= 1e-10
    assert _rel(Mend[0, 0], M2) <= 1e-10
    assert _rel(out[0, 0], out2) <= 1e-12


def test_alpha_is_gamma_mode_matches_closed_form():
    rng = np.random.default_rng(7)
    d, h, C, L = 3, 4, 4, 12
    q, k, v, eta, alpha, beta, W0, M0 = _rand_problem(rng, oracle.SWIGLU, L, d, h)
    alpha = 0.5 + 0.5 * rng.random((1, 1, L))
    _, Wend, Mend = oracle.chunk_forward(oracle.SWIGLU, q, k, v, eta, alpha, beta, W0, M0, C, h,
                                         decay_mode=oracle.ALPHA_IS_GAMMA)
    _, W2, M2 = closed_form_forward(oracle.SWIGLU, q[0, 0], k[0, 0], v[0, 0], eta[0, 0],
                                    alpha[0, 0], beta[0, 0], W0[0, 0], M0[0, 0], C, d, h,
                                    alpha_is_gamma=True)
    assert _rel(Wend[0, 0], W2) <= 1e-10 and _rel(Mend[0, 0], M2) <= 1e-10


@pytest.mark.parametrize("kind,d,h", [(oracle.LINEAR, 5, 0), (oracle.SWIGLU, 4, 7)])
def test_descent_direction_matches_autograd(kind, d, h):
    rng = np.random.default_rng(3)
    for _ in range(5):
        P = d * d if kind == oracle.LINEAR else 3 * d * h
        W = rng.standard_normal(P)
        k = rng.standard_normal(d)
        v = rng.standard_normal(d)
        G = oracle.token_descent(kind, W, k, v, d, h)
        Ga = autograd_descent(kind, W, k, v, d, h)
        assert np.max(np.abs(G - Ga)) <= 1e-12 * max(1.0, np.max(np.abs(Ga)))


def test_descent_direction_matches_finite_differences():
    rng = np.random.default_rng(4)
    d, h = 3, 4
    W = rng.standard_normal(3 * d * h) * 0.7
    k = rng.standard_normal(d)
    v = rng.standard_normal(d)

    def loss(Wv):
        y = oracle.fast_forward(oracle.SWIGLU, Wv, k, d, h)
        return 0.5 * np.sum((y - v) ** 2)

    G = oracle.token_descent(oracle.SWIGLU, W, k, v, d, h)
    eps = 1e-6
    fd = np.empty_like(W)
    for i in range(W.size):
        e = np.zeros_like(W)
        e[i] = eps
        fd[i] = -(loss(W + e) - loss(W - e)) / (2 * eps)
    assert np.max(np.abs(G - fd)) <= 1e-7


def test_no_momentum_no_decay_is_summed_gradient_step():
    """beta = 0, alpha = 0 (gamma = 1): W_C = W_0 - grad sum_t eta_t l_t(W_0),
    M_C = eta_C G_C (one chunk)."""
    rng = np.random.default_rng(5)
    d, h, C = 4, 6, 9
    q, k, v, eta, alpha, beta, W0, M0 = _rand_problem(rng, oracle.SWIGLU, C, d, h, m0=False)
    alpha[:] = 0.0
    beta[:] = 0.0
    _, Wend, Mend = oracle.chunk_forward(oracle.SWIGLU, q, k, v, eta, alpha, beta, W0, M0, C, h)
    Wt = torch.tensor(W0[0, 0], requires_grad=True)
    total = 0.0
    for t in range(C):
        y = learner_forward(1, Wt, torch.tensor(k[0, 0, t]), d, h)
        total = total + eta[0, 0, t] * 0.5 * ((y - torch.tensor(v[0, 0, t])) ** 2).sum()
    (g,) = torch.autograd.grad(total, Wt)
    assert np.max(np.abs(Wend[0, 0] - (W0[0, 0] - g.numpy()))) <= 1e-12
    GC = autograd_descent(1, W0[0, 0], k[0, 0, C - 1], v[0, 0, C - 1], d, h)
    assert np.max(np.abs(Mend[0, 0] - eta[0, 0, C - 1] * GC)) <= 1e-12


def test_gamma_zero_makes_weight_equal_momentum():
    rng = np.random.default_rng(6)
    d, h, C, L = 3, 5, 4, 8
    q, k, v, eta, alpha, beta, W0, M0 = _rand_problem(rng, oracle.SWIGLU, L, d, h)
    alpha[:] = 0.0  # gamma = alpha = 0
    _, Wend, Mend = oracle.chunk_forward(oracle.SWIGLU, q, k, v, eta, alpha, beta, W0, M0, C, h,
                                         decay_mode=oracle.ALPHA_IS_GAMMA)
    assert np.max(np.abs(Wend - Mend)) <= 1e-14
    kw, km, coef = oracle.scalar_kernels(eta[0, :, :4], alpha[0, :, :4], beta[0, :, :4],
                                         decay_mode=oracle.ALPHA_IS_GAMMA)
    assert np.array_equal(kw, km) and coef[0, 0] == 0.0 and coef[0, 1] == coef[0, 2]


@pytest.mark.parametrize("kind,d,h", [(oracle.LINEAR, 3, 0), (oracle.SWIGLU, 3, 4)])
def test_chunk_of_one_is_online_descent_with_momentum(kind, d, h):
    """C = 1: the gradient of each token is taken at the current weights."""
    rng = np.random.default_rng(8)
    L = 10
    q, k, v, eta, alpha, beta, W0, M0 = _rand_problem(rng, kind, L, d, h)
    out, Wend, Mend = oracle.chunk_forward(kind, q, k, v, eta, alpha, beta, W0, M0, 1, h)
    W = W0[0, 0].copy()
    M = M0[0, 0].copy()
    for t in range(L):
        o = learner_forward(kind, torch.tensor(W), torch.tensor(q[0, 0, t]), d, h).numpy()
        assert np.max(np.abs(o - out[0, 0, t])) <= 1e-12
        G = autograd_descent(kind, W, k[0, 0, t], v[0, 0, t], d, h)
        M = beta[0, 0, t] * M + eta[0, 0, t] * G
        W = (1.0 - eta[0, 0, t] * alpha[0, 0, t]) * W + M
    assert np.max(np.abs(Wend[0, 0] - W)) <= 1e-12
    assert np.max(np.abs(Mend[0, 0] - M)) <= 1e-12


@pytest.mark.parametrize("b,g", [(0.5, 0.9), (0.9, 0.5), (0.7, 0.7), (0.999, 0.9995)])
def test_constant_scalars_kernels_are_geometric(b, g):
    n = 37
    eta = np.full((1, n), 0.25)
    beta = np.full((1, n), b)
    alpha = np.full((1, n), g)
    kw, km, coef = oracle.scalar_kernels(eta, alpha, beta, decay_mode=oracle.ALPHA_IS_GAMMA)
    m = n - 1 - np.arange(n)  # later tokens in the chunk
    assert np.max(np.abs(km[0] - 0.25 * b ** m)) <= 1e-12
    if b != g:
        P = (g ** (m + 1) - b ** (m + 1)) / (g - b)
    else:
        P = (m + 1) * b ** m
    assert np.max(np.abs(kw[0] - 0.25 * P) / (0.25 * P)) <= 1e-12
    assert abs(coef[0, 0] - g ** n) <= 1e-14
    assert abs(coef[0, 1] - b ** n) <= 1e-14
    # M_0 enters W_C like an impulse one token before the first, decayed by beta.
    P0 = (g ** n - b ** n) / (g - b) if b != g else n * b ** (n - 1)
    assert abs(coef[0, 2] - b * P0) <= 1e-12 * max(1.0, b * P0)


def test_near_unit_kernel_limit():
    """beta, gamma -> 1: K^M -> eta, K^W/eta -> number of remaining updates
    (App. A.3 regime (i))."""
    n = 64
    eta = np.full((1, n), 0.5)
    one = np.ones((1, n))
    kw, km, coef = oracle.scalar_kernels(eta, one, one, decay_mode=oracle.ALPHA_IS_GAMMA)
    assert np.array_equal(km[0], eta[0])
    assert np.array_equal(kw[0], 0.5 * (n - np.arange(n)))
    assert coef[0].tolist() == [1.0, 1.0, float(n)]


def test_scalar_kernels_match_paper_ratio_sums():
    rng = np.random.default_rng(9)
    n = 24
    eta = 0.1 * rng.random((3, n))
    alpha = rng.random((3, n))
    beta = 0.3 + 0.7 * rng.random((3, n))
    kw, km, coef = oracle.scalar_kernels(eta, alpha, beta)
    for s in range(3):
        KW, KM, cW, cM, cWM = paper_kernels(eta[s], 1 - eta[s] * alpha[s], beta[s])
        assert np.max(np.abs(kw[s] - KW) / KW) <= 1e-12
        assert np.max(np.abs(km[s] - KM) / KM) <= 1e-12
        assert np.allclose(coef[s], [cW, cM, cWM], rtol=1e-12, atol=0)


def test_readout_uses_chunk_start_weights():
    rng = np.random.default_rng(10)
    d, h, C, L = 4, 6, 5, 15
    q, k, v, eta, alpha, beta, W0, M0 = _rand_problem(rng, oracle.SWIGLU, L, d, h)
    out, _, _ = oracle.chunk_forward(oracle.SWIGLU, q, k, v, eta, alpha, beta, W0, M0, C, h)
    for r in range(3):
        if r == 0:
            Ws = W0[0, 0]
        else:
            _, Wp, _ = oracle.chunk_forward(oracle.SWIGLU, q[..., :r * C, :], k[..., :r * C, :],
                                            v[..., :r * C, :], eta[..., :r * C], alpha[..., :r * C],
                                            beta[..., :r * C], W0, M0, C, h)
            Ws = Wp[0, 0]
        Wt = torch.tensor(Ws)
        Q = torch.tensor(q[0, 0, r * C:(r + 1) * C])
        W1 = Wt[: h * d].reshape(h, d)
        W3 = Wt[h * d: 2 * h * d].reshape(h, d)
        W2 = Wt[2 * h * d:].reshape(d, h)
        ref = (torch.nn.functional.silu(Q @ W1.T) * (Q @ W3.T)) @ W2.T
        assert np.max(np.abs(out[0, 0, r * C:(r + 1) * C] - ref.numpy())) <= 1e-12


def test_linear_learner_is_linear_in_state_and_values():
    rng = np.random.default_rng(11)
    d, C, L = 4, 3, 9
    q, k, v, eta, alpha, beta, W0, M0 = _rand_problem(rng, oracle.LINEAR, L, d, 0)
    _, _, v2, _, _, _, W0b, M0b = _rand_problem(rng, oracle.LINEAR, L, d, 0)
    a, b = 0.7, -1.3
    r1 = oracle.chunk_forward(0, q, k, v, eta, alpha, beta, W0, M0, C)
    r2 = oracle.chunk_forward(0, q, k, v2, eta, alpha, beta, W0b, M0b, C)
    r3 = oracle.chunk_forward(0, q, k, a * v + b * v2, eta, alpha, beta, a * W0 + b * W0b,
                              a * M0 + b * M0b, C)
    for x1, x2, x3 in zip(r1, r2, r3):
        assert np.max(np.abs(x3 - (a * x1 + b * x2))) <= 1e-12


@pytest.mark.parametrize("kind,d,h", [(oracle.LINEAR, 4, 0), (oracle.SWIGLU, 4, 6)])
def test_resume_at_chunk_boundary_is_exact(kind, d, h):
    rng = np.random.default_rng(12)
    C, L, L1 = 4, 14, 8
    q, k, v, eta, alpha, beta, W0, M0 = _rand_problem(rng, kind, L, d, h)
    out, W, M = oracle.chunk_forward(kind, q, k, v, eta, alpha, beta, W0, M0, C, h)
    oa, Wa, Ma = oracle.chunk_forward(kind, q[..., :L1, :], k[..., :L1, :], v[..., :L1, :],
                                      eta[..., :L1], alpha[..., :L1], beta[..., :L1], W0, M0, C, h)
    ob, Wb, Mb = oracle.chunk_forward(kind, q[..., L1:, :], k[..., L1:, :], v[..., L1:, :],
                                      eta[..., L1:], alpha[..., L1:], beta[..., L1:], Wa, Ma, C, h)
    assert np.array_equal(np.concatenate([oa, ob], axis=2), out)
    assert np.array_equal(Wb, W) and np.array_equal(Mb, M)


def test_units_are_independent_and_empty_sequence_copies_state():
    rng = np.random.default_rng(13)
    d, h, C, L = 3, 4, 3, 7
    probs = [_rand_problem(rng, oracle.SWIGLU, L, d, h) for _ in range(4)]
    cat = [np.concatenate([p[i] for p in probs], axis=0).reshape((2, 2) + probs[0][i].shape[2:])
           for i in range(8)]
    out, W, M = oracle.chunk_forward(oracle.SWIGLU, *cat, C, h)
    for u, p in enumerate(probs):
        o1, W1, M1 = oracle.chunk_forward(oracle.SWIGLU, *p, C, h)
        assert np.array_equal(out.reshape(4, L, d)[u], o1[0, 0])
        assert np.array_equal(W.reshape(4, -1)[u], W1[0, 0])
    e = [x[..., :0, :] if x.ndim == 4 and x.shape[-2] == L else x for x in cat[:3]]
    s = [x[..., :0] for x in cat[3:6]]
    out0, W0e, M0e = oracle.chunk_forward(oracle.SWIGLU, *e, *s, cat[6], cat[7], C, h)
    assert out0.size == 0 and np.array_equal(W0e, cat[6]) and np.array_equal(M0e, cat[7])


def test_handworked_linear_example():
    with open(os.path.join(GOLDEN, "linear_d2_handworked.json")) as f:
        g = json.load(f)
    L, d = len(g["eta"]), g["d"]
    arr = lambda x: np.asarray(x, dtype=np.float64)
    out, W, M = oracle.chunk_forward(
        oracle.LINEAR, arr(g["q"]).reshape(1, 1, L, d), arr(g["k"]).reshape(1, 1, L, d),
        arr(g["v"]).reshape(1, 1, L, d), arr(g["eta"]).reshape(1, 1, L),
        arr(g["alpha"]).reshape(1, 1, L), arr(g["beta"]).reshape(1, 1, L),
        arr(g["W0"]).reshape(1, 1, d * d), arr(g["M0"]).reshape(1, 1, d * d), g["chunk"])
    assert np.array_equal(out[0, 0], arr(g["expected_out"]))
    assert np.array_equal(W[0, 0].reshape(d, d), arr(g["expected_Wend"]))
    assert np.array_equal(M[0, 0].reshape(d, d), arr(g["expected_Mend"]))


def test_planted_mistakes_are_caught():
    """A wrong sign or a dropped decay in a copy of the recurrence breaks the
    closed-form agreement by far more than the 1e-10 bar."""
    rng = np.random.default_rng(14)
    d, C, L = 3, 4, 8
    q, k, v, eta, alpha, beta, W0, M0 = _rand_problem(rng, oracle.LINEAR, L, d, 0)
    _, Wref, _ = closed_form_forward(0, q[0, 0], k[0, 0], v[0, 0], eta[0, 0], alpha[0, 0],
                                     beta[0, 0], W0[0, 0], M0[0, 0], C, d)

    def mutated(sign=1.0, use_decay=True):
        W = W0[0, 0].copy()
        M = M0[0, 0].copy()
        for t0 in range(0, L, C):
            Ws = W.copy().reshape(d, d)
            for t in range(t0, t0 + C):
                G = np.outer(v[0, 0, t] - Ws @ k[0, 0, t], k[0, 0, t]).ravel()
                M = beta[0, 0, t] * M + sign * eta[0, 0, t] * G
                gam = 1 - eta[0, 0, t] * alpha[0, 0, t] if use_decay else 1.0
                W = gam * W + M
        return W

    assert _rel(mutated(), Wref) <= 1e-10
    assert _rel(mutated(sign=-1.0), Wref) > 1e-3
    assert _rel(mutated(use_decay=False), Wref) > 1e-3


# --- Chunk-averaged variant (the ablation of §5.4 / App. B.3 of the E2-TTT
# page: per-token beta_t, gamma_t collapsed to chunk-level scalars; reading:
# arithmetic means over the chunk's tokens).

def _chunk_means(x, C):
    """Per-token array whose entries are the means of x over each chunk."""
    y = np.empty_like(x)
    L = x.shape[-1]
    for t0 in range(0, L, C):
        y[..., t0:t0 + C] = np.mean(x[..., t0:t0 + C], axis=-1, keepdims=True)
    return y


@pytest.mark.parametrize("kind,d,h", [(oracle.LINEAR, 4, 0), (oracle.SWIGLU, 3, 5)])
@pytest.mark.parametrize("C,L", [(3, 9), (7, 17), (5, 5)])
def test_chunk_averaged_is_recurrence_on_averaged_factors(kind, d, h, C, L):
    """The averaged run equals the plain recurrence fed the chunk means of beta
    and of gamma = 1 - eta*alpha (passed as gamma directly), means by numpy."""
    rng = np.random.default_rng(7 + C)
    q, k, v, eta, alpha, beta, W0, M0 = _rand_problem(rng, kind, L, d, h)
    out, Wend, Mend = oracle.chunk_forward(kind, q, k, v, eta, alpha, beta, W0, M0, C, h,
                                           averaged=True)
    gbar = _chunk_means(1.0 - eta * alpha, C)
    bbar = _chunk_means(beta, C)
    out2, W2, M2 = oracle.chunk_forward(kind, q, k, v, eta, gbar, bbar, W0, M0, C, h,
                                        decay_mode=oracle.ALPHA_IS_GAMMA)
    assert _rel(Wend, W2) <= 1e-12 and _rel(Mend, M2) <= 1e-12
    assert np.array_equal(out, out2)  # the readout does not depend on the factors
    # and it differs from the per-token rule once the factors vary
    _, W3, _ = oracle.chunk_forward(kind, q, k, v, eta, alpha, beta, W0, M0, C, h)
    assert _rel(Wend, W3) > 1e-6


def test_chunk_averaged_kernels_are_geometric_in_the_means():
    """Closed form with constant factors, evaluated at numpy's chunk means."""
    rng = np.random.default_rng(11)
    n = 29
    eta = 0.05 + 0.2 * rng.random((2, n))
    alpha = rng.random((2, n))
    beta = 0.3 + 0.6 * rng.random((2, n))
    kw, km, coef = oracle.scalar_kernels(eta, alpha, beta, averaged=True)
    for sg in range(2):
        b = float(np.mean(beta[sg]))
        g = float(np.mean(1.0 - eta[sg] * alpha[sg]))
        m = n - 1 - np.arange(n)
        assert np.max(np.abs(km[sg] - eta[sg] * b ** m) / (eta[sg] * b ** m)) <= 1e-12
        P = (g ** (m + 1) - b ** (m + 1)) / (g - b)
        assert np.max(np.abs(kw[sg] - eta[sg] * P) / (eta[sg] * P)) <= 1e-12
        assert abs(coef[sg, 0] - g ** n) <= 1e-13 * g ** n
        assert abs(coef[sg, 1] - b ** n) <= 1e-13 * b ** n
        P0 = (g ** n - b ** n) / (g - b)
        assert abs(coef[sg, 2] - b * P0) <= 1e-12 * b * P0


# --- q/k prologue (§4 "Overall Architecture" of the E2-TTT page: SiLU on the
# queries and keys, then L2 normalisation per token).

@pytest.mark.parametrize("kind,d,h", [(oracle.LINEAR, 5, 0), (oracle.SWIGLU, 4, 6)])
def test_qk_prologue_is_silu_then_l2_normalisation(kind, d, h):
    """The option equals the plain run on inputs prepared by the library
    routines torch.nn.functional.silu and .normalize (eps 1e-12)."""
    rng = np.random.default_rng(21)
    L, C = 11, 4
    q, k, v, eta, alpha, beta, W0, M0 = _rand_problem(rng, kind, L, d, h)
    q = 3.0 * rng.standard_normal(q.shape)  # raw projections, not normalised
    k = 3.0 * rng.standard_normal(k.shape)
    q[0, 0, 2] = 0.0                        # a zero row stays zero
    out, Wend, Mend = oracle.chunk_forward(kind, q, k, v, eta, alpha, beta, W0, M0, C, h,
                                           qk_norm=True)
    F = torch.nn.functional
    prep = lambda x: F.normalize(F.silu(torch.from_numpy(x)), dim=-1, eps=1e-12).numpy()
    out2, W2, M2 = oracle.chunk_forward(kind, prep(q), prep(k), v, eta, alpha, beta, W0, M0,
                                        C, h)
    assert _rel(out, out2) <= 1e-13 and _rel(Wend, W2) <= 1e-13 and _rel(Mend, M2) <= 1e-13
    assert np.all(out[0, 0, 2] == 0.0)


@pytest.mark.parametrize("kind,d,h", [(oracle.LINEAR, 5, 0), (oracle.SWIGLU, 4, 6)])
def test_qk_prologue_rounded_to_bf16(kind, d, h):
    """With qk_round_bf16 the option equals the plain run on inputs prepared
    by torch's silu and normalize, then rounded to bf16 by torch's own
    conversion (fp32, then bf16 to nearest even); the rounding changes the
    result (it is not a no-op on these inputs)."""
    rng = np.random.default_rng(22)
    L, C = 13, 5
    q, k, v, eta, alpha, beta, W0, M0 = _rand_problem(rng, kind, L, d, h)
    q = 3.0 * rng.standard_normal(q.shape)
    k = 3.0 * rng.standard_normal(k.shape)
    out, Wend, Mend = oracle.chunk_forward(kind, q, k, v, eta, alpha, beta, W0, M0, C, h,
                                           qk_norm=True, qk_round_bf16=True)
    F = torch.nn.functional
    prep = lambda x: (F.normalize(F.silu(torch.from_numpy(x)), dim=-1, eps=1e-12)
                      .float().to(torch.bfloat16).double().numpy())
    out2, W2, M2 = oracle.chunk_forward(kind, prep(q), prep(k), v, eta, alpha, beta, W0, M0,
                                        C, h)
    assert _rel(out, out2) <= 1e-13 and _rel(Wend, W2) <= 1e-13 and _rel(Mend, M2) <= 1e-13
    out3, W3, M3 = oracle.chunk_forward(kind, q, k, v, eta, alpha, beta, W0, M0, C, h,
                                        qk_norm=True)
    assert _rel(Wend, W3) > 1e-5


def _normalise_rows_np(kind, W, d, h):
    """Rows of every fast-weight matrix divided by max(||row||, 1e-12) (numpy)."""
    W = np.array(W, dtype=np.float64)
    parts = [(0, d, d)] if kind == oracle.LINEAR else [(0, 2 * h, d), (2 * h * d, d, h)]
    for off, rows, cols in parts:
        blk = W[..., off:off + rows * cols].reshape(W.shape[:-1] + (rows, cols))
        nrm = np.maximum(np.linalg.norm(blk, axis=-1, keepdims=True), 1e-12)
        W[..., off:off + rows * cols] = (blk / nrm).reshape(W.shape[:-1] + (rows * cols,))
    return W


@pytest.mark.parametrize("kind,d,h", [(oracle.LINEAR, 4, 0), (oracle.SWIGLU, 3, 5)])
@pytest.mark.parametrize("C,L", [(3, 10), (4, 4), (1, 3)])
def test_row_norm_is_chunkwise_row_normalisation(kind, d, h, C, L):
    """Chunk-boundary normalisation (App. B.1): the run with the option equals
    chunk-by-chunk runs without it, with every fast-weight row divided by its
    norm (numpy) between chunks and after the last; readouts of later chunks
    see the normalised weights, and M is untouched by the normalisation."""
    rng = np.random.default_rng(31 + C + L + d)
    q, k, v, eta, alpha, beta, W0, M0 = _rand_problem(rng, kind, L, d, h)
    out, We, Me = oracle.chunk_forward(kind, q, k, v, eta, alpha, beta, W0, M0, C, h,
                                       row_norm=True)
    W, M, outs = W0, M0, []
    for t0 in range(0, L, C):
        sl = slice(t0, min(L, t0 + C))
        o, W, M = oracle.chunk_forward(kind, q[:, :, sl], k[:, :, sl], v[:, :, sl],
                                       eta[:, :, sl], alpha[:, :, sl], beta[:, :, sl], W, M,
                                       C, h)
        W = _normalise_rows_np(kind, W, d, h)
        outs.append(o)
    assert _rel(out, np.concatenate(outs, axis=2)) <= 1e-13
    assert _rel(We, W) <= 1e-13
    assert _rel(Me, M) <= 1e-13
    assert np.allclose(_normalise_rows_np(kind, We, d, h), We, rtol=0, atol=1e-14)
    # the option changes the result (the normalisation is not a no-op here)
    _, W_plain, _ = oracle.chunk_forward(kind, q, k, v, eta, alpha, beta, W0, M0, C, h)
    assert _rel(We, W_plain) > 1e-3
