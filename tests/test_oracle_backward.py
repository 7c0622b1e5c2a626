"""Pins of the oracle's reverse mode (linear and SwiGLU learners, CPU only).

The outer-loop backward of the chunk forward is pinned to two things other
than itself:
  - central finite differences of the oracle's own forward (the literal
    recurrence of App. A.5, itself pinned in test_oracle.py), one input class
    at a time, so a wrong or missing term in any one gradient fails;
  - torch autograd through an independent fp64 closed form of the chunk
    update (the kernels of §3.2 / Appendix A: suffix products, the affine
    reverse scan P_t = c_t + beta_{t+1} P_{t+1}, and the aggregation
    E^T diag(K) K), written here in torch and differentiated by the library.
"""
import numpy as np
import pytest
import torch

import oracle

NAMES = ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")


def _problem(rng, B, H, L, d, mode):
    q = rng.standard_normal((B, H, L, d))
    k = rng.standard_normal((B, H, L, d)) / np.sqrt(d)
    v = rng.standard_normal((B, H, L, d))
    eta = 0.3 * rng.random((B, H, L)) + 0.05
    alpha = rng.random((B, H, L)) if mode == oracle.GAMMA_1_MINUS_ETA_ALPHA else \
        0.5 + 0.5 * rng.random((B, H, L))
    beta = rng.random((B, H, L))
    W0 = rng.standard_normal((B, H, d * d)) * 0.5
    M0 = rng.standard_normal((B, H, d * d)) * 0.3
    return dict(q=q, k=k, v=v, eta=eta, alpha=alpha, beta=beta, W0=W0, M0=M0)


def _loss(x, C, mode, dout, dWe, dMe):
    o, We, Me = oracle.chunk_forward(oracle.LINEAR, x["q"], x["k"], x["v"], x["eta"],
                                     x["alpha"], x["beta"], x["W0"], x["M0"], C,
                                     decay_mode=mode)
    return float((dout * o).sum() + (dWe * We).sum() + (dMe * Me).sum())


@pytest.mark.parametrize("mode", [oracle.GAMMA_1_MINUS_ETA_ALPHA, oracle.ALPHA_IS_GAMMA])
@pytest.mark.parametrize("L,C", [(7, 3), (6, 6), (5, 1)])
def test_backward_matches_finite_differences(mode, L, C):
    rng = np.random.default_rng(100 + L + 10 * C + mode)
    B, H, d = 1, 2, 3
    x = _problem(rng, B, H, L, d, mode)
    dout = rng.standard_normal((B, H, L, d))
    dWe = rng.standard_normal((B, H, d * d))
    dMe = rng.standard_normal((B, H, d * d))
    g = oracle.chunk_backward(oracle.LINEAR, *[x[n] for n in NAMES], dout, dWe, dMe, C,
                              decay_mode=mode)
    h = 1e-6
    for name in NAMES:
        dl = rng.standard_normal(x[name].shape)
        xp = dict(x); xp[name] = x[name] + h * dl
        xm = dict(x); xm[name] = x[name] - h * dl
        fd = (_loss(xp, C, mode, dout, dWe, dMe) - _loss(xm, C, mode, dout, dWe, dMe)) / (2 * h)
        an = float((g[name] * dl).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def _closed_form_torch(x, C, mode):
    """Chunk forward of the linear learner by the closed form, in torch fp64."""
    q, k, v = x["q"], x["k"], x["v"]
    eta, alpha, beta = x["eta"], x["alpha"], x["beta"]
    B, H, L, d = q.shape
    W = x["W0"].reshape(B, H, d, d)
    M = x["M0"].reshape(B, H, d, d)
    gam = 1.0 - eta * alpha if mode == oracle.GAMMA_1_MINUS_ETA_ALPHA else alpha
    outs = []
    for t0 in range(0, L, C):
        n = min(C, L - t0)
        sl = slice(t0, t0 + n)
        Q, K, V = q[:, :, sl], k[:, :, sl], v[:, :, sl]
        be, ga, et = beta[:, :, sl], gam[:, :, sl], eta[:, :, sl]
        # exclusive suffix products b_t = prod_{s>t} beta_s, c_t likewise
        ones = torch.ones_like(be[..., :1])
        b_all = torch.flip(torch.cumprod(torch.flip(torch.cat([be[..., 1:], ones], -1), [-1]), -1), [-1])
        c_all = torch.flip(torch.cumprod(torch.flip(torch.cat([ga[..., 1:], ones], -1), [-1]), -1), [-1])
        # P_t = c_t + beta_{t+1} P_{t+1}, P of the last token = 1
        Ps = [None] * n
        Ps[n - 1] = c_all[..., n - 1]
        for t in range(n - 2, -1, -1):
            Ps[t] = c_all[..., t] + be[..., t + 1] * Ps[t + 1]
        Pt = torch.stack(Ps, -1)
        KW, KM = et * Pt, et * b_all
        cW = torch.prod(ga, -1)
        cM = torch.prod(be, -1)
        cWM = be[..., 0] * Pt[..., 0]
        E = V - torch.einsum("bhij,bhtj->bhti", W, K)
        outs.append(torch.einsum("bhij,bhtj->bhti", W, Q))
        AW = torch.einsum("bhti,bht,bhtj->bhij", E, KW, K)
        AM = torch.einsum("bhti,bht,bhtj->bhij", E, KM, K)
        W, M = (cW[..., None, None] * W + cWM[..., None, None] * M + AW,
                cM[..., None, None] * M + AM)
    return torch.cat(outs, 2), W.reshape(B, H, d * d), M.reshape(B, H, d * d)


@pytest.mark.parametrize("mode", [oracle.GAMMA_1_MINUS_ETA_ALPHA, oracle.ALPHA_IS_GAMMA])
@pytest.mark.parametrize("L,C,d", [(9, 4, 3), (16, 16, 4), (11, 3, 5)])
def test_backward_matches_autograd_of_closed_form(mode, L, C, d):
    rng = np.random.default_rng(200 + L + C + d + mode)
    B, H = 2, 1
    x = _problem(rng, B, H, L, d, mode)
    dout = rng.standard_normal((B, H, L, d))
    dWe = rng.standard_normal((B, H, d * d))
    dMe = rng.standard_normal((B, H, d * d))
    xt = {n: torch.tensor(x[n], dtype=torch.float64, requires_grad=True) for n in NAMES}
    o, We, Me = _closed_form_torch(xt, C, mode)
    loss = (torch.tensor(dout) * o).sum() + (torch.tensor(dWe) * We).sum() + \
        (torch.tensor(dMe) * Me).sum()
    loss.backward()
    g = oracle.chunk_backward(oracle.LINEAR, *[x[n] for n in NAMES], dout, dWe, dMe, C,
                              decay_mode=mode)
    for n in NAMES:
        ref = xt[n].grad.numpy()
        err = np.linalg.norm(g[n] - ref) / max(np.linalg.norm(ref), 1e-300)
        assert err <= 1e-10, (n, err)


def test_backward_without_state_gradients_and_empty_sequence():
    """dWend = dMend = None means zero; L = 0 passes the state gradients
    through unchanged (Wend = W0, Mend = M0)."""
    rng = np.random.default_rng(7)
    B, H, L, d, C = 1, 1, 5, 3, 2
    x = _problem(rng, B, H, L, d, 0)
    dout = rng.standard_normal((B, H, L, d))
    z = np.zeros((B, H, d * d))
    g0 = oracle.chunk_backward(oracle.LINEAR, *[x[n] for n in NAMES], dout, None, None, C)
    g1 = oracle.chunk_backward(oracle.LINEAR, *[x[n] for n in NAMES], dout, z, z, C)
    for n in NAMES:
        np.testing.assert_array_equal(g0[n], g1[n])
    e = {n: (x[n][:, :, :0] if n not in ("W0", "M0") else x[n]) for n in NAMES}
    dWe = rng.standard_normal((B, H, d * d))
    dMe = rng.standard_normal((B, H, d * d))
    ge = oracle.chunk_backward(oracle.LINEAR, *[e[n] for n in NAMES],
                               np.zeros((B, H, 0, d)), dWe, dMe, C)
    np.testing.assert_array_equal(ge["W0"], dWe)
    np.testing.assert_array_equal(ge["M0"], dMe)


# --------------------------------------------------------------------------
# SwiGLU learner f(x) = W2 (silu(W1 x) * (W3 x)), state [W1 | W3 | W2].

def _problem_sw(rng, B, H, L, d, hd, mode):
    x = _problem(rng, B, H, L, d, mode)
    P = 3 * d * hd
    x["k"] = rng.standard_normal((B, H, L, d)) / np.sqrt(d)
    x["W0"] = rng.standard_normal((B, H, P)) * 0.6
    x["M0"] = rng.standard_normal((B, H, P)) * 0.3
    return x


def _loss_sw(x, C, mode, hd, dout, dWe, dMe):
    o, We, Me = oracle.chunk_forward(oracle.SWIGLU, x["q"], x["k"], x["v"], x["eta"],
                                     x["alpha"], x["beta"], x["W0"], x["M0"], C,
                                     hidden=hd, decay_mode=mode)
    return float((dout * o).sum() + (dWe * We).sum() + (dMe * Me).sum())


@pytest.mark.parametrize("mode", [oracle.GAMMA_1_MINUS_ETA_ALPHA, oracle.ALPHA_IS_GAMMA])
@pytest.mark.parametrize("L,C", [(7, 3), (5, 5), (4, 1)])
def test_swiglu_backward_matches_finite_differences(mode, L, C):
    rng = np.random.default_rng(300 + L + 10 * C + mode)
    B, H, d, hd = 1, 2, 3, 4
    x = _problem_sw(rng, B, H, L, d, hd, mode)
    P = 3 * d * hd
    dout = rng.standard_normal((B, H, L, d))
    dWe = rng.standard_normal((B, H, P))
    dMe = rng.standard_normal((B, H, P))
    g = oracle.chunk_backward(oracle.SWIGLU, *[x[n] for n in NAMES], dout, dWe, dMe, C,
                              decay_mode=mode, hidden=hd)
    eps = 1e-6
    for name in NAMES:
        dl = rng.standard_normal(x[name].shape)
        xp = dict(x); xp[name] = x[name] + eps * dl
        xm = dict(x); xm[name] = x[name] - eps * dl
        fd = (_loss_sw(xp, C, mode, hd, dout, dWe, dMe) -
              _loss_sw(xm, C, mode, hd, dout, dWe, dMe)) / (2 * eps)
        an = float((g[name] * dl).sum())
        assert abs(fd - an) <= 2e-7 * max(1.0, abs(an)), (name, fd, an)


def _closed_form_swiglu_torch(x, C, mode, hd):
    """Chunk forward of the SwiGLU learner by the closed form, in torch fp64:
    per-token descent factors at the chunk-start weights, the two kernels
    from suffix products and the reverse affine scan, and the aggregations
    U^T diag(K) X per matrix."""
    q, k, v = x["q"], x["k"], x["v"]
    eta, alpha, beta = x["eta"], x["alpha"], x["beta"]
    B, H, L, d = q.shape

    def split(S):
        return (S[..., :hd * d].reshape(B, H, hd, d), S[..., hd * d:2 * hd * d].reshape(B, H, hd, d),
                S[..., 2 * hd * d:].reshape(B, H, d, hd))

    def join(W1, W3, W2):
        return torch.cat([W1.reshape(B, H, -1), W3.reshape(B, H, -1), W2.reshape(B, H, -1)], -1)

    def silu(a):
        return a * torch.sigmoid(a)

    def f(W1, W3, W2, X):
        a1 = X @ W1.transpose(-1, -2)
        a3 = X @ W3.transpose(-1, -2)
        z = silu(a1) * a3
        return a1, a3, z, z @ W2.transpose(-1, -2)

    W1, W3, W2 = split(x["W0"])
    M1, M3, M2 = split(x["M0"])
    gam = 1.0 - eta * alpha if mode == oracle.GAMMA_1_MINUS_ETA_ALPHA else alpha
    outs = []
    for t0 in range(0, L, C):
        n = min(C, L - t0)
        sl = slice(t0, t0 + n)
        Q, K, V = q[:, :, sl], k[:, :, sl], v[:, :, sl]
        be, ga, et = beta[:, :, sl], gam[:, :, sl], eta[:, :, sl]
        ones = torch.ones_like(be[..., :1])
        b_all = torch.flip(torch.cumprod(torch.flip(torch.cat([be[..., 1:], ones], -1), [-1]), -1), [-1])
        c_all = torch.flip(torch.cumprod(torch.flip(torch.cat([ga[..., 1:], ones], -1), [-1]), -1), [-1])
        Ps = [None] * n
        Ps[n - 1] = c_all[..., n - 1]
        for t in range(n - 2, -1, -1):
            Ps[t] = c_all[..., t] + be[..., t + 1] * Ps[t + 1]
        Pt = torch.stack(Ps, -1)
        KW, KM = et * Pt, et * b_all
        cW, cM, cWM = torch.prod(ga, -1), torch.prod(be, -1), be[..., 0] * Pt[..., 0]
        outs.append(f(W1, W3, W2, Q)[3])
        a1, a3, z, y = f(W1, W3, W2, K)
        e = V - y                                   # descent factor of W2: e z^T
        w = e @ W2                                  # W2^T e per token
        sg = torch.sigmoid(a1)
        u1 = w * a3 * (sg * (1.0 + a1 * (1.0 - sg)))  # factor of W1: u1 k^T
        u3 = w * silu(a1)                            # factor of W3: u3 k^T

        def agg(Kv, U, X):
            return (U * Kv[..., None]).transpose(-1, -2) @ X

        cw, cm, cwm = cW[..., None, None], cM[..., None, None], cWM[..., None, None]
        nW1 = cw * W1 + cwm * M1 + agg(KW, u1, K)
        nW3 = cw * W3 + cwm * M3 + agg(KW, u3, K)
        nW2 = cw * W2 + cwm * M2 + agg(KW, e, z)
        M1, M3, M2 = cm * M1 + agg(KM, u1, K), cm * M3 + agg(KM, u3, K), cm * M2 + agg(KM, e, z)
        W1, W3, W2 = nW1, nW3, nW2
    return torch.cat(outs, 2), join(W1, W3, W2), join(M1, M3, M2)


def test_swiglu_closed_form_reproduces_the_oracle_forward():
    """The torch closed form used below is itself the oracle's forward."""
    rng = np.random.default_rng(11)
    B, H, L, d, hd, C = 1, 2, 10, 4, 5, 4
    x = _problem_sw(rng, B, H, L, d, hd, 0)
    o, We, Me = oracle.chunk_forward(oracle.SWIGLU, *[x[n] for n in NAMES], C, hidden=hd)
    xt = {n: torch.tensor(x[n], dtype=torch.float64) for n in NAMES}
    ot, Wt, Mt = _closed_form_swiglu_torch(xt, C, 0, hd)
    for a, b in ((o, ot), (We, Wt), (Me, Mt)):
        assert np.linalg.norm(a - b.numpy()) <= 1e-12 * np.linalg.norm(a)


@pytest.mark.parametrize("mode", [oracle.GAMMA_1_MINUS_ETA_ALPHA, oracle.ALPHA_IS_GAMMA])
@pytest.mark.parametrize("L,C,d,hd", [(9, 4, 3, 5), (8, 8, 4, 6), (10, 3, 2, 3)])
def test_swiglu_backward_matches_autograd_of_closed_form(mode, L, C, d, hd):
    rng = np.random.default_rng(400 + L + C + d + hd + mode)
    B, H = 2, 1
    P = 3 * d * hd
    x = _problem_sw(rng, B, H, L, d, hd, mode)
    dout = rng.standard_normal((B, H, L, d))
    dWe = rng.standard_normal((B, H, P))
    dMe = rng.standard_normal((B, H, P))
    xt = {n: torch.tensor(x[n], dtype=torch.float64, requires_grad=True) for n in NAMES}
    o, We, Me = _closed_form_swiglu_torch(xt, C, mode, hd)
    loss = (torch.tensor(dout) * o).sum() + (torch.tensor(dWe) * We).sum() + \
        (torch.tensor(dMe) * Me).sum()
    loss.backward()
    g = oracle.chunk_backward(oracle.SWIGLU, *[x[n] for n in NAMES], dout, dWe, dMe, C,
                              decay_mode=mode, hidden=hd)
    for n in NAMES:
        ref = xt[n].grad.numpy()
        err = np.linalg.norm(g[n] - ref) / max(np.linalg.norm(ref), 1e-300)
        assert err <= 1e-10, (n, err)


@pytest.mark.parametrize("kind", [oracle.LINEAR, oracle.SWIGLU])
def test_backward_through_qk_prologue_matches_finite_differences(kind):
    """With the q/k prologue (SiLU, then L2 per token) dq and dk are mapped
    back through it; checked, with every other input, against central
    differences of the oracle's forward with the prologue."""
    rng = np.random.default_rng(500 + kind)
    B, H, L, d, hd, C = 1, 2, 7, 3, 4, 3
    if kind == oracle.LINEAR:
        x, hd, P = _problem(rng, B, H, L, d, 0), 0, d * d
    else:
        x, P = _problem_sw(rng, B, H, L, d, hd, 0), 3 * d * hd
    x["q"] = rng.standard_normal((B, H, L, d))   # raw inputs: the prologue normalises them
    x["k"] = rng.standard_normal((B, H, L, d))
    dout = rng.standard_normal((B, H, L, d))
    dWe = rng.standard_normal((B, H, P))
    dMe = rng.standard_normal((B, H, P))
    g = oracle.chunk_backward(kind, *[x[n] for n in NAMES], dout, dWe, dMe, C, hidden=hd,
                              qk_norm=True)

    def loss(xx):
        o, We, Me = oracle.chunk_forward(kind, *[xx[n] for n in NAMES], C, hidden=hd,
                                         qk_norm=True)
        return float((dout * o).sum() + (dWe * We).sum() + (dMe * Me).sum())
    eps = 1e-6
    for name in NAMES:
        dl = rng.standard_normal(x[name].shape)
        xp = dict(x); xp[name] = x[name] + eps * dl
        xm = dict(x); xm[name] = x[name] - eps * dl
        fd = (loss(xp) - loss(xm)) / (2 * eps)
        an = float((g[name] * dl).sum())
        assert abs(fd - an) <= 2e-7 * max(1.0, abs(an)), (name, fd, an)


@pytest.mark.parametrize("kind,mode", [(oracle.LINEAR, oracle.GAMMA_1_MINUS_ETA_ALPHA),
                                       (oracle.SWIGLU, oracle.ALPHA_IS_GAMMA)])
def test_backward_chunk_averaged_matches_finite_differences(kind, mode):
    """Chunk-averaged variant: every token of a chunk uses the chunk means of
    beta and gamma; checked against central differences of the oracle's
    forward in that variant (a ragged last chunk included)."""
    rng = np.random.default_rng(600 + kind)
    B, H, L, d, hd, C = 1, 2, 8, 3, 4, 3
    if kind == oracle.LINEAR:
        x, hd, P = _problem(rng, B, H, L, d, mode), 0, d * d
    else:
        x, P = _problem_sw(rng, B, H, L, d, hd, mode), 3 * d * hd
    dout = rng.standard_normal((B, H, L, d))
    dWe = rng.standard_normal((B, H, P))
    dMe = rng.standard_normal((B, H, P))
    g = oracle.chunk_backward(kind, *[x[n] for n in NAMES], dout, dWe, dMe, C, hidden=hd,
                              decay_mode=mode, averaged=True)

    def loss(xx):
        o, We, Me = oracle.chunk_forward(kind, *[xx[n] for n in NAMES], C, hidden=hd,
                                         decay_mode=mode, averaged=True)
        return float((dout * o).sum() + (dWe * We).sum() + (dMe * Me).sum())
    eps = 1e-6
    for name in NAMES:
        dl = rng.standard_normal(x[name].shape)
        xp = dict(x); xp[name] = x[name] + eps * dl
        xm = dict(x); xm[name] = x[name] - eps * dl
        fd = (loss(xp) - loss(xm)) / (2 * eps)
        an = float((g[name] * dl).sum())
        assert abs(fd - an) <= 2e-7 * max(1.0, abs(an)), (name, fd, an)


@pytest.mark.parametrize("kind", [oracle.LINEAR, oracle.SWIGLU])
def test_backward_row_normalisation_matches_finite_differences(kind):
    """Chunk-boundary normalisation: W normalised after every chunk (the last
    included); the adjoint goes back through each normalisation."""
    rng = np.random.default_rng(700 + kind)
    B, H, L, d, hd, C = 1, 2, 8, 3, 4, 3
    if kind == oracle.LINEAR:
        x, hd, P = _problem(rng, B, H, L, d, 0), 0, d * d
    else:
        x, P = _problem_sw(rng, B, H, L, d, hd, 0), 3 * d * hd
    dout = rng.standard_normal((B, H, L, d))
    dWe = rng.standard_normal((B, H, P))
    dMe = rng.standard_normal((B, H, P))
    g = oracle.chunk_backward(kind, *[x[n] for n in NAMES], dout, dWe, dMe, C, hidden=hd,
                              row_norm=True)

    def loss(xx):
        o, We, Me = oracle.chunk_forward(kind, *[xx[n] for n in NAMES], C, hidden=hd,
                                         row_norm=True)
        return float((dout * o).sum() + (dWe * We).sum() + (dMe * Me).sum())
    eps = 1e-6
    for name in NAMES:
        dl = rng.standard_normal(x[name].shape)
        xp = dict(x); xp[name] = x[name] + eps * dl
        xm = dict(x); xm[name] = x[name] - eps * dl
        fd = (loss(xp) - loss(xm)) / (2 * eps)
        an = float((g[name] * dl).sum())
        assert abs(fd - an) <= 2e-7 * max(1.0, abs(an)), (name, fd, an)
