"""Pins of the oracle's reverse mode for the MLP learner (E2-TTT_MLP,
f(x) = W2 silu(W1 x)) and for the LaCT rule (one step per chunk on the
eta-weighted sum of the descent directions, with the chunk means of beta and
gamma), CPU only.

Each is pinned, as the default rule's reverse mode is, to two things other
than itself:
  - central finite differences of the oracle's own forward (pinned in
    test_oracle_mlp.py and test_oracle_lact.py), one input class at a time;
  - torch autograd through an independent fp64 closed form written here:
    per-token descent factors at the chunk-start weights, then either the
    kernels of the default rule (suffix products and the reverse affine scan
    of §3.2 / App. A) or the LaCT step (K^W = K^M = eta, chunk means as the
    coefficients), and the aggregations U^T diag(K) X per matrix.
"""
import numpy as np
import pytest
import torch

import oracle

NAMES = ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")


def _state_size(kind, d, hd):
    return d * d if kind == oracle.LINEAR else (2 if kind == oracle.MLP else 3) * d * hd


def _problem(rng, kind, B, H, L, d, hd, mode):
    P = _state_size(kind, d, hd)
    alpha = rng.random((B, H, L)) if mode == oracle.GAMMA_1_MINUS_ETA_ALPHA else \
        0.5 + 0.5 * rng.random((B, H, L))
    return dict(q=rng.standard_normal((B, H, L, d)),
                k=rng.standard_normal((B, H, L, d)) / np.sqrt(d),
                v=rng.standard_normal((B, H, L, d)),
                eta=0.3 * rng.random((B, H, L)) + 0.05, alpha=alpha,
                beta=rng.random((B, H, L)),
                W0=rng.standard_normal((B, H, P)) * 0.6,
                M0=rng.standard_normal((B, H, P)) * 0.3)


def _closed_form_torch(x, C, mode, kind, hd, lact):
    """The chunk forward in torch fp64 by the closed form (see the module
    docstring); returns out, W_end, M_end."""
    q, k, v = x["q"], x["k"], x["v"]
    eta, alpha, beta = x["eta"], x["alpha"], x["beta"]
    B, H, L, d = q.shape
    gated = kind == oracle.SWIGLU

    def split(S):
        if kind == oracle.LINEAR:
            return [S.reshape(B, H, d, d)]
        W1 = S[..., :hd * d].reshape(B, H, hd, d)
        if gated:
            return [W1, S[..., hd * d:2 * hd * d].reshape(B, H, hd, d),
                    S[..., 2 * hd * d:].reshape(B, H, d, hd)]
        return [W1, S[..., hd * d:].reshape(B, H, d, hd)]

    def join(parts):
        return torch.cat([p.reshape(B, H, -1) for p in parts], -1)

    def silu(a):
        return a * torch.sigmoid(a)

    def forward(W, X):  # hidden pre-activations, z and y for rows X
        if kind == oracle.LINEAR:
            return None, None, None, X @ W[0].transpose(-1, -2)
        a1 = X @ W[0].transpose(-1, -2)
        a3 = X @ W[1].transpose(-1, -2) if gated else torch.ones_like(a1)
        z = silu(a1) * a3
        return a1, a3, z, z @ W[-1].transpose(-1, -2)

    def factors(W, K, V):  # (left, right) factor pairs of the descent direction, per matrix
        a1, a3, z, y = forward(W, K)
        e = V - y
        if kind == oracle.LINEAR:
            return [(e, K)]
        w = e @ W[-1]
        sg = torch.sigmoid(a1)
        u1 = w * a3 * (sg * (1.0 + a1 * (1.0 - sg)))
        if gated:
            return [(u1, K), (w * silu(a1), K), (e, z)]
        return [(u1, K), (e, z)]

    W, M = split(x["W0"]), split(x["M0"])
    gam = 1.0 - eta * alpha if mode == oracle.GAMMA_1_MINUS_ETA_ALPHA else alpha
    outs = []
    for t0 in range(0, L, C):
        n = min(C, L - t0)
        sl = slice(t0, t0 + n)
        be, ga, et = beta[:, :, sl], gam[:, :, sl], eta[:, :, sl]
        if lact:
            KW = KM = et
            cW, cM = ga.mean(-1), be.mean(-1)
            cWM = cM
        else:
            ones = torch.ones_like(be[..., :1])
            b_all = torch.flip(torch.cumprod(torch.flip(torch.cat([be[..., 1:], ones], -1), [-1]),
                                             -1), [-1])
            c_all = torch.flip(torch.cumprod(torch.flip(torch.cat([ga[..., 1:], ones], -1), [-1]),
                                             -1), [-1])
            Ps = [None] * n
            Ps[n - 1] = c_all[..., n - 1]
            for t in range(n - 2, -1, -1):
                Ps[t] = c_all[..., t] + be[..., t + 1] * Ps[t + 1]
            Pt = torch.stack(Ps, -1)
            KW, KM = et * Pt, et * b_all
            cW, cM, cWM = torch.prod(ga, -1), torch.prod(be, -1), be[..., 0] * Pt[..., 0]
        outs.append(forward(W, q[:, :, sl])[3])
        fac = factors(W, k[:, :, sl], v[:, :, sl])

        def agg(Kv, U, X):
            return (U * Kv[..., None]).transpose(-1, -2) @ X

        cw, cm, cwm = cW[..., None, None], cM[..., None, None], cWM[..., None, None]
        W_new = [cw * Wi + cwm * Mi + agg(KW, U, X) for Wi, Mi, (U, X) in zip(W, M, fac)]
        M = [cm * Mi + agg(KM, U, X) for Mi, (U, X) in zip(M, fac)]
        W = W_new
    return torch.cat(outs, 2), join(W), join(M)


CASES = [(oracle.MLP, False), (oracle.LINEAR, True), (oracle.SWIGLU, True), (oracle.MLP, True)]


@pytest.mark.parametrize("kind,lact", CASES)
def test_closed_form_reproduces_the_oracle_forward(kind, lact):
    """The torch closed form below is itself the oracle's forward."""
    rng = np.random.default_rng(21 + kind + 10 * lact)
    B, H, L, d, hd, C = 1, 2, 10, 4, 5, 4
    x = _problem(rng, kind, B, H, L, d, hd, 0)
    o, We, Me = oracle.chunk_forward(kind, *[x[n] for n in NAMES], C, hidden=hd, lact=lact)
    xt = {n: torch.tensor(x[n], dtype=torch.float64) for n in NAMES}
    ot, Wt, Mt = _closed_form_torch(xt, C, 0, kind, hd, lact)
    for a, b in ((o, ot), (We, Wt), (Me, Mt)):
        assert np.linalg.norm(a - b.numpy()) <= 1e-12 * np.linalg.norm(a)


@pytest.mark.parametrize("kind,lact", CASES)
@pytest.mark.parametrize("mode", [oracle.GAMMA_1_MINUS_ETA_ALPHA, oracle.ALPHA_IS_GAMMA])
@pytest.mark.parametrize("L,C", [(7, 3), (5, 5), (4, 1)])
def test_backward_matches_finite_differences(kind, lact, mode, L, C):
    rng = np.random.default_rng(800 + L + 10 * C + mode + 3 * kind + 7 * lact)
    B, H, d, hd = 1, 2, 3, 4
    x = _problem(rng, kind, B, H, L, d, hd, mode)
    P = _state_size(kind, d, hd)
    dout = rng.standard_normal((B, H, L, d))
    dWe = rng.standard_normal((B, H, P))
    dMe = rng.standard_normal((B, H, P))
    g = oracle.chunk_backward(kind, *[x[n] for n in NAMES], dout, dWe, dMe, C, decay_mode=mode,
                              hidden=hd, lact=lact)

    def loss(xx):
        o, We, Me = oracle.chunk_forward(kind, *[xx[n] for n in NAMES], C, hidden=hd,
                                         decay_mode=mode, lact=lact)
        return float((dout * o).sum() + (dWe * We).sum() + (dMe * Me).sum())
    eps = 1e-6
    for name in NAMES:
        dl = rng.standard_normal(x[name].shape)
        xp = dict(x); xp[name] = x[name] + eps * dl
        xm = dict(x); xm[name] = x[name] - eps * dl
        fd = (loss(xp) - loss(xm)) / (2 * eps)
        an = float((g[name] * dl).sum())
        assert abs(fd - an) <= 2e-7 * max(1.0, abs(an)), (name, fd, an)


@pytest.mark.parametrize("kind,lact", CASES)
@pytest.mark.parametrize("mode", [oracle.GAMMA_1_MINUS_ETA_ALPHA, oracle.ALPHA_IS_GAMMA])
@pytest.mark.parametrize("L,C,d,hd", [(9, 4, 3, 5), (8, 8, 4, 6), (10, 3, 2, 3)])
def test_backward_matches_autograd_of_closed_form(kind, lact, mode, L, C, d, hd):
    rng = np.random.default_rng(900 + L + C + d + hd + mode + 3 * kind + 7 * lact)
    B, H = 2, 1
    P = _state_size(kind, d, hd)
    x = _problem(rng, kind, B, H, L, d, hd, mode)
    dout = rng.standard_normal((B, H, L, d))
    dWe = rng.standard_normal((B, H, P))
    dMe = rng.standard_normal((B, H, P))
    xt = {n: torch.tensor(x[n], dtype=torch.float64, requires_grad=True) for n in NAMES}
    o, We, Me = _closed_form_torch(xt, C, mode, kind, hd, lact)
    loss = (torch.tensor(dout) * o).sum() + (torch.tensor(dWe) * We).sum() + \
        (torch.tensor(dMe) * Me).sum()
    loss.backward()
    g = oracle.chunk_backward(kind, *[x[n] for n in NAMES], dout, dWe, dMe, C, decay_mode=mode,
                              hidden=hd, lact=lact)
    for n in NAMES:
        ref = xt[n].grad.numpy()
        err = np.linalg.norm(g[n] - ref) / max(np.linalg.norm(ref), 1e-300)
        assert err <= 1e-10, (n, err)


@pytest.mark.parametrize("kind,lact,qk_norm,row_norm", [
    (oracle.MLP, False, True, False), (oracle.MLP, False, False, True),
    (oracle.SWIGLU, True, False, True), (oracle.LINEAR, True, True, True),
    (oracle.MLP, True, True, True)])
def test_backward_with_prologue_and_row_normalisation(kind, lact, qk_norm, row_norm):
    """The q/k prologue and the chunk-boundary normalisation combined with the
    MLP learner and the LaCT rule (a ragged last chunk), against central
    differences of the oracle's forward with the same options."""
    rng = np.random.default_rng(1000 + kind + 2 * lact + 4 * qk_norm + 8 * row_norm)
    B, H, L, d, hd, C = 1, 2, 8, 3, 4, 3
    x = _problem(rng, kind, B, H, L, d, hd, 0)
    P = _state_size(kind, d, hd)
    dout = rng.standard_normal((B, H, L, d))
    dWe = rng.standard_normal((B, H, P))
    dMe = rng.standard_normal((B, H, P))
    g = oracle.chunk_backward(kind, *[x[n] for n in NAMES], dout, dWe, dMe, C, hidden=hd,
                              qk_norm=qk_norm, row_norm=row_norm, lact=lact)

    def loss(xx):
        o, We, Me = oracle.chunk_forward(kind, *[xx[n] for n in NAMES], C, hidden=hd,
                                         qk_norm=qk_norm, row_norm=row_norm, lact=lact)
        return float((dout * o).sum() + (dWe * We).sum() + (dMe * Me).sum())
    eps = 1e-6
    for name in NAMES:
        dl = rng.standard_normal(x[name].shape)
        xp = dict(x); xp[name] = x[name] + eps * dl
        xm = dict(x); xm[name] = x[name] - eps * dl
        fd = (loss(xp) - loss(xm)) / (2 * eps)
        an = float((g[name] * dl).sum())
        assert abs(fd - an) <= 5e-7 * max(1.0, abs(an)), (name, fd, an)
