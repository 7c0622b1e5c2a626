"""Independent fp64 closed form of the E2-TTT chunk update (tests only).

Written from the kernel formulas of §3.2 of "Rethinking Expressivity and
Efficiency in Test-Time Training" (E2-TTT), in their printed ratio-sum form:

    K^M_t = eta_t * beta~_t
    K^W_t = eta_t * beta~_t * R_t,    R_t = sum_{i >= t} gamma~_i / beta~_i

with beta~_t, gamma~_t the products of beta_s, gamma_s over the later tokens
s > t of the chunk (suffix products, App. A.2), gamma_t = 1 - eta_t alpha_t
(Eq. 14).  The chunk-end states are the two weighted aggregations of §3.2 and
App. A.4 plus the carried terms of the inherited state:

    M_C = beta~_0 M_0 + sum_t K^M_t G_t
    W_C = gamma~_0 W_0 + beta~_0 R_1 M_0 + sum_t K^W_t G_t

(index 0 is the inherited state, 1 the first token of the chunk: M_0 enters
the momentum like a gradient placed before token 1, decayed by beta_1 first,
so its weight factor is beta~_0 R_1 instead of beta~_1 R_1).  The per-token descent directions G_t are
taken from torch autograd in fp64 at the chunk-start weights, so neither the
recurrence nor the gradient code of the oracle is reused.  The ratio-sum form
overflows for long chunks with beta < gamma, so this is only used on tiny
inputs with moderate scalars.
"""
from __future__ import annotations

import numpy as np
import torch


def learner_forward(kind, W, x, d, h):
    """f_W(x) on torch fp64 tensors; W is the packed state vector (kind 0
    linear, 1 SwiGLU [W1 | W3 | W2], 2 MLP [W1 | W2] = W2 silu(W1 x))."""
    if kind == 0:
        return W.reshape(d, d) @ x
    if kind == 2:
        return W[h * d:].reshape(d, h) @ torch.nn.functional.silu(W[: h * d].reshape(h, d) @ x)
    W1 = W[: h * d].reshape(h, d)
    W3 = W[h * d: 2 * h * d].reshape(h, d)
    W2 = W[2 * h * d:].reshape(d, h)
    return W2 @ (torch.nn.functional.silu(W1 @ x) * (W3 @ x))


def autograd_descent(kind, W, k, v, d, h):
    """-grad_W 0.5 ||f_W(k) - v||^2 via torch autograd (fp64)."""
    Wt = torch.tensor(np.asarray(W, dtype=np.float64), requires_grad=True)
    kt = torch.tensor(np.asarray(k, dtype=np.float64))
    vt = torch.tensor(np.asarray(v, dtype=np.float64))
    loss = 0.5 * ((learner_forward(kind, Wt, kt, d, h) - vt) ** 2).sum()
    (g,) = torch.autograd.grad(loss, Wt)
    return -g.numpy()


def paper_kernels(eta, gamma, beta):
    """K^W, K^M and the carried-state factors of one chunk (ratio-sum form)."""
    n = len(eta)
    bt = np.array([np.prod(beta[t + 1:]) for t in range(n)])    # beta~_t
    gt = np.array([np.prod(gamma[t + 1:]) for t in range(n)])   # gamma~_t
    R = np.array([np.sum(gt[t:] / bt[t:]) for t in range(n)])
    KM = eta * bt
    KW = eta * bt * R
    b0 = np.prod(beta)
    g0 = np.prod(gamma)
    return KW, KM, g0, b0, b0 * R[0]


def closed_form_forward(kind, q, k, v, eta, alpha, beta, W0, M0, C, d, h=0,
                        alpha_is_gamma=False):
    """Closed-form chunk forward for one (batch, head): q,k,v [L,d]."""
    L = q.shape[0]
    W = np.array(W0, dtype=np.float64)
    M = np.array(M0, dtype=np.float64)
    out = np.zeros((L, d))
    for t0 in range(0, L, C):
        t1 = min(t0 + C, L)
        Wt = torch.tensor(W)
        for t in range(t0, t1):
            out[t] = learner_forward(kind, Wt, torch.tensor(q[t]), d, h).numpy()
        G = np.stack([autograd_descent(kind, W, k[t], v[t], d, h) for t in range(t0, t1)])
        e = np.asarray(eta[t0:t1], dtype=np.float64)
        a = np.asarray(alpha[t0:t1], dtype=np.float64)
        gam = a.copy() if alpha_is_gamma else 1.0 - e * a
        KW, KM, cW, cM, cWM = paper_kernels(e, gam, np.asarray(beta[t0:t1], dtype=np.float64))
        W, M = (cW * W + cWM * M + KW @ G, cM * M + KM @ G)
    return out, W, M
