"""fp64 CPU oracle of the E2-TTT chunk forward (and, for the linear learner,
its reverse mode) -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and has
no fallback to it.

The arithmetic lives in ``e2ttt_oracle.c`` (plain C, fp64, OpenMP); this
module only compiles it with gcc and marshals numpy arrays.  Every input is
widened to fp64 from exactly the values the GPU receives (bf16 inputs are
widened after their rounding), so input rounding is never charged to the GPU.

Citations are to "Rethinking Expressivity and Efficiency in Test-Time
Training" (E2-TTT): the token-wise recurrence with chunk-start gradients is
the optimisation-style view of App. A.5 (Eq. 7), the decay coupling is Eq. 14
(App. A.3), the readout is Eq. 6 (§3.2).

Parity pins (tests/test_oracle.py) tie every function here to something other
than itself: the paper's kernel formulas of §3.2 in their ratio-sum form,
torch autograd and finite differences for the gradients, the
momentum-free/decay-free reduction to a summed-gradient update, the C = 1
reduction to token-wise online descent (App. B.3), the gamma = 0 limit of
App. A.3, geometric-series closed forms for constant scalars, and a worked
example by hand under tests/golden/.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "e2ttt_oracle.c")
# E2TTT_ORACLE_LIBRARY selects a prebuilt oracle library (the sanitizer
# build); it is then loaded as it is, never rebuilt.
_LIB_ENV = os.environ.get("E2TTT_ORACLE_LIBRARY")
_LIB = _LIB_ENV or os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

LINEAR = 0
SWIGLU = 1
MLP = 2
GAMMA_1_MINUS_ETA_ALPHA = 0
ALPHA_IS_GAMMA = 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-shared", "-fPIC", "-std=c99", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not _LIB_ENV and (not os.path.exists(_LIB) or (
                    os.path.getmtime(_LIB) < os.path.getmtime(_SRC))):
                build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.POINTER(ctypes.c_double)
            i64 = ctypes.c_int64
            lib.oracle_chunk_forward.argtypes = (
                [ctypes.c_int, ctypes.c_int] + [i64] * 6 + [P] * 11 + [ctypes.c_int] * 3)
            lib.oracle_chunk_forward.restype = ctypes.c_int
            lib.oracle_token_descent.argtypes = [ctypes.c_int, i64, i64, P, P, P, P]
            lib.oracle_token_descent.restype = ctypes.c_int
            lib.oracle_fast_forward.argtypes = [ctypes.c_int, i64, i64, P, P, P]
            lib.oracle_fast_forward.restype = ctypes.c_int
            lib.oracle_scalar_kernels.argtypes = [ctypes.c_int, i64, i64] + [P] * 6 + [ctypes.c_int]
            lib.oracle_scalar_kernels.restype = ctypes.c_int
            lib.oracle_chunk_backward.argtypes = (
                [ctypes.c_int, ctypes.c_int] + [i64] * 6 + [P] * 19 + [ctypes.c_int] * 3)
            lib.oracle_chunk_backward.restype = ctypes.c_int
            lib.oracle_scalar_heads.argtypes = [i64] * 4 + [P] * 3 + [ctypes.c_double] * 2 + [P] * 3
            lib.oracle_scalar_heads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _variant(averaged: bool, lact: bool) -> int:
    """Variant code of the C functions: 0 the E2-TTT recurrence, 1 its
    chunk-averaged ablation, 2 the LaCT rule."""
    if averaged and lact:
        raise ValueError("averaged and lact are exclusive")
    return 2 if lact else int(bool(averaged))


def state_size(kind: int, d: int, h: int) -> int:
    return d * d if kind == LINEAR else (2 if kind == MLP else 3) * d * h


def set_threads(n: int) -> None:
    """Set the OpenMP thread count used by the oracle (process-wide)."""
    os.environ["OMP_NUM_THREADS"] = str(int(n))
    try:
        libgomp = ctypes.CDLL("libgomp.so.1")
        libgomp.omp_set_num_threads(ctypes.c_int(int(n)))
    except OSError:
        pass


def chunk_forward(kind, q, k, v, eta, alpha, beta, W0, M0, chunk, hidden=0,
                  decay_mode=GAMMA_1_MINUS_ETA_ALPHA, averaged=False, qk_norm=False,
                  row_norm=False, lact=False, qk_round_bf16=False):
    """Run the literal recurrence.  q,k,v: [B,H,L,d]; eta/alpha/beta: [B,H,L];
    W0, M0: [B,H,P].  averaged: the chunk-averaged variant (beta, gamma
    replaced by their means over each chunk).  lact: the LaCT rule instead
    (one step per chunk on the eta-weighted sum of the descent directions,
    with the chunk means of beta and gamma; exclusive with averaged).  qk_norm: the q/k prologue (SiLU,
    then L2 normalisation per token) before use; with qk_round_bf16 its
    outputs are rounded to bf16 (the precision a bf16 layer keeps q and k in,
    so that, as for bf16 inputs, that rounding is not charged to the GPU).
    row_norm: every row of every
    fast-weight matrix divided by its L2 norm after each chunk (the
    chunk-boundary stabiliser of App. B.1).  Returns (out [B,H,L,d],
    Wend, Mend), all float64."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    eta, alpha, beta = _f64(eta), _f64(alpha), _f64(beta)
    W0, M0 = _f64(W0), _f64(M0)
    B, H, L, d = q.shape
    P = state_size(kind, d, hidden)
    assert k.shape == q.shape and v.shape == q.shape
    assert eta.shape == (B, H, L) and alpha.shape == (B, H, L) and beta.shape == (B, H, L)
    assert W0.shape == (B, H, P) and M0.shape == (B, H, P)
    out = np.empty_like(q)
    Wend = np.empty_like(W0)
    Mend = np.empty_like(M0)
    rc = lib.oracle_chunk_forward(kind, decay_mode, B, H, L, d, hidden, chunk,
                                  _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                                  _ptr(alpha), _ptr(beta), _ptr(W0), _ptr(M0),
                                  _ptr(out), _ptr(Wend), _ptr(Mend),
                                  _variant(averaged, lact),
                                  (2 if qk_round_bf16 else 1) if qk_norm else 0,
                                  int(bool(row_norm)))
    if rc != 0:
        raise RuntimeError(f"oracle_chunk_forward failed with code {rc}")
    return out, Wend, Mend


def token_descent(kind, W, k, v, d, hidden=0):
    """Dense descent direction -grad_W 0.5||f_W(k)-v||^2 for one token."""
    lib = _load()
    W, k, v = _f64(W), _f64(k), _f64(v)
    G = np.empty_like(W)
    rc = lib.oracle_token_descent(kind, d, hidden, _ptr(W), _ptr(k), _ptr(v), _ptr(G))
    if rc != 0:
        raise RuntimeError(f"oracle_token_descent failed with code {rc}")
    return G


def fast_forward(kind, W, x, d, hidden=0):
    """f_W(x) for one vector."""
    lib = _load()
    W, x = _f64(W), _f64(x)
    y = np.empty(d, dtype=np.float64)
    rc = lib.oracle_fast_forward(kind, d, hidden, _ptr(W), _ptr(x), _ptr(y))
    if rc != 0:
        raise RuntimeError(f"oracle_fast_forward failed with code {rc}")
    return y


def scalar_kernels(eta, alpha, beta, decay_mode=GAMMA_1_MINUS_ETA_ALPHA, averaged=False,
                   lact=False):
    """Impulse-response kernels of each segment.  eta/alpha/beta: [nseg, n].
    Returns kw [nseg,n], km [nseg,n], coef [nseg,3] = (cW, cM, cWM)."""
    lib = _load()
    eta, alpha, beta = _f64(eta), _f64(alpha), _f64(beta)
    nseg, n = eta.shape
    kw = np.empty_like(eta)
    km = np.empty_like(eta)
    coef = np.empty((nseg, 3), dtype=np.float64)
    rc = lib.oracle_scalar_kernels(decay_mode, nseg, n, _ptr(eta), _ptr(alpha),
                                   _ptr(beta), _ptr(kw), _ptr(km), _ptr(coef),
                                   _variant(averaged, lact))
    if rc != 0:
        raise RuntimeError(f"oracle_scalar_kernels failed with code {rc}")
    return kw, km, coef


def chunk_backward(kind, q, k, v, eta, alpha, beta, W0, M0, dout, dWend, dMend, chunk,
                   decay_mode=GAMMA_1_MINUS_ETA_ALPHA, hidden=0, qk_norm=False, averaged=False,
                   row_norm=False, lact=False):
    """Reverse mode of ``chunk_forward`` (linear, SwiGLU and MLP learners; the
    default rule, the chunk-averaged variant or the LaCT rule): gradients of
    <dout, out> + <dWend, Wend> + <dMend, Mend> with respect to every input.
    dWend / dMend may be None (zero).  Returns a dict with keys q, k, v, eta,
    alpha, beta, W0, M0 (float64 arrays of the inputs' shapes)."""
    assert not (averaged and lact), "the LaCT rule and the chunk-averaged variant are exclusive"
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    eta, alpha, beta = _f64(eta), _f64(alpha), _f64(beta)
    W0, M0, dout = _f64(W0), _f64(M0), _f64(dout)
    B, H, L, d = q.shape
    P = state_size(kind, d, hidden)
    assert k.shape == q.shape and v.shape == q.shape and dout.shape == q.shape
    assert eta.shape == (B, H, L) and alpha.shape == (B, H, L) and beta.shape == (B, H, L)
    assert W0.shape == (B, H, P) and M0.shape == (B, H, P)
    null = ctypes.POINTER(ctypes.c_double)()
    dWp = _f64(dWend) if dWend is not None else None
    dMp = _f64(dMend) if dMend is not None else None
    g = {n: np.empty_like(a) for n, a in
         (("q", q), ("k", k), ("v", v), ("eta", eta), ("alpha", alpha), ("beta", beta),
          ("W0", W0), ("M0", M0))}
    rc = lib.oracle_chunk_backward(
        kind, decay_mode, B, H, L, d, hidden, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
        _ptr(alpha), _ptr(beta), _ptr(W0), _ptr(M0), _ptr(dout),
        _ptr(dWp) if dWp is not None else null, _ptr(dMp) if dMp is not None else null,
        _ptr(g["q"]), _ptr(g["k"]), _ptr(g["v"]), _ptr(g["eta"]), _ptr(g["alpha"]),
        _ptr(g["beta"]), _ptr(g["W0"]), _ptr(g["M0"]), int(bool(qk_norm)),
        2 if lact else int(bool(averaged)), int(bool(row_norm)))
    if rc != 0:
        raise RuntimeError(f"oracle_chunk_backward failed with code {rc}")
    return g


def scalar_heads(x, w, bias, heads, eta_base, alpha_base):
    """The per-token scalar heads: x [B, L, D] layer input, w [3H, D] (eta,
    alpha, beta heads in that order), bias [3H].  Returns eta, alpha, beta
    [B, H, L] (float64): eta_base * sigma(.), alpha_base * sigma(.), sigma(.)."""
    lib = _load()
    x, w, bias = _f64(x), _f64(w), _f64(bias)
    B, L, D = x.shape
    H = int(heads)
    assert w.shape == (3 * H, D) and bias.shape == (3 * H,)
    eta = np.empty((B, H, L))
    alpha = np.empty((B, H, L))
    beta = np.empty((B, H, L))
    rc = lib.oracle_scalar_heads(B, L, D, H, _ptr(x), _ptr(w), _ptr(bias), float(eta_base),
                                 float(alpha_base), _ptr(eta), _ptr(alpha), _ptr(beta))
    if rc != 0:
        raise RuntimeError(f"oracle_scalar_heads failed with code {rc}")
    return eta, alpha, beta

