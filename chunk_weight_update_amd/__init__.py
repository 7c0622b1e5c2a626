"""E2-TTT chunk-parallel fast-weight update on AMD MI355X (gfx950).

Thin Python binding of the C ABI in ``include/e2ttt.h`` (``libe2ttt.so``,
built in-tree by ``chunk_weight_update_amd.build``).  This module only
marshals arguments: every step of the computation runs in the HIP kernels.
There is no CPU fallback; if the library is missing, calls raise.

The names mirror the C entry points: ``validate``, ``workspace_bytes``,
``chunk_forward``, ``scalar_kernels``, ``status_string``.  Tensors are torch
tensors on the GPU (PyTorch supplies device memory and streams).
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# E2TTT_LIBRARY selects another build of the same library (the sanitizer
# build of the host code); it must exist like the default one.
LIB_PATH = os.environ.get("E2TTT_LIBRARY") or os.path.join(_HERE, "libe2ttt.so")

OK, EINVAL, EWORKSPACE, EUNSUPPORTED, EHIP = 0, 1, 2, 3, 4
LINEAR, SWIGLU, MLP = 0, 1, 2
F32, BF16 = 0, 1
GAMMA_1_MINUS_ETA_ALPHA, ALPHA_IS_GAMMA = 0, 1
FLAG_COMPENSATED_WEIGHTS = 1
FLAG_CHUNK_AVERAGED_DECAY = 2
FLAG_QK_SILU_L2 = 4
FLAG_POST_CHUNK_ROW_L2 = 8
FLAG_PLAIN_BF16_WEIGHTS = 16
FLAG_LACT_RULE = 32


class Problem(ctypes.Structure):
    """Mirror of ``e2ttt_problem``."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("kind", ctypes.c_int32),
        ("batch", ctypes.c_int64),
        ("heads", ctypes.c_int64),
        ("seq_len", ctypes.c_int64),
        ("dim", ctypes.c_int64),
        ("hidden", ctypes.c_int64),
        ("chunk", ctypes.c_int64),
        ("io_dtype", ctypes.c_int32),
        ("decay_mode", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


def make_problem(kind: int, batch: int, heads: int, seq_len: int, dim: int, hidden: int,
                 chunk: int, io_dtype: int, decay_mode: int = GAMMA_1_MINUS_ETA_ALPHA,
                 flags: int = 0) -> Problem:
    return Problem(ctypes.sizeof(Problem), kind, batch, heads, seq_len, dim, hidden, chunk,
                   io_dtype, decay_mode, flags, 0)


class E2tttError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


_lock = threading.Lock()
_lib = None

EXPORTED = ("e2ttt_validate", "e2ttt_workspace_bytes", "e2ttt_chunk_forward",
            "e2ttt_scalar_kernels", "e2ttt_chunk_forward_timed", "e2ttt_status_string",
            "e2ttt_decode_workspace_bytes", "e2ttt_decode_step",
            "e2ttt_backward_workspace_bytes", "e2ttt_chunk_backward",
            "e2ttt_chunk_forward_states", "e2ttt_chunk_backward_states",
            "e2ttt_chunk_forward_noalloc", "e2ttt_scalar_heads")
# Scratch size built into e2ttt_chunk_forward_noalloc (E2TTT_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20

# e2ttt_kernel_class
KERNEL_SCAN, KERNEL_PREP, KERNEL_FWD13, KERNEL_FWD2, KERNEL_BWD, KERNEL_AGG = range(6)
KERNEL_LINEAR_FWD, KERNEL_LINEAR_AGG, KERNEL_PHASE_A, KERNEL_PHASE_B = 6, 7, 8, 9
KERNEL_STATE, KERNEL_PROLOGUE = 10, 11
KERNEL_NUM_CLASSES = 12
KERNEL_NAMES = ("scan", "prep", "fwd13", "fwd2", "bwd", "agg", "linear_fwd", "linear_agg",
                "phase_a", "phase_b", "state", "prologue")


def lib() -> ctypes.CDLL:
    """Load libe2ttt.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it first (python -m "
                    "chunk_weight_update_amd.build or __graft_entry__.build()); there is no "
                    "fallback implementation")
            L = ctypes.CDLL(LIB_PATH)
            P = ctypes.POINTER(Problem)
            vp = ctypes.c_void_p
            L.e2ttt_validate.argtypes = [P]
            L.e2ttt_validate.restype = ctypes.c_int
            L.e2ttt_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
            L.e2ttt_workspace_bytes.restype = ctypes.c_int
            L.e2ttt_chunk_forward.argtypes = [P] + [vp] * 12 + [ctypes.c_size_t, vp]
            L.e2ttt_chunk_forward.restype = ctypes.c_int
            L.e2ttt_scalar_heads.argtypes = ([P, vp, ctypes.c_int64, vp, vp, ctypes.c_float,
                                              ctypes.c_float] + [vp] * 4)
            L.e2ttt_scalar_heads.restype = ctypes.c_int
            L.e2ttt_chunk_forward_noalloc.argtypes = [P] + [vp] * 12
            L.e2ttt_chunk_forward_noalloc.restype = ctypes.c_int
            L.e2ttt_chunk_forward_timed.argtypes = ([P] + [vp] * 12 + [ctypes.c_size_t, vp] +
                                                    [ctypes.c_int, ctypes.POINTER(vp),
                                                     ctypes.c_int,
                                                     ctypes.POINTER(ctypes.c_int)])
            L.e2ttt_chunk_forward_timed.restype = ctypes.c_int
            L.e2ttt_scalar_kernels.argtypes = [P] + [vp] * 7
            L.e2ttt_scalar_kernels.restype = ctypes.c_int
            L.e2ttt_decode_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
            L.e2ttt_decode_workspace_bytes.restype = ctypes.c_int
            L.e2ttt_decode_step.argtypes = ([P] + [vp] * 9 + [ctypes.c_int64, ctypes.c_int, vp,
                                                                ctypes.c_size_t, vp])
            L.e2ttt_decode_step.restype = ctypes.c_int
            L.e2ttt_backward_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
            L.e2ttt_backward_workspace_bytes.restype = ctypes.c_int
            L.e2ttt_chunk_backward.argtypes = [P] + [vp] * 20 + [ctypes.c_size_t, vp]
            L.e2ttt_chunk_backward.restype = ctypes.c_int
            L.e2ttt_chunk_forward_states.argtypes = [P] + [vp] * 14 + [ctypes.c_size_t, vp]
            L.e2ttt_chunk_forward_states.restype = ctypes.c_int
            L.e2ttt_chunk_backward_states.argtypes = [P] + [vp] * 22 + [ctypes.c_size_t, vp]
            L.e2ttt_chunk_backward_states.restype = ctypes.c_int
            L.e2ttt_status_string.argtypes = [ctypes.c_int]
            L.e2ttt_status_string.restype = ctypes.c_char_p
            _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().e2ttt_status_string(int(status)).decode()


def validate(prob: Problem) -> int:
    return lib().e2ttt_validate(ctypes.byref(prob))


def workspace_bytes(prob: Problem) -> int:
    n = ctypes.c_size_t(0)
    st = lib().e2ttt_workspace_bytes(ctypes.byref(prob), ctypes.byref(n))
    if st != OK:
        raise E2tttError(st, "e2ttt_workspace_bytes")
    return int(n.value)


def state_size(kind: int, d: int, h: int) -> int:
    """Floats of one (batch, head) state: d*d (linear), 3dh (SwiGLU), 2dh (MLP)."""
    return d * d if kind == LINEAR else (2 if kind == MLP else 3) * d * h


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def chunk_forward(prob: Problem, q, k, v, eta, alpha, beta, W0, M0, out, W_end, M_end,
                  workspace, workspace_nbytes: Optional[int] = None, stream=None,
                  check: bool = True) -> int:
    """Call ``e2ttt_chunk_forward`` on device tensors (or raw pointers).
    Returns the status; raises E2tttError on failure when ``check``."""
    if workspace_nbytes is None:
        workspace_nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().e2ttt_chunk_forward(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(alpha), _ptr(beta),
        _ptr(W0), _ptr(M0), _ptr(out), _ptr(W_end), _ptr(M_end), _ptr(workspace),
        int(workspace_nbytes), _stream(stream))
    if check and st != OK:
        raise E2tttError(st, "e2ttt_chunk_forward")
    return st


def chunk_forward_noalloc(prob: Problem, q, k, v, eta, alpha, beta, W0, M0, out, W_end, M_end,
                          stream=None, check: bool = True) -> int:
    """Call ``e2ttt_chunk_forward_noalloc``: chunk_forward on the library's
    built-in per-GPU scratch instead of a caller workspace.  Returns the
    status; raises E2tttError on failure when ``check``."""
    st = lib().e2ttt_chunk_forward_noalloc(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(alpha), _ptr(beta),
        _ptr(W0), _ptr(M0), _ptr(out), _ptr(W_end), _ptr(M_end), _stream(stream))
    if check and st != OK:
        raise E2tttError(st, "e2ttt_chunk_forward_noalloc")
    return st


def chunk_forward_states(prob: Problem, q, k, v, eta, alpha, beta, W0, M0, out, W_end,
                         M_end, W_starts, M_starts, workspace,
                         workspace_nbytes: Optional[int] = None, stream=None,
                         check: bool = True) -> int:
    """Call ``e2ttt_chunk_forward_states``: chunk_forward that also writes the
    states at the starts of chunks 1 .. nC-1 ([nC-1, B, H, P] fp32 each), for
    e2ttt_chunk_backward_states.  Returns the status."""
    if workspace_nbytes is None:
        workspace_nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().e2ttt_chunk_forward_states(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(alpha), _ptr(beta),
        _ptr(W0), _ptr(M0), _ptr(out), _ptr(W_end), _ptr(M_end), _ptr(W_starts), _ptr(M_starts),
        _ptr(workspace), int(workspace_nbytes), _stream(stream))
    if check and st != OK:
        raise E2tttError(st, "e2ttt_chunk_forward_states")
    return st


def chunk_forward_timed(prob: Problem, q, k, v, eta, alpha, beta, W0, M0, out, W_end, M_end,
                        workspace, kernel_class: int, events, workspace_nbytes=None,
                        stream=None, check: bool = True):
    """Call ``e2ttt_chunk_forward_timed``: same work as chunk_forward, with the
    HIP events ``events`` (raw hipEvent_t handles as ints) recorded around
    each launch of ``kernel_class``.  Returns (status, n_recorded)."""
    if workspace_nbytes is None:
        workspace_nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    arr = (ctypes.c_void_p * max(len(events), 1))(*[ctypes.c_void_p(e) for e in events])
    nrec = ctypes.c_int(0)
    st = lib().e2ttt_chunk_forward_timed(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(alpha), _ptr(beta),
        _ptr(W0), _ptr(M0), _ptr(out), _ptr(W_end), _ptr(M_end), _ptr(workspace),
        int(workspace_nbytes), _stream(stream), int(kernel_class), arr, len(events),
        ctypes.byref(nrec))
    if check and st != OK:
        raise E2tttError(st, "e2ttt_chunk_forward_timed")
    return st, int(nrec.value)


def scalar_kernels(prob: Problem, eta, alpha, beta, k_w, k_m, chunk_coef, stream=None,
                   check: bool = True) -> int:
    """Call ``e2ttt_scalar_kernels`` on device tensors."""
    st = lib().e2ttt_scalar_kernels(ctypes.byref(prob), _ptr(eta), _ptr(alpha), _ptr(beta),
                                    _ptr(k_w), _ptr(k_m), _ptr(chunk_coef), _stream(stream))
    if check and st != OK:
        raise E2tttError(st, "e2ttt_scalar_kernels")
    return st


def scalar_heads(prob: Problem, x, model_dim: int, w_heads, b_heads, eta_base: float,
                 alpha_base: float, eta, alpha, beta, stream=None, check: bool = True) -> int:
    """Call ``e2ttt_scalar_heads``: eta, alpha, beta [B, H, L] from the layer
    input x [B, L, model_dim] and the head weights w_heads [3H, model_dim],
    b_heads [3H].  Returns the status; raises on failure when ``check``."""
    st = lib().e2ttt_scalar_heads(ctypes.byref(prob), _ptr(x), int(model_dim), _ptr(w_heads),
                                  _ptr(b_heads), float(eta_base), float(alpha_base), _ptr(eta),
                                  _ptr(alpha), _ptr(beta), _stream(stream))
    if check and st != OK:
        raise E2tttError(st, "e2ttt_scalar_heads")
    return st


def decode_workspace_bytes(prob: Problem) -> int:
    n = ctypes.c_size_t(0)
    st = lib().e2ttt_decode_workspace_bytes(ctypes.byref(prob), ctypes.byref(n))
    if st != OK:
        raise E2tttError(st, "e2ttt_decode_workspace_bytes")
    return int(n.value)


def decode_step(prob: Problem, q, k, v, eta, alpha, beta, W, M, out, pos: int, chunk_end: bool,
                workspace, workspace_nbytes: Optional[int] = None, stream=None,
                check: bool = True) -> int:
    """Call ``e2ttt_decode_step``: the token at position ``pos`` of the current
    chunk for every (b, h) unit; W, M (the chunk-start state) are replaced by
    the chunk-end state when ``chunk_end``.  The workspace must be the same,
    unmodified, for all calls of a chunk.  Returns the status; raises on
    failure when ``check``."""
    if workspace_nbytes is None:
        workspace_nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().e2ttt_decode_step(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(alpha), _ptr(beta),
        _ptr(W), _ptr(M), _ptr(out), int(pos), int(bool(chunk_end)), _ptr(workspace),
        int(workspace_nbytes), _stream(stream))
    if check and st != OK:
        raise E2tttError(st, "e2ttt_decode_step")
    return st


def backward_workspace_bytes(prob: Problem) -> int:
    n = ctypes.c_size_t(0)
    st = lib().e2ttt_backward_workspace_bytes(ctypes.byref(prob), ctypes.byref(n))
    if st != OK:
        raise E2tttError(st, "e2ttt_backward_workspace_bytes")
    return int(n.value)


def chunk_backward(prob: Problem, q, k, v, eta, alpha, beta, W0, M0, dout, dW_end, dM_end,
                   dq, dk, dv, deta, dalpha, dbeta, dW0, dM0, workspace,
                   workspace_nbytes: Optional[int] = None, stream=None,
                   check: bool = True, W_starts=None, M_starts=None) -> int:
    """Call ``e2ttt_chunk_backward`` (linear and SwiGLU learners, fp32 or bf16
    io): gradients of a loss with respect to every input of the chunk
    forward, given its gradients dout, dW_end, dM_end (the last two may be
    None).  With ``W_starts``/``M_starts`` (the chunk-start states kept by
    ``chunk_forward_states``) it calls ``e2ttt_chunk_backward_states``, which
    skips the forward re-run.  Returns the status; raises on failure when
    ``check``."""
    if workspace_nbytes is None:
        workspace_nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if W_starts is None and M_starts is None:
        name = "e2ttt_chunk_backward"
        st = lib().e2ttt_chunk_backward(
            ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(alpha), _ptr(beta),
            _ptr(W0), _ptr(M0), _ptr(dout), _ptr(dW_end), _ptr(dM_end), _ptr(dq), _ptr(dk),
            _ptr(dv), _ptr(deta), _ptr(dalpha), _ptr(dbeta), _ptr(dW0), _ptr(dM0),
            _ptr(workspace), int(workspace_nbytes), _stream(stream))
    else:
        name = "e2ttt_chunk_backward_states"
        st = lib().e2ttt_chunk_backward_states(
            ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(alpha), _ptr(beta),
            _ptr(W0), _ptr(M0), _ptr(W_starts), _ptr(M_starts), _ptr(dout), _ptr(dW_end),
            _ptr(dM_end), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(deta), _ptr(dalpha), _ptr(dbeta),
            _ptr(dW0), _ptr(dM0), _ptr(workspace), int(workspace_nbytes), _stream(stream))
    if check and st != OK:
        raise E2tttError(st, name)
    return st


class ChunkForward:
    """Holds the output and workspace tensors of one problem shape, so that
    repeated calls allocate nothing."""

    def __init__(self, prob: Problem, device="cuda"):
        import torch
        self.prob = prob
        B, H, L, d = prob.batch, prob.heads, prob.seq_len, prob.dim
        P = state_size(prob.kind, d, prob.hidden)
        io = torch.bfloat16 if prob.io_dtype == BF16 else torch.float32
        self.out = torch.empty((B, H, L, d), dtype=io, device=device)
        self.W_end = torch.empty((B, H, P), dtype=torch.float32, device=device)
        self.M_end = torch.empty((B, H, P), dtype=torch.float32, device=device)
        nbytes = workspace_bytes(prob)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)

    def __call__(self, q, k, v, eta, alpha, beta, W0, M0, stream=None):
        chunk_forward(self.prob, q, k, v, eta, alpha, beta, W0, M0, self.out, self.W_end,
                      self.M_end, self.workspace, stream=stream)
        return self.out, self.W_end, self.M_end
