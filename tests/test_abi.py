"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/e2ttt.h, and rejects bad arguments on the host before
anything is enqueued (fake device pointers are never dereferenced there)."""
import ctypes
import os
import re
import subprocess

import pytest

import chunk_weight_update_amd as cwu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "e2ttt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(e2ttt_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_entry_point():
    names = declared_functions()
    assert set(names) == set(cwu.EXPORTED)
    L = cwu.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", cwu.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (e2ttt_\w+)", out))
    assert set(names) <= exported


def test_problem_struct_layout_matches_header():
    # uint32, int32, 6 x int64, int32, int32, uint32, uint32
    assert ctypes.sizeof(cwu.Problem) == 4 + 4 + 6 * 8 + 4 * 4


def swiglu(**kw):
    a = dict(kind=cwu.SWIGLU, batch=2, heads=4, seq_len=4096, dim=128, hidden=256, chunk=512,
             io_dtype=cwu.BF16)
    a.update(kw)
    return cwu.make_problem(**a)


def linear(**kw):
    a = dict(kind=cwu.LINEAR, batch=1, heads=1, seq_len=256, dim=64, hidden=0, chunk=64,
             io_dtype=cwu.F32)
    a.update(kw)
    return cwu.make_problem(**a)


def test_status_strings():
    for s in range(5):
        assert cwu.status_string(s).startswith("E2TTT")
    assert "unknown" in cwu.status_string(99)


@pytest.mark.parametrize("prob,expected", [
    (swiglu(), cwu.OK),
    (linear(), cwu.OK),
    (swiglu(dim=768, hidden=1536, chunk=8192, seq_len=57344, batch=1, heads=1), cwu.OK),
    (swiglu(io_dtype=cwu.F32), cwu.OK),
    (swiglu(flags=cwu.FLAG_COMPENSATED_WEIGHTS), cwu.OK),
    (swiglu(seq_len=0), cwu.OK),
    (swiglu(seq_len=1000), cwu.OK),  # short last chunk
    (swiglu(chunk=100), cwu.OK),  # chunk not a multiple of the tile
    (swiglu(batch=0), cwu.EINVAL),
    (swiglu(heads=-1), cwu.EINVAL),
    (swiglu(seq_len=-5), cwu.EINVAL),
    (swiglu(chunk=0), cwu.EINVAL),
    (swiglu(hidden=0), cwu.EINVAL),
    (swiglu(kind=7), cwu.EINVAL),
    (swiglu(kind=cwu.MLP), cwu.OK),
    (swiglu(kind=cwu.MLP, dim=768, hidden=1536, chunk=8192, seq_len=57344, batch=1, heads=1),
     cwu.OK),
    (swiglu(kind=cwu.MLP, dim=96), cwu.EUNSUPPORTED),
    (swiglu(io_dtype=5), cwu.EINVAL),
    (swiglu(decay_mode=3), cwu.EINVAL),
    (swiglu(flags=cwu.FLAG_CHUNK_AVERAGED_DECAY), cwu.OK),
    (swiglu(flags=cwu.FLAG_QK_SILU_L2), cwu.OK),
    (swiglu(flags=cwu.FLAG_POST_CHUNK_ROW_L2), cwu.OK),
    (linear(flags=cwu.FLAG_POST_CHUNK_ROW_L2), cwu.OK),
    (swiglu(flags=cwu.FLAG_PLAIN_BF16_WEIGHTS), cwu.OK),
    (swiglu(flags=cwu.FLAG_PLAIN_BF16_WEIGHTS | cwu.FLAG_COMPENSATED_WEIGHTS), cwu.EINVAL),
    (swiglu(flags=cwu.FLAG_LACT_RULE), cwu.OK),
    (linear(flags=cwu.FLAG_LACT_RULE), cwu.OK),
    (swiglu(flags=cwu.FLAG_LACT_RULE | cwu.FLAG_CHUNK_AVERAGED_DECAY), cwu.EINVAL),
    (swiglu(flags=64), cwu.EINVAL),
    (linear(hidden=3), cwu.EINVAL),
    (swiglu(dim=96), cwu.EUNSUPPORTED),
    (swiglu(hidden=200), cwu.EUNSUPPORTED),
    (swiglu(dim=2048), cwu.EUNSUPPORTED),
    (linear(dim=72), cwu.EUNSUPPORTED),
    (linear(dim=256), cwu.EUNSUPPORTED),
    (swiglu(chunk=20000), cwu.EUNSUPPORTED),
    (swiglu(batch=1 << 40, heads=1 << 20), cwu.EUNSUPPORTED),
])
def test_validate(prob, expected):
    assert cwu.validate(prob) == expected


def test_struct_size_and_reserved_checked():
    p = swiglu()
    p.struct_size = 12
    assert cwu.validate(p) == cwu.EINVAL
    p = swiglu()
    p.reserved = 1
    assert cwu.validate(p) == cwu.EINVAL
    assert cwu.lib().e2ttt_validate(None) == cwu.EINVAL


def test_workspace_bytes():
    n = cwu.workspace_bytes(swiglu())
    assert n > 0 and n % 256 == 0
    # d = 128 bf16: the default shadows carry hi/lo pairs (as with compensated
    # weights); plain bf16 weights need half of that shadow space
    assert cwu.workspace_bytes(swiglu(flags=cwu.FLAG_COMPENSATED_WEIGHTS)) == n
    assert cwu.workspace_bytes(swiglu(flags=cwu.FLAG_PLAIN_BF16_WEIGHTS)) < n
    big = dict(dim=768, hidden=1536, chunk=8192, seq_len=57344, batch=1, heads=1)
    assert (cwu.workspace_bytes(swiglu(flags=cwu.FLAG_COMPENSATED_WEIGHTS, **big))
            > cwu.workspace_bytes(swiglu(**big)))
    assert cwu.workspace_bytes(swiglu(io_dtype=cwu.F32)) > n
    assert cwu.workspace_bytes(swiglu(seq_len=0)) == 0
    with pytest.raises(cwu.E2tttError):
        cwu.workspace_bytes(swiglu(dim=96))
    assert cwu.lib().e2ttt_workspace_bytes(ctypes.byref(swiglu()), None) == cwu.EINVAL


class Fake:
    """Non-overlapping, 256-aligned fake device addresses."""

    def __init__(self):
        self.next = 1 << 40

    def __call__(self, nbytes):
        a = self.next
        self.next += (int(nbytes) + (1 << 20)) & ~255
        return a


def fake_args(prob):
    f = Fake()
    B, H, L, d = prob.batch, prob.heads, prob.seq_len, prob.dim
    P = d * d if prob.kind == cwu.LINEAR else 3 * d * prob.hidden
    io = 2 if prob.io_dtype == cwu.BF16 else 4
    a = dict(q=f(B * H * L * d * io), k=f(B * H * L * d * io), v=f(B * H * L * d * io),
             eta=f(B * H * L * 4), alpha=f(B * H * L * 4), beta=f(B * H * L * 4),
             W0=f(B * H * P * 4), M0=f(B * H * P * 4), out=f(B * H * L * d * io),
             W_end=f(B * H * P * 4), M_end=f(B * H * P * 4))
    nws = cwu.workspace_bytes(prob)
    a["workspace"] = f(nws)
    a["nws"] = nws
    return a


def call(prob, a):
    return cwu.chunk_forward(prob, a["q"], a["k"], a["v"], a["eta"], a["alpha"], a["beta"],
                             a["W0"], a["M0"], a["out"], a["W_end"], a["M_end"],
                             a["workspace"], a["nws"], stream=0, check=False)


@pytest.mark.parametrize("mutate,expected", [
    (lambda a: a.update(q=None), cwu.EINVAL),
    (lambda a: a.update(W_end=None), cwu.EINVAL),
    (lambda a: a.update(workspace=None), cwu.EINVAL),
    (lambda a: a.update(k=a["k"] + 4), cwu.EINVAL),            # misaligned
    (lambda a: a.update(workspace=a["workspace"] + 16), cwu.EINVAL),  # not 256-aligned
    (lambda a: a.update(nws=a["nws"] - 256), cwu.EWORKSPACE),
    (lambda a: a.update(out=a["q"]), cwu.EINVAL),               # out aliases q
    (lambda a: a.update(W_end=a["W0"] + 256), cwu.EINVAL),      # partial overlap
    (lambda a: a.update(M_end=a["W_end"]), cwu.EINVAL),         # outputs alias
    (lambda a: a.update(workspace=a["out"]), cwu.EINVAL),       # workspace aliases out
    (lambda a: a.update(W_end=a["M0"]), cwu.EINVAL),            # W_end over M0
])
def test_forward_host_errors(mutate, expected):
    prob = swiglu()
    a = fake_args(prob)
    mutate(a)
    assert call(prob, a) == expected


def test_forward_rejects_bad_problem_before_pointers():
    a = fake_args(swiglu())
    assert call(swiglu(dim=96), a) == cwu.EUNSUPPORTED
    assert call(swiglu(batch=0), a) == cwu.EINVAL


def test_scalar_kernels_host_errors():
    prob = swiglu()
    f = Fake()
    n = prob.batch * prob.heads * prob.seq_len * 4
    e, al, b, kw, km, cf = (f(n) for _ in range(6))
    assert cwu.scalar_kernels(prob, e, al, b, kw, None, cf, stream=0, check=False) == cwu.EINVAL
    assert cwu.scalar_kernels(prob, e, al, b, e, km, cf, stream=0, check=False) == cwu.EINVAL
    assert cwu.scalar_kernels(prob, e + 8, al, b, kw, km, cf, stream=0, check=False) == cwu.EINVAL
    assert cwu.scalar_kernels(swiglu(chunk=0), e, al, b, kw, km, cf, stream=0,
                              check=False) == cwu.EINVAL


def test_timed_entry_host_errors():
    prob = swiglu()
    a = fake_args(prob)
    L = cwu.lib()

    def timed(kclass, events, n):
        arr = (ctypes.c_void_p * max(n, 1))(*events)
        return L.e2ttt_chunk_forward_timed(
            ctypes.byref(prob), a["q"], a["k"], a["v"], a["eta"], a["alpha"], a["beta"],
            a["W0"], a["M0"], a["out"], a["W_end"], a["M_end"], a["workspace"], a["nws"], 0,
            kclass, arr, n, None)

    assert timed(99, [], 0) == cwu.EINVAL
    assert timed(-1, [], 0) == cwu.EINVAL
    assert timed(cwu.KERNEL_AGG, [None, None], 2) == cwu.EINVAL
    assert timed(cwu.KERNEL_AGG, [], -2) == cwu.EINVAL


def test_decode_host_checks():
    """Host-side checks of the decode entry points (no device call): the
    workspace holds the chunk buffer (grows with the chunk length), and bad
    positions or null tensors are rejected before anything touches a device."""
    base = swiglu()
    n = cwu.decode_workspace_bytes(base)
    B, H, d, h, C = base.batch, base.heads, base.dim, base.hidden, base.chunk
    assert n >= 4 * B * H * (7 * h + 4 * d) * C and n % 256 == 0
    assert cwu.decode_workspace_bytes(swiglu(chunk=2 * C)) > n
    lin = linear()
    assert cwu.decode_workspace_bytes(lin) >= 4 * 4 * lin.dim * lin.chunk
    assert cwu.decode_workspace_bytes(swiglu(flags=cwu.FLAG_CHUNK_AVERAGED_DECAY)) == n
    assert cwu.decode_workspace_bytes(swiglu(flags=cwu.FLAG_LACT_RULE)) == n
    with pytest.raises(cwu.E2tttError):
        cwu.decode_workspace_bytes(swiglu(flags=cwu.FLAG_LACT_RULE |
                                          cwu.FLAG_CHUNK_AVERAGED_DECAY))
    assert cwu.decode_workspace_bytes(swiglu(flags=cwu.FLAG_POST_CHUNK_ROW_L2)) == n
    step = cwu.lib().e2ttt_decode_step
    f = Fake()
    nx, ns, np_ = B * H * d * 2, B * H * 4, B * H * 3 * d * h * 4
    args = [f(nx), f(nx), f(nx), f(ns), f(ns), f(ns), f(np_), f(np_), f(nx)]
    ws = f(n)
    # null tensors
    assert step(ctypes.byref(base), *([None] * 9), 0, 0, None, 0, None) == cwu.EINVAL
    # positions outside the chunk, and the chunk's last slot without chunk_end
    assert step(ctypes.byref(base), *args, -1, 0, ws, n, None) == cwu.EINVAL
    assert step(ctypes.byref(base), *args, C, 1, ws, n, None) == cwu.EINVAL
    assert step(ctypes.byref(base), *args, C - 1, 0, ws, n, None) == cwu.EINVAL
    # a workspace too small for the chunk buffer
    assert step(ctypes.byref(base), *args, 0, 0, ws, n - 256, None) == cwu.EWORKSPACE


def bwd_fake_args(prob):
    f = Fake()
    B, H, L, d = prob.batch, prob.heads, prob.seq_len, prob.dim
    P = d * d if prob.kind == cwu.LINEAR else 3 * d * prob.hidden
    nx, ns, np_ = B * H * L * d * 4, B * H * L * 4, B * H * P * 4
    a = dict(q=f(nx), k=f(nx), v=f(nx), eta=f(ns), alpha=f(ns), beta=f(ns), W0=f(np_),
             M0=f(np_), dout=f(nx), dW_end=f(np_), dM_end=f(np_), dq=f(nx), dk=f(nx), dv=f(nx),
             deta=f(ns), dalpha=f(ns), dbeta=f(ns), dW0=f(np_), dM0=f(np_))
    nws = cwu.backward_workspace_bytes(prob)
    a["workspace"] = f(nws)
    a["nws"] = nws
    return a


def bwd_call(prob, a):
    return cwu.chunk_backward(prob, a["q"], a["k"], a["v"], a["eta"], a["alpha"], a["beta"],
                              a["W0"], a["M0"], a["dout"], a["dW_end"], a["dM_end"], a["dq"],
                              a["dk"], a["dv"], a["deta"], a["dalpha"], a["dbeta"], a["dW0"],
                              a["dM0"], a["workspace"], a["nws"], stream=0, check=False)


def test_backward_support_and_workspace():
    lin = linear()
    n = cwu.backward_workspace_bytes(lin)
    assert n > cwu.workspace_bytes(lin) and n % 256 == 0
    assert cwu.backward_workspace_bytes(linear(seq_len=0)) == 0
    sw = swiglu(io_dtype=cwu.F32)
    n = cwu.backward_workspace_bytes(sw)
    assert n > cwu.workspace_bytes(sw) and n % 256 == 0
    assert cwu.backward_workspace_bytes(swiglu(io_dtype=cwu.F32, seq_len=0)) == 0
    for ok in (swiglu(), linear(io_dtype=cwu.BF16),  # bf16 io: widened at the boundary
               linear(flags=cwu.FLAG_QK_SILU_L2), swiglu(flags=cwu.FLAG_QK_SILU_L2)):
        assert cwu.backward_workspace_bytes(ok) > 0
    assert cwu.backward_workspace_bytes(linear(flags=cwu.FLAG_CHUNK_AVERAGED_DECAY)) > 0
    assert cwu.backward_workspace_bytes(swiglu(flags=cwu.FLAG_POST_CHUNK_ROW_L2)) > 0
    assert cwu.backward_workspace_bytes(swiglu(flags=cwu.FLAG_COMPENSATED_WEIGHTS)) > 0
    assert cwu.backward_workspace_bytes(linear(flags=cwu.FLAG_LACT_RULE)) > 0
    for bad in (linear(dim=128), linear(dim=80)):
        with pytest.raises(cwu.E2tttError) as e:
            cwu.backward_workspace_bytes(bad)
        assert e.value.status == cwu.EUNSUPPORTED
    assert cwu.lib().e2ttt_backward_workspace_bytes(ctypes.byref(lin), None) == cwu.EINVAL


@pytest.mark.parametrize("mutate,expected", [
    (lambda a: a.update(q=None), cwu.EINVAL),
    (lambda a: a.update(dout=None), cwu.EINVAL),
    (lambda a: a.update(dW0=None), cwu.EINVAL),
    (lambda a: a.update(deta=None), cwu.EINVAL),
    (lambda a: a.update(workspace=None), cwu.EINVAL),
    (lambda a: a.update(dk=a["dk"] + 4), cwu.EINVAL),            # misaligned
    (lambda a: a.update(workspace=a["workspace"] + 16), cwu.EINVAL),
    (lambda a: a.update(nws=a["nws"] - 256), cwu.EWORKSPACE),
    (lambda a: a.update(dq=a["q"]), cwu.EINVAL),                  # output over an input
    (lambda a: a.update(dW0=a["dW_end"]), cwu.EINVAL),            # in-place not allowed
    (lambda a: a.update(dM0=a["dW0"]), cwu.EINVAL),               # outputs alias
    (lambda a: a.update(workspace=a["dv"]), cwu.EINVAL),
])
def test_backward_host_errors(mutate, expected):
    for prob in (linear(), swiglu(io_dtype=cwu.F32, seq_len=300, batch=1, heads=2),
                 swiglu(seq_len=100, batch=1, heads=1)):
        a = bwd_fake_args(prob)
        mutate(a)
        assert bwd_call(prob, a) == expected
    bad = linear(dim=128)
    assert bwd_call(bad, bwd_fake_args(linear())) == cwu.EUNSUPPORTED


def test_state_keeping_entry_points_host_checks():
    """e2ttt_chunk_forward_states needs both state buffers when there is more
    than one chunk; e2ttt_chunk_backward_states takes both or neither; kept
    states may not overlap an output."""
    f = Fake()
    prob = linear()  # L = 256, C = 64: 4 chunks, 3 kept states
    B, H, L, d = prob.batch, prob.heads, prob.seq_len, prob.dim
    nx, ns, np_ = B * H * L * d * 4, B * H * L * 4, B * H * d * d * 4
    args = [f(nx), f(nx), f(nx), f(ns), f(ns), f(ns), f(np_), f(np_), f(nx), f(np_), f(np_)]
    Ws, Ms = f(3 * np_), f(3 * np_)
    nws = cwu.workspace_bytes(prob)
    ws = f(nws)
    call = lambda W, M: cwu.chunk_forward_states(prob, *args, W, M, ws, nws, stream=0,
                                                 check=False)
    assert call(None, Ms) == cwu.EINVAL
    assert call(Ws, None) == cwu.EINVAL
    assert call(Ws, Ws + 16) == cwu.EINVAL          # the two overlap
    assert call(Ws, args[9]) == cwu.EINVAL          # M_starts over W_end
    a = bwd_fake_args(prob)
    bcall = lambda W, M: cwu.chunk_backward(
        prob, a["q"], a["k"], a["v"], a["eta"], a["alpha"], a["beta"], a["W0"], a["M0"],
        a["dout"], a["dW_end"], a["dM_end"], a["dq"], a["dk"], a["dv"], a["deta"],
        a["dalpha"], a["dbeta"], a["dW0"], a["dM0"], a["workspace"], a["nws"], stream=0,
        check=False, W_starts=W, M_starts=M)
    assert bcall(Ws, None) == cwu.EINVAL
    assert bcall(a["dq"], Ms) == cwu.EINVAL         # kept states over an output
    assert bcall(Ws + 4, Ms) == cwu.EINVAL          # misaligned


def test_backward_kept_states_with_row_normalisation_unsupported():
    """The reverse of the row normalisation needs each chunk's end state before
    it; the kept (normalised) states do not carry it."""
    f = Fake()
    prob = linear(flags=cwu.FLAG_POST_CHUNK_ROW_L2)
    a = bwd_fake_args(prob)
    np_ = prob.dim * prob.dim * 4
    st = cwu.chunk_backward(
        prob, a["q"], a["k"], a["v"], a["eta"], a["alpha"], a["beta"], a["W0"], a["M0"],
        a["dout"], a["dW_end"], a["dM_end"], a["dq"], a["dk"], a["dv"], a["deta"], a["dalpha"],
        a["dbeta"], a["dW0"], a["dM0"], a["workspace"], a["nws"], stream=0, check=False,
        W_starts=f(3 * np_), M_starts=f(3 * np_))
    assert st == cwu.EUNSUPPORTED


def test_noalloc_size_and_problem_checked_on_the_host():
    """e2ttt_chunk_forward_noalloc checks the problem and the scratch size
    before any HIP call: EWORKSPACE for a problem whose workspace exceeds the
    built-in scratch, EINVAL for a malformed problem."""
    L = cwu.lib()
    big = swiglu(batch=8, heads=16, chunk=2048)
    assert cwu.workspace_bytes(big) > cwu.NOALLOC_SCRATCH_BYTES
    args = [None] * 11 + [None]
    assert L.e2ttt_chunk_forward_noalloc(ctypes.byref(big), *args) == cwu.EWORKSPACE
    assert L.e2ttt_chunk_forward_noalloc(ctypes.byref(swiglu(chunk=0)), *args) == cwu.EINVAL
    assert cwu.workspace_bytes(swiglu()) <= cwu.NOALLOC_SCRATCH_BYTES


def test_scalar_heads_checked_on_the_host():
    """e2ttt_scalar_heads rejects unsupported model dims and head counts, and
    null or misaligned pointers, before any HIP call."""
    L = cwu.lib()
    p = swiglu()
    assert L.e2ttt_scalar_heads(ctypes.byref(p), None, 96, None, None, 0.01, 0.1,
                                None, None, None, None) == cwu.EUNSUPPORTED
    assert L.e2ttt_scalar_heads(ctypes.byref(swiglu(heads=65)), None, 512, None, None, 0.01,
                                0.1, None, None, None, None) == cwu.EUNSUPPORTED
    assert L.e2ttt_scalar_heads(ctypes.byref(p), None, 512, None, None, 0.01, 0.1,
                                None, None, None, None) == cwu.EINVAL
    assert L.e2ttt_scalar_heads(ctypes.byref(swiglu(seq_len=0)), None, 512, None, None, 0.01,
                                0.1, None, None, None, None) == cwu.OK
    assert L.e2ttt_scalar_heads(ctypes.byref(swiglu(chunk=0)), None, 512, None, None, 0.01,
                                0.1, None, None, None, None) == cwu.EINVAL


def test_mlp_learner_entry_points():
    """The MLP learner: its own (larger, SwiGLU-layout) forward workspace;
    the decode step's workspace adds the state in that layout (for the
    chunk-end update); the backward's holds W0, M0 and their adjoints in that
    layout on top of the SwiGLU backward's at the same shape, less its own
    states' W3 blocks (none: the states are carried at 3dh too)."""
    assert cwu.workspace_bytes(swiglu(kind=cwu.MLP)) > cwu.workspace_bytes(
        swiglu(kind=cwu.MLP, seq_len=0))
    p = swiglu(kind=cwu.MLP)
    assert cwu.decode_workspace_bytes(p) >= (cwu.decode_workspace_bytes(swiglu()) +
                                             2 * 4 * p.batch * p.heads * 3 * p.dim * p.hidden)
    pm = swiglu(kind=cwu.MLP, io_dtype=cwu.F32)
    ps = swiglu(io_dtype=cwu.F32)
    extra = 4 * 4 * pm.batch * pm.heads * 3 * pm.dim * pm.hidden
    assert cwu.backward_workspace_bytes(pm) >= cwu.backward_workspace_bytes(ps) + extra


def test_problems_beyond_the_dispatch_limit_are_unsupported():
    """A launch of more than 2^32 work-items cannot be dispatched: such
    problems are EUNSUPPORTED before anything is enqueued (here the q/k
    prologue over 2^27 rows, which needs 2^33 work-items), while the same
    sequence without it fits."""
    big = linear(dim=16, seq_len=1 << 27, chunk=64)
    assert cwu.validate(big) == cwu.OK
    assert cwu.workspace_bytes(big) > 0
    with pytest.raises(cwu.E2tttError):
        cwu.workspace_bytes(linear(dim=16, seq_len=1 << 27, chunk=64, flags=cwu.FLAG_QK_SILU_L2))
