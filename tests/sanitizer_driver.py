"""Run by tests/test_sanitizers.py in a child process whose libraries are the
AddressSanitizer + UndefinedBehaviorSanitizer builds of the host library and
of the oracle (E2TTT_LIBRARY, E2TTT_ORACLE_LIBRARY; the ASan runtime
preloaded).  No torch and no GPU: it exercises the library's host-side
argument checks and planning for every entry point, and the oracle's
functions on small inputs, comparing the latter with reference results the
parent computed with the regular oracle build (argv[1], an .npz)."""
import ctypes
import sys

import numpy as np

import chunk_weight_update_amd as cwu
import oracle
from chunk_weight_update_amd.inputs import (BF16, F32, LINEAR, MLP, SWIGLU, make_head_inputs,
                                            make_inputs)


def host_checks():
    L = cwu.lib()
    probs = []
    for kind, d, h in ((LINEAR, 64, 0), (SWIGLU, 128, 256), (SWIGLU, 768, 1536), (MLP, 256, 512)):
        for io in (F32, BF16):
            for flags in (0, 1, 2, 4, 8, 16, 32, 2 | 4 | 8, 1 | 16, 2 | 32):
                for L_ in (0, 1000, 4096):
                    probs.append(cwu.make_problem(kind, 2, 3, L_, d, h, 512, io, flags & 1, flags))
    probs.append(cwu.make_problem(SWIGLU, 1, 1, 1 << 27, 128, 256, 64, BF16, 0, 4))
    probs.append(cwu.make_problem(7, 1, 1, 8, 16, 0, 4, F32))
    n = ctypes.c_size_t(0)
    for p in probs:
        b = ctypes.byref(p)
        L.e2ttt_validate(b)
        L.e2ttt_workspace_bytes(b, ctypes.byref(n))
        L.e2ttt_decode_workspace_bytes(b, ctypes.byref(n))
        L.e2ttt_backward_workspace_bytes(b, ctypes.byref(n))
        # Null tensors: rejected on the host, before any HIP call.
        L.e2ttt_chunk_forward(b, *([None] * 12), 0, None)
        L.e2ttt_chunk_forward_noalloc(b, *([None] * 11), None)
        L.e2ttt_scalar_heads(b, None, 512, None, None, 0.01, 0.1, None, None, None, None)
        L.e2ttt_scalar_heads(b, None, 96, None, None, 0.01, 0.1, None, None, None, None)
    L.e2ttt_validate(None)
    for s in range(-1, 7):
        L.e2ttt_status_string(s)


def oracle_runs():
    out = {}
    for kind, d, h in ((LINEAR, 4, 0), (SWIGLU, 3, 5), (MLP, 4, 3)):
        inp = make_inputs(kind, 1, 2, 13, d, h, F32, seed=kind, m0_scale=0.1)
        a = (inp["q64"], inp["k64"], inp["v64"], inp["eta"], inp["alpha"], inp["beta"],
             inp["W0"], inp["M0"])
        for name, kw in (("plain", {}), ("avg", {"averaged": True}), ("lact", {"lact": True}),
                         ("qk_row", {"qk_norm": True, "row_norm": True}),
                         ("mode1", {"decay_mode": 1})):
            for i, x in enumerate(oracle.chunk_forward(kind, *a, 5, h, **kw)):
                out[f"fwd_{kind}_{name}_{i}"] = x
        if kind != MLP:
            rng = np.random.default_rng(3)
            up = [rng.standard_normal(x.shape) for x in (inp["q64"], inp["W0"], inp["W0"])]
            g = oracle.chunk_backward(kind, *a, *up, 5, hidden=h, qk_norm=True, row_norm=True)
            for n_, x in g.items():
                out[f"bwd_{kind}_{n_}"] = x
    kw, km, cf = oracle.scalar_kernels(inp["eta"][0], inp["alpha"][0], inp["beta"][0])
    out["sk_kw"], out["sk_km"], out["sk_cf"] = kw, km, cf
    hin = make_head_inputs(2, 9, 64, 3, BF16, seed=1)
    for i, x in enumerate(oracle.scalar_heads(hin["x64"], hin["w64"], hin["bias"], 3, 0.01, 0.1)):
        out[f"heads_{i}"] = x
    return out


if __name__ == "__main__":
    host_checks()
    got = oracle_runs()
    if len(sys.argv) > 2 and sys.argv[2] == "write":
        np.savez(sys.argv[1], **got)
    else:
        ref = np.load(sys.argv[1])
        for k, v in got.items():
            r = ref[k]
            err = float(np.max(np.abs(v - r))) if v.size else 0.0
            assert err <= 1e-13 * max(1.0, float(np.max(np.abs(r)))), (k, err)
    print("sanitizer driver: ok", flush=True)
