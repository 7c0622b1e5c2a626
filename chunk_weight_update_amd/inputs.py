"""Seeded synthetic inputs for the E2-TTT chunk forward.

This module draws inputs only; it holds none of the method's arithmetic, so
both the oracle-side tests and the HIP side may use it.

Recipe (all draws from numpy's PCG64 ``default_rng(seed)``, in this order):
  1. q, k, v ~ N(0, 1) of shape [B, H, L, d] in fp64, each token L2-normalised
     over d (the E2-TTT branch normalises q and k, §4; the workloads normalise
     v too), then cast to fp32 and, for bf16 workloads, rounded to bf16
     (round-to-nearest-even).
  2. z_eta, z_alpha, z_beta ~ N(0, 1) of shape [B, H, L]; the per-token
     scalars are sigmoid transforms of them (``SCALARS`` below), stored fp32.
  3. Fast weights, per tensor over all (b, h): W1 [B,H,h,d], W3 [B,H,h,d],
     W2 [B,H,d,h] ~ N(0, 1/fan_in) (fan_in = d for W1, W3 and the linear W;
     h for W2), fp32, packed [W1 | W3 | W2] per (b, h); the MLP learner
     draws W1 then W2, packed [W1 | W2].
  4. M0 = 0, or with ``m0_scale`` > 0: M0 ~ N(0, m0_scale/fan_in) drawn in the
     same tensor order, so the M0 terms of the chunk-end state are exercised.

The two scalar regimes: "default" (eta = 0.1*s(z), alpha = 1 - 0.05*s(z),
beta = 0.9*s(z)) and "nearunit", which uses the base scalars of App. B.1/B.3
(eta_base = 1e-2, alpha_base = 1e-1) with beta close to one, the near-unit
retention regime (i) of App. A.3.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

LINEAR = 0
SWIGLU = 1
MLP = 2
F32 = 0
BF16 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: int
    B: int
    H: int
    L: int
    d: int
    h: int
    C: int
    io: int
    regime: str = "default"

    @property
    def P(self) -> int:
        if self.kind == LINEAR:
            return self.d * self.d
        return (2 if self.kind == MLP else 3) * self.d * self.h

    @property
    def n_chunks(self) -> int:
        return -(-self.L // self.C) if self.L > 0 else 0

    def describe(self) -> Dict:
        return {"workload": self.name,
                "learner": {LINEAR: "linear", SWIGLU: "swiglu", MLP: "mlp"}[self.kind],
                "batch": self.B, "heads": self.H, "seq_len": self.L,
                "dim": self.d, "hidden": self.h, "chunk": self.C,
                "io_dtype": "bf16" if self.io == BF16 else "fp32",
                "scalars": self.regime}


WORKLOADS = {w.name: w for w in [
    Workload("linear-d64-b1h1-l256-c64-fp32", LINEAR, 1, 1, 256, 64, 0, 64, F32),
    Workload("swiglu-d128h256-b2h4-l4096-c512-bf16", SWIGLU, 2, 4, 4096, 128, 256, 512, BF16),
    Workload("swiglu-d128h256-b8h16-l4096-c2048-bf16", SWIGLU, 8, 16, 4096, 128, 256, 2048, BF16),
    Workload("swiglu-d128h256-b1h16-l32768-c2048-bf16", SWIGLU, 1, 16, 32768, 128, 256, 2048, BF16),
    Workload("swiglu-d768h1536-b1h1-l57344-c8192-bf16", SWIGLU, 1, 1, 57344, 768, 1536, 8192, BF16),
    Workload("swiglu-d128h256-b1h1-l65536-c512-fp32-nearunit", SWIGLU, 1, 1, 65536, 128, 256, 512,
             F32, "nearunit"),
    Workload("swiglu-d128h256-b2h4-l4096-c512-bf16-nearunit", SWIGLU, 2, 4, 4096, 128, 256, 512, BF16,
             "nearunit"),
    Workload("swiglu-d128h256-b1h16-l32768-c2048-bf16-nearunit", SWIGLU, 1, 16, 32768, 128, 256,
             2048, BF16, "nearunit"),
    Workload("swiglu-d768h1536-b1h1-l24576-c8192-bf16-nearunit", SWIGLU, 1, 1, 24576, 768, 1536,
             8192, BF16, "nearunit"),
]}

# The workload the benchmark line is quoted on.
BENCH_WORKLOAD = "swiglu-d768h1536-b1h1-l57344-c8192-bf16"


def _sig(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


SCALARS = {
    "default": lambda ze, za, zb: (0.1 * _sig(ze), 1.0 - 0.05 * _sig(za), 0.9 * _sig(zb)),
    "nearunit": lambda ze, za, zb: (0.01 * _sig(ze), 0.1 * _sig(za), 1.0 - 0.01 * _sig(zb)),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _unit_rows(rng, shape) -> np.ndarray:
    x = rng.standard_normal(shape)
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    n[n == 0] = 1.0
    return x / n


def make_inputs(kind: int, B: int, H: int, L: int, d: int, h: int, io: int,
                seed: int = 0, regime: str = "default", m0_scale: float = 0.0,
                ) -> Dict[str, np.ndarray]:
    """Draw one problem.  Returns numpy arrays:
      q, k, v      : io representation ([B,H,L,d] float32, or uint16 bf16 bits)
      q64,k64,v64  : the same values widened to float64 (what the oracle sees)
      eta, alpha, beta : [B,H,L] float32
      W0, M0       : [B,H,P] float32
    """
    rng = np.random.default_rng(seed)
    out: Dict[str, np.ndarray] = {}
    for name in ("q", "k", "v"):
        x32 = _unit_rows(rng, (B, H, L, d)).astype(np.float32)
        if io == BF16:
            bits = f32_to_bf16_bits(x32)
            out[name] = bits
            out[name + "64"] = bf16_bits_to_f32(bits).astype(np.float64)
        else:
            out[name] = x32
            out[name + "64"] = x32.astype(np.float64)
    ze = rng.standard_normal((B, H, L))
    za = rng.standard_normal((B, H, L))
    zb = rng.standard_normal((B, H, L))
    eta, alpha, beta = SCALARS[regime](ze, za, zb)
    out["eta"] = eta.astype(np.float32)
    out["alpha"] = alpha.astype(np.float32)
    out["beta"] = beta.astype(np.float32)

    def draw_state(scale: float) -> np.ndarray:
        if kind == LINEAR:
            return (rng.standard_normal((B, H, d, d)) * np.sqrt(scale / d)
                    ).reshape(B, H, d * d).astype(np.float32)
        W1 = rng.standard_normal((B, H, h, d)) * np.sqrt(scale / d)
        if kind == MLP:  # [W1 | W2]
            W2 = rng.standard_normal((B, H, d, h)) * np.sqrt(scale / h)
            return np.concatenate([W1.reshape(B, H, -1), W2.reshape(B, H, -1)],
                                  axis=-1).astype(np.float32)
        W3 = rng.standard_normal((B, H, h, d)) * np.sqrt(scale / d)
        W2 = rng.standard_normal((B, H, d, h)) * np.sqrt(scale / h)
        return np.concatenate([W1.reshape(B, H, -1), W3.reshape(B, H, -1),
                               W2.reshape(B, H, -1)], axis=-1).astype(np.float32)

    out["W0"] = draw_state(1.0)
    P = out["W0"].shape[-1]
    out["M0"] = draw_state(m0_scale) if m0_scale > 0 else np.zeros((B, H, P), np.float32)
    return out


def make_workload_inputs(w: Workload, seed: int = 0, m0_scale: float = 0.0,
                         L: Optional[int] = None, B: Optional[int] = None,
                         H: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs shaped like workload ``w`` (optionally with fewer tokens/units)."""
    return make_inputs(w.kind, B or w.B, H or w.H, w.L if L is None else L, w.d, w.h,
                       w.io, seed=seed, regime=w.regime, m0_scale=m0_scale)


def make_head_inputs(B: int, L: int, D: int, H: int, io: int, seed: int = 0,
                     ) -> Dict[str, np.ndarray]:
    """Inputs of the per-token scalar heads (numpy PCG64, in this order):
      x [B, L, D] ~ N(0, 1), the layer input (unit-variance hidden states);
      w [3H, D] ~ N(0, 1/D), the eta, alpha and beta head weights, so that
        every pre-activation <w, x> is ~ N(0, 1) like the workloads' z draws;
      bias [3H] ~ N(0, 0.25).
    x and w are rounded to bf16 (RNE) for bf16 problems; the bias stays fp32.
    Returns the io representations (x, w) and their fp64 widenings (x64,
    w64), and bias (fp32)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, L, D)).astype(np.float32)
    w = (rng.standard_normal((3 * H, D)) / np.sqrt(D)).astype(np.float32)
    bias = (0.5 * rng.standard_normal(3 * H)).astype(np.float32)
    out: Dict[str, np.ndarray] = {"bias": bias}
    for name, a in (("x", x), ("w", w)):
        if io == BF16:
            bits = f32_to_bf16_bits(a)
            out[name] = bits
            out[name + "64"] = bf16_bits_to_f32(bits).astype(np.float64)
        else:
            out[name] = a
            out[name + "64"] = a.astype(np.float64)
    return out

