"""Seeded synthetic inputs for the delta-rule forward pass and decode step.

This module is shared by the fp64 oracle's tests and the GPU path's tests and
benchmark.  It draws random numbers and shapes them like the activations of the
models the pages describe; it contains none of the method's arithmetic (no state,
no recurrence, no chunking).

Distributions (per the pages' model descriptions):
  * q, k: Gaussian then L2-normalised per head (Gated DeltaNet layer design,
    "q/k path ... L2 Norm" on the delta-rule/DPLR page, section 3).
  * DeltaProduct keys: SiLU of a Gaussian, then L2-normalised; beta = 2*sigmoid
    (DeltaProduct notes, section 2.2, key/value/beta generation).
  * beta = sigmoid(N(0,1)) in (0,1) (write strength, section 1.1 / 3).
  * gate: log g = -softplus(N(0,1) + 2) (Mamba-2 style scalar decay, section 3),
    delivered in log space as the pages' chunk code takes it.
  * "weak" gate: log g = -softplus(N(0,1) - 4), a stress set that keeps the
    cross-chunk state alive.

Seeds: numpy PCG64 streams from SeedSequence([2026, cfg_id, stream]) with
streams q=0, k=1, v=2, beta=3, g=4, S0=5, dO=6, dS_final=7, KDA decays=8, decode step t -> 100 + t,
KDA decay of decode step t -> 300 + t.  Values are
drawn in fp64, cast to fp32, and for bf16 workloads rounded to the nearest bf16
(ties to even); both the oracle and the GPU consume exactly those values.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "CONFIGS", "make_inputs", "make_decode_inputs", "round_bf16", "get"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int              # tokens (not expanded)
    dk: int
    dv: int
    n_h: int = 1        # Householder steps per token
    chunk: int = 64     # in expanded positions
    dtype: str = "bf16"  # "f32" or "bf16": dtype of q, k, v, O
    gate: Optional[str] = None   # None | "cfg3" | "weak"
    key: str = "l2n"             # "l2n" | "silu_l2n"
    beta: str = "sigmoid"        # "sigmoid" | "2sigmoid" | "zero" | "one" | "two"
    s0: Optional[float] = None   # std of a Gaussian S0, or None for S0 = 0
    cfg_id: int = 0              # seed namespace

    @property
    def Lx(self) -> int:
        return self.L * self.n_h

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the build target (names say what they are).
CONFIGS = {
    "tiny_deltanet_f32": Workload("tiny_deltanet_f32", B=1, H=1, L=64, dk=16, dv=16, chunk=16,
                                  dtype="f32", cfg_id=1),
    "deltanet_b4h8_l2k": Workload("deltanet_b4h8_l2k", B=4, H=8, L=2048, dk=128, dv=128, chunk=64,
                                  cfg_id=2),
    "gdn_b2h16_l8k": Workload("gdn_b2h16_l8k", B=2, H=16, L=8192, dk=128, dv=128, chunk=64,
                              gate="cfg3", s0=0.1, cfg_id=3),
    "gdp2_b2h16_l4k": Workload("gdp2_b2h16_l4k", B=2, H=16, L=4096, dk=128, dv=128, n_h=2, chunk=64,
                               gate="cfg3", key="silu_l2n", beta="2sigmoid", cfg_id=4),
    "gdn_b1h16_l64k": Workload("gdn_b1h16_l64k", B=1, H=16, L=65536, dk=128, dv=128, chunk=64,
                               gate="cfg3", s0=0.1, cfg_id=5),
}
# Decode workload: 256 single-token steps at batch 64 from S ~ 0.1*N(0,1).
DECODE = Workload("gdn_decode_b64h16", B=64, H=16, L=1, dk=128, dv=128, chunk=64,
                  gate="cfg3", s0=0.1, cfg_id=5)
DECODE_STEPS = 256


def get(name: str) -> Workload:
    if name == DECODE.name:
        return DECODE
    return CONFIGS[name]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _rng(cfg_id: int, stream: int, salt: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([2026, cfg_id, stream, salt])))


def _l2n(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x)


def _draw(w: Workload, stream: int, shape, salt: int) -> np.ndarray:
    return _rng(w.cfg_id, stream, salt).standard_normal(size=shape)


def make_inputs(w: Workload, salt: int = 0) -> dict:
    """Inputs of one forward call, as float32 numpy arrays (bf16-exact for bf16).

    Layouts (token-major, contiguous):
      q [B, L, H, dk]; k [B, L*n_h, H, dk]; v [B, L*n_h, H, dv];
      beta [B, L*n_h, H] (f32); g_log [B, L, H] (f32) or None; S0 [B, H, dk, dv] or None.
    `salt` selects an independent draw of the same workload (stress variants).
    """
    B, L, H, dk, dv, Lx = w.B, w.L, w.H, w.dk, w.dv, w.Lx
    q = _l2n(_draw(w, 0, (B, L, H, dk), salt))
    kr = _draw(w, 1, (B, Lx, H, dk), salt)
    k = _l2n(_silu(kr)) if w.key == "silu_l2n" else _l2n(kr)
    v = _draw(w, 2, (B, Lx, H, dv), salt)
    bz = _draw(w, 3, (B, Lx, H), salt)
    if w.beta == "sigmoid":
        beta = _sigmoid(bz)
    elif w.beta == "2sigmoid":
        beta = 2.0 * _sigmoid(bz)
    elif w.beta == "zero":
        beta = np.zeros_like(bz)
    elif w.beta == "one":
        beta = np.ones_like(bz)
    elif w.beta == "two":
        beta = np.full_like(bz, 2.0)
    else:
        raise ValueError(w.beta)
    g_log = None
    if w.gate is not None:
        gz = _draw(w, 4, (B, L, H), salt)
        shift = {"cfg3": 2.0, "weak": -4.0}[w.gate]
        g_log = (-_softplus(gz + shift)).astype(np.float32)
    S0 = None
    if w.s0 is not None:
        S0 = (w.s0 * _draw(w, 5, (B, H, dk, dv), salt)).astype(np.float32)
    return {
        "q": _cast(q, w.dtype), "k": _cast(k, w.dtype), "v": _cast(v, w.dtype),
        "beta": beta.astype(np.float32), "g_log": g_log, "S0": S0,
    }


def make_cotangents(w: Workload, salt: int = 0) -> dict:
    """Gradients fed to a backward call: dO [B, L, H, dv] ~ N(0,1) in the workload's dtype
    (bf16-exact for bf16) and dS_final [B, H, dk, dv] ~ N(0,1) float32 (streams 6 and 7)."""
    dO = _draw(w, 6, (w.B, w.L, w.H, w.dv), salt)
    dS = _draw(w, 7, (w.B, w.H, w.dk, w.dv), salt).astype(np.float32)
    return {"dO": _cast(dO, w.dtype), "dS_final": dS}


def make_decode_inputs(w: Workload, step: int) -> dict:
    """Inputs of decode step `step` (one token per (b, h)), same layouts as make_inputs with L = 1."""
    B, H, dk, dv, nh = w.B, w.H, w.dk, w.dv, w.n_h
    rng = _rng(w.cfg_id, 100 + step)
    q = _l2n(rng.standard_normal((B, 1, H, dk)))
    kr = rng.standard_normal((B, nh, H, dk))
    k = _l2n(_silu(kr)) if w.key == "silu_l2n" else _l2n(kr)
    v = rng.standard_normal((B, nh, H, dv))
    bz = rng.standard_normal((B, nh, H))
    beta = 2.0 * _sigmoid(bz) if w.beta == "2sigmoid" else _sigmoid(bz)
    g_log = None
    if w.gate is not None:
        shift = {"cfg3": 2.0, "weak": -4.0}[w.gate]
        g_log = (-_softplus(rng.standard_normal((B, 1, H)) + shift)).astype(np.float32)
    return {"q": _cast(q, w.dtype), "k": _cast(k, w.dtype), "v": _cast(v, w.dtype),
            "beta": beta.astype(np.float32), "g_log": g_log}


def make_kda_decay(w: Workload, step: int) -> np.ndarray:
    """Per-key-channel log decay of decode step `step` for the KDA recurrence, [B, 1, H, dk]
    float32: -softplus(N(0,1) + shift) per channel (the scalar gate's distribution, drawn for
    every channel; shift as the workload's gate, cfg3 when it has none)."""
    rng = _rng(w.cfg_id, 300 + step)
    shift = {"cfg3": 2.0, "weak": -4.0}[w.gate or "cfg3"]
    return (-_softplus(rng.standard_normal((w.B, 1, w.H, w.dk)) + shift)).astype(np.float32)


def make_kda_decays(w: Workload, salt: int = 0) -> np.ndarray:
    """Per-key-channel log decays of a whole sequence for the KDA recurrence, [B, L, H, dk]
    float32 (stream 8): -softplus(N(0,1) + shift) per channel and token, shift as the workload's
    gate (cfg3 when it has none)."""
    shift = {"cfg3": 2.0, "weak": -4.0}[w.gate or "cfg3"]
    return (-_softplus(_draw(w, 8, (w.B, w.L, w.H, w.dk), salt) + shift)).astype(np.float32)


def make_decode_state(w: Workload) -> np.ndarray:
    """Initial decode state S ~ s0 * N(0,1), [B, H, dk, dv] float32."""
    return (w.s0 * _rng(w.cfg_id, 5).standard_normal((w.B, w.H, w.dk, w.dv))).astype(np.float32)
