"""Shared helpers of the GPU parity tests: move seeded inputs to the GPU, run the library,
run the oracle on the same values, and compare with the error measure below.

err(X) = max over (b, h) of max|X - X_ref| / max|X_ref|, separately for O and S_final
(a per-head relative error that stays meaningful where individual entries are near 0).
Tolerances: 1e-4 for float32 inputs, 2e-2 for bf16 inputs with float32 state.
"""
from __future__ import annotations

import sys

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def head_rel_err(x, ref, head_axes):
    """max over heads of max|x - ref| / max|ref|; head_axes are the axes indexing (b, h)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    other = tuple(i for i in range(ref.ndim) if i not in head_axes)
    num = np.abs(x - ref).max(axis=other) if other else np.abs(x - ref)
    den = np.abs(ref).max(axis=other) if other else np.abs(ref)
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return float(np.max(rel)) if rel.size else 0.0


def to_dev(x, dtype):
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def inputs_to_dev(inp, dtype):
    return {
        "q": to_dev(inp["q"], dtype), "k": to_dev(inp["k"], dtype), "v": to_dev(inp["v"], dtype),
        "beta": to_dev(inp["beta"], "f32"), "g_log": to_dev(inp["g_log"], "f32"),
        "S0": to_dev(inp["S0"], "f32"),
    }


def to_np(t):
    return t.float().cpu().numpy()
