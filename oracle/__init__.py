"""fp64 CPU oracle of the delta-rule forward pass, decode step and UT/WY factors.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product library (which must fail
loudly when its HIP library is missing rather than fall back to this code).
The oracle shares no code with the GPU path.

Functions
---------
fwd(...)        the token-by-token recurrence in fp64 (oracle.c); the definition
                of what delta_fwd and delta_decode compute.
bwd(...)        its gradients by reverse-mode differentiation of the same recurrence
                (oracle.c), for the backward pass.
fwd_kda(...)    the KDA recurrence (per-key-channel decay, then the delta-rule write),
                in fp64 (oracle.c); decode_kda is its one-token step.
ut_factors(...) the per-chunk UT transform T = (I + strictLower(diag(beta)
                (Gamma * K K^T)))^-1 diag(beta) and the WY factors
                W = T (gamma * K), U = T V, written from their definitions with a
                library triangular solve (what delta_chunk_wy computes).

layer (module)  the layer steps around the token mixer: causal depthwise ShortConv, SiLU,
                per-head L2 norm (prologue), RMS norm times a SiLU gate (epilogue), in
                numpy fp64; pinned in tests/test_oracle_layer.py.

All of them are pinned in tests/test_oracle_pins.py (closed forms, brute force,
independent formulations, finite differences); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import scipy.linalg

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile oracle.c into liboracle.so (plain C, fp64, OpenMP)."""
    import subprocess
    src = os.path.join(_HERE, "oracle.c")
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        lib.oracle_fwd.argtypes = [ctypes.c_int] * 6 + [ctypes.c_double] + [P] * 8 + [ctypes.c_int]
        lib.oracle_fwd.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_bwd.argtypes = [ctypes.c_int] * 6 + [ctypes.c_double] + [P] * 14 + [ctypes.c_int]
        lib.oracle_bwd.restype = ctypes.c_int
        lib.oracle_fwd_kda.argtypes = [ctypes.c_int] * 5 + [ctypes.c_double] + [P] * 8 + [ctypes.c_int]
        lib.oracle_fwd_kda.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f32(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float32)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def fwd(q, k, v, beta, g_log=None, S0=None, n_h: int = 1, scale: float = 1.0,
        nthreads: int = 0):
    """fp64 recurrence.  Shapes: q [B,L,H,dk], k [B,L*n_h,H,dk], v [B,L*n_h,H,dv],
    beta [B,L*n_h,H], g_log [B,L,H] or None, S0 [B,H,dk,dv] or None.
    Inputs are taken as float32 (exact for bf16 values).  Returns (O, S_final) in fp64.
    """
    q, k, v, beta, g_log, S0 = map(_f32, (q, k, v, beta, g_log, S0))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    Lx = L * n_h
    assert k.shape == (B, Lx, H, dk), (k.shape, (B, Lx, H, dk))
    assert v.shape == (B, Lx, H, dv)
    assert beta.shape == (B, Lx, H)
    assert g_log is None or g_log.shape == (B, L, H)
    assert S0 is None or S0.shape == (B, H, dk, dv)
    O = np.empty((B, L, H, dv), dtype=np.float64)
    S_final = np.empty((B, H, dk, dv), dtype=np.float64)
    rc = _load().oracle_fwd(B, L, H, dk, dv, n_h, float(scale), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(beta), _ptr(g_log), _ptr(S0), _ptr(O), _ptr(S_final),
                            int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_fwd failed (%d)" % rc)
    return O, S_final


def bwd(q, k, v, beta, g_log, S0, dO, dS_final=None, n_h: int = 1, scale: float = 1.0,
        nthreads: int = 0):
    """Gradients of fwd (oracle.c, oracle_bwd: reverse-mode differentiation of the same
    recurrence in fp64) for the loss <O, dO> + <S_final, dS_final>.  Inputs as fwd, plus dO
    [B,L,H,dv] and dS_final [B,H,dk,dv] or None (taken as float32).  Returns a dict of fp64
    arrays dq, dk, dv, dbeta, dg_log (None when ungated), dS0."""
    q, k, v, beta, g_log, S0, dO, dS_final = map(_f32, (q, k, v, beta, g_log, S0, dO, dS_final))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    Lx = L * n_h
    assert k.shape == (B, Lx, H, dk) and v.shape == (B, Lx, H, dv) and beta.shape == (B, Lx, H)
    assert g_log is None or g_log.shape == (B, L, H)
    assert S0 is None or S0.shape == (B, H, dk, dv)
    assert dO.shape == (B, L, H, dv)
    assert dS_final is None or dS_final.shape == (B, H, dk, dv)
    out = {"dq": np.empty((B, L, H, dk)), "dk": np.empty((B, Lx, H, dk)), "dv": np.empty((B, Lx, H, dv)),
           "dbeta": np.empty((B, Lx, H)), "dg_log": np.empty((B, L, H)) if g_log is not None else None,
           "dS0": np.empty((B, H, dk, dv))}
    rc = _load().oracle_bwd(B, L, H, dk, dv, n_h, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                            _ptr(g_log), _ptr(S0), _ptr(dO), _ptr(dS_final), _ptr(out["dq"]),
                            _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]), _ptr(out["dg_log"]),
                            _ptr(out["dS0"]), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_bwd failed (%d)" % rc)
    return out


def fwd_kda(q, k, v, beta, a_log, S0=None, scale: float = 1.0, nthreads: int = 0):
    """The KDA recurrence in fp64 (oracle.c, oracle_fwd_kda): per token, the state's key
    channels decay by exp(a_log) (vector), then the delta-rule write, then the readout.
    q, k [B,L,H,dk], v [B,L,H,dv], beta [B,L,H], a_log [B,L,H,dk], S0 [B,H,dk,dv] or None.
    Returns (O, S_final) in fp64."""
    q, k, v, beta, a_log, S0 = map(_f32, (q, k, v, beta, a_log, S0))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, L, H, dk) and v.shape == (B, L, H, dv) and beta.shape == (B, L, H)
    assert a_log.shape == (B, L, H, dk)
    assert S0 is None or S0.shape == (B, H, dk, dv)
    O = np.empty((B, L, H, dv))
    S_final = np.empty((B, H, dk, dv))
    rc = _load().oracle_fwd_kda(B, L, H, dk, dv, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                _ptr(a_log), _ptr(S0), _ptr(O), _ptr(S_final), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_fwd_kda failed (%d)" % rc)
    return O, S_final


def decode_kda(q, k, v, beta, a_log, S, scale: float = 1.0):
    """One KDA decode step per (b, h): q, k [B,1,H,dk], v [B,1,H,dv], beta [B,1,H],
    a_log [B,1,H,dk], S [B,H,dk,dv].  Returns (O [B,1,H,dv], S_new) in fp64."""
    return fwd_kda(q, k, v, beta, a_log, S, scale=scale)


def decode(q, k, v, beta, g_log, S, n_h: int = 1, scale: float = 1.0):
    """One decode step per (b, h): the recurrence body for a single token.
    q [B,1,H,dk], k [B,n_h,H,dk], v [B,n_h,H,dv], beta [B,n_h,H], g_log [B,1,H] or None,
    S [B,H,dk,dv].  Returns (O [B,1,H,dv], S_new) in fp64."""
    return fwd(q, k, v, beta, g_log, S, n_h=n_h, scale=scale)


def ut_factors(k, v, beta, g_log=None, n_h: int = 1, chunk: int = 64):
    """Per-chunk UT transform and WY factors, in fp64, from their definitions.

    "08 linear delta rule & DPLR" page, section 2.2 (UT transform:
    T = [I + strictLower(diag(beta) K K^T)]^-1 diag(beta), W = T K, U = T V) and
    section 3 (gated form: the Gram matrix is multiplied elementwise by
    Gamma_ij = gamma_i / gamma_j, and W uses keys decayed to the chunk start,
    gamma_r k_r, where gamma_r is the product of the gates up to position r of the
    chunk, restarting at every chunk).  For n_h > 1 the keys, values and betas are
    the expanded sequence and the log gate sits at each token's first sub-step
    (DeltaProduct notes, section 4.1).  A tail chunk is padded with k = v = beta = 0
    and log g = 0.

    Returns dict of fp64 arrays: T [B,H,NT,C,C], W [B,H,NT,C,dk], U [B,H,NT,C,dv],
    gc [B,H,NT,C] (cumulative log gate within the chunk).
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, Lx, H, dk = k.shape
    dv = v.shape[-1]
    C = chunk
    NT = -(-Lx // C)
    pad = NT * C - Lx
    # expanded-sequence log gate: g at the first sub-step of each token, 0 elsewhere
    glx = np.zeros((B, Lx, H))
    if g_log is not None:
        glx[:, ::n_h, :] = np.asarray(g_log, dtype=np.float64)

    def chunked(x):  # [B, Lx, H, ...] -> [B, H, NT, C, ...]
        x = np.concatenate([x, np.zeros((B, pad) + x.shape[2:])], axis=1) if pad else x
        x = np.moveaxis(x, 2, 1)
        return x.reshape((B, H, NT, C) + x.shape[3:])

    kc, vc, bc, gcl = chunked(k), chunked(v), chunked(beta), chunked(glx)
    gc = np.cumsum(gcl, axis=-1)
    T = np.zeros((B, H, NT, C, C))
    W = np.zeros((B, H, NT, C, dk))
    U = np.zeros((B, H, NT, C, dv))
    eye = np.eye(C)
    for b in range(B):
        for h in range(H):
            for n in range(NT):
                K, V, bt, g = kc[b, h, n], vc[b, h, n], bc[b, h, n], gc[b, h, n]
                gam = np.exp(g[:, None] - g[None, :])
                A = np.tril(bt[:, None] * (gam * (K @ K.T)), -1)
                Tn = scipy.linalg.solve_triangular(eye + A, np.diag(bt), lower=True,
                                                   unit_diagonal=True)
                T[b, h, n] = Tn
                W[b, h, n] = Tn @ (np.exp(g)[:, None] * K)
                U[b, h, n] = Tn @ V
    return {"T": T, "W": W, "U": U, "gc": gc}
