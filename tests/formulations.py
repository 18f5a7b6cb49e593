"""Independent fp64 formulations of the delta rule, used only to pin the oracle.

Each routine takes a different route to the same mathematical object than the
oracle's token loop (oracle/oracle.c) or its UT-factor routine
(oracle.ut_factors), so that a slip in either one shows up as a disagreement:

  brute_force   materialised d_k x d_k transition products per token
                (DeltaProduct notes, section 2.3: A_i = F_{n_h}...F_1,
                B_i = sum_j F_{n_h}...F_{j+1} C_j; gated form, section 2.6)
  chunked       the chunkwise WY/UT algorithm ("08 linear delta rule & DPLR"
                page, sections 2.2-2.3, gated form in section 3) with T obtained
                by row-by-row forward substitution
  dplr          the generic diagonal-plus-low-rank recurrence of the same page,
                section 5, under the DeltaNet / Gated DeltaNet reductions
  erase_write_step, gd_step
                one update in the erase-write form (section 1.1) and as one
                gradient-descent step on 1/2 ||S^T k - v||^2 (section 1.3)
  wy_recursive  the sequential w/u recursions of the WY representation
                (section 2.1), with the gate weights of section 3
  one_chunk_closed_form
                the fully parallel form O = (Q K^T * M) T V of section 2.4
                (S0 = 0, ungated, one chunk)
"""
from __future__ import annotations

import numpy as np
import scipy.linalg


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def brute_force(q, k, v, beta, g_log=None, S0=None, n_h=1, scale=1.0):
    q, k, v, beta, g_log, S0 = map(_f64, (q, k, v, beta, g_log, S0))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    O = np.zeros((B, L, H, dv))
    SF = np.zeros((B, H, dk, dv))
    I = np.eye(dk)
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[b, h].copy()
            for i in range(L):
                F = [I - beta[b, i * n_h + j, h] * np.outer(k[b, i * n_h + j, h], k[b, i * n_h + j, h])
                     for j in range(n_h)]
                Cw = [beta[b, i * n_h + j, h] * np.outer(k[b, i * n_h + j, h], v[b, i * n_h + j, h])
                      for j in range(n_h)]
                A = I.copy()
                for j in range(n_h):
                    A = F[j] @ A
                if g_log is not None:
                    A = np.exp(g_log[b, i, h]) * A
                Bm = np.zeros((dk, dv))
                for j in range(n_h):
                    P = I.copy()
                    for jj in range(j + 1, n_h):
                        P = F[jj] @ P
                    Bm += P @ Cw[j]
                S = A @ S + Bm
                O[b, i, h] = scale * (S.T @ q[b, i, h])
            SF[b, h] = S
    return O, SF


def transition(k_steps, beta_steps, g=1.0):
    """A = g * F_{n_h} ... F_1 for one token (DeltaProduct notes, sections 2.3 / 2.6)."""
    dk = k_steps.shape[-1]
    A = np.eye(dk)
    for kk, bb in zip(k_steps, beta_steps):
        A = (np.eye(dk) - bb * np.outer(kk, kk)) @ A
    return g * A


def _forward_substitution_inverse(A):
    """(I + A)^-1 for strictly-lower A, row by row: N_i = e_i - sum_{j<i} A_ij N_j."""
    C = A.shape[0]
    N = np.zeros((C, C))
    for i in range(C):
        row = np.zeros(C)
        row[i] = 1.0
        for j in range(i):
            row -= A[i, j] * N[j]
        N[i] = row
    return N


def chunked(q, k, v, beta, g_log=None, S0=None, n_h=1, C=16, scale=1.0):
    """Chunkwise algorithm in fp64 on the expanded sequence; T by forward substitution."""
    q, k, v, beta, g_log, S0 = map(_f64, (q, k, v, beta, g_log, S0))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    Lx = L * n_h
    NT = -(-Lx // C)
    O = np.zeros((B, L, H, dv))
    SF = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[b, h].copy()
            for n in range(NT):
                pos = np.arange(n * C, min((n + 1) * C, Lx))
                c = len(pos)
                K = k[b, pos, h]
                V = v[b, pos, h]
                bt = beta[b, pos, h]
                lg = np.zeros(c)
                if g_log is not None:
                    first = (pos % n_h) == 0
                    lg[first] = g_log[b, pos[first] // n_h, h]
                gc = np.cumsum(lg)
                gam = np.exp(gc)
                lower = np.tril(np.ones((c, c), dtype=bool))
                Gam = np.exp(np.where(lower, gc[:, None] - gc[None, :], -np.inf))
                A = np.tril(bt[:, None] * Gam * (K @ K.T), -1)
                T = _forward_substitution_inverse(A) * bt[None, :]
                W = T @ (gam[:, None] * K)
                U = T @ V
                Vt = U - W @ S                                    # pseudo-values
                Qfull = np.zeros((c, dk))
                last = (pos % n_h) == n_h - 1
                Qfull[last] = q[b, pos[last] // n_h, h] * scale
                Aqk = (Qfull @ K.T) * Gam                         # Gam is lower incl. diagonal
                Oc = (gam[:, None] * Qfull) @ S + Aqk @ Vt
                for r in np.nonzero(last)[0]:
                    O[b, pos[r] // n_h, h] = Oc[r]
                gC = gam[-1]
                S = gC * S + (np.exp(gc[-1] - gc)[:, None] * K).T @ Vt
            SF[b, h] = S
    return O, SF


def dplr(q, w_log, a, bvec, kk, vv, S0=None, scale=1.0):
    """S_t = (Diag(w_t) + a_t b_t^T) S_{t-1} + kk_t vv_t^T, o_t = S_t^T (q_t scale).
    w_log [B,T,H,dk] (log of the diagonal), a/bvec/kk [B,T,H,dk], vv [B,T,H,dv]."""
    q, w_log, a, bvec, kk, vv, S0 = map(_f64, (q, w_log, a, bvec, kk, vv, S0))
    B, T, H, dk = q.shape
    dv = vv.shape[-1]
    O = np.zeros((B, T, H, dv))
    SF = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[b, h].copy()
            for t in range(T):
                S = (np.exp(w_log[b, t, h])[:, None] * S
                     + np.outer(a[b, t, h], bvec[b, t, h] @ S)
                     + np.outer(kk[b, t, h], vv[b, t, h]))
                O[b, t, h] = S.T @ (q[b, t, h] * scale)
            SF[b, h] = S
    return O, SF


def erase_write_step(S, k, v, beta):
    """Erase the value bound to k, write the beta-interpolation of old and new."""
    v_old = S.T @ k
    v_new = beta * v + (1.0 - beta) * v_old
    return S - np.outer(k, v_old) + np.outer(k, v_new)


def gd_step(S, k, v, beta):
    """One gradient-descent step with learning rate beta on 1/2 ||S^T k - v||^2."""
    grad = np.outer(k, S.T @ k - v)
    return S - beta * grad


def wy_recursive(K, V, beta, gc=None):
    """Sequential WY vectors of one chunk (gated: weights Gamma_ri = exp(gc_r - gc_i)).
    w_r = beta_r (gamma_r k_r - sum_{i<r} Gamma_ri (k_r . k_i) w_i),
    u_r = beta_r (v_r - sum_{i<r} Gamma_ri (k_r . k_i) u_i)."""
    K, V, beta = _f64(K), _f64(V), _f64(beta)
    C = K.shape[0]
    gc = np.zeros(C) if gc is None else _f64(gc)
    Wv = np.zeros_like(K)
    Uv = np.zeros_like(V)
    for r in range(C):
        wr = np.exp(gc[r]) * K[r].copy()
        ur = V[r].copy()
        for i in range(r):
            cf = np.exp(gc[r] - gc[i]) * (K[r] @ K[i])
            wr -= cf * Wv[i]
            ur -= cf * Uv[i]
        Wv[r] = beta[r] * wr
        Uv[r] = beta[r] * ur
    return Wv, Uv


def one_chunk_closed_form(q, k, v, beta):
    """O = (Q K^T * M) T V for a single chunk from S = 0, ungated (M inclusive causal)."""
    Q, K, V, bt = map(_f64, (q, k, v, beta))
    C = K.shape[0]
    A = np.tril(bt[:, None] * (K @ K.T), -1)
    T = scipy.linalg.solve_triangular(np.eye(C) + A, np.diag(bt), lower=True, unit_diagonal=True)
    return np.tril(Q @ K.T) @ T @ V
