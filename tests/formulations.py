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
  chunked_kda   a chunkwise form of KDA (a decay per key channel), derived below
                from the recurrence of the page's section 1.4 table and section 5;
                it pins oracle.fwd_kda
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


def chunked_kda(q, k, v, beta, a_log, S0=None, C=16, scale=1.0):
    """Chunkwise KDA in fp64.  The pages give KDA's recurrence, S_t = (I - b_t k_t k_t^T) D_t
    S_{t-1} + b_t k_t v_t^T with D_t = Diag(alpha_t) ("08 linear delta rule & DPLR", section 1.4
    table and section 5), but not a chunk algorithm; this one follows from it.

    Write the update as S_t = D_t S_{t-1} + k_t u_t^T with u_t = b_t (v_t - S_{t-1}^T D_t k_t).
    Inside a chunk that starts from S, with G_r = D_1 ... D_r (cumulative, restarting each chunk),
    S_r = G_r S + sum_{j<=r} G_r G_j^-1 k_j u_j^T, so
        u_r + b_r sum_{j<r} (k_r^T G_r G_j^-1 k_j) u_j = b_r (v_r - S^T G_r k_r),
    i.e. U = T (V - (K G) S) with T = (I + A)^-1 diag(b), A_rj = b_r k_r^T G_r G_j^-1 k_j (j < r):
    the UT transform of section 2.2 with the Gram matrix decayed per channel.  The readout
    o_r = S_r^T q_r gives O = scale ((Q G) S + Aqk U), Aqk_rj = q_r^T G_r G_j^-1 k_j (j <= r), and
    the chunk ends at S' = G_C S + (K G_C G^-1)^T U.  The ratios G_r G_j^-1 are formed only for
    j <= r, where they are products of decays (no overflow).  A log decay of -inf (alpha = 0) is
    taken as -800, whose exponential is exactly 0 in fp64 (so a reset stays exact)."""
    q, k, v, beta, a_log, S0 = map(_f64, (q, k, v, beta, a_log, S0))
    a_log = np.maximum(a_log, -800.0)
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    NT = -(-L // C)
    O = np.zeros((B, L, H, dv))
    SF = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[b, h].copy()
            for n in range(NT):
                pos = np.arange(n * C, min((n + 1) * C, L))
                c = len(pos)
                K, V, Q, bt = k[b, pos, h], v[b, pos, h], q[b, pos, h] * scale, beta[b, pos, h]
                Gc = np.cumsum(a_log[b, pos, h], axis=0)                       # [c, dk]
                lower = np.tril(np.ones((c, c), dtype=bool))
                diff = np.where(lower[:, :, None], Gc[:, None, :] - Gc[None, :, :], -np.inf)
                R = np.exp(diff)                                              # [r, j, dk], j <= r
                A = np.tril(bt[:, None] * np.einsum("rc,jc,rjc->rj", K, K, R), -1)
                T = _forward_substitution_inverse(A) * bt[None, :]
                U = T @ (V - (K * np.exp(Gc)) @ S)
                Aqk = np.einsum("rc,jc,rjc->rj", Q, K, R)
                O[b, pos, h] = (Q * np.exp(Gc)) @ S + Aqk @ U
                S = np.exp(Gc[-1])[:, None] * S + (K * np.exp(Gc[-1][None, :] - Gc)).T @ U
            SF[b, h] = S
    return O, SF


def dplr(q, w_log, a, bvec, kk, vv, S0=None, scale=1.0):
    """The generic diagonal-plus-low-rank state transition of the "08 linear delta rule & DPLR"
    page, section 5, applied token by token: S_t = (Diag(w_t) + a_t b_t^T) S_{t-1} + kk_t vv_t^T,
    o_t = S_t^T (q_t scale), with the section's reductions (DeltaNet: w = 1, a = -beta k, b = k;
    Gated DeltaNet: w = g, b = g k; KDA: w = alpha) supplied by the caller.
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


def chunked_bwd(q, k, v, beta, g_log=None, S0=None, dO=None, dS_final=None, n_h=1, C=16, scale=1.0):
    """Gradients of `chunked` for <O, dO> + <S_final, dS_final>, chunk by chunk, in fp64: the
    chunkwise backward the GPU kernels are to compute.  Per chunk, with the forward's
    Y = V - gam K S, V~ = T Y, T = N diag(beta), N = (I + A)^-1, O = (gam Q) S + (Q K^T * Gam) V~
    and S' = gam_C S + K^T (w V~), w = gam_C / gam, given G' = dS' and dO (Q and dO rows only
    at each token's last sub-step):
        dV~ = w K G' + (Q K^T * Gam)^T dO,   dY = T^T dV~,   dT = dV~ Y^T,   dN = dT diag(beta)
        dA  = -strictLower(N^T dN N^T),      dG = diag(beta) (Gam * dA)   (A = diag(beta)(Gam * K K^T))
        dS  = gam_C G' - K^T (gam dY) + (gam Q)^T dO                    (carried to the previous chunk)
        dQ  = gam (dO S^T) + (Gam * dO V~^T) K
        dK  = -gam (dY S^T) + w (V~ G'^T) + (Gam * dO V~^T)^T Q + (dG + dG^T) K
        dbeta = diag(N^T dT) + rowsum(dA * Gam * K K^T),   dV = dY
    and the log-gate prefix gc (gam = exp(gc)) collects every gamma-dependent factor; the log
    gates are its reverse cumulative sum within the chunk (at each token's first sub-step)."""
    q, k, v, beta, g_log, S0, dO, dS_final = map(_f64, (q, k, v, beta, g_log, S0, dO, dS_final))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    Lx = L * n_h
    NT = -(-Lx // C)
    out = {"dq": np.zeros((B, L, H, dk)), "dk": np.zeros((B, Lx, H, dk)), "dv": np.zeros((B, Lx, H, dv)),
           "dbeta": np.zeros((B, Lx, H)), "dg_log": np.zeros((B, L, H)), "dS0": np.zeros((B, H, dk, dv))}
    for b in range(B):
        for h in range(H):
            # forward, keeping each chunk's start state and pieces
            S = np.zeros((dk, dv)) if S0 is None else S0[b, h].copy()
            saved = []
            for n in range(NT):
                pos = np.arange(n * C, min((n + 1) * C, Lx))
                c = len(pos)
                K, V, bt = k[b, pos, h], v[b, pos, h], beta[b, pos, h]
                lg = np.zeros(c)
                first = (pos % n_h) == 0
                if g_log is not None:
                    lg[first] = g_log[b, pos[first] // n_h, h]
                gc = np.cumsum(lg)
                gam = np.exp(gc)
                lower = np.tril(np.ones((c, c), dtype=bool))
                Gam = np.exp(np.where(lower, gc[:, None] - gc[None, :], -np.inf))
                Gm = K @ K.T
                A = np.tril(bt[:, None] * Gam * Gm, -1)
                N = _forward_substitution_inverse(A)
                T = N * bt[None, :]
                Y = V - gam[:, None] * (K @ S)
                Vt = T @ Y
                last = (pos % n_h) == n_h - 1
                Qf = np.zeros((c, dk))
                Qf[last] = q[b, pos[last] // n_h, h] * scale
                w = np.exp(gc[-1] - gc)
                saved.append((pos, K, V, bt, lg, gc, gam, Gam, Gm, N, T, Y, Vt, Qf, last, first, w, S.copy()))
                S = gam[-1] * S + (w[:, None] * K).T @ Vt
            # backward over chunks, last first
            G = np.zeros((dk, dv)) if dS_final is None else dS_final[b, h].copy()
            for n in range(NT - 1, -1, -1):
                pos, K, V, bt, lg, gc, gam, Gam, Gm, N, T, Y, Vt, Qf, last, first, w, Sn = saved[n]
                c = len(pos)
                dOc = np.zeros((c, dv))
                if dO is not None:
                    dOc[last] = dO[b, pos[last] // n_h, h]
                QK = (Qf @ K.T) * Gam
                dVt = w[:, None] * (K @ G) + QK.T @ dOc
                dY = T.T @ dVt
                dT = dVt @ Y.T
                dN = dT * bt[None, :]
                dA = -np.tril(N.T @ dN @ N.T, -1)
                dGm = bt[:, None] * Gam * dA
                dOV = dOc @ Vt.T                                   # (dO V~^T)
                dQf = gam[:, None] * (dOc @ Sn.T) + (Gam * dOV) @ K
                dK = (-gam[:, None] * (dY @ Sn.T) + w[:, None] * (Vt @ G.T) + (Gam * dOV).T @ Qf
                      + (dGm + dGm.T) @ K)
                dbeta = np.diag(N.T @ dT) + np.sum(dA * Gam * Gm, axis=1)
                # the log-gate prefix: every factor that depends on gc
                dgc = np.zeros(c)
                dgc += gam * np.sum(-(K @ Sn) * dY, axis=1)           # Y = V - gam K S
                dgc += gam * np.sum((Qf @ Sn) * dOc, axis=1)          # O's gam Q S
                dGam = np.where(np.tril(np.ones((c, c), dtype=bool), -1), bt[:, None] * Gm * dA, 0.0)
                dGam += (Qf @ K.T) * dOV * np.tril(np.ones((c, c)))  # O's (Q K^T * Gam) V~
                t = Gam * dGam
                dgc += t.sum(axis=1) - t.sum(axis=0)
                dw = np.sum((K @ G) * Vt, axis=1)                     # S' = gam_C S + K^T (w V~)
                dgc[-1] += gam[-1] * np.sum(G * Sn) + np.sum(w * dw)
                dgc -= w * dw
                dlg = np.cumsum(dgc[::-1])[::-1]
                # carry the state gradient to the previous chunk
                G = gam[-1] * G - K.T @ (gam[:, None] * dY) + (gam[:, None] * Qf).T @ dOc
                out["dk"][b, pos, h] = dK
                out["dv"][b, pos, h] = dY
                out["dbeta"][b, pos, h] = dbeta
                out["dq"][b, pos[last] // n_h, h] = dQf[last] * scale
                if g_log is not None:
                    out["dg_log"][b, pos[first] // n_h, h] = dlg[first]
            out["dS0"][b, h] = G
    if g_log is None:
        out["dg_log"] = None
    return out
