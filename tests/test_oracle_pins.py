"""Pins of the fp64 oracle (oracle.fwd, oracle.ut_factors) to what the pages and
the mathematics fix.  CPU only.

Every check compares the oracle with something other than itself: a closed form,
a worked example the pages print (tests/golden/), brute-force materialised
products, or an independent formulation from tests/formulations.py.
"""
import os

import numpy as np
import pytest

import oracle
import formulations as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
f32 = np.float32


def rnd(seed):
    return np.random.default_rng(seed)


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_inputs(seed, B=1, L=8, H=1, dk=6, dv=5, n_h=1, gate=True, s0=True, beta_hi=1.0):
    r = rnd(seed)
    q = unit(r.standard_normal((B, L, H, dk))).astype(f32)
    k = unit(r.standard_normal((B, L * n_h, H, dk))).astype(f32)
    v = r.standard_normal((B, L * n_h, H, dv)).astype(f32)
    beta = (beta_hi * r.uniform(0.05, 1.0, (B, L * n_h, H))).astype(f32)
    g = (-np.logaddexp(0, r.standard_normal((B, L, H)) - 1.0)).astype(f32) if gate else None
    S0 = (0.5 * r.standard_normal((B, H, dk, dv))).astype(f32) if s0 else None
    return q, k, v, beta, g, S0


def single_token_transition(k_steps, beta_steps, g_log=None):
    """The oracle's transition for one token: start from S0 = I, v = 0 => S_final = A."""
    n_h, dk = k_steps.shape
    q = np.zeros((1, 1, 1, dk), f32)
    k = k_steps.reshape(1, n_h, 1, dk).astype(f32)
    v = np.zeros((1, n_h, 1, dk), f32)
    beta = np.asarray(beta_steps, f32).reshape(1, n_h, 1)
    g = None if g_log is None else np.full((1, 1, 1), g_log, f32)
    S0 = np.eye(dk, dtype=f32)[None, None]
    _, S = oracle.fwd(q, k, v, beta, g, S0, n_h=n_h)
    return S[0, 0]


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("beta", [0.0, 0.3, 1.0, 1.7, 2.0])
def test_householder_eigenvalues(beta):
    """Delta-rule/DPLR page, section 1.2: eig(I - beta k k^T) = {1 - beta (once), 1 (d_k - 1 times)}."""
    dk = 8
    kk = unit(rnd(1).standard_normal(dk)).astype(f32)
    A = single_token_transition(kk[None], [beta])
    ev = np.sort(np.linalg.eigvalsh((A + A.T) / 2))
    assert np.allclose(A, A.T, atol=1e-12)
    expect = np.sort(np.r_[1.0 - np.float64(f32(beta)) * np.dot(kk.astype(np.float64), kk), np.ones(dk - 1)])
    assert np.allclose(ev, expect, atol=1e-12)
    # and explicitly: A k = (1 - beta) k, A u = u for u orthogonal to k
    k64 = kk.astype(np.float64)
    assert np.allclose(A @ k64, (1 - np.float64(f32(beta)) * (k64 @ k64)) * k64, atol=1e-12)


@pytest.mark.parametrize("gated", [False, True])
def test_exact_write_beta_one(gated):
    """DeltaProduct notes, section 2.1: unit key, beta = 1 => S_t^T k_t = v_t exactly;
    reading with q = k_t returns v_t."""
    r = rnd(2)
    dk, dv = 16, 7
    kk = unit(r.standard_normal(dk))
    kk = (kk / np.linalg.norm(kk)).astype(f32)
    q = kk.reshape(1, 1, 1, dk)
    k = kk.reshape(1, 1, 1, dk)
    v = r.standard_normal((1, 1, 1, dv)).astype(f32)
    S0 = r.standard_normal((1, 1, dk, dv)).astype(f32)
    g = np.full((1, 1, 1), -0.7, f32) if gated else None
    O, S = oracle.fwd(q, k, v, np.ones((1, 1, 1), f32), g, S0)
    kn2 = float(np.dot(kk.astype(np.float64), kk))
    # with ||k||^2 = kn2 (1 up to fp32 rounding): S^T k = v + (1 - kn2) * (stuff); exact when kn2 == 1
    g0 = np.exp(-0.7) if gated else 1.0
    pred = kn2 * v[0, 0, 0] + (1 - kn2) * g0 * (S0[0, 0].astype(np.float64).T @ kk)
    assert np.allclose(S[0, 0].T @ kk.astype(np.float64), pred, atol=1e-12)
    assert abs(kn2 - 1) < 1e-6
    assert np.allclose(O[0, 0, 0], pred, atol=1e-12)


def test_mod3_rotation_golden():
    """DeltaProduct notes, section 2.4: k1 = (1,0), k2 = (1/2, sqrt3/2), beta = 2 gives a
    120-degree rotation; the state returns to e1 every three tokens (tests/golden)."""
    rows = {}
    for line in open(os.path.join(GOLDEN, "mod3_rotation.txt")):
        if line.strip() and not line.startswith("#"):
            p = line.split()
            rows[p[0]] = np.array([float(x) for x in p[1:]])
    k1 = np.array([1.0, 0.0])
    k2 = np.array([0.5, np.sqrt(3) / 2])
    A = single_token_transition(np.stack([k1, k2]), [2.0, 2.0])
    assert np.allclose(A.reshape(-1), rows["F2F1"], atol=1e-7)
    L = 6
    k = np.tile(np.stack([k1, k2]), (L, 1)).reshape(1, 2 * L, 1, 2).astype(f32)
    v = np.zeros((1, 2 * L, 1, 1), f32)
    beta = np.full((1, 2 * L, 1), 2.0, f32)
    S0 = np.array([1.0, 0.0], f32).reshape(1, 1, 2, 1)
    for qi, col in ((np.array([1.0, 0.0]), 0), (np.array([0.0, 1.0]), 1)):
        q = np.tile(qi, (L, 1)).reshape(1, L, 1, 2).astype(f32)
        O, S = oracle.fwd(q, k, v, beta, None, S0, n_h=2)
        got = O[0, :, 0, 0]
        want = np.array([rows["S%d" % (i + 1)][col] for i in range(L)])
        assert np.allclose(got, want, atol=1e-6), (got, want)
    assert np.allclose(S[0, 0, :, 0], [1.0, 0.0], atol=1e-6)


@pytest.mark.parametrize("betas", [(0.3, 1.5, 0.7), (2.0, 0.4), (1.0, 1.0, 1.0, 0.2)])
def test_identical_keys_collapse(betas):
    """DeltaProduct notes, section 2.4: identical keys => one factor with
    beta_eff = 1 - prod_j (1 - beta_j)."""
    dk = 6
    kk = unit(rnd(3).standard_normal(dk)).astype(f32).astype(np.float64)
    kk = kk / np.linalg.norm(kk)
    A = single_token_transition(np.tile(kk, (len(betas), 1)), betas)
    b = np.array(betas, f32).astype(np.float64)
    k32 = kk.astype(f32).astype(np.float64)
    # exact for the fp32-rounded key: each factor is I - b_j k k^T with ||k||^2 = n2
    n2 = k32 @ k32
    # product of (I - b_j P') with P' = k k^T, (k k^T)^2 = n2 k k^T  =>  I - c k k^T,
    # c = (1 - prod(1 - b_j n2)) / n2
    c = (1 - np.prod(1 - b * n2)) / n2
    assert np.allclose(A, np.eye(dk) - c * np.outer(k32, k32), atol=1e-12)
    assert abs(n2 - 1) < 1e-6
    beta_eff = 1 - np.prod(1 - b)
    assert np.allclose(A, np.eye(dk) - beta_eff * np.outer(k32, k32), atol=1e-5)


def test_orthogonal_keys_commute():
    """DeltaProduct notes, section 2.4: pairwise orthogonal keys => A = I - sum_j beta_j k_j k_j^T."""
    dk = 7
    Qm, _ = np.linalg.qr(rnd(4).standard_normal((dk, dk)))
    ks = Qm[:, :3].T
    betas = [0.4, 1.9, 1.1]
    A = single_token_transition(ks, betas)
    k32 = ks.astype(f32).astype(np.float64)
    b = np.array(betas, f32).astype(np.float64)
    want = np.eye(dk) - sum(b[j] * np.outer(k32[j], k32[j]) for j in range(3))
    assert np.allclose(A, want, atol=1e-6)
    # reversed order gives the same matrix
    A2 = single_token_transition(ks[::-1], betas[::-1])
    assert np.allclose(A, A2, atol=1e-6)


def test_same_key_twice_beta2_is_identity():
    """DeltaProduct notes, section 2.5: the same key twice at beta = 2 gives I (a plain sum of the
    two rank-1 terms would give eigenvalue -3)."""
    kk = np.zeros(5)
    kk[2] = 1.0
    A = single_token_transition(np.stack([kk, kk]), [2.0, 2.0])
    assert np.allclose(A, np.eye(5), atol=0)
    kk = unit(rnd(5).standard_normal(5))
    A = single_token_transition(np.stack([kk, kk]), [2.0, 2.0])
    assert np.allclose(A, np.eye(5), atol=1e-6)


def test_nh2_cross_term():
    """DeltaProduct notes, section 2.3: A = I - b1 k1k1^T - b2 k2k2^T + b1 b2 (k2.k1) k2 k1^T."""
    r = rnd(6)
    dk = 9
    k1, k2 = unit(r.standard_normal((2, dk))).astype(f32).astype(np.float64)
    b1, b2 = np.float64(f32(0.8)), np.float64(f32(1.6))
    A = single_token_transition(np.stack([k1, k2]), [b1, b2])
    want = (np.eye(dk) - b1 * np.outer(k1, k1) - b2 * np.outer(k2, k2)
            + b1 * b2 * (k2 @ k1) * np.outer(k2, k1))
    assert np.allclose(A, want, atol=1e-12)
    assert not np.allclose(A, A.T, atol=1e-3)   # order matters: not symmetric


@pytest.mark.parametrize("n_h", [1, 2, 3, 5])
def test_rank_bounds(n_h):
    """DeltaProduct notes, sections 2.3 and 2.6: rank(A - I) <= n_h, rank(A - g I) <= n_h."""
    r = rnd(10 + n_h)
    dk = 12
    ks = unit(r.standard_normal((n_h, dk)))
    bs = r.uniform(0.1, 2.0, n_h)
    A = single_token_transition(ks, bs)
    assert np.linalg.matrix_rank(A - np.eye(dk), tol=1e-9) == n_h
    g = -0.4
    Ag = single_token_transition(ks, bs, g_log=g)
    assert np.linalg.matrix_rank(Ag - np.exp(np.float64(f32(g))) * np.eye(dk), tol=1e-9) == n_h
    assert np.linalg.matrix_rank(A, tol=1e-9) == dk or np.any(np.isclose(bs, 1.0))


def test_spectral_norm_bound():
    """DeltaProduct notes, section 2.5: unit keys, beta in [0, 2] => ||A||_2 <= 1, also for
    products over tokens; beta > 2 can exceed it."""
    r = rnd(20)
    dk = 8
    for trial in range(50):
        n_h = 1 + trial % 4
        ks = unit(r.standard_normal((n_h, dk)))
        ks = ks.astype(f32).astype(np.float64)
        ks = ks / np.linalg.norm(ks, axis=1, keepdims=True)
        bs = r.uniform(0, 2, n_h)
        A = single_token_transition(ks, bs)
        assert np.linalg.norm(A, 2) <= 1 + 1e-6
    # product over 40 tokens via the state from S0 = I
    L, n_h = 40, 2
    k = unit(r.standard_normal((1, L * n_h, 1, dk))).astype(f32)
    beta = r.uniform(0, 2, (1, L * n_h, 1)).astype(f32)
    _, S = oracle.fwd(np.zeros((1, L, 1, dk), f32), k, np.zeros((1, L * n_h, 1, dk), f32), beta,
                      None, np.eye(dk, dtype=f32)[None, None], n_h=n_h)
    assert np.linalg.norm(S[0, 0], 2) <= 1 + 1e-5
    kk = unit(r.standard_normal(dk))
    assert np.linalg.norm(single_token_transition(kk[None], [2.5]), 2) > 1.4


def test_complex_eigenvalue_condition():
    """DeltaProduct notes, section 2.4: in the plane of k1, k2 (c = k1.k2),
    tau = 2 - b1 - b2 + b1 b2 c^2, delta = (1 - b1)(1 - b2); complex pair iff tau^2 - 4 delta < 0."""
    r = rnd(21)
    seen = {True: 0, False: 0}
    for _ in range(200):
        k1, k2 = unit(r.standard_normal((2, 2)))
        b1, b2 = r.uniform(0, 2, 2)
        A = single_token_transition(np.stack([k1, k2]), [b1, b2])
        k1r, k2r = (x.astype(f32).astype(np.float64) for x in (k1, k2))
        b1r, b2r = np.float64(f32(b1)), np.float64(f32(b2))
        c = (k1r @ k2r) / np.linalg.norm(k1r) / np.linalg.norm(k2r)
        tau = 2 - b1r - b2r + b1r * b2r * c * c
        delta = (1 - b1r) * (1 - b2r)
        disc = tau * tau - 4 * delta
        if abs(disc) < 1e-6:
            continue
        ev = np.linalg.eigvals(A)
        assert np.isclose(np.trace(A), tau, atol=1e-6) and np.isclose(np.linalg.det(A), delta, atol=1e-6)
        is_complex = np.max(np.abs(ev.imag)) > 1e-9
        assert is_complex == (disc < 0)
        seen[is_complex] += 1
    assert seen[True] > 5 and seen[False] > 5


def test_swap_permutations():
    """DeltaProduct notes, section 3.1: k = (e_a - e_b)/sqrt2 with beta = 2 swaps coordinates a, b;
    n - 1 swaps per token realise any permutation of S_n.  S0 = (1..n)^T tracks the composition."""
    n = 5
    r = rnd(22)
    L = 12
    ks, perms = [], []
    cur = np.arange(1, n + 1, dtype=np.float64)
    tracked = []
    for i in range(L):
        pairs = [tuple(r.choice(n, 2, replace=False)) for _ in range(n - 1)]
        for a, b in pairs:
            kk = np.zeros(n)
            kk[a], kk[b] = 1 / np.sqrt(2), -1 / np.sqrt(2)
            ks.append(kk)
            cur[[a, b]] = cur[[b, a]]
        tracked.append(cur.copy())
    n_h = n - 1
    k = np.array(ks).reshape(1, L * n_h, 1, n).astype(f32)
    v = np.zeros((1, L * n_h, 1, 1), f32)
    beta = np.full((1, L * n_h, 1), 2.0, f32)
    S0 = np.arange(1, n + 1, dtype=f32).reshape(1, 1, n, 1)
    outs = []
    for j in range(n):
        q = np.zeros((1, L, 1, n), f32)
        q[..., j] = 1
        O, S = oracle.fwd(q, k, v, beta, None, S0, n_h=n_h)
        outs.append(O[0, :, 0, 0])
    got = np.stack(outs, 1)
    assert np.allclose(got, np.array(tracked), atol=1e-5)
    assert np.allclose(np.round(got), got, atol=1e-5)


def test_erase_write_and_gd_forms():
    """Delta-rule/DPLR page, sections 1.1-1.3: erase-write form = Householder form = one GD step."""
    r = rnd(23)
    dk, dv = 10, 6
    for beta in (0.0, 0.35, 1.0, 1.8):
        kk = unit(r.standard_normal(dk)).astype(f32)
        vv = r.standard_normal(dv).astype(f32)
        S0 = r.standard_normal((dk, dv)).astype(f32)
        _, S = oracle.fwd(np.zeros((1, 1, 1, dk), f32), kk.reshape(1, 1, 1, dk),
                          vv.reshape(1, 1, 1, dv), np.full((1, 1, 1), beta, f32), None,
                          S0[None, None])
        Sd, kd, vd = S0.astype(np.float64), kk.astype(np.float64), vv.astype(np.float64)
        b = np.float64(f32(beta))
        assert np.allclose(S[0, 0], F.erase_write_step(Sd, kd, vd, b), atol=1e-12)
        assert np.allclose(S[0, 0], F.gd_step(Sd, kd, vd, b), atol=1e-12)


# ---------------------------------------------------------------- brute force & cross-forms

@pytest.mark.parametrize("n_h,gate,s0", [(1, False, False), (1, True, True), (2, True, True),
                                         (3, False, True), (2, True, False)])
def test_brute_force_products(n_h, gate, s0):
    """DeltaProduct notes, sections 2.3 / 2.6: materialise A_i = g_i F_{n_h}...F_1 and
    B_i = sum_j F_{n_h}...F_{j+1} C_{i,j} (d_k x d_k) and step S_i = A_i S_{i-1} + B_i."""
    q, k, v, beta, g, S0 = rand_inputs(30 + n_h, B=2, L=9, H=2, dk=5, dv=4, n_h=n_h,
                                       gate=gate, s0=s0, beta_hi=2.0)
    O, S = oracle.fwd(q, k, v, beta, g, S0, n_h=n_h, scale=0.7)
    Ob, Sb = F.brute_force(q, k, v, beta, g, S0, n_h=n_h, scale=0.7)
    assert np.max(np.abs(O - Ob)) < 1e-12 and np.max(np.abs(S - Sb)) < 1e-12


@pytest.mark.parametrize("C", [4, 8, 16])
@pytest.mark.parametrize("n_h,gate", [(1, False), (1, True), (2, True), (4, True)])
def test_chunked_form_matches(C, n_h, gate):
    """Delta-rule/DPLR page, section 2.3 (and section 3 for the gated form): the chunkwise UT/WY
    algorithm reaches the recurrent result; the page reports 1.4e-14 (DeltaNet) and 1.7e-15 (GDN)
    relative error in fp64 at C = 16.  Ragged lengths exercise a partial last chunk."""
    if C % n_h:
        pytest.skip("chunk must hold whole tokens")
    L = 37 if n_h == 1 else 19
    q, k, v, beta, g, S0 = rand_inputs(40 + C + n_h, B=1, L=L, H=2, dk=8, dv=6, n_h=n_h,
                                       gate=gate, s0=True)
    O, S = oracle.fwd(q, k, v, beta, g, S0, n_h=n_h)
    Oc, Sc = F.chunked(q, k, v, beta, g, S0, n_h=n_h, C=C)
    rel = max(np.abs(O - Oc).max() / np.abs(O).max(), np.abs(S - Sc).max() / np.abs(S).max())
    assert rel < 1e-12, rel


def test_dplr_reductions():
    """Delta-rule/DPLR page, section 5: DeltaNet = DPLR(w = 1, a = -beta k, b = k, beta k v^T) and
    GDN = DPLR(w = alpha, a = -beta k, b = alpha k, beta k v^T); the page reports <= 5.2e-16."""
    q, k, v, beta, g, S0 = rand_inputs(50, B=2, L=11, H=2, dk=6, dv=5, gate=True, s0=True)
    dk = k.shape[-1]
    bv = beta[..., None].astype(np.float64)
    k64 = k.astype(np.float64)
    zeros = np.zeros(k.shape)
    # DeltaNet
    O, S = oracle.fwd(q, k, v, beta, None, S0)
    Od, Sd = F.dplr(q, zeros, -bv * k64, k64, bv * k64, v, S0)
    assert np.abs(O - Od).max() < 1e-12 and np.abs(S - Sd).max() < 1e-12
    # Gated DeltaNet
    gl = np.repeat(g.astype(np.float64)[..., None], dk, axis=-1)
    O, S = oracle.fwd(q, k, v, beta, g, S0)
    Od, Sd = F.dplr(q, gl, -bv * k64, k64 * np.exp(gl), bv * k64, v, S0)
    assert np.abs(O - Od).max() < 1e-12 and np.abs(S - Sd).max() < 1e-12


def test_one_chunk_closed_form():
    """Delta-rule/DPLR page, section 2.4: from S = 0, ungated, O = (Q K^T * M) T V."""
    q, k, v, beta, _, _ = rand_inputs(51, B=1, L=24, H=1, dk=7, dv=5, gate=False, s0=False)
    O, _ = oracle.fwd(q, k, v, beta)
    Oc = F.one_chunk_closed_form(q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0])
    assert np.abs(O[0, :, 0] - Oc).max() < 1e-12


# ---------------------------------------------------------------- special cases & invariants

def test_special_cases():
    """n_h = 1 DeltaProduct is DeltaNet; log g = 0 is ungated; beta = 0 leaves S = g-decayed S0;
    the output is linear in scale."""
    q, k, v, beta, g, S0 = rand_inputs(60, B=1, L=10, H=3, dk=6, dv=4, gate=True, s0=True)
    O1, S1 = oracle.fwd(q, k, v, beta, None, S0)
    O0, S0g = oracle.fwd(q, k, v, beta, np.zeros_like(g), S0)
    assert np.array_equal(O1, O0) and np.array_equal(S1, S0g)
    Ob, Sb = oracle.fwd(q, k, v, np.zeros_like(beta), g, S0)
    decay = np.exp(g.astype(np.float64).sum(axis=1))       # [B, H]
    assert np.allclose(Sb, decay[:, :, None, None] * S0.astype(np.float64), atol=1e-14)
    Os, _ = oracle.fwd(q, k, v, beta, g, S0, scale=0.125)
    Og, _ = oracle.fwd(q, k, v, beta, g, S0)
    assert np.allclose(Os, 0.125 * Og, atol=1e-15)


def test_expanded_sequence_equivalence():
    """DeltaProduct notes, section 4.1: DeltaProduct = DeltaNet on the expanded sequence with the
    gate (g_1, 1, ..., 1, g_2, ...) and only the last sub-step's output kept."""
    n_h = 3
    q, k, v, beta, g, S0 = rand_inputs(61, B=2, L=7, H=2, dk=6, dv=4, n_h=n_h, gate=True, s0=True)
    O, S = oracle.fwd(q, k, v, beta, g, S0, n_h=n_h)
    B, L, H, dk = q.shape
    qx = np.zeros((B, L * n_h, H, dk), f32)
    qx[:, n_h - 1::n_h] = q
    gx = np.zeros((B, L * n_h, H), f32)
    gx[:, ::n_h] = g
    Ox, Sx = oracle.fwd(qx, k, v, beta, gx, S0, n_h=1)
    assert np.abs(Ox[:, n_h - 1::n_h] - O).max() < 1e-13 and np.abs(Sx - S).max() < 1e-13


def test_hard_reset():
    """DeltaProduct notes, section 3.3: g = 0 (log g = -inf) resets the state; afterwards only
    the current token's writes remain."""
    q, k, v, beta, g, S0 = rand_inputs(62, B=1, L=6, H=1, dk=5, dv=3, gate=True, s0=True)
    g = g.copy()
    g[0, 3, 0] = -np.inf
    O, S = oracle.fwd(q, k, v, beta, g, S0)
    Ot, St = oracle.fwd(q[:, 3:], k[:, 3:], v[:, 3:], beta[:, 3:], np.where(np.isinf(g), 0, g)[:, 3:], None)
    assert np.abs(O[:, 3:] - Ot).max() < 1e-14 and np.abs(S - St).max() < 1e-14
    Ob, Sb = F.brute_force(q, k, v, beta, g, S0)
    assert np.abs(O - Ob).max() < 1e-12


def test_segment_split():
    """The state is the resume point: S_final of the first segment as S0 of the second
    reproduces the single call."""
    n_h = 2
    q, k, v, beta, g, S0 = rand_inputs(63, B=2, L=14, H=2, dk=6, dv=5, n_h=n_h, gate=True, s0=True)
    O, S = oracle.fwd(q, k, v, beta, g, S0, n_h=n_h)
    c = 5
    Oa, Sa = oracle.fwd(q[:, :c], k[:, :c * n_h], v[:, :c * n_h], beta[:, :c * n_h], g[:, :c], S0, n_h=n_h)
    Ob, Sb = oracle.fwd(q[:, c:], k[:, c * n_h:], v[:, c * n_h:], beta[:, c * n_h:], g[:, c:],
                        Sa.astype(f32), n_h=n_h)
    # Sa is rounded to fp32 to pass it back in: compare at fp32 resolution
    assert np.abs(np.concatenate([Oa, Ob], 1) - O).max() < 1e-5 and np.abs(Sb - S).max() < 1e-5


# ---------------------------------------------------------------- UT/WY factors (oracle.ut_factors)

@pytest.mark.parametrize("n_h,gate,C", [(1, False, 16), (1, True, 16), (2, True, 8), (1, True, 32)])
def test_ut_factors_match_wy_recursion(n_h, gate, C):
    """Delta-rule/DPLR page, section 2.1 (sequential WY vectors) vs section 2.2 (UT transform):
    rows of T K and T V equal the recursively built w and u (gated weights from section 3)."""
    L = 21 if n_h == 1 else 11
    q, k, v, beta, g, _ = rand_inputs(70 + C, B=1, L=L, H=2, dk=6, dv=5, n_h=n_h, gate=gate,
                                      s0=False, beta_hi=2.0)
    f = oracle.ut_factors(k, v, beta, g, n_h=n_h, chunk=C)
    Lx = L * n_h
    NT = f["T"].shape[2]
    assert NT == -(-Lx // C)
    for h in range(2):
        for n in range(NT):
            pos = np.arange(n * C, min((n + 1) * C, Lx))
            gc = f["gc"][0, h, n, :len(pos)]
            Wr, Ur = F.wy_recursive(k[0, pos, h], v[0, pos, h], beta[0, pos, h], gc)
            assert np.abs(f["W"][0, h, n, :len(pos)] - Wr).max() < 1e-12
            assert np.abs(f["U"][0, h, n, :len(pos)] - Ur).max() < 1e-12
            # padded rows are zero, T is lower triangular with diag(beta) on the diagonal
            assert np.all(f["T"][0, h, n, len(pos):] == 0)
            T = f["T"][0, h, n]
            assert np.all(np.triu(T, 1) == 0)
            assert np.allclose(np.diag(T)[:len(pos)], beta[0, pos, h], atol=0)


def test_ut_factors_orthogonal_keys():
    """With mutually orthogonal keys the strictly-lower Gram part vanishes: T = diag(beta),
    W = gamma * beta * K, U = beta * V."""
    C, dk = 8, 8
    Qm, _ = np.linalg.qr(rnd(80).standard_normal((dk, dk)))
    k = Qm.T.reshape(1, C, 1, dk)
    v = rnd(81).standard_normal((1, C, 1, 3))
    beta = rnd(82).uniform(0.1, 1.9, (1, C, 1))
    g = -rnd(83).uniform(0, 1, (1, C, 1))
    f = oracle.ut_factors(k, v, beta, g, chunk=C)
    assert np.allclose(f["T"][0, 0, 0], np.diag(beta[0, :, 0]), atol=1e-12)
    gam = np.exp(np.cumsum(g[0, :, 0]))
    assert np.allclose(f["W"][0, 0, 0], (gam * beta[0, :, 0])[:, None] * k[0, :, 0], atol=1e-12)
    assert np.allclose(f["U"][0, 0, 0], beta[0, :, 0][:, None] * v[0, :, 0], atol=1e-12)


def test_ut_factors_drive_chunk_recurrence():
    """Using oracle.ut_factors' W, U in the chunk recurrence of the delta-rule/DPLR page
    (section 2.3 / section 3: V~ = U - W S, O = (gamma Q) S + (Q K^T * Gamma * M) V~,
    S <- gamma_C S + ((gamma_C / gamma) K)^T V~) reproduces the token-by-token oracle."""
    C = 8
    q, k, v, beta, g, S0 = rand_inputs(84, B=1, L=29, H=1, dk=6, dv=4, gate=True, s0=True)
    f = oracle.ut_factors(k, v, beta, g, chunk=C)
    O, S = oracle.fwd(q, k, v, beta, g, S0)
    Sc = S0[0, 0].astype(np.float64)
    L = q.shape[1]
    Oc = np.zeros((L, 4))
    for n in range(f["T"].shape[2]):
        pos = np.arange(n * C, min((n + 1) * C, L))
        c = len(pos)
        gc = f["gc"][0, 0, n, :c]
        W, U = f["W"][0, 0, n, :c], f["U"][0, 0, n, :c]
        Q, K = q[0, pos, 0].astype(np.float64), k[0, pos, 0].astype(np.float64)
        Vt = U - W @ Sc
        mask = np.tril(np.ones((c, c), bool))
        Gam = np.exp(np.where(mask, gc[:, None] - gc[None, :], -np.inf))
        Oc[pos] = (np.exp(gc)[:, None] * Q) @ Sc + ((Q @ K.T) * Gam) @ Vt
        Sc = np.exp(gc[-1]) * Sc + (np.exp(gc[-1] - gc)[:, None] * K).T @ Vt
    assert np.abs(Oc - O[0, :, 0]).max() < 1e-12 and np.abs(Sc - S[0, 0]).max() < 1e-12


# ---------------------------------------------------------------- backward (oracle.bwd)

def _loss(inp, dO, dS, n_h, scale):
    """<O, dO> + <S_final, dS> of the forward oracle, in fp64."""
    q, k, v, beta, g, S0 = inp
    O, S = oracle.fwd(q, k, v, beta, g, S0, n_h=n_h, scale=scale)
    return float(np.sum(O * dO) + np.sum(S * dS))


@pytest.mark.parametrize("n_h,gate,s0", [(1, False, False), (1, True, True), (2, True, True), (3, False, True)])
def test_bwd_matches_finite_differences(n_h, gate, s0):
    """Every gradient of oracle.bwd against central differences of oracle.fwd (an independent
    function, itself pinned above).  Perturbations are float32-exact (h = 2^-11 on inputs of
    magnitude < 8), so oracle.fwd sees exactly x +- h; the O(h^2) truncation error is ~1e-7."""
    inp = list(rand_inputs(40 + 7 * n_h + gate, B=1, L=4, H=1, dk=3, dv=2, n_h=n_h, gate=gate, s0=s0,
                           beta_hi=1.9))
    r = rnd(5)
    dO = r.standard_normal((1, 4, 1, 2)).astype(f32)
    dS = r.standard_normal((1, 1, 3, 2)).astype(f32)
    scale = 0.75
    got = oracle.bwd(*inp, dO, dS, n_h=n_h, scale=scale)
    h = 2.0 ** -11
    names = [("dq", 0), ("dk", 1), ("dv", 2), ("dbeta", 3), ("dg_log", 4), ("dS0", 5)]
    for name, idx in names:
        x = inp[idx]
        if x is None:
            assert name in ("dg_log", "dS0") and (name != "dg_log" or got["dg_log"] is None)
            continue
        num = np.zeros(x.shape)
        for pos in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += f32(h)
            xm[pos] -= f32(h)
            assert float(xp[pos]) - float(x[pos]) == h  # exact perturbation
            ip, im = list(inp), list(inp)
            ip[idx], im[idx] = xp, xm
            num[pos] = (_loss(ip, dO, dS, n_h, scale) - _loss(im, dO, dS, n_h, scale)) / (2 * h)
        err = np.max(np.abs(num - got[name])) / max(1.0, np.max(np.abs(num)))
        assert err < 1e-6, (name, err)


def test_bwd_one_token_closed_form():
    """One token, n_h = 1, gate g, state S0: S = g S0 + beta k (v - g S0^T k)^T, o = scale S^T q.
    The gradients written out by hand for <o, do>:
      dq = scale S do;  dv = scale beta (k.q) do;  dbeta = scale (k.q) (e.do), e = v - g S0^T k;
      dk = scale beta [(e.do) q - (k.q) g S0 do];  dlog g = scale [<S0, q do^T> g - beta (k.q) g (S0^T k).do];
      dS0 = scale g [q do^T - beta k (k.q) do^T]."""
    r = rnd(77)
    dk, dv = 4, 3
    q = r.standard_normal((1, 1, 1, dk)).astype(f32)
    k = r.standard_normal((1, 1, 1, dk)).astype(f32)
    v = r.standard_normal((1, 1, 1, dv)).astype(f32)
    beta = np.array([[[0.6]]], f32)
    glog = np.array([[[-0.4]]], f32)
    S0 = r.standard_normal((1, 1, dk, dv)).astype(f32)
    do = r.standard_normal((1, 1, 1, dv)).astype(f32)
    scale = 1.3
    got = oracle.bwd(q, k, v, beta, glog, S0, do, None, n_h=1, scale=scale)
    Q, K, V, D = (x.astype(np.float64).ravel() for x in (q, k, v, do))
    Z = S0[0, 0].astype(np.float64)
    g, b = np.exp(np.float64(glog.ravel()[0])), np.float64(beta.ravel()[0])
    e = V - g * Z.T @ K
    S = g * Z + b * np.outer(K, e)
    kq = K @ Q
    want = {
        "dq": scale * S @ D,
        "dv": scale * b * kq * D,
        "dbeta": scale * kq * (e @ D),
        "dk": scale * b * ((e @ D) * Q - kq * g * (Z @ D)),
        "dg_log": scale * (g * (Q @ Z @ D) - b * kq * g * ((Z.T @ K) @ D)),
        "dS0": scale * g * (np.outer(Q, D) - b * kq * np.outer(K, D)),
    }
    for name, w in want.items():
        assert np.allclose(np.asarray(got[name]).ravel(), np.asarray(w).ravel(), rtol=1e-12, atol=1e-12), name


@pytest.mark.parametrize("n_h,C,gate,s0", [(1, 8, True, True), (1, 16, False, False), (2, 8, True, True),
                                            (3, 12, True, False)])
def test_chunked_backward_matches_oracle_bwd(n_h, C, gate, s0):
    """The chunkwise backward (formulations.chunked_bwd: per-chunk transposed products, the
    triangular-inverse gradient, the reverse state recurrence, the gate prefix) reproduces the
    token-level reverse-mode oracle (pinned by finite differences above) on several chunks with
    a ragged tail."""
    L = 23
    inp = rand_inputs(90 + n_h + C, B=2, L=L, H=2, dk=5, dv=4, n_h=n_h, gate=gate, s0=s0, beta_hi=1.6)
    r = rnd(91)
    dO = r.standard_normal((2, L, 2, 4)).astype(f32)
    dS = r.standard_normal((2, 2, 5, 4)).astype(f32)
    want = oracle.bwd(*inp, dO, dS, n_h=n_h, scale=0.8)
    got = F.chunked_bwd(*inp, dO=dO, dS_final=dS, n_h=n_h, C=C, scale=0.8)
    for name in ("dq", "dk", "dv", "dbeta", "dg_log", "dS0"):
        if want[name] is None:
            assert got[name] is None
            continue
        err = np.max(np.abs(got[name] - want[name])) / max(1.0, np.max(np.abs(want[name])))
        assert err < 1e-10, (name, err)


# ---------------------------------------------------------------- KDA (oracle.fwd_kda)

def _kda_inputs(seed, B=2, L=9, H=2, dk=6, dv=5, s0=True):
    r = rnd(seed)
    q = unit(r.standard_normal((B, L, H, dk))).astype(f32)
    k = unit(r.standard_normal((B, L, H, dk))).astype(f32)
    v = r.standard_normal((B, L, H, dv)).astype(f32)
    beta = r.uniform(0.05, 1.0, (B, L, H)).astype(f32)
    a = (-np.logaddexp(0, r.standard_normal((B, L, H, dk)) - 1.0)).astype(f32)
    S0 = (0.5 * r.standard_normal((B, H, dk, dv))).astype(f32) if s0 else None
    return q, k, v, beta, a, S0


def test_kda_dplr_reduction():
    """Delta-rule/DPLR page, section 5: KDA = DPLR(w = log alpha (vector), a = -beta k,
    b = alpha * k, beta k v^T) — the diagonal decay applied before the low-rank erase (the page
    reports <= 5.2e-16 for this reduction)."""
    q, k, v, beta, a, S0 = _kda_inputs(120)
    O, S = oracle.fwd_kda(q, k, v, beta, a, S0, scale=0.7)
    bv = beta[..., None].astype(np.float64)
    k64, a64 = k.astype(np.float64), a.astype(np.float64)
    Od, Sd = F.dplr(q, a64, -bv * k64, k64 * np.exp(a64), bv * k64, v, S0, scale=0.7)
    assert np.abs(O - Od).max() < 1e-12 and np.abs(S - Sd).max() < 1e-12


def test_kda_equal_channels_is_gated_deltanet():
    """With the same decay on every key channel KDA is Gated DeltaNet (same page, section 1.4
    table): fwd_kda with a_log = g for all channels equals fwd with the scalar log gate g."""
    q, k, v, beta, _, S0 = _kda_inputs(121)
    g = (-np.logaddexp(0, rnd(122).standard_normal(beta.shape) - 1.0)).astype(f32)
    a = np.repeat(g[..., None], q.shape[-1], axis=-1)
    O1, S1 = oracle.fwd_kda(q, k, v, beta, a, S0)
    O2, S2 = oracle.fwd(q, k, v, beta, g, S0)
    assert np.abs(O1 - O2).max() < 1e-13 and np.abs(S1 - S2).max() < 1e-13


def test_kda_zero_channel_decay_erases_row():
    """alpha_r = 0 (log alpha = -inf) erases key channel r of the state before the write: after
    one token S[r] = beta k_r e with e = v - (Diag(alpha) S0)^T k, and row r of S0 is gone."""
    q, k, v, beta, a, S0 = _kda_inputs(123, B=1, L=1, H=1)
    a = a.copy()
    a[0, 0, 0, 2] = -np.inf
    _, S = oracle.fwd_kda(q, k, v, beta, a, S0)
    al = np.exp(a[0, 0, 0].astype(np.float64))
    Sd = al[:, None] * S0[0, 0].astype(np.float64)
    assert np.all(Sd[2] == 0.0)
    e = v[0, 0, 0].astype(np.float64) - Sd.T @ k[0, 0, 0].astype(np.float64)
    want = Sd + float(beta[0, 0, 0]) * np.outer(k[0, 0, 0].astype(np.float64), e)
    assert np.allclose(S[0, 0], want, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("C,L,s0,reset", [(4, 9, True, False), (16, 37, True, False), (8, 30, False, True),
                                          (32, 70, True, True), (1, 5, True, False)])
def test_kda_chunked_form_matches_oracle(C, L, s0, reset):
    """The chunkwise KDA form (tests/formulations.py, derived from the page's recurrence) and the
    oracle's token loop agree to fp64 rounding, for chunks of 1..32 positions, ragged tails,
    strong per-channel decays and channel resets (log alpha = -inf)."""
    q, k, v, beta, a, S0 = _kda_inputs(130 + C, L=L, dk=8, dv=5, s0=s0)
    a = (a * 3.0).astype(f32)                       # stronger decays: cumulative logs reach ~-60
    if reset:
        a[0, L // 3, 1, 2] = -np.inf
        a[1, L // 2, 0, :] = -np.inf
    O, S = oracle.fwd_kda(q, k, v, beta, a, S0, scale=0.8)
    Oc, Sc = F.chunked_kda(q, k, v, beta, a, S0, C=C, scale=0.8)
    assert np.abs(O - Oc).max() <= 1e-10 * max(1.0, np.abs(O).max())
    assert np.abs(S - Sc).max() <= 1e-10 * max(1.0, np.abs(S).max())
