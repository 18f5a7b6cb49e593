"""GPU path against results the pages fix in closed form (not against the oracle).

Each case runs the HIP path through the C ABI on inputs whose exact answer the pages state:
  - the n_h = 2 mod-3 rotation of the DeltaProduct notes, section 2.4, against the page's printed
    matrix (tests/golden/mod3_rotation.txt), embedded in d_k = d_v = 16;
  - swap permutations at beta = 2 (DeltaProduct notes, section 3.1): (e_a - e_b)/sqrt2 keys, n_h = 4
    swaps per token, integer-valued outputs that track the composed permutation;
  - the exact write at beta = 1 with a unit key (DeltaProduct notes, section 2.1: the write makes
    S_t^T k_t = v_t), read back with q_t = k_t, gated and with S0;
  - the same key twice at beta = 2 is the identity (DeltaProduct notes, section 2.5);
  - one Householder transition: S0 = I, v = 0 gives I - beta k k^T ("08 linear delta rule &
    DPLR", section 1.2).
All in float32 (the page values need exact unit keys; bf16 keys are not unit-norm)."""
import os

import numpy as np
import pytest

from parity import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import chunkwise_delta_rule_chunked_amd as D  # noqa: E402

f32 = np.float32
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def gpu(q, k, v, beta, g_log, S0, n_h, chunk, **kw):
    t = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=f32)).cuda()
    O, S = D.fwd(t(q), t(k), t(v), t(beta), t(g_log), t(S0), n_h=n_h, chunk=chunk, **kw)
    torch.cuda.synchronize()
    return O.cpu().numpy().astype(np.float64), S.cpu().numpy().astype(np.float64)


def golden_rows():
    rows = {}
    for line in open(os.path.join(GOLDEN, "mod3_rotation.txt")):
        if line.strip() and not line.startswith("#"):
            p = line.split()
            rows[p[0]] = np.array([float(x) for x in p[1:]])
    return rows


@pytest.mark.parametrize("L,chunk", [(6, 16), (99, 16), (99, 64), (400, 32)])
def test_mod3_rotation(L, chunk):
    """Head 0 reads with q = e1, head 1 with q = e2; state column 0 starts at e1 and rotates by
    120 degrees per token, so the outputs repeat the page's three states."""
    rows = golden_rows()
    dk = dv = 16
    H = 2
    k = np.zeros((1, 2 * L, H, dk), f32)
    k[0, 0::2, :, 0] = 1.0                                  # k1 = (1, 0)
    k[0, 1::2, :, 0] = 0.5                                  # k2 = (1/2, sqrt3/2)
    k[0, 1::2, :, 1] = np.sqrt(3.0) / 2
    v = np.zeros((1, 2 * L, H, dv), f32)
    beta = np.full((1, 2 * L, H), 2.0, f32)
    S0 = np.zeros((1, H, dk, dv), f32)
    S0[0, :, 0, 0] = 1.0                                    # column 0 = e1
    q = np.zeros((1, L, H, dk), f32)
    q[0, :, 0, 0] = 1.0
    q[0, :, 1, 1] = 1.0
    O, S = gpu(q, k, v, beta, None, S0, n_h=2, chunk=chunk)
    want = np.array([rows["S%d" % (i % 3 + 1)] for i in range(L)])   # [L, 2]: S_i = (F2F1)^i e1
    err = max(np.abs(O[0, :, 0, 0] - want[:, 0]).max(), np.abs(O[0, :, 1, 0] - want[:, 1]).max())
    say("mod3 L=%d chunk=%d: max |O - page| %.2e" % (L, chunk, err))
    assert err <= 1e-4
    assert np.abs(O[0, :, :, 1:]).max() == 0.0             # the zero columns stay zero
    last = rows["S%d" % ((L - 1) % 3 + 1)]
    assert np.allclose(S[0, 0, :2, 0], last, atol=1e-4) and np.abs(S[0, 0, 2:, 0]).max() <= 1e-6


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_swap_permutations(chunk):
    """n = 5 coordinates embedded in d_k = 16; each token applies 4 random transpositions
    (k = (e_a - e_b)/sqrt2, beta = 2).  Head h reads coordinate h (q = e_h), so O[:, t, h, 0] is
    the value at coordinate h after token t of the tracked vector (1..5)."""
    n, n_h, L, dk, dv = 5, 4, 40, 16, 16
    r = np.random.default_rng(31)
    k1 = np.zeros((L * n_h, dk), f32)
    cur = np.arange(1, n + 1, dtype=np.float64)
    tracked = []
    for i in range(L):
        for j in range(n_h):
            a, b = r.choice(n, 2, replace=False)
            k1[i * n_h + j, a], k1[i * n_h + j, b] = 1 / np.sqrt(2), -1 / np.sqrt(2)
            cur[[a, b]] = cur[[b, a]]
        tracked.append(cur.copy())
    tracked = np.array(tracked)                             # [L, n]
    H = n
    k = np.repeat(k1[None, :, None, :], H, axis=2)
    v = np.zeros((1, L * n_h, H, dv), f32)
    beta = np.full((1, L * n_h, H), 2.0, f32)
    S0 = np.zeros((1, H, dk, dv), f32)
    S0[0, :, :n, 0] = np.arange(1, n + 1)
    q = np.zeros((1, L, H, dk), f32)
    for h in range(H):
        q[0, :, h, h] = 1.0
    O, S = gpu(q, k, v, beta, None, S0, n_h=n_h, chunk=chunk)
    got = O[0, :, :, 0]                                     # [L, n]
    err = np.abs(got - tracked).max()
    say("swaps chunk=%d: max |O - tracked| %.2e, max |O - round(O)| %.2e" % (chunk, err,
                                                                           np.abs(got - np.round(got)).max()))
    assert err <= 1e-4
    assert np.array_equal(np.round(got), tracked)
    assert np.allclose(S[0, 0, :n, 0], tracked[-1], atol=1e-4)


@pytest.mark.parametrize("n_h,gated,chunk", [(1, False, 64), (1, True, 32), (2, True, 16), (3, False, 48)])
def test_beta_one_exact_write(n_h, gated, chunk):
    """beta = 1 with unit keys: after each token's last write S_t^T k = v for that key, so reading
    with q_t = that key returns v exactly, whatever S0 and the gate were."""
    B, H, L, dk, dv = 1, 3, 150, 64, 32
    r = np.random.default_rng(5)
    k = r.standard_normal((B, L * n_h, H, dk))
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(f32)
    v = r.standard_normal((B, L * n_h, H, dv)).astype(f32)
    beta = np.ones((B, L * n_h, H), f32)
    g = -np.log1p(np.exp(r.standard_normal((B, L, H)) - 1.0)).astype(f32) if gated else None
    S0 = (0.1 * r.standard_normal((B, H, dk, dv))).astype(f32)
    q = np.ascontiguousarray(k[:, n_h - 1::n_h])            # the last sub-step's key of each token
    O, _ = gpu(q, k, v, beta, g, S0, n_h=n_h, chunk=chunk)
    want = v[:, n_h - 1::n_h].astype(np.float64)
    # exact up to the float32 key norm (|k|^2 = 1 within a few ulp) and float32 arithmetic
    err = np.abs(O - want).max() / np.abs(want).max()
    say("beta=1 write n_h=%d gated=%s: rel err %.2e" % (n_h, gated, err))
    assert err <= 1e-4


@pytest.mark.parametrize("chunk", [16, 64])
def test_same_key_twice_beta2_is_identity(chunk):
    """n_h = 2, both sub-steps the same unit key at beta = 2, v = 0: each token's transition is I,
    so S_final = S0 and o_t = S0^T q_t."""
    B, H, L, dk, dv = 2, 2, 120, 32, 48
    r = np.random.default_rng(9)
    kk = r.standard_normal((B, L, H, dk))
    kk = (kk / np.linalg.norm(kk, axis=-1, keepdims=True)).astype(f32)
    k = np.repeat(kk, 2, axis=1)                            # sub-steps 2i and 2i+1 share key i
    v = np.zeros((B, 2 * L, H, dv), f32)
    beta = np.full((B, 2 * L, H), 2.0, f32)
    S0 = r.standard_normal((B, H, dk, dv)).astype(f32)
    q = r.standard_normal((B, L, H, dk)).astype(f32)
    O, S = gpu(q, k, v, beta, None, S0, n_h=2, chunk=chunk)
    want = np.einsum("bhkv,blhk->blhv", S0.astype(np.float64), q.astype(np.float64))
    eo = np.abs(O - want).max() / np.abs(want).max()
    es = np.abs(S - S0).max() / np.abs(S0).max()
    say("same key twice chunk=%d: rel err O %.2e S %.2e" % (chunk, eo, es))
    assert eo <= 1e-4 and es <= 1e-4


@pytest.mark.parametrize("dk", [16, 64, 128])
def test_single_householder_transition(dk):
    """S0 = I, v = 0, one token: S_final = I - beta k k^T, whose eigenvalues are 1 - beta (along k)
    and 1 (d_k - 1 times)."""
    r = np.random.default_rng(dk)
    H = 4
    kk = r.standard_normal((1, 1, H, dk))
    kk = (kk / np.linalg.norm(kk, axis=-1, keepdims=True)).astype(f32)
    beta = np.array([0.3, 1.0, 1.7, 2.0], f32).reshape(1, 1, H)
    S0 = np.tile(np.eye(dk, dtype=f32), (1, H, 1, 1))
    v = np.zeros((1, 1, H, dk), f32)
    q = np.zeros((1, 1, H, dk), f32)
    _, S = gpu(q, kk, v, beta, None, S0, n_h=1, chunk=16)
    for h in range(H):
        k64 = kk[0, 0, h].astype(np.float64)
        want = np.eye(dk) - float(beta[0, 0, h]) * np.outer(k64, k64)
        assert np.abs(S[0, h] - want).max() <= 1e-5
        ev = np.sort(np.linalg.eigvalsh((S[0, h] + S[0, h].T) / 2))
        assert abs(ev[0] - min(1 - beta[0, 0, h], 1.0)) <= 1e-4 and abs(ev[-1] - max(1 - beta[0, 0, h], 1.0)) <= 1e-4
