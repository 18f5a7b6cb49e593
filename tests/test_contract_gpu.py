"""GPU checks of the library's contract beyond plain parity:
  - g = 0 (log g = -inf), the hard reset of the DeltaProduct notes (section 3.3), inside chunks and
    across segments, against the oracle (which takes it exactly);
  - the opt-in DELTA_VALIDATE=1 pass: out-of-contract beta or log gates return
    DELTA_ERR_BAD_VALUE (-8) and leave every output untouched; -inf log gates pass;
  - DELTA_FAULT=launch: DELTA_ERR_HIP (-7) with nothing written;
  - workspace contents on entry are ignored: a NaN-filled workspace gives bitwise the results of a
    zero-filled one (no kernel reads a workspace byte it did not write in the same call);
  - NaN inputs propagate to the outputs they reach and no further;
  - the in-place update S_final == S0 with the sequence split into segments."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import TOL, head_rel_err, inputs_to_dev, say, to_np
from test_parity_gpu import wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import chunkwise_delta_rule_chunked_amd as D  # noqa: E402


def with_resets(inp, where):
    """Copy of the inputs with log g = -inf at the (b, token, h) triples in `where`."""
    g = inp["g_log"].copy()
    for b, t, h in where:
        g[b, t, h] = -np.inf
    return dict(inp, g_log=g)


RESET_CASES = [
    # dtype, n_h, chunk, tokens reset on head 0 (and a few on head 1)
    ("f32", 1, 64, [0, 37, 63, 64, 100, 101, 640]),
    ("bf16", 1, 64, [5, 200, 201, 511, 512, 699]),
    ("f32", 2, 16, [0, 3, 7, 8, 150]),
    ("bf16", 2, 64, [31, 32, 33, 340]),
    ("f32", 1, 48, [47, 48, 333]),
]


@pytest.mark.parametrize("dt,n_h,chunk,toks", RESET_CASES)
def test_hard_reset(dt, n_h, chunk, toks):
    """Weak gate (the state carries far), resets at a chunk's first and last position, mid-chunk,
    twice in a row, and in later segments: GPU against the oracle's exact g = 0."""
    L = 700 if n_h == 1 else 350
    w = wl("reset", B=1, H=2, L=L, dk=64, dv=64, chunk=chunk, n_h=n_h, dtype=dt, gate="weak", s0=0.1,
           key="silu_l2n" if n_h > 1 else "l2n", beta="2sigmoid" if n_h > 1 else "sigmoid")
    P, _ = D.segments(w.B, w.L, w.H, w.dk, w.dv, n_h, chunk, D.BF16 if dt == "bf16" else D.F32)
    inp = with_resets(W.make_inputs(w), [(0, t, 0) for t in toks if t < L] + [(0, t, 1) for t in (1, L // 2)])
    say("case reset", w, "segments", P, "resets", toks)
    d = inputs_to_dev(inp, dt)
    O, S = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], n_h=n_h, chunk=chunk)
    torch.cuda.synchronize()
    Or, Sr = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g_log"], inp["S0"], n_h=n_h)
    O, S = to_np(O), to_np(S)
    assert np.isfinite(O).all() and np.isfinite(S).all()
    eo, es = head_rel_err(O, Or, (0, 2)), head_rel_err(S, Sr, (0, 1))
    say("  err O %.3e S %.3e" % (eo, es))
    assert eo <= TOL[dt] and es <= TOL[dt]
    # right after a reset the output no longer depends on anything before it: the token's readout
    # equals the oracle's run of that token's own writes from a zero state
    t = toks[1]
    sub = {kk: (None if x is None else x[:, t:t + 1] if kk in ("q", "g_log") else
                x[:, t * n_h:(t + 1) * n_h] if kk in ("k", "v", "beta") else None)
           for kk, x in inp.items()}
    O1, _ = oracle.fwd(sub["q"][:, :, :1], sub["k"][:, :, :1], sub["v"][:, :, :1], sub["beta"][:, :, :1],
                       None, None, n_h=n_h)
    assert np.abs(O[0, t, 0] - O1[0, 0, 0]).max() <= TOL[dt] * np.abs(Or[0, :, 0]).max()


def test_decode_hard_reset():
    """A decode step with log g = -inf on some heads: the state is cleared before the write."""
    w = W.Workload("dec_reset", B=4, H=3, L=1, dk=64, dv=64, dtype="f32", gate="cfg3", s0=0.1, cfg_id=97)
    S0 = W.make_decode_state(w)
    x = W.make_decode_inputs(w, 0)
    x["g_log"][1, 0, 2] = -np.inf
    x["g_log"][3, 0, 0] = -np.inf
    d = inputs_to_dev(dict(x, S0=None), "f32")
    S = torch.from_numpy(S0).cuda()
    O = D.decode(d["q"], d["k"], d["v"], d["beta"], d["g_log"], S)
    torch.cuda.synchronize()
    Or, Sr = oracle.fwd(x["q"], x["k"], x["v"], x["beta"], x["g_log"], S0)
    assert head_rel_err(to_np(O), Or, (0, 2)) <= TOL["f32"]
    assert head_rel_err(S.cpu().numpy(), Sr, (0, 1)) <= TOL["f32"]


# ---------------------------------------------------------------- DELTA_VALIDATE / DELTA_FAULT

def sentinel(shape, dtype):
    return torch.full(shape, 7.0, dtype=dtype, device="cuda")


def fwd_call(w, d, **kw):
    O = sentinel((w.B, w.L, w.H, w.dv), torch.bfloat16 if w.dtype == "bf16" else torch.float32)
    S = sentinel((w.B, w.H, w.dk, w.dv), torch.float32)
    D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], n_h=w.n_h, chunk=w.chunk, O=O, S_final=S, **kw)
    torch.cuda.synchronize()
    return O, S


@pytest.mark.parametrize("what", ["nan_gate", "posinf_gate", "nan_beta", "inf_beta", "neginf_beta"])
def test_validate_rejects(monkeypatch, what):
    w = wl("validate", B=1, H=2, L=300, dk=64, dv=64, chunk=64, gate="cfg3", s0=0.1, dtype="bf16")
    inp = W.make_inputs(w)
    key, val = {"nan_gate": ("g_log", np.nan), "posinf_gate": ("g_log", np.inf), "nan_beta": ("beta", np.nan),
                "inf_beta": ("beta", np.inf), "neginf_beta": ("beta", -np.inf)}[what]
    bad = inp[key].copy()
    bad[0, 217, 1] = val
    d = inputs_to_dev(dict(inp, **{key: bad}), "bf16")
    monkeypatch.setenv("DELTA_VALIDATE", "1")
    with pytest.raises(D.DeltaError) as e:
        O, S = fwd_call(w, d)
    assert e.value.code == -8
    # nothing written: run again into sentinel buffers and inspect them
    O = sentinel((w.B, w.L, w.H, w.dv), torch.bfloat16)
    S = sentinel((w.B, w.H, w.dk, w.dv), torch.float32)
    ws = torch.empty(D.workspace_bytes(w.B, w.L, w.H, w.dk, w.dv, 1, w.chunk), dtype=torch.uint8, device="cuda")
    with pytest.raises(D.DeltaError):
        D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], chunk=w.chunk, O=O, S_final=S, workspace=ws)
    torch.cuda.synchronize()
    assert bool((O.float() == 7.0).all()) and bool((S == 7.0).all())
    # the backward and the intra-chunk phase check the same inputs
    dO = torch.ones_like(d["q"])
    with pytest.raises(D.DeltaError) as e:
        D.bwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], dO, None, chunk=w.chunk)
    assert e.value.code == -8
    with pytest.raises(D.DeltaError) as e:
        D.fwd_intra(d["k"], d["beta"], d["g_log"], ws, chunk=w.chunk, dv=w.dv)
    assert e.value.code == -8


def test_validate_accepts_resets(monkeypatch):
    """-inf log gates are resets, inside the contract: the validated call runs and gives exactly
    the unvalidated result."""
    w = wl("validate_ok", B=1, H=2, L=300, dk=64, dv=64, chunk=64, gate="weak", s0=0.1, dtype="bf16")
    inp = with_resets(W.make_inputs(w), [(0, 10, 0), (0, 250, 1)])
    d = inputs_to_dev(inp, "bf16")
    O1, S1 = fwd_call(w, d)
    monkeypatch.setenv("DELTA_VALIDATE", "1")
    O2, S2 = fwd_call(w, d)
    assert torch.equal(O1, O2) and torch.equal(S1, S2)


def test_validate_decode(monkeypatch):
    w = W.Workload("dec_val", B=2, H=2, L=1, dk=32, dv=32, dtype="bf16", gate="cfg3", s0=0.1, cfg_id=98)
    x = W.make_decode_inputs(w, 0)
    S0 = torch.from_numpy(W.make_decode_state(w)).cuda()
    monkeypatch.setenv("DELTA_VALIDATE", "1")
    for key in ("beta", "g_log"):
        bad = dict(x)
        bad[key] = x[key].copy()
        bad[key][1, 0, 1] = np.nan
        d = inputs_to_dev(dict(bad, S0=None), "bf16")
        S = S0.clone()
        O = sentinel((w.B, 1, w.H, w.dv), torch.bfloat16)
        with pytest.raises(D.DeltaError) as e:
            D.decode(d["q"], d["k"], d["v"], d["beta"], d["g_log"], S, O=O)
        torch.cuda.synchronize()
        assert e.value.code == -8 and torch.equal(S, S0) and bool((O.float() == 7.0).all())
    a = np.zeros((w.B, 1, w.H, w.dk), np.float32)
    a[0, 0, 1, 3] = np.inf
    d = inputs_to_dev(dict(x, S0=None), "bf16")
    with pytest.raises(D.DeltaError) as e:
        D.decode_kda(d["q"], d["k"], d["v"], d["beta"], torch.from_numpy(a).cuda(), S0.clone())
    assert e.value.code == -8


def test_fault_injection(monkeypatch):
    """DELTA_FAULT=launch: -7 from every entry point with work, and nothing written."""
    w = wl("fault", B=1, H=2, L=100, dk=32, dv=32, chunk=32, gate="cfg3", s0=0.1, dtype="f32")
    d = inputs_to_dev(W.make_inputs(w), "f32")
    monkeypatch.setenv("DELTA_FAULT", "launch")
    O = sentinel((w.B, w.L, w.H, w.dv), torch.float32)
    S = sentinel((w.B, w.H, w.dk, w.dv), torch.float32)
    with pytest.raises(D.DeltaError) as e:
        D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], chunk=w.chunk, O=O, S_final=S)
    torch.cuda.synchronize()
    assert e.value.code == -7 and bool((O == 7.0).all()) and bool((S == 7.0).all())
    Sd = sentinel((1, 2, 32, 32), torch.float32)
    x = inputs_to_dev(dict(W.make_decode_inputs(w.replace(L=1), 0), S0=None), "f32")
    with pytest.raises(D.DeltaError) as e:
        D.decode(x["q"], x["k"], x["v"], x["beta"], x["g_log"], Sd)
    torch.cuda.synchronize()
    assert e.value.code == -7 and bool((Sd == 7.0).all())
    monkeypatch.delenv("DELTA_FAULT")
    D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], chunk=w.chunk, O=O, S_final=S)
    torch.cuda.synchronize()
    assert not bool((O == 7.0).all())


# ---------------------------------------------------------------- workspace and NaN handling

POISON_CASES = [
    wl("poison_gdn", B=2, H=2, L=1000, dk=128, dv=128, chunk=64, gate="cfg3", s0=0.1),        # fast summary
    wl("poison_dp2", B=1, H=2, L=333, dk=64, dv=96, chunk=32, n_h=2, gate="weak", s0=0.1,
       key="silu_l2n", beta="2sigmoid"),
    wl("poison_f32", B=1, H=3, L=257, dk=32, dv=48, chunk=16, dtype="f32", gate="weak", s0=0.1),
    wl("poison_unsplit", B=32, H=8, L=130, dk=32, dv=32, chunk=32, gate="cfg3", s0=0.1),
]


@pytest.mark.parametrize("w", POISON_CASES, ids=lambda w: w.name)
def test_nan_workspace_is_ignored(w):
    d = inputs_to_dev(W.make_inputs(w), w.dtype)
    nbytes = D.workspace_bytes(w.B, w.L, w.H, w.dk, w.dv, w.n_h, w.chunk, D.BF16 if w.dtype == "bf16" else D.F32)
    res = []
    for fill in (0.0, float("nan")):
        ws = torch.empty(max(nbytes, 4) // 4, dtype=torch.float32, device="cuda").fill_(fill)
        res.append(D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], n_h=w.n_h, chunk=w.chunk,
                         workspace=ws))
    torch.cuda.synchronize()
    (O0, S0), (O1, S1) = res
    assert torch.isfinite(O1.float()).all() and torch.isfinite(S1).all()
    assert torch.equal(O0, O1) and torch.equal(S0, S1)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_nan_propagates(dt):
    """NaN in one value row of head 1 reaches that head's output from its token on (and its final
    state); the other head, and head 1's tokens before that token's chunk, stay finite.  (Inside
    the chunk it may reach earlier tokens too: the zeros above the diagonal of T and of the causal
    Q K^T multiply it, and 0 * NaN is NaN.)"""
    w = wl("nan", B=1, H=2, L=300, dk=64, dv=64, chunk=64, gate="weak", s0=0.1, dtype=dt)
    inp = W.make_inputs(w)
    t = 150
    v = inp["v"].copy()
    v[0, t, 1, 5] = np.nan
    d = inputs_to_dev(dict(inp, v=v), dt)
    O, S = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], chunk=w.chunk)
    torch.cuda.synchronize()
    O, S = to_np(O), to_np(S)
    assert np.isfinite(O[0, :, 0]).all() and np.isfinite(S[0, 0]).all()
    assert np.isfinite(O[0, :t // w.chunk * w.chunk, 1]).all()
    assert np.isnan(O[0, t, 1]).any() and np.isnan(O[0, -1, 1]).any() and np.isnan(S[0, 1]).any()


@pytest.mark.parametrize("dt,dv", [("bf16", 128), ("f32", 64)])
def test_in_place_many_segments(dt, dv):
    """S_final == S0 with the sequence split into many segments: the same result as with a separate
    S_final buffer (the outputs launch must not read S0 while its last segment writes it)."""
    w = wl("inplace_seg", B=1, H=4, L=2000, dk=128, dv=dv, chunk=64, gate="weak", s0=0.1, dtype=dt)
    P, _ = D.segments(w.B, w.L, w.H, w.dk, w.dv, 1, w.chunk, D.BF16 if dt == "bf16" else D.F32)
    assert P > 8
    d = inputs_to_dev(W.make_inputs(w), dt)
    O1, S1 = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], chunk=w.chunk)
    Sin = d["S0"].clone()
    O2, S2 = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], Sin, chunk=w.chunk, S_final=Sin)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(S1, S2)
