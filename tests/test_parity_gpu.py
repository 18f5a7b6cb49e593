"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded
inputs.  Bar: err <= 1e-4 (float32 inputs) or <= 2e-2 (bf16 inputs, fp32 state), with err the
per-head relative error defined in tests/parity.py."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import TOL, head_rel_err, inputs_to_dev, say, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import chunkwise_delta_rule_chunked_amd as D  # noqa: E402


def run_gpu(w, inp, chunk=None, **kw):
    d = inputs_to_dev(inp, w.dtype)
    O, S = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], n_h=w.n_h,
                 chunk=chunk or w.chunk, **kw)
    torch.cuda.synchronize()
    return to_np(O), to_np(S)


def check(w, inp, chunk=None, tol=None, heads=None):
    """Run GPU and oracle; compare O and S_final.  heads: optional list of (b, h) to sample."""
    say("case", w, "chunk", chunk or w.chunk)
    O, S = run_gpu(w, inp, chunk)
    if heads is None:
        Or, Sr = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g_log"], inp["S0"], n_h=w.n_h)
    else:
        Or = np.zeros(O.shape[:1] + O.shape[1:])
        outs = []
        for b, h in heads:
            q = inp["q"][b:b + 1, :, h:h + 1]
            k = inp["k"][b:b + 1, :, h:h + 1]
            v = inp["v"][b:b + 1, :, h:h + 1]
            be = inp["beta"][b:b + 1, :, h:h + 1]
            g = None if inp["g_log"] is None else inp["g_log"][b:b + 1, :, h:h + 1]
            S0 = None if inp["S0"] is None else inp["S0"][b:b + 1, h:h + 1]
            outs.append(oracle.fwd(q, k, v, be, g, S0, n_h=w.n_h))
        O = np.concatenate([O[b:b + 1, :, h:h + 1] for b, h in heads], axis=2)
        S = np.concatenate([S[b:b + 1, h:h + 1] for b, h in heads], axis=1)
        Or = np.concatenate([o for o, _ in outs], axis=2)
        Sr = np.concatenate([s for _, s in outs], axis=1)
    eo = head_rel_err(O, Or, (0, 2))
    es = head_rel_err(S, Sr, (0, 1))
    tol = tol if tol is not None else TOL[w.dtype]
    say("  err O %.3e  S %.3e  (tol %.0e)" % (eo, es, tol))
    assert np.isfinite(O).all() and np.isfinite(S).all()
    assert eo <= tol and es <= tol, (eo, es)
    return eo, es


# ---------------------------------------------------------------- small cases (whole oracle)

def wl(name, **kw):
    base = dict(B=2, H=2, L=100, dk=64, dv=64, chunk=32, dtype="bf16", cfg_id=90)
    base.update(kw)
    return W.Workload(name, **base)


F32_CASES = [
    W.CONFIGS["tiny_deltanet_f32"],
    wl("f32_gated_ragged", dtype="f32", L=77, dk=32, dv=48, chunk=32, gate="weak", s0=0.1),
    wl("f32_dp3_c48", dtype="f32", L=50, dk=64, dv=16, chunk=48, n_h=3, gate="cfg3", key="silu_l2n",
       beta="2sigmoid", s0=0.1),
    wl("f32_d128_c64", dtype="f32", B=1, L=130, dk=128, dv=128, chunk=64, gate="cfg3", s0=0.1),
    wl("f32_dk16_dv256_c16_dp2", dtype="f32", B=1, H=3, L=41, dk=16, dv=256, chunk=16, n_h=2,
       gate="weak"),
    wl("f32_nh4_c16", dtype="f32", B=1, L=23, dk=32, dv=32, chunk=16, n_h=4, beta="2sigmoid"),
]

BF16_CASES = [
    wl("bf16_deltanet_d128", B=2, H=2, L=333, dk=128, dv=128, chunk=64),
    wl("bf16_gdn_d128", B=2, H=2, L=333, dk=128, dv=128, chunk=64, gate="cfg3", s0=0.1),
    wl("bf16_gdn_weak_d128", B=1, H=2, L=700, dk=128, dv=128, chunk=64, gate="weak", s0=0.1),
    wl("bf16_gdp2_d128", B=1, H=2, L=300, dk=128, dv=128, chunk=64, n_h=2, gate="cfg3",
       key="silu_l2n", beta="2sigmoid"),
    wl("bf16_gdp2_weak_s0", B=1, H=2, L=257, dk=128, dv=128, chunk=64, n_h=2, gate="weak",
       key="silu_l2n", beta="2sigmoid", s0=0.1),
    wl("bf16_dp4_c32", B=1, H=3, L=90, dk=64, dv=64, chunk=32, n_h=4, key="silu_l2n", beta="2sigmoid",
       gate="weak"),
    wl("bf16_dp3_c48", B=2, H=1, L=95, dk=32, dv=80, chunk=48, n_h=3, gate="cfg3", key="silu_l2n",
       beta="2sigmoid", s0=0.1),
    wl("bf16_c16_dk16", B=2, H=2, L=61, dk=16, dv=16, chunk=16, gate="weak", s0=0.1),
    wl("bf16_c48_dk32_dv256", B=1, H=2, L=150, dk=32, dv=256, chunk=48, gate="cfg3"),
    wl("bf16_nh16_c16", B=1, H=2, L=20, dk=64, dv=32, chunk=16, n_h=16, key="silu_l2n", beta="2sigmoid"),
]


@pytest.mark.parametrize("w", F32_CASES, ids=lambda w: w.name)
def test_fwd_f32(w):
    check(w, W.make_inputs(w))


@pytest.mark.parametrize("w", BF16_CASES, ids=lambda w: w.name)
def test_fwd_bf16(w):
    check(w, W.make_inputs(w))


@pytest.mark.parametrize("chunk", [16, 32, 48, 64])
def test_chunk_size_invariance(chunk):
    """Results do not depend on the chunk beyond rounding: every chunk size meets the bar."""
    w = wl("bf16_weak_chunks", B=1, H=2, L=200, dk=64, dv=64, gate="weak", s0=0.1)
    check(w, W.make_inputs(w), chunk=chunk)
    wf = w.replace(dtype="f32")
    check(wf, W.make_inputs(wf), chunk=chunk)


@pytest.mark.parametrize("L", [1, 5, 16, 17, 63, 64, 65])
def test_short_and_ragged(L):
    for dt in ("f32", "bf16"):
        w = wl("short", B=1, H=2, L=L, dk=64, dv=32, chunk=64 if L > 16 else 16, dtype=dt, gate="cfg3",
               s0=0.1)
        check(w, W.make_inputs(w))


@pytest.mark.parametrize("beta", ["zero", "one", "two"])
def test_beta_extremes(beta):
    for dt in ("f32", "bf16"):
        w = wl("beta_" + beta, B=1, H=2, L=130, dk=64, dv=32, chunk=64, dtype=dt, gate="weak", s0=0.1,
               beta=beta)
        check(w, W.make_inputs(w))


def test_empty_sequence_copies_state():
    w = wl("empty", B=2, H=2, L=0, dk=32, dv=32, dtype="f32", s0=0.1)
    inp = W.make_inputs(w)
    d = inputs_to_dev(inp, "f32")
    O, S = D.fwd(d["q"], d["k"], d["v"], d["beta"], None, d["S0"], chunk=32)
    torch.cuda.synchronize()
    assert O.numel() == 0 and np.array_equal(to_np(S), inp["S0"])
    O, S = D.fwd(d["q"], d["k"], d["v"], d["beta"], None, None, chunk=32)
    torch.cuda.synchronize()
    assert np.all(to_np(S) == 0)


def test_in_place_state_and_determinism():
    w = wl("inplace", B=2, H=2, L=150, dk=128, dv=64, chunk=64, gate="weak", s0=0.1)
    inp = W.make_inputs(w)
    d = inputs_to_dev(inp, "bf16")
    O1, S1 = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], chunk=64)
    O2, S2 = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], chunk=64)
    Sin = d["S0"].clone()
    O3, S3 = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], Sin, chunk=64, S_final=Sin)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(S1, S2)      # bitwise deterministic
    assert torch.equal(O1, O3) and torch.equal(S1, S3) and S3.data_ptr() == Sin.data_ptr()


@pytest.mark.parametrize("dk", [32, 128])
def test_chunk48_repeatable(dk):
    """Chunk 48 mixes 32- and 16-deep contractions; repeated calls must agree bitwise and meet the
    bar (a dependent 16x16x32 -> 16x16x16 MFMA pair on one accumulator once gave intermittent
    wrong sums here)."""
    w = wl("c48_repeat", B=1, H=2, L=150, dk=dk, dv=32, chunk=48, gate="weak", s0=0.1)
    inp = W.make_inputs(w)
    d = inputs_to_dev(inp, "bf16")
    runs = []
    for _ in range(6):
        O, S = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], chunk=48)
        runs.append((O.clone(), S.clone()))
    torch.cuda.synchronize()
    for O, S in runs[1:]:
        assert torch.equal(O, runs[0][0]) and torch.equal(S, runs[0][1])
    Or, Sr = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g_log"], inp["S0"])
    assert head_rel_err(to_np(runs[0][0]), Or, (0, 2)) <= TOL["bf16"]
    assert head_rel_err(to_np(runs[0][1]), Sr, (0, 1)) <= TOL["bf16"]


def test_segment_split():
    """S_final of one call as S0 of the next reproduces a single call (the state is the resume point)."""
    w = wl("split", B=1, H=2, L=300, dk=64, dv=64, chunk=64, gate="weak", s0=0.1, n_h=2,
           key="silu_l2n", beta="2sigmoid")
    inp = W.make_inputs(w)
    d = inputs_to_dev(inp, "bf16")
    c = 111
    Oa, Sa = D.fwd(d["q"][:, :c].contiguous(), d["k"][:, :2 * c].contiguous(), d["v"][:, :2 * c].contiguous(),
                   d["beta"][:, :2 * c].contiguous(), d["g_log"][:, :c].contiguous(), d["S0"], n_h=2)
    Ob, Sb = D.fwd(d["q"][:, c:].contiguous(), d["k"][:, 2 * c:].contiguous(), d["v"][:, 2 * c:].contiguous(),
                   d["beta"][:, 2 * c:].contiguous(), d["g_log"][:, c:].contiguous(), Sa, n_h=2)
    torch.cuda.synchronize()
    Or, Sr = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g_log"], inp["S0"], n_h=2)
    O = np.concatenate([to_np(Oa), to_np(Ob)], axis=1)
    assert head_rel_err(O, Or, (0, 2)) <= TOL["bf16"]
    assert head_rel_err(to_np(Sb), Sr, (0, 1)) <= TOL["bf16"]


def test_phase_calls_match_fwd():
    """intra, then the three scan launches called one by one, reproduce fwd bitwise (with a
    readout scale, which the outputs launch folds into its on-chip Q K^T)."""
    w = wl("phases", B=1, H=2, L=400, dk=64, dv=96, chunk=32, gate="weak", s0=0.1)
    P, NS = D.segments(w.B, w.L, w.H, w.dk, w.dv, 1, w.chunk)
    assert P > 1
    inp = W.make_inputs(w)
    d = inputs_to_dev(inp, "bf16")
    O1, S1 = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], chunk=w.chunk, scale=0.5)
    ws = torch.empty(D.workspace_bytes(w.B, w.L, w.H, w.dk, w.dv, 1, w.chunk), dtype=torch.uint8, device="cuda")
    O2, S2 = torch.empty_like(O1), torch.empty_like(S1)
    D.fwd_intra(d["k"], d["beta"], d["g_log"], ws, chunk=w.chunk, dv=w.dv)
    D.scan_summary(d["k"], d["v"], d["S0"], ws, chunk=w.chunk)
    D.scan_combine(ws, B=w.B, L=w.L, H=w.H, dk=w.dk, dv=w.dv, chunk=w.chunk)
    D.scan_outputs(d["q"], d["k"], d["v"], d["S0"], ws, chunk=w.chunk, scale=0.5, O=O2, S_final=S2)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(S1, S2)


@pytest.mark.parametrize("dt,chunk", [("bf16", 16), ("f32", 64), ("bf16", 48)])
def test_many_segments_weak_gate(dt, chunk):
    """One head, a long sequence and a weak gate: the state carries across ~100 segments, so
    every segment's transition and the chained start states matter."""
    L = {16: 1500, 64: 3000, 48: 2400}[chunk]
    w = wl("many_seg", B=1, H=1, L=L, dk=128, dv=128, chunk=chunk, dtype=dt, gate="weak", s0=0.1)
    P, NS = D.segments(w.B, w.L, w.H, w.dk, w.dv, 1, chunk, D.BF16 if dt == "bf16" else D.F32)
    say("segments", P, "x", NS, "chunks")
    assert P >= 40
    check(w, W.make_inputs(w))


def test_unsplit_many_heads():
    """Enough heads to fill the GPU: one segment per sequence (no summary or combine launch)."""
    w = wl("unsplit", B=32, H=8, L=130, dk=32, dv=32, chunk=32, gate="cfg3", s0=0.1)
    assert D.segments(w.B, w.L, w.H, w.dk, w.dv, 1, w.chunk) == (1, 5)
    check(w, W.make_inputs(w), heads=[(0, 0), (7, 3), (31, 7)])


def test_scale():
    w = wl("scale", B=1, H=2, L=70, dk=32, dv=32, chunk=32, dtype="f32", gate="cfg3")
    inp = W.make_inputs(w)
    d = inputs_to_dev(inp, "f32")
    O, _ = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], None, chunk=32, scale=0.125)
    torch.cuda.synchronize()
    Or, _ = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g_log"], None, scale=0.125)
    assert head_rel_err(to_np(O), Or, (0, 2)) <= TOL["f32"]


# ---------------------------------------------------------------- intra-chunk factors

@pytest.mark.parametrize("dt,chunk,n_h,gate", [("f32", 16, 1, None), ("f32", 64, 2, "cfg3"),
                                               ("bf16", 64, 1, "cfg3"), ("bf16", 48, 3, "weak"),
                                               ("bf16", 32, 1, None)])
def test_chunk_wy_factors(dt, chunk, n_h, gate):
    """T, W, U, gc of the intra-chunk kernel against oracle.ut_factors (fp64 definitions).
    Inputs are the same (bf16-rounded) values on both sides; T is computed in fp32 on the GPU."""
    w = wl("wy", B=1, H=2, L=(150 // n_h), dk=64, dv=48, chunk=chunk, n_h=n_h, gate=gate, dtype=dt,
           key="silu_l2n", beta="2sigmoid")
    inp = W.make_inputs(w)
    say("case chunk_wy", w)
    d = inputs_to_dev(inp, dt)
    f = D.chunk_wy(d["k"], d["v"], d["beta"], d["g_log"], L=w.L, n_h=n_h, chunk=chunk)
    torch.cuda.synchronize()
    ref = oracle.ut_factors(inp["k"], inp["v"], inp["beta"], inp["g_log"], n_h=n_h, chunk=chunk)
    for name in ("gc", "T", "W", "U"):
        got, want = to_np(f[name]), ref[name]
        err = np.abs(got - want).max() / max(np.abs(want).max(), 1e-30)
        say("  %s err %.3e" % (name, err))
        assert err < 1e-4, (name, err)


# ---------------------------------------------------------------- decode

def decode_sequence(w, S, steps, heads=None):
    """Run `steps` decode calls on the GPU from state S; return per-step O, final S (GPU) and the
    oracle's O and S_final for the same tokens taken as one sequence (optionally only `heads`)."""
    Sd = torch.from_numpy(S).cuda()
    Os, stack = [], []
    for step in range(steps):
        inp = W.make_decode_inputs(w, step)
        d = inputs_to_dev(dict(inp, S0=None), w.dtype)
        Os.append(to_np(D.decode(d["q"], d["k"], d["v"], d["beta"], d["g_log"], Sd, n_h=w.n_h)))
        stack.append(inp)
    torch.cuda.synchronize()
    cat = lambda key: None if stack[0][key] is None else np.concatenate([x[key] for x in stack], axis=1)
    q, k, v, beta, g = (cat(x) for x in ("q", "k", "v", "beta", "g_log"))
    O = np.concatenate(Os, axis=1)
    Sg = Sd.cpu().numpy()
    if heads is not None:
        bs = [b for b, _ in heads]
        hs = [h for _, h in heads]
        pick = lambda x: None if x is None else np.stack([x[b, :, h] for b, h in heads], 1)[None]
        q, k, v, beta, g = (pick(x) for x in (q, k, v, beta, g))
        S = np.stack([S[b, h] for b, h in heads])[None]
        O = np.stack([O[b, :, h] for b, h in heads], 1)[None]
        Sg = np.stack([Sg[b, h] for b, h in heads])[None]
    Or, Sr = oracle.fwd(q, k, v, beta, g, S, n_h=w.n_h)
    return O, Sg, Or, Sr


@pytest.mark.parametrize("dt,n_h,dk,dv,gate", [("f32", 1, 128, 128, "cfg3"), ("bf16", 1, 128, 128, "cfg3"),
                                               ("bf16", 2, 128, 128, "weak"), ("f32", 3, 64, 48, None),
                                               ("bf16", 1, 16, 16, "cfg3"), ("f32", 2, 32, 96, "weak")])
def test_decode_steps(dt, n_h, dk, dv, gate):
    w = W.Workload("dec", B=3, H=2, L=1, dk=dk, dv=dv, n_h=n_h, dtype=dt, gate=gate, s0=0.1, cfg_id=91,
                   key="silu_l2n" if n_h > 1 else "l2n", beta="2sigmoid" if n_h > 1 else "sigmoid")
    say("case decode", w)
    O, S, Or, Sr = decode_sequence(w, W.make_decode_state(w), steps=7)
    eo, es = head_rel_err(O, Or, (0, 2)), head_rel_err(S, Sr, (0, 1))
    say("  err O %.3e S %.3e" % (eo, es))
    assert eo <= TOL[dt] and es <= TOL[dt]


# ---------------------------------------------------------------- HIP graph capture

def test_decode_graph_replay():
    """Decode steps captured in a HIP graph: every replay (with eager work and synchronisation
    between replays) matches the same steps run eagerly."""
    w = W.Workload("dec_graph", B=4, H=2, L=1, dk=128, dv=128, dtype="bf16", gate="cfg3", s0=0.1, cfg_id=93)
    steps = [inputs_to_dev(dict(W.make_decode_inputs(w, t), S0=None), w.dtype) for t in range(3)]
    S0 = torch.from_numpy(W.make_decode_state(w)).cuda()
    Sg, Se = S0.clone(), S0.clone()
    Og = torch.empty((w.B, 1, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    Oe = torch.empty_like(Og)

    def run(S, O):
        for d in steps:
            D.decode(d["q"], d["k"], d["v"], d["beta"], d["g_log"], S, O=O)

    # warm the library up outside the capture, on a scratch state
    run(S0.clone(), torch.empty_like(Og))
    torch.cuda.synchronize()
    Sg.copy_(S0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(Sg, Og)
    Sg.copy_(S0)  # capture does not execute; start the replays from S0
    torch.cuda.synchronize()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        run(Se, Oe)
        torch.cuda.synchronize()
        es = (Sg - Se).abs().max().item()
        eo = (Og.float() - Oe.float()).abs().max().item()
        say("  replay %d: |S - S_eager| %.3e, |O - O_eager| %.3e" % (rep, es, eo))
        assert es == 0.0 and eo == 0.0, (rep, es, eo)


def test_fwd_graph_replay():
    """A whole forward pass (intra-chunk, summary, combine and output launches) captured in a HIP
    graph: every replay matches the eager call exactly."""
    w = wl("fwd_graph", B=1, H=2, L=1000, dk=128, dv=128, chunk=64, gate="cfg3", s0=0.1, cfg_id=94)
    d = inputs_to_dev(W.make_inputs(w), w.dtype)
    code = D.BF16
    ws = torch.empty(D.workspace_bytes(w.B, w.L, w.H, w.dk, w.dv, w.n_h, w.chunk, code), dtype=torch.uint8, device="cuda")
    Og = torch.empty((w.B, w.L, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    Sg = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    call = lambda O, S: D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], n_h=w.n_h, chunk=w.chunk,
                              O=O, S_final=S, workspace=ws)
    Oe, Se = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], n_h=w.n_h, chunk=w.chunk)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(Og, Sg)
    for rep in range(3):
        Og.zero_()
        Sg.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eo = (Og.float() - Oe.float()).abs().max().item()
        es = (Sg - Se).abs().max().item()
        say("  replay %d: |O - O_eager| %.3e, |S - S_eager| %.3e" % (rep, eo, es))
        assert eo == 0.0 and es == 0.0, (rep, eo, es)


# ---------------------------------------------------------------- KDA decode (per-channel decay)

def kda_sequence(w, S, steps):
    """`steps` KDA decode calls on the GPU from state S; returns per-step O and the final S, and
    the KDA oracle's O and S_final for the same tokens as one sequence."""
    Sd = torch.from_numpy(S).cuda()
    Os, stack, decays = [], [], []
    for step in range(steps):
        inp = W.make_decode_inputs(w, step)
        a = W.make_kda_decay(w, step)
        d = inputs_to_dev(dict(inp, S0=None), w.dtype)
        Os.append(to_np(D.decode_kda(d["q"], d["k"], d["v"], d["beta"], torch.from_numpy(a).cuda(), Sd, scale=0.9)))
        stack.append(inp)
        decays.append(a)
    torch.cuda.synchronize()
    cat = lambda key: np.concatenate([x[key] for x in stack], axis=1)
    Or, Sr = oracle.fwd_kda(cat("q"), cat("k"), cat("v"), cat("beta"), np.concatenate(decays, axis=1), S, scale=0.9)
    return np.concatenate(Os, axis=1), Sd.cpu().numpy(), Or, Sr


@pytest.mark.parametrize("dt,dk,dv", [("f32", 128, 128), ("bf16", 128, 128), ("bf16", 16, 16), ("f32", 64, 48),
                                      ("bf16", 32, 256)])
def test_decode_kda_steps(dt, dk, dv):
    w = W.Workload("kda", B=3, H=2, L=1, dk=dk, dv=dv, dtype=dt, gate="cfg3", s0=0.1, cfg_id=95)
    say("case kda decode", w)
    O, S, Or, Sr = kda_sequence(w, W.make_decode_state(w), steps=6)
    eo, es = head_rel_err(O, Or, (0, 2)), head_rel_err(S, Sr, (0, 1))
    say("  err O %.3e S %.3e" % (eo, es))
    assert eo <= TOL[dt] and es <= TOL[dt]


def test_decode_kda_equal_channels_is_gated_decode():
    """The same decay on every key channel is the scalar gate: delta_decode_kda with a_log = g
    for all channels gives exactly what delta_decode gives with log gate g."""
    w = W.Workload("kda_eq", B=2, H=3, L=1, dk=64, dv=64, dtype="bf16", gate="cfg3", s0=0.1, cfg_id=96)
    S0 = torch.from_numpy(W.make_decode_state(w)).cuda()
    S1, S2 = S0.clone(), S0.clone()
    for step in range(3):
        d = inputs_to_dev(dict(W.make_decode_inputs(w, step), S0=None), w.dtype)
        a = d["g_log"][..., None].expand(w.B, 1, w.H, w.dk).contiguous()
        O1 = D.decode(d["q"], d["k"], d["v"], d["beta"], d["g_log"], S1)
        O2 = D.decode_kda(d["q"], d["k"], d["v"], d["beta"], a, S2)
        torch.cuda.synchronize()
        assert torch.equal(O1, O2) and torch.equal(S1, S2), step
