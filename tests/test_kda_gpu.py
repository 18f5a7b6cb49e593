"""GPU parity of the KDA forward over a sequence (delta_fwd_kda, the token recurrence with a decay
per key channel) against the fp64 oracle (oracle.fwd_kda), through the C ABI.  Bar as for the
scalar-gated path: per-head relative error <= 1e-4 (float32 inputs), <= 2e-2 (bf16 inputs)."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import TOL, head_rel_err, inputs_to_dev, say, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import chunkwise_delta_rule_chunked_amd as D  # noqa: E402


def kda_case(name, **kw):
    base = dict(B=2, H=2, L=100, dk=64, dv=64, dtype="bf16", gate="cfg3", s0=0.1, cfg_id=110)
    base.update(kw)
    return W.Workload(name, **base)


def run_kda(w, inp, a, scale=1.0, S_final=None):
    d = inputs_to_dev(inp, w.dtype)
    ad = torch.from_numpy(a).cuda()
    O, S = D.fwd_kda(d["q"], d["k"], d["v"], d["beta"], ad, d["S0"] if S_final is None else S_final,
                     scale=scale, S_final=S_final)
    torch.cuda.synchronize()
    return to_np(O), to_np(S)


def check_kda(w, inp=None, a=None, scale=1.0, tol=None):
    inp = inp if inp is not None else W.make_inputs(w)
    a = a if a is not None else W.make_kda_decays(w)
    say("case kda", w)
    O, S = run_kda(w, inp, a, scale)
    Or, Sr = oracle.fwd_kda(inp["q"], inp["k"], inp["v"], inp["beta"], a, inp["S0"], scale=scale)
    eo, es = head_rel_err(O, Or, (0, 2)), head_rel_err(S, Sr, (0, 1))
    say("  err O %.3e S %.3e" % (eo, es))
    assert np.isfinite(O).all() and np.isfinite(S).all()
    tol = tol if tol is not None else TOL[w.dtype]
    assert eo <= tol and es <= tol, (eo, es)


CASES = [
    kda_case("kda_f32_d128", dtype="f32", B=1, L=300, dk=128, dv=128),
    kda_case("kda_bf16_d128", B=2, L=333, dk=128, dv=128),
    kda_case("kda_bf16_weak", B=1, L=700, dk=128, dv=128, gate="weak"),
    kda_case("kda_f32_dk16_dv256", dtype="f32", B=2, L=77, dk=16, dv=256),
    kda_case("kda_bf16_dk32_dv48", B=3, H=1, L=65, dk=32, dv=48, s0=None),
    kda_case("kda_f32_dk64_dv16", dtype="f32", B=1, H=3, L=17, dk=64, dv=16),
    kda_case("kda_bf16_L1", B=2, H=2, L=1, dk=128, dv=32),
    kda_case("kda_f32_L16", dtype="f32", B=1, H=1, L=16, dk=32, dv=32, gate="weak"),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_kda_fwd(w):
    check_kda(w, scale=0.9)


def test_kda_long_sequence():
    """8192 tokens with the weak decay (the state carries far): the chain of 8K dependent steps
    stays within the bar."""
    check_kda(kda_case("kda_long", B=1, H=2, L=8192, dk=128, dv=128, gate="weak"))


def test_kda_full_shape_all_heads():
    """The 32-head, 8K-token shape of the Gated DeltaNet workload with per-channel decays, every
    head against the oracle."""
    check_kda(kda_case("kda_b2h16_l8k", B=2, H=16, L=8192, dk=128, dv=128, cfg_id=3))


def test_kda_channel_resets():
    """log alpha = -inf on single channels and on whole tokens: the channel's state rows (or the
    whole state) are erased before the write, exactly as in the oracle."""
    w = kda_case("kda_reset", B=1, H=2, L=200, dk=64, dv=64, gate="weak", dtype="f32")
    a = W.make_kda_decays(w)
    a[0, 50, 0, 7] = -np.inf
    a[0, 120, 1, :] = -np.inf
    check_kda(w, a=a)


def test_kda_equal_channels_matches_scalar_gate():
    """The same decay on every channel is Gated DeltaNet ("08 linear delta rule & DPLR", section
    1.4 table): delta_fwd_kda with a_log = g broadcast agrees with the oracle's scalar-gated run and,
    within the bar, with the chunkwise delta_fwd on the same inputs."""
    w = kda_case("kda_eq", B=1, H=2, L=500, dk=128, dv=128, gate="weak")
    inp = W.make_inputs(w)
    a = np.repeat(inp["g_log"][..., None], w.dk, axis=-1)
    O, S = run_kda(w, inp, a)
    Or, Sr = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g_log"], inp["S0"])
    assert head_rel_err(O, Or, (0, 2)) <= TOL["bf16"] and head_rel_err(S, Sr, (0, 1)) <= TOL["bf16"]
    d = inputs_to_dev(inp, w.dtype)
    Oc, Sc = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], chunk=64)
    torch.cuda.synchronize()
    assert head_rel_err(O, to_np(Oc).astype(np.float64), (0, 2)) <= TOL["bf16"]


def test_kda_in_place_and_empty():
    w = kda_case("kda_inplace", B=1, H=2, L=90, dk=64, dv=64, dtype="f32")
    inp, a = W.make_inputs(w), W.make_kda_decays(w)
    O1, S1 = run_kda(w, inp, a)
    Sin = torch.from_numpy(inp["S0"]).cuda()
    O2, S2 = run_kda(w, inp, a, S_final=Sin)
    assert np.array_equal(O1, O2) and np.array_equal(S1, S2) and np.array_equal(Sin.cpu().numpy(), S1)
    # L = 0: S_final = S0
    w0 = w.replace(L=0)
    inp0 = W.make_inputs(w0)
    d = inputs_to_dev(inp0, "f32")
    O, S = D.fwd_kda(d["q"], d["k"], d["v"], d["beta"], torch.zeros((1, 0, 2, 64), device="cuda"), d["S0"])
    torch.cuda.synchronize()
    assert O.numel() == 0 and np.array_equal(S.cpu().numpy(), inp0["S0"])


def test_kda_prefill_then_decode():
    """A prefill of 200 tokens followed by 5 decode steps (delta_decode_kda on the returned state)
    continues the same recurrence: the oracle over all 205 tokens agrees with both."""
    w = kda_case("kda_pd", B=2, H=2, L=205, dk=64, dv=64, dtype="f32", gate="weak")
    inp, a = W.make_inputs(w), W.make_kda_decays(w)
    d = inputs_to_dev(inp, "f32")
    ad = torch.from_numpy(a).cuda()
    P = 200
    O1, S = D.fwd_kda(d["q"][:, :P].contiguous(), d["k"][:, :P].contiguous(), d["v"][:, :P].contiguous(),
                      d["beta"][:, :P].contiguous(), ad[:, :P].contiguous(), d["S0"])
    outs = [to_np(O1)]
    for t in range(P, w.L):
        sl = lambda x: x[:, t:t + 1].contiguous()
        outs.append(to_np(D.decode_kda(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["beta"]), sl(ad), S)))
    torch.cuda.synchronize()
    Or, Sr = oracle.fwd_kda(inp["q"], inp["k"], inp["v"], inp["beta"], a, inp["S0"])
    assert head_rel_err(np.concatenate(outs, axis=1), Or, (0, 2)) <= TOL["f32"]
    assert head_rel_err(S.cpu().numpy(), Sr, (0, 1)) <= TOL["f32"]


# ---------------------------------------------------------------- KDA in chunks
def run_kda_chunked(w, inp, a, scale=1.0, S_final=None):
    d = inputs_to_dev(inp, w.dtype)
    ad = torch.from_numpy(a).cuda()
    O, S = D.fwd_kda_chunked(d["q"], d["k"], d["v"], d["beta"], ad, d["S0"] if S_final is None else S_final,
                             scale=scale, S_final=S_final)
    torch.cuda.synchronize()
    return to_np(O), to_np(S)


def check_kda_chunked(w, inp=None, a=None, scale=1.0):
    """delta_fwd_kda_chunked against the oracle (bar 2e-2, bf16 inputs) and against the token
    recurrence delta_fwd_kda on the same inputs (same bar)."""
    inp = inp if inp is not None else W.make_inputs(w)
    a = a if a is not None else W.make_kda_decays(w)
    say("case kda chunked", w, "segments", D.segments(w.B, w.L, w.H, w.dk, w.dv))
    O, S = run_kda_chunked(w, inp, a, scale)
    Or, Sr = oracle.fwd_kda(inp["q"], inp["k"], inp["v"], inp["beta"], a, inp["S0"], scale=scale)
    eo, es = head_rel_err(O, Or, (0, 2)), head_rel_err(S, Sr, (0, 1))
    Ot, St = run_kda(w, inp, a, scale)
    et = head_rel_err(O, Ot.astype(np.float64), (0, 2))
    say("  err O %.3e S %.3e; against the recurrence %.3e" % (eo, es, et))
    assert np.isfinite(O).all() and np.isfinite(S).all()
    assert eo <= TOL["bf16"] and es <= TOL["bf16"] and et <= TOL["bf16"], (eo, es, et)


CHUNKED = [
    kda_case("kdac_bf16_333", B=2, L=333, dk=128, dv=128),
    kda_case("kdac_weak_700", B=1, L=700, dk=128, dv=128, gate="weak"),
    kda_case("kdac_one_chunk", B=2, H=3, L=64, dk=128, dv=128, s0=None),
    kda_case("kdac_short", B=1, L=5, dk=128, dv=128),
    # the scan's segment split: none (256 heads fill the GPU), and 41 one-chunk segments
    kda_case("kdac_unsplit", B=2, H=128, L=70, dk=128, dv=128),
    kda_case("kdac_41_segments", B=1, H=1, L=64 * 40 + 17, dk=128, dv=128, gate="weak"),
]


@pytest.mark.parametrize("w", CHUNKED, ids=lambda w: w.name)
def test_kda_chunked(w):
    check_kda_chunked(w, scale=0.9)


def test_kda_chunked_full_shape_all_heads():
    check_kda_chunked(kda_case("kda_b2h16_l8k", B=2, H=16, L=8192, dk=128, dv=128, cfg_id=3))


def test_kda_chunked_decay_spans_around_the_diagonal_bound():
    """Decays 1.9 times the default (about 65 nats over 16 tokens on average per channel): the
    intra kernel's diagonal blocks take the MFMA route or the entry-by-entry one, block by block,
    both against the oracle."""
    w = kda_case("kdac_spans", B=1, H=4, L=500, dk=128, dv=128)
    check_kda_chunked(w, a=W.make_kda_decays(w) * np.float32(1.9))


def test_kda_chunked_resets_and_in_place():
    """log alpha = -inf on one channel, on a whole token at a chunk start and mid-chunk: exact
    erasure as in the oracle; then S_final = S0 in place gives the same O and state."""
    w = kda_case("kdac_reset", B=1, H=2, L=300, dk=128, dv=128, gate="weak")
    inp, a = W.make_inputs(w), W.make_kda_decays(w)
    a[0, 50, 0, 7] = -np.inf
    a[0, 128, 1, :] = -np.inf
    a[0, 201, 0, :] = -np.inf
    check_kda_chunked(w, inp=inp, a=a)
    O1, S1 = run_kda_chunked(w, inp, a)
    Sin = torch.from_numpy(inp["S0"]).cuda()
    O2, S2 = run_kda_chunked(w, inp, a, S_final=Sin)
    assert np.array_equal(O1, O2) and np.array_equal(S1, S2) and np.array_equal(Sin.cpu().numpy(), S1)


def test_kda_chunked_nan_workspace_is_ignored():
    """A workspace filled with NaN gives the same result, bit for bit, as a zeroed one (every
    workspace byte the launches read is written first in the same call)."""
    w = kda_case("kdac_ws", B=1, H=4, L=700, dk=128, dv=128, gate="weak")
    inp, a = W.make_inputs(w), W.make_kda_decays(w)
    d = inputs_to_dev(inp, w.dtype)
    ad = torch.from_numpy(a).cuda()
    nbytes = D.kda_chunked_workspace_bytes(w.B, w.L, w.H)
    res = []
    for fill in (0.0, float("nan")):
        ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(fill)
        res.append(D.fwd_kda_chunked(d["q"], d["k"], d["v"], d["beta"], ad, d["S0"], workspace=ws))
    torch.cuda.synchronize()
    (O0, S0), (O1, S1) = res
    assert torch.isfinite(O1.float()).all() and torch.isfinite(S1).all()
    assert torch.equal(O0, O1) and torch.equal(S0, S1)


@pytest.mark.parametrize("where", ["v", "a_log"])
def test_kda_chunked_nan_propagates(where):
    """NaN in one value, or in one channel's log decay, of head 1 at token t reaches that head's
    output at t and at the end, and its final state; head 0, and head 1's tokens before t's chunk,
    stay finite (inside the chunk it may reach earlier tokens: the zeros above the diagonal of T
    and Aqk multiply it)."""
    w = kda_case("kdac_nan", B=1, H=2, L=300, dk=128, dv=128, gate="weak")
    inp, a = W.make_inputs(w), W.make_kda_decays(w)
    t = 150
    if where == "v":
        v = inp["v"].copy()
        v[0, t, 1, 5] = np.nan
        inp = dict(inp, v=v)
    else:
        a[0, t, 1, 7] = np.nan
    O, S = run_kda_chunked(w, inp, a)
    assert np.isfinite(O[0, :, 0]).all() and np.isfinite(S[0, 0]).all()
    assert np.isfinite(O[0, :t // 64 * 64, 1]).all()
    assert np.isnan(O[0, t, 1]).any() and np.isnan(O[0, -1, 1]).any() and np.isnan(S[0, 1]).any()


@pytest.mark.parametrize("what", ["nan_decay", "posinf_decay", "nan_beta", "ok_neginf_decay"])
def test_kda_chunked_validate(monkeypatch, what):
    """With DELTA_VALIDATE=1, a NaN or +inf log decay or a non-finite beta returns
    DELTA_ERR_BAD_VALUE (-8) and leaves the outputs untouched; a -inf log decay (a reset) passes."""
    w = kda_case("kdac_validate", B=1, H=2, L=300, dk=128, dv=128, gate="weak")
    inp, a = W.make_inputs(w), W.make_kda_decays(w)
    beta = inp["beta"].copy()
    if what == "nan_decay":
        a[0, 217, 1, 9] = np.nan
    elif what == "posinf_decay":
        a[0, 217, 1, 9] = np.inf
    elif what == "nan_beta":
        beta[0, 217, 1] = np.nan
    else:
        a[0, 217, 1, 9] = -np.inf
    d = inputs_to_dev(dict(inp, beta=beta), w.dtype)
    ad = torch.from_numpy(a).cuda()
    O = torch.full((w.B, w.L, w.H, w.dv), 7.0, dtype=torch.bfloat16, device="cuda")
    S = torch.full((w.B, w.H, w.dk, w.dv), 7.0, dtype=torch.float32, device="cuda")
    monkeypatch.setenv("DELTA_VALIDATE", "1")
    if what == "ok_neginf_decay":
        D.fwd_kda_chunked(d["q"], d["k"], d["v"], d["beta"], ad, d["S0"], O=O, S_final=S)
        torch.cuda.synchronize()
        assert torch.isfinite(O.float()).all() and torch.isfinite(S).all()
        return
    with pytest.raises(D.DeltaError) as e:
        D.fwd_kda_chunked(d["q"], d["k"], d["v"], d["beta"], ad, d["S0"], O=O, S_final=S)
    torch.cuda.synchronize()
    assert e.value.code == -8
    assert bool((O.float() == 7.0).all()) and bool((S == 7.0).all())
