"""GPU parity of the backward pass: delta_bwd (through the C ABI) against the fp64 oracle's
reverse-mode gradients (oracle_bwd) on the same seeded inputs and cotangents.

Bars (per-head relative error, tests/parity.py):
  - shapes whose per-chunk gradients run on the float32 vector ALUs (every float32 case, and bf16
    outside d_k = d_v = 128, chunk 64): 1e-4, the log-gate gradient (a sum of up to C * d_v
    products per token) 5e-4;
  - bf16 inputs with d_k = d_v = 128 and chunk 64, whose per-chunk gradients run on the bf16
    MFMA with float32 accumulation (states and intermediate tiles rounded to bf16 as operands):
    2e-2, the bar the forward pass holds bf16 inputs to."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import head_rel_err, inputs_to_dev, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import chunkwise_delta_rule_chunked_amd as D  # noqa: E402

TOL = 1e-4
TOL_G = 5e-4
AXES = {"dq": (0, 2), "dk": (0, 2), "dv": (0, 2), "dbeta": (0, 2), "dg_log": (0, 2), "dS0": (0, 1)}


def wl(name, **kw):
    base = dict(B=2, H=2, L=100, dk=64, dv=64, chunk=32, dtype="bf16", cfg_id=91)
    base.update(kw)
    return W.Workload(name, **base)


CASES = [
    wl("bwd_f32_deltanet", dtype="f32", L=70, dk=32, dv=32, chunk=16),
    wl("bwd_f32_gated_ragged", dtype="f32", L=77, dk=32, dv=48, chunk=32, gate="weak", s0=0.1),
    wl("bwd_f32_dp3_c48", dtype="f32", L=50, dk=64, dv=16, chunk=48, n_h=3, gate="cfg3", key="silu_l2n",
       beta="2sigmoid", s0=0.1),
    wl("bwd_f32_d128_c64", dtype="f32", B=1, L=130, dk=128, dv=128, chunk=64, gate="cfg3", s0=0.1),
    wl("bwd_f32_dk16_dv256_dp2", dtype="f32", B=1, H=3, L=41, dk=16, dv=256, chunk=16, n_h=2, gate="weak"),
    wl("bwd_bf16_gdn_d128", B=2, H=2, L=333, dk=128, dv=128, chunk=64, gate="cfg3", s0=0.1),
    wl("bwd_bf16_gdp2_d128", B=1, H=2, L=300, dk=128, dv=128, chunk=64, n_h=2, gate="weak",
       key="silu_l2n", beta="2sigmoid"),
    wl("bwd_bf16_one_chunk", B=1, H=1, L=5, dk=64, dv=32, chunk=64, gate="cfg3"),
    # the state scans' segment split: none (256 heads fill the GPU), one chunk per segment over
    # 41 chunks (40 combine steps, a ragged last chunk), ungated with a start state
    wl("bwd_bf16_d128_unsplit", B=2, H=128, L=70, dk=128, dv=128, chunk=64, gate="cfg3", s0=0.1),
    wl("bwd_bf16_d128_41_segments", B=1, H=1, L=64 * 40 + 17, dk=128, dv=128, chunk=64, gate="weak", s0=0.1),
    wl("bwd_bf16_d128_ungated", B=1, H=3, L=200, dk=128, dv=128, chunk=64, s0=0.1),
]


def run(w, inp, cot, chunk=None, scale=1.0, with_dS=True):
    d = inputs_to_dev(inp, w.dtype)
    dO = to_dev(cot["dO"], w.dtype)
    dS = to_dev(cot["dS_final"], "f32") if with_dS else None
    g = D.bwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], dO, dS, n_h=w.n_h,
              chunk=chunk or w.chunk, scale=scale)
    torch.cuda.synchronize()
    return {n: (None if t is None else t.cpu().numpy()) for n, t in g.items()}


def mfma_path(w, chunk=None):
    return w.dtype == "bf16" and w.dk == 128 and w.dv == 128 and (chunk or w.chunk) == 64


def compare(got, want, tol=TOL, tol_g=TOL_G):
    errs = {}
    for n, ax in AXES.items():
        if want[n] is None:
            assert got[n] is None, n
            continue
        assert got[n] is not None and np.isfinite(got[n]).all(), n
        errs[n] = head_rel_err(got[n], want[n], ax)
    say("  errs " + "  ".join("%s %.2e" % kv for kv in errs.items()))
    for n, e in errs.items():
        assert e <= (tol_g if n == "dg_log" else tol), (n, e)
    return errs


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_bwd_matches_oracle(w):
    say("case", w)
    inp, cot = W.make_inputs(w), W.make_cotangents(w)
    got = run(w, inp, cot, scale=0.7)
    want = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g_log"], inp["S0"], cot["dO"],
                      cot["dS_final"], n_h=w.n_h, scale=0.7)
    compare(got, want, *((2e-2, 2e-2) if mfma_path(w) else (TOL, TOL_G)))


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_bwd_chunk_independent(chunk):
    # results do not depend on the chunk length beyond rounding
    w = wl("bwd_chunks", dtype="f32", B=1, L=90, dk=32, dv=32, gate="cfg3", s0=0.2)
    inp, cot = W.make_inputs(w), W.make_cotangents(w)
    say("case", w, "chunk", chunk)
    want = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g_log"], inp["S0"], cot["dO"],
                      cot["dS_final"], n_h=1)
    compare(run(w, inp, cot, chunk=chunk), want)


def test_bwd_without_state_gradient():
    w = wl("bwd_no_dS", dtype="f32", B=1, L=64, dk=32, dv=32, chunk=32, gate="cfg3")
    inp, cot = W.make_inputs(w), W.make_cotangents(w)
    say("case", w)
    want = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g_log"], inp["S0"], cot["dO"],
                      None, n_h=1)
    compare(run(w, inp, cot, with_dS=False), want)


def test_bwd_zero_beta_passes_state_through():
    # beta = 0 everywhere: nothing is written, the state only decays; dv and dk vanish exactly
    # while dbeta does not
    w = wl("bwd_beta0", dtype="f32", B=1, L=40, dk=32, dv=32, chunk=16, gate="cfg3", beta="zero", s0=0.5)
    inp, cot = W.make_inputs(w), W.make_cotangents(w)
    say("case", w)
    got = run(w, inp, cot)
    want = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g_log"], inp["S0"], cot["dO"],
                      cot["dS_final"], n_h=1)
    compare(got, want)
    assert np.abs(got["dv"]).max() == 0.0 and np.abs(got["dk"]).max() == 0.0
    assert np.abs(got["dbeta"]).max() > 0.0


def test_bwd_empty_sequence():
    # L = 0: no chunks; dS0 = dS_final
    w = wl("bwd_empty", dtype="f32", B=2, H=2, L=0, dk=32, dv=32, chunk=16, gate="cfg3", s0=0.1)
    inp, cot = W.make_inputs(w), W.make_cotangents(w)
    say("case", w)
    got = run(w, inp, cot)
    assert np.array_equal(got["dS0"], cot["dS_final"])


@pytest.mark.parametrize("hb", [(0, 0), (0, 3), (1, 14), (1, 15)])
def test_bwd_full_size_sampled_heads(hb):
    # the prefill workload at full size, one launch for all heads; the oracle on two sampled heads
    w = W.get("gdn_b2h16_l8k")
    inp, cot = W.make_inputs(w), W.make_cotangents(w)
    b, h = hb
    say("case", w.name, "head", hb)
    got = run(w, inp, cot)
    sl = lambda x: None if x is None else x[b:b + 1, :, h:h + 1]
    want = oracle.bwd(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta"]), sl(inp["g_log"]),
                      None if inp["S0"] is None else inp["S0"][b:b + 1, h:h + 1], sl(cot["dO"]),
                      cot["dS_final"][b:b + 1, h:h + 1], n_h=w.n_h)
    sub = {n: (None if v is None else (v[b:b + 1, h:h + 1] if n == "dS0" else v[b:b + 1, :, h:h + 1]))
           for n, v in got.items()}
    compare(sub, want, *((2e-2, 2e-2) if mfma_path(w) else (TOL, TOL_G)))
