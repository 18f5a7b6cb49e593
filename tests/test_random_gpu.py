"""Seeded random sweep of the shape space through the C ABI, against the fp64 oracle.

The hand-picked cases in the other parity files each pin one feature; this file draws whole
configurations at random (fixed seed, so every case is reproducible by its name): both dtypes,
every d_k, d_v from 16 to 256 in steps of 16, every chunk length, 1 to 4 Householder steps per
token where the chunk allows, ragged lengths from a single token up, no gate / a weak gate / the
prefill workloads' gate, start states or none, beta in (0, 1) or (0, 2).  The forward pass is
compared on every draw and the backward pass on the first BWD_CASES of them, each at the bar the
rest of the suite holds that route to (tests/parity.py, tests/test_bwd_gpu.py).  The KDA forward
over a sequence and the two decode steps get draws of their own shape ranges.  Sizes stay small
enough for the oracle to take well under a second per case."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import TOL, head_rel_err, inputs_to_dev, say, to_dev, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import chunkwise_delta_rule_chunked_amd as D  # noqa: E402

SEED = 20261202
FWD_CASES = 32
BWD_CASES = 16


def draw_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = ("f32", "bf16")[int(rng.integers(2))]
        dk = int(rng.choice([16, 32, 64, 128]))
        dv = 16 * int(rng.integers(1, 17))
        chunk = int(rng.choice([16, 32, 48, 64]))
        steps = [h for h in (1, 2, 3, 4) if chunk % h == 0]
        n_h = int(steps[0] if rng.random() < 0.5 else rng.choice(steps))
        L = int(rng.integers(1, 240 // n_h + 1))
        gate = (None, "weak", "cfg3")[int(rng.integers(3))]
        key = "silu_l2n" if n_h > 1 else "l2n"
        beta = "2sigmoid" if n_h > 1 or rng.random() < 0.3 else "sigmoid"
        s0 = 0.1 if rng.random() < 0.5 else None
        name = "r%02d_%s_dk%d_dv%d_c%d_nh%d_L%d_%s%s" % (i, dtype, dk, dv, chunk, n_h, L, gate or "ungated",
                                                         "_s0" if s0 else "")
        cases.append(W.Workload(name, B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), L=L, dk=dk, dv=dv,
                                n_h=n_h, chunk=chunk, dtype=dtype, gate=gate, key=key, beta=beta, s0=s0,
                                cfg_id=300 + i))
    return cases


CASES = draw_cases(FWD_CASES, SEED)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_random_fwd(w):
    say("case", w)
    inp = W.make_inputs(w)
    d = inputs_to_dev(inp, w.dtype)
    O, S = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], n_h=w.n_h, chunk=w.chunk)
    torch.cuda.synchronize()
    O, S = to_np(O), to_np(S)
    Or, Sr = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g_log"], inp["S0"], n_h=w.n_h)
    eo, es = head_rel_err(O, Or, (0, 2)), head_rel_err(S, Sr, (0, 1))
    say("  err O %.3e  S %.3e" % (eo, es))
    assert np.isfinite(O).all() and np.isfinite(S).all()
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype], (eo, es)


BWD_AXES = {"dq": (0, 2), "dk": (0, 2), "dv": (0, 2), "dbeta": (0, 2), "dg_log": (0, 2), "dS0": (0, 1)}


@pytest.mark.parametrize("w", CASES[:BWD_CASES], ids=lambda w: w.name)
def test_random_bwd(w):
    say("case", w)
    inp, cot = W.make_inputs(w), W.make_cotangents(w)
    d = inputs_to_dev(inp, w.dtype)
    g = D.bwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], to_dev(cot["dO"], w.dtype),
              to_dev(cot["dS_final"], "f32"), n_h=w.n_h, chunk=w.chunk)
    torch.cuda.synchronize()
    want = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g_log"], inp["S0"], cot["dO"],
                      cot["dS_final"], n_h=w.n_h)
    # bf16 inputs at d_k = d_v = 128, chunk 64 take the bf16-MFMA route (2e-2); every other shape
    # the float32 vector-ALU route (1e-4, the log-gate gradient 5e-4)
    mfma = w.dtype == "bf16" and w.dk == 128 and w.dv == 128 and w.chunk == 64
    errs = {}
    for n, ax in BWD_AXES.items():
        if want[n] is None:
            assert g[n] is None, n
            continue
        got = g[n].cpu().numpy()
        assert np.isfinite(got).all(), n
        errs[n] = head_rel_err(got, want[n], ax)
    say("  errs " + "  ".join("%s %.2e" % kv for kv in errs.items()))
    for n, e in errs.items():
        bar = 2e-2 if mfma else (5e-4 if n == "dg_log" else 1e-4)
        assert e <= bar, (n, e)


# ---------------------------------------------------------------- KDA recurrence and decode steps

def draw_kda(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = ("f32", "bf16")[int(rng.integers(2))]
        dk, dv = int(rng.choice([16, 32, 64, 128])), 16 * int(rng.integers(1, 17))
        L = int(rng.integers(1, 241))
        gate = ("weak", "cfg3")[int(rng.integers(2))]
        s0 = 0.1 if rng.random() < 0.5 else None
        out.append(W.Workload("k%02d_%s_dk%d_dv%d_L%d_%s%s" % (i, dtype, dk, dv, L, gate, "_s0" if s0 else ""),
                              B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), L=L, dk=dk, dv=dv,
                              dtype=dtype, gate=gate, s0=s0, cfg_id=400 + i))
    return out


@pytest.mark.parametrize("w", draw_kda(10, SEED + 1), ids=lambda w: w.name)
def test_random_kda_fwd(w):
    from test_kda_gpu import check_kda
    check_kda(w, scale=0.9)


def draw_decode(n, seed, kda):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = ("f32", "bf16")[int(rng.integers(2))]
        dk, dv = int(rng.choice([16, 32, 64, 128])), 16 * int(rng.integers(1, 17))
        n_h = 1 if kda or rng.random() < 0.5 else int(rng.integers(2, 5))
        gate = (None, "weak", "cfg3")[int(rng.integers(1 if kda else 0, 3))]
        steps = int(rng.integers(1, 9))
        out.append((W.Workload("d%02d_%s_%s_dk%d_dv%d_nh%d_%s" % (i, "kda" if kda else "gdn", dtype, dk, dv, n_h,
                                                                 gate or "ungated"),
                               B=int(rng.integers(1, 5)), H=int(rng.integers(1, 4)), L=1, dk=dk, dv=dv, n_h=n_h,
                               dtype=dtype, gate=gate, s0=0.1, cfg_id=500 + 50 * kda + i,
                               key="silu_l2n" if n_h > 1 else "l2n", beta="2sigmoid" if n_h > 1 else "sigmoid"),
                    steps))
    return out


@pytest.mark.parametrize("w,steps", draw_decode(8, SEED + 2, False), ids=lambda x: getattr(x, "name", str(x)))
def test_random_decode(w, steps):
    from test_parity_gpu import decode_sequence
    say("case decode", w, "steps", steps)
    O, S, Or, Sr = decode_sequence(w, W.make_decode_state(w), steps=steps)
    eo, es = head_rel_err(O, Or, (0, 2)), head_rel_err(S, Sr, (0, 1))
    say("  err O %.3e  S %.3e" % (eo, es))
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype], (eo, es)


@pytest.mark.parametrize("w,steps", draw_decode(6, SEED + 3, True), ids=lambda x: getattr(x, "name", str(x)))
def test_random_decode_kda(w, steps):
    from test_parity_gpu import kda_sequence
    say("case kda decode", w, "steps", steps)
    O, S, Or, Sr = kda_sequence(w, W.make_decode_state(w), steps=steps)
    eo, es = head_rel_err(O, Or, (0, 2)), head_rel_err(S, Sr, (0, 1))
    say("  err O %.3e  S %.3e" % (eo, es))
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype], (eo, es)
