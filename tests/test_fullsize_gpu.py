"""Parity at the full workload sizes, in the launch configuration the benchmark times: every
(b, h) sequence of every output is compared with the oracle (OpenMP over the sequences on the
host cores; the largest workload takes about a second there)."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import TOL, head_rel_err, inputs_to_dev, say, to_np
from test_parity_gpu import check, decode_sequence

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import chunkwise_delta_rule_chunked_amd as D  # noqa: E402

FULL = ["deltanet_b4h8_l2k", "gdn_b2h16_l8k", "gdp2_b2h16_l4k", "gdn_b1h16_l64k"]


@pytest.mark.parametrize("name", FULL)
def test_full_workload_all_heads(name):
    w = W.CONFIGS[name]
    check(w, W.make_inputs(w))


def test_full_workload_in_place_state():
    """The metric workload with S_final == S0 (the state updated in place; 8 segments per
    sequence): the same bits as with a separate S_final, and within the bar of the oracle."""
    w = W.CONFIGS["gdn_b2h16_l8k"]
    inp = W.make_inputs(w)
    d = inputs_to_dev(inp, w.dtype)
    O1, S1 = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], chunk=w.chunk)
    Sin = d["S0"].clone()
    O2, S2 = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], Sin, chunk=w.chunk, S_final=Sin)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(S1, S2)


def test_tiny_config_whole():
    w = W.CONFIGS["tiny_deltanet_f32"]
    check(w, W.make_inputs(w))


def test_decode_full_256_steps_all_heads():
    w = W.DECODE
    say("case decode full", w)
    O, S, Or, Sr = decode_sequence(w, W.make_decode_state(w), steps=W.DECODE_STEPS)
    eo, es = head_rel_err(O, Or, (0, 2)), head_rel_err(S, Sr, (0, 1))
    say("  err O %.3e S %.3e" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
