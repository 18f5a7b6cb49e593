"""Parity at the full workload sizes, in the launch configuration the benchmark times.
The oracle runs on a sample of (b, h) sequences (each sequence is independent, so its
outputs are exact samples of the full result); the GPU runs the whole workload."""
import numpy as np
import pytest

import workloads as W
from parity import TOL, head_rel_err, say
from test_parity_gpu import check, decode_sequence

pytestmark = pytest.mark.gpu

FULL = ["deltanet_b4h8_l2k", "gdn_b2h16_l8k", "gdp2_b2h16_l4k", "gdn_b1h16_l64k"]


@pytest.mark.parametrize("name", FULL)
def test_full_workload_sampled_heads(name):
    w = W.CONFIGS[name]
    inp = W.make_inputs(w)
    BH = w.B * w.H
    n = 2 if w.L >= 65536 else 4
    idx = sorted({0, BH - 1} | set(np.random.default_rng(7).choice(BH, n, replace=False).tolist()))[:n + 1]
    heads = [(i // w.H, i % w.H) for i in idx]
    say("heads", heads)
    check(w, inp, heads=heads)


def test_tiny_config_whole():
    w = W.CONFIGS["tiny_deltanet_f32"]
    check(w, W.make_inputs(w))


def test_decode_full_256_steps_sampled_heads():
    w = W.DECODE
    heads = [(0, 0), (17, 5), (40, 9), (63, 15)]
    say("case decode full", w, heads)
    O, S, Or, Sr = decode_sequence(w, W.make_decode_state(w), steps=W.DECODE_STEPS, heads=heads)
    eo, es = head_rel_err(O, Or, (0, 2)), head_rel_err(S, Sr, (0, 1))
    say("  err O %.3e S %.3e" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
