"""delta_fwd_noalloc (the forward pass with its workspace in the library's fixed device array)
against delta_fwd with a caller workspace, through the C ABI: two calls in a row, the second on a
smaller problem, each bitwise equal to delta_fwd and within the bar of the oracle; and shapes
beyond the fixed array rejected before any work."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as W
from parity import TOL, head_rel_err, inputs_to_dev, say, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import chunkwise_delta_rule_chunked_amd as D  # noqa: E402


def run_pair(w):
    """(O, S) from delta_fwd_noalloc and from delta_fwd on the same inputs."""
    inp = W.make_inputs(w)
    d = inputs_to_dev(inp, w.dtype)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    code = D.BF16 if w.dtype == "bf16" else D.F32
    need = D.workspace_bytes(w.B, w.L, w.H, w.dk, w.dv, w.n_h, w.chunk, code)
    assert need <= D.NOALLOC_MAX_BYTES
    On = torch.empty((w.B, w.L, w.H, w.dv), dtype=dt, device="cuda")
    Sn = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    sh = D.make_shape(w.B, w.L, w.H, w.dk, w.dv, w.n_h, w.chunk, code, 1.0)
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    rc = D.load_library().delta_fwd_noalloc(ctypes.byref(sh), ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(d["beta"]),
                                            ptr(d["g_log"]), ptr(d["S0"]), ptr(On), ptr(Sn),
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, D.strerror(rc)
    Of, Sf = D.fwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], n_h=w.n_h, chunk=w.chunk)
    torch.cuda.synchronize()
    return inp, (On, Sn), (Of, Sf), need


def test_two_calls_second_smaller():
    big = W.CONFIGS["gdn_b2h16_l8k"]              # the metric workload: 81 MiB of workspace, 8 segments
    small = W.Workload("noalloc_small", B=1, H=3, L=333, dk=64, dv=96, n_h=2, chunk=32, dtype="bf16",
                       gate="weak", key="silu_l2n", beta="2sigmoid", s0=0.1, cfg_id=99)
    for w in (big, small):
        inp, (On, Sn), (Of, Sf), need = run_pair(w)
        say("case noalloc", w.name, "workspace %.1f MiB" % (need / 2**20))
        assert torch.equal(On, Of) and torch.equal(Sn, Sf)
        Or, Sr = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g_log"], inp["S0"], n_h=w.n_h)
        eo, es = head_rel_err(to_np(On), Or, (0, 2)), head_rel_err(to_np(Sn), Sr, (0, 1))
        say("  err O %.3e S %.3e" % (eo, es))
        assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


def test_f32_and_unsplit():
    for w in (W.CONFIGS["tiny_deltanet_f32"],
              W.Workload("noalloc_unsplit", B=32, H=8, L=130, dk=32, dv=32, chunk=32, dtype="bf16", gate="cfg3",
                         s0=0.1, cfg_id=99)):
        _, (On, Sn), (Of, Sf), _ = run_pair(w)
        assert torch.equal(On, Of) and torch.equal(Sn, Sf)


def test_too_large_rejected():
    w = W.CONFIGS["gdn_b1h16_l64k"]                # 180 MiB of workspace
    need = D.workspace_bytes(w.B, w.L, w.H, w.dk, w.dv, w.n_h, w.chunk, D.BF16)
    assert need > D.NOALLOC_MAX_BYTES
    sh = D.make_shape(w.B, w.L, w.H, w.dk, w.dv, w.n_h, w.chunk, D.BF16, 1.0)
    rc = D.load_library().delta_fwd_noalloc(ctypes.byref(sh), *[None] * 8, None)
    assert rc == -9 and "DELTA_NOALLOC_MAX_BYTES" in D.strerror(rc)
