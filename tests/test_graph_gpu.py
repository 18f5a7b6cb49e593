"""HIP graph capture of the multi-launch entry points: the backward pass (both routes), KDA in
chunks and the layer prologue.  Each is captured once with preallocated outputs and workspace,
replayed several times with eager work and synchronisation between the replays, and every
replay is compared with the eager call bit for bit (the kernels are deterministic, and no launch
records a memset node).  The forward pass and the decode steps have the same test in
test_parity_gpu.py."""
import pytest

import workloads as W
from parity import inputs_to_dev, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import chunkwise_delta_rule_chunked_amd as D  # noqa: E402

REPLAYS = 3


def replay_and_compare(capture_call, outputs, expected, reset):
    """Capture capture_call() into a graph, then replay it REPLAYS times; after each replay the
    tensors in `outputs` must equal `expected` exactly.  `reset` runs eagerly before each replay."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture_call()
    for rep in range(REPLAYS):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in outputs.items():
            e = expected[name]
            if t is None:
                assert e is None, name
                continue
            diff = (t.float() - e.float()).abs().max().item() if t.numel() else 0.0
            say("  replay %d %s: max |graph - eager| %.3e" % (rep, name, diff))
            assert diff == 0.0, (rep, name, diff)


@pytest.mark.parametrize("dt,dk,dv,chunk", [("bf16", 128, 128, 64), ("f32", 64, 48, 32)])
def test_bwd_graph_replay(dt, dk, dv, chunk):
    w = W.Workload("bwd_graph", B=1, H=2, L=300, dk=dk, dv=dv, chunk=chunk, dtype=dt, gate="cfg3", s0=0.1,
                   cfg_id=96)
    say("case", w)
    inp, cot = W.make_inputs(w), W.make_cotangents(w)
    d = inputs_to_dev(inp, w.dtype)
    dO, dS = to_dev(cot["dO"], w.dtype), to_dev(cot["dS_final"], "f32")
    code = D.BF16 if dt == "bf16" else D.F32
    ws = torch.empty(D.bwd_workspace_bytes(w.B, w.L, w.H, dk, dv, w.n_h, chunk, code), dtype=torch.uint8,
                     device="cuda")
    call = lambda grads=None: D.bwd(d["q"], d["k"], d["v"], d["beta"], d["g_log"], d["S0"], dO, dS, n_h=w.n_h,
                                    chunk=chunk, scale=0.7, grads=grads, workspace=ws)
    eager = {n: (None if t is None else t.clone()) for n, t in call().items()}
    torch.cuda.synchronize()
    graph_out = {n: (None if t is None else torch.empty_like(t)) for n, t in eager.items()}

    def reset():
        for t in graph_out.values():
            if t is not None:
                t.zero_()

    replay_and_compare(lambda: call(graph_out), graph_out, eager, reset)


def test_kda_chunked_graph_replay():
    w = W.Workload("kda_graph", B=1, H=2, L=500, dk=128, dv=128, dtype="bf16", gate="cfg3", s0=0.1, cfg_id=97)
    say("case", w)
    inp = W.make_inputs(w)
    d = inputs_to_dev(inp, w.dtype)
    a = torch.from_numpy(W.make_kda_decays(w)).cuda()
    ws = torch.empty(D.kda_chunked_workspace_bytes(w.B, w.L, w.H), dtype=torch.uint8, device="cuda")
    Oe, Se = D.fwd_kda_chunked(d["q"], d["k"], d["v"], d["beta"], a, d["S0"], scale=0.9, workspace=ws)
    Oe, Se = Oe.clone(), Se.clone()
    torch.cuda.synchronize()
    Og, Sg = torch.empty_like(Oe), torch.empty_like(Se)
    call = lambda: D.fwd_kda_chunked(d["q"], d["k"], d["v"], d["beta"], a, d["S0"], scale=0.9, O=Og, S_final=Sg,
                                     workspace=ws)

    def reset():
        Og.zero_()
        Sg.zero_()

    replay_and_compare(call, {"O": Og, "S_final": Sg}, {"O": Oe, "S_final": Se}, reset)


def test_layer_prologue_graph_replay():
    B, L, H, d, width = 2, 200, 3, 128, 4
    g = torch.Generator().manual_seed(98)
    x = {n: torch.randn((B, L, H, d), generator=g).to(torch.bfloat16).cuda() for n in ("q", "k", "v")}
    wts = {n: (0.5 * torch.randn((H * d, width), generator=g)).cuda() for n in ("q", "k", "v")}
    outs_e = D.layer_prologue(x["q"], x["k"], x["v"], wts["q"], wts["k"], wts["v"])
    outs_e = [t.clone() for t in outs_e]
    torch.cuda.synchronize()
    outs_g = [torch.empty_like(t) for t in outs_e]
    call = lambda: D.layer_prologue(x["q"], x["k"], x["v"], wts["q"], wts["k"], wts["v"], q=outs_g[0], k=outs_g[1],
                                    v=outs_g[2])

    def reset():
        for t in outs_g:
            t.zero_()

    replay_and_compare(call, dict(zip("qkv", outs_g)), dict(zip("qkv", outs_e)), reset)
