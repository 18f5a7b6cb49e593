"""GPU parity of the layer prologue/epilogue (delta_layer_prologue / delta_layer_epilogue through
the C ABI) against the fp64 oracle in oracle/layer.py on the same seeded inputs.  Bar: max
absolute error <= 2e-5 for float32 (unit-scale outputs) and <= 1.6e-2 for bf16 (one bf16 rounding
of the output: half an ulp of values below 4 is at most 2^-7 / 2 * 4), elementwise."""
import numpy as np
import pytest

from oracle import layer as Lr
from parity import say, to_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import chunkwise_delta_rule_chunked_amd as D  # noqa: E402

TOLS = {"f32": 2e-5, "bf16": 1.6e-2}


def draw(seed, shape, dtype):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    if dtype == "bf16":
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    return x


@pytest.mark.parametrize("B,L,H,dk,dv,n_h,width,dtype", [
    (2, 37, 3, 64, 32, 1, 4, "f32"),
    (1, 50, 2, 16, 256, 2, 3, "f32"),
    (2, 333, 4, 128, 128, 1, 4, "bf16"),
    (1, 3, 2, 32, 48, 3, 4, "bf16"),      # shorter than the filter
    (1, 64, 2, 128, 128, 1, 1, "bf16"),   # one tap
    # one launch for the three tensors: row widths of 1..64 16-byte lanes, every filter width,
    # runs cut by the sequence end, DeltaProduct rows
    (2, 100, 3, 64, 128, 1, 2, "bf16"),
    (1, 70, 2, 128, 256, 2, 3, "f32"),    # 32 and 64 lanes per row
    (3, 33, 5, 16, 16, 1, 4, "bf16"),     # one lane per row
    (1, 257, 16, 128, 128, 2, 4, "bf16"),
    (2, 31, 1, 32, 64, 4, 2, "f32"),
    (1, 2, 3, 64, 64, 1, 4, "f32"),       # two tokens, four taps
])
def test_prologue(B, L, H, dk, dv, n_h, width, dtype):
    say("prologue", B, L, H, dk, dv, n_h, width, dtype)
    Lx = L * n_h
    xq, xk, xv = draw(1, (B, L, H, dk), dtype), draw(2, (B, Lx, H, dk), dtype), draw(3, (B, Lx, H, dv), dtype)
    wq, wk, wv = (0.5 * draw(4 + i, (H * d, width), "f32") for i, d in enumerate((dk, dk, dv)))
    q, k, v = D.layer_prologue(to_dev(xq, dtype), to_dev(xk, dtype), to_dev(xv, dtype), to_dev(wq, "f32"),
                               to_dev(wk, "f32"), to_dev(wv, "f32"), n_h=n_h)
    torch.cuda.synchronize()
    rq, rk, rv = Lr.prologue(xq, xk, xv, wq, wk, wv, eps=1e-6)
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        err = np.abs(got.float().cpu().numpy() - ref).max()
        say("  %s max abs err %.2e" % (name, err))
        assert err <= TOLS[dtype] * max(1.0, np.abs(ref).max() / 4), (name, err)


@pytest.mark.parametrize("B,L,H,dv,dtype", [(2, 41, 3, 64, "f32"), (2, 300, 4, 128, "bf16"), (1, 5, 2, 256, "bf16")])
def test_epilogue(B, L, H, dv, dtype):
    say("epilogue", B, L, H, dv, dtype)
    o, g = draw(11, (B, L, H, dv), dtype), draw(12, (B, L, H, dv), dtype)
    w = (1.0 + 0.1 * draw(13, (dv,), "f32")).astype(np.float32)
    y = D.layer_epilogue(to_dev(o, dtype), to_dev(g, dtype), to_dev(w, "f32"))
    torch.cuda.synchronize()
    ref = Lr.epilogue(o, g, w, eps=1e-6)
    err = np.abs(y.float().cpu().numpy() - ref).max()
    say("  y max abs err %.2e (max |y| %.2f)" % (err, np.abs(ref).max()))
    assert err <= TOLS[dtype] * max(1.0, np.abs(ref).max() / 4)


def test_epilogue_in_place():
    o, g = draw(21, (1, 17, 2, 64), "f32"), draw(22, (1, 17, 2, 64), "f32")
    w = np.ones(64, dtype=np.float32)
    od = to_dev(o, "f32")
    y = D.layer_epilogue(od, to_dev(g, "f32"), to_dev(w, "f32"), y=od)
    torch.cuda.synchronize()
    assert y.data_ptr() == od.data_ptr()
    assert np.abs(y.cpu().numpy() - Lr.epilogue(o, g, w)).max() <= 2e-5


@pytest.mark.parametrize("n_h,width,dk,dv,dtype", [(1, 4, 128, 128, "bf16"), (2, 3, 64, 32, "f32"),
                                                   (1, 1, 32, 48, "f32"), (3, 2, 16, 256, "bf16")])
def test_prologue_decode_steps(n_h, width, dk, dv, dtype):
    """A prefill of L tokens through delta_layer_prologue, then T tokens one at a time through
    delta_layer_prologue_step with the filters' state taken from the prefill's last inputs: the
    outputs equal the oracle's prologue over all L + T tokens, and the state ends as the last
    width - 1 inputs."""
    B, H, L, T = 2, 3, 9, 6
    say("prologue steps", n_h, width, dk, dv, dtype)
    N = L + T
    xq, xk, xv = draw(31, (B, N, H, dk), dtype), draw(32, (B, N * n_h, H, dk), dtype), draw(33, (B, N * n_h, H, dv), dtype)
    wq, wk, wv = (0.5 * draw(34 + i, (H * d, width), "f32") for i, d in enumerate((dk, dk, dv)))
    dev = lambda x: to_dev(x, dtype)
    wqd, wkd, wvd = to_dev(wq, "f32"), to_dev(wk, "f32"), to_dev(wv, "f32")
    q0, k0, v0 = D.layer_prologue(dev(xq[:, :L]), dev(xk[:, :L * n_h]), dev(xv[:, :L * n_h]), wqd, wkd, wvd, n_h=n_h)
    W1 = width - 1

    def state(x, rows):  # the last width-1 input rows before `rows`, oldest first
        return dev(np.ascontiguousarray(x[:, rows - W1:rows])) if W1 else None

    cq, ck, cv = state(xq, L), state(xk, L * n_h), state(xv, L * n_h)
    outs = [(q0, k0, v0)]
    for t in range(L, N):
        outs.append(D.layer_prologue_step(dev(xq[:, t:t + 1]), dev(xk[:, t * n_h:(t + 1) * n_h]),
                                          dev(xv[:, t * n_h:(t + 1) * n_h]), wqd, wkd, wvd, cq, ck, cv, n_h=n_h))
    torch.cuda.synchronize()
    got = [torch.cat([o[i] for o in outs], dim=1).float().cpu().numpy() for i in range(3)]
    ref = Lr.prologue(xq, xk, xv, wq, wk, wv, eps=1e-6)
    for name, g, r in zip("qkv", got, ref):
        err = np.abs(g - r).max()
        say("  %s max abs err %.2e" % (name, err))
        assert err <= TOLS[dtype] * max(1.0, np.abs(r).max() / 4), (name, err)
    if W1:
        for c, x, rows in ((cq, xq, N), (ck, xk, N * n_h), (cv, xv, N * n_h)):
            assert np.array_equal(c.float().cpu().numpy(), x[:, rows - W1:rows])
