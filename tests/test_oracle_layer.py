"""Pins of the layer prologue/epilogue oracle (oracle/layer.py) against facts fixed outside it:
numpy's convolution, closed forms of SiLU, unit norms, causality, scale invariance."""
import numpy as np
import pytest

from oracle import layer as Lr


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_silu_closed_forms():
    assert Lr.silu(0.0) == 0.0
    assert abs(Lr.silu(1.0) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-15
    assert abs(Lr.silu(40.0) - 40.0) < 1e-12 and abs(Lr.silu(-40.0)) < 1e-15
    # silu(x) - silu(-x) = x
    x = rnd(1, 50)
    assert np.allclose(Lr.silu(x) - Lr.silu(-x), x, atol=1e-14)


@pytest.mark.parametrize("width", [1, 2, 3, 4])
def test_conv_matches_numpy_convolve(width):
    B, T, H, d = 2, 11, 2, 3
    x, w = rnd(2, B, T, H, d), rnd(3, H * d, width)
    y = Lr.short_conv(x, w)
    for b in range(B):
        for h in range(H):
            for i in range(d):
                ref = np.convolve(x[b, :, h, i], w[h * d + i, ::-1])[:T]
                assert np.allclose(y[b, :, h, i], ref, atol=1e-13)


def test_conv_current_tap_is_identity_and_causal():
    x = rnd(4, 1, 9, 2, 4)
    w = np.zeros((8, 4))
    w[:, 3] = 1.0
    assert np.array_equal(Lr.short_conv(x, w), x)
    w = rnd(5, 8, 4)
    y0 = Lr.short_conv(x, w)
    x2 = x.copy()
    x2[:, 5] += 3.0
    y2 = Lr.short_conv(x2, w)
    assert np.array_equal(y0[:, :5], y2[:, :5]) and not np.allclose(y0[:, 5:], y2[:, 5:])
    # a one-token sequence sees only the current tap
    assert np.allclose(Lr.short_conv(x[:, :1], w), x[:, :1] * w[:, 3].reshape(1, 1, 2, 4))


def test_prologue_unit_norm_and_direction():
    xq, xk, xv = rnd(6, 2, 7, 3, 16), rnd(7, 2, 7, 3, 16), rnd(8, 2, 7, 3, 8)
    wq, wk, wv = rnd(9, 48, 4), rnd(10, 48, 4), rnd(11, 24, 4)
    q, k, v = Lr.prologue(xq, xk, xv, wq, wk, wv, eps=0.0)
    assert np.allclose(np.linalg.norm(q, axis=-1), 1.0, atol=1e-12)
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, atol=1e-12)
    a = Lr.silu(Lr.short_conv(xq, wq))
    assert np.allclose(q * np.linalg.norm(a, axis=-1, keepdims=True), a, atol=1e-12)
    assert np.allclose(v, Lr.silu(Lr.short_conv(xv, wv)))
    # eps keeps an all-zero row at zero instead of dividing by zero
    q0, _, _ = Lr.prologue(np.zeros((1, 2, 1, 16)), xk[:1, :2, :1], xv[:1, :2, :1], wq[:16], wk[:16], wv[:8])
    assert np.array_equal(q0, np.zeros_like(q0))


def test_epilogue_rms_gate_and_scale_invariance():
    o, g = rnd(12, 2, 5, 3, 16), rnd(13, 2, 5, 3, 16)
    one = np.ones(16)
    y = Lr.epilogue(o, np.full_like(g, 60.0), one, eps=0.0)      # SiLU(60) = 60 to 1e-24
    assert np.allclose(np.sqrt(np.mean((y / 60.0) ** 2, axis=-1)), 1.0, atol=1e-12)
    assert np.array_equal(Lr.epilogue(o, np.zeros_like(g), one), np.zeros_like(o))
    w = rnd(14, 16)
    assert np.allclose(Lr.epilogue(7.5 * o, g, w, eps=0.0), Lr.epilogue(o, g, w, eps=0.0), atol=1e-12)
    # a row with a single nonzero entry a: rms = |a| / 4, so the entry becomes 4 sign(a) w_i SiLU(g_i)
    o1 = np.zeros((1, 1, 1, 16))
    o1[0, 0, 0, 5] = -2.5
    y1 = Lr.epilogue(o1, g[:1, :1, :1], w, eps=0.0)
    assert abs(y1[0, 0, 0, 5] - (-4.0) * w[5] * Lr.silu(g[0, 0, 0, 5])) < 1e-12
