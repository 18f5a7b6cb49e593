"""fp64 oracle of the layer steps on either side of the delta-rule token mixer.

TEST INFRASTRUCTURE ONLY (as the rest of this package): used by tests/ and the benchmark's
CPU-baseline leg, never by the product library.

The Gated DeltaNet layer design ("08 linear delta rule & DPLR" page, the layer-design figure
after section 3) runs, after the input projections:
  q, k:  ShortConv -> SiLU -> L2 norm (per head)
  v:     ShortConv -> SiLU
and, after the token mixer, Norm -> output gate (a projection passed through SiLU) before the
output projection.  The page does not spell the pieces out; this module takes the plainest
readings:
  ShortConv  a causal depthwise convolution along time, one filter of `width` taps per channel
             (channel = head * d + i), no bias, zeros before the first token:
             y[t, c] = sum_s w[c, s] * x[t - (width - 1) + s, c]   (tap width-1 = current token)
  SiLU       x * sigmoid(x)
  L2 norm    x / sqrt(sum_i x_i^2 + eps) over the d channels of one head of one token
  Norm       RMS norm over the d_v channels of one head: o / sqrt(mean(o^2) + eps) * weight,
             weight [d_v] shared by the heads
  gate       y = Norm(o) * SiLU(g), g the gate projection [B, L, H, d_v]
Each function is the definition written out with numpy, pinned in tests/test_oracle_layer.py.
"""
from __future__ import annotations

import numpy as np


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def short_conv(x, w):
    """x [B, T, H, d], w [H * d, width] -> [B, T, H, d] (fp64), causal depthwise along T."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, T, H, d = x.shape
    width = w.shape[1]
    wc = w.reshape(H, d, width)
    y = np.zeros((B, T, H, d))
    for s in range(width):
        lag = width - 1 - s          # tap s reads the token `lag` steps back
        if lag >= T:
            continue
        y[:, lag:] += x[:, :T - lag] * wc[None, None, :, :, s]
    return y


def l2_norm(x, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def prologue(xq, xk, xv, wq, wk, wv, eps=1e-6):
    """q = L2(SiLU(conv(xq))), k = L2(SiLU(conv(xk))), v = SiLU(conv(xv)); fp64."""
    q = l2_norm(silu(short_conv(xq, wq)), eps)
    k = l2_norm(silu(short_conv(xk, wk)), eps)
    v = silu(short_conv(xv, wv))
    return q, k, v


def epilogue(o, g, weight, eps=1e-6):
    """y = o / sqrt(mean(o^2) + eps) * weight * SiLU(g) per (token, head); fp64."""
    o = np.asarray(o, dtype=np.float64)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o / rms * np.asarray(weight, dtype=np.float64) * silu(g)
