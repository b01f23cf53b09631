"""FP64 CPU oracle for the short causal conv1d + SiLU front-end (test infrastructure).

TEST INFRASTRUCTURE ONLY. Only the test suite and the benchmark's CPU-baseline leg use this
module; the product path (the HIP library and its binding) never imports it, and it imports
nothing from the product.

What is computed. The pages time the gated delta rule together with a short causal convolution
over the packed q/k/v channels (flashinfer PR #8542, "Conventions": shape B23 runs the short causal
convolution over the 10,240 packed q/k/v channels on every timed call; flashinfer PR #7117 text:
the causal conv1d + SiLU training backend of the same kernel family; the README saved-set table
keeps at most 3 convolution history rows per fragment, so the window is 4 taps). They never write
the operation down. The plainest reading is the depthwise causal convolution of each channel
within each document, followed by SiLU:

    pre[t, c] = bias[c] + sum_{i=0}^{W-1} weight[c, i] * x[t - (W-1) + i, c]
    y[t, c]   = SiLU(pre[t, c]) = pre / (1 + exp(-pre))          (pre itself when silu is off)

where x at a position before the first token of t's document is zero (documents delimited by
cu_seqlens never see each other's tokens). The backward, for an upstream gradient dy of y:

    dpre[t, c] = dy[t, c] * s * (1 + pre (1 - s)),  s = 1 / (1 + exp(-pre))   (dy when silu is off)
    dx[t, c]   = sum_{i} weight[c, i] * dpre[t + (W-1) - i, c]   over positions in t's document
    dweight[c, i] = sum_t dpre[t, c] * x[t - (W-1) + i, c],   dbias[c] = sum_t dpre[t, c]

Everything here is float64 numpy: shifts of whole documents for the window taps, no blocking.
"""
from __future__ import annotations

import numpy as np


def _docs(cu):
    cu = np.asarray(cu, dtype=np.int64)
    return [(int(cu[n]), int(cu[n + 1])) for n in range(cu.shape[0] - 1)]


def conv_fwd(cu_seqlens, x, weight, bias=None, silu=True):
    """Returns (y, pre), both float64 [T, C]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    T, C = x.shape
    W = w.shape[1]
    assert w.shape == (C, W)
    pre = np.zeros((T, C))
    for s, e in _docs(cu_seqlens):
        L = e - s
        xs = x[s:e]
        for i in range(W):
            shift = W - 1 - i  # tap i reads the token `shift` positions back
            if shift < L:
                pre[s + shift:e] += w[:, i] * xs[:L - shift]
    if bias is not None:
        pre += np.asarray(bias, dtype=np.float64)
    y = pre / (1.0 + np.exp(-pre)) if silu else pre.copy()
    return y, pre


def conv_bwd(cu_seqlens, x, weight, bias, dy, silu=True):
    """Returns dict dx [T, C], dweight [C, W], dbias [C] (float64)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    T, C = x.shape
    W = w.shape[1]
    _, pre = conv_fwd(cu_seqlens, x, w, bias, silu=False)
    if silu:
        s = 1.0 / (1.0 + np.exp(-pre))
        dpre = dy * s * (1.0 + pre * (1.0 - s))
    else:
        dpre = dy
    dx = np.zeros((T, C))
    dw = np.zeros((C, W))
    for s0, e in _docs(cu_seqlens):
        L = e - s0
        xs, ds = x[s0:e], dpre[s0:e]
        for i in range(W):
            shift = W - 1 - i
            if shift < L:
                # pre[t] gets w_i x[t - shift]: x[t'] feeds pre[t' + shift]
                dx[s0:e - shift] += w[:, i] * ds[shift:]
                dw[:, i] += np.sum(ds[shift:] * xs[:L - shift], axis=0)
    return dict(dx=dx, dweight=dw, dbias=dpre.sum(axis=0))
