"""Pins of the conv1d + SiLU oracle (oracle/conv_oracle.py) against what fixes it independently:
library routines (numpy.convolve per document and channel; torch's float64 conv1d and SiLU with
autograd), central finite differences, document isolation and closed forms. Each pin takes the
oracle module as an argument, so the mutant test can run them on planted mistakes."""
from __future__ import annotations

import numpy as np
import torch

CU = np.array([0, 5, 5, 17, 18, 30], dtype=np.int32)  # ragged documents, one empty, one of 1 token


def _inputs(C=6, W=4, seed=0, cu=CU):
    rng = np.random.default_rng(seed)
    T = int(cu[-1])
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W)) * 0.7
    b = rng.standard_normal(C) * 0.3
    dy = rng.standard_normal((T, C))
    return x, w, b, dy


def pin_numpy_convolve(mod):
    """Without SiLU and bias, each document's channel is numpy's full convolution with the
    reversed window, cut to the document's length (zeros before the document's first token)."""
    for W in (1, 2, 3, 4):
        x, w, _, _ = _inputs(W=W, seed=W)
        y, _ = mod.conv_fwd(CU, x, w, None, silu=False)
        for n in range(len(CU) - 1):
            s, e = int(CU[n]), int(CU[n + 1])
            if e == s:
                continue
            for c in range(x.shape[1]):
                ref = np.convolve(x[s:e, c], w[c, ::-1])[: e - s]
                np.testing.assert_allclose(y[s:e, c], ref, rtol=1e-13, atol=1e-13)


def _torch_ref(x, w, b, dy, silu=True):
    """torch float64: per document, conv1d with groups = channels and left padding W - 1, plus bias,
    then SiLU; gradients by autograd."""
    C, W = w.shape
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
    outs = []
    for n in range(len(CU) - 1):
        s, e = int(CU[n]), int(CU[n + 1])
        if e == s:
            continue
        seg = xt[s:e].t().unsqueeze(0)  # [1, C, L]
        pre = torch.nn.functional.conv1d(torch.nn.functional.pad(seg, (W - 1, 0)), wt.unsqueeze(1), bt, groups=C)
        y = torch.nn.functional.silu(pre) if silu else pre
        outs.append(y[0].t())
    y = torch.cat(outs)
    (y * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    return y.detach().numpy(), xt.grad.numpy(), wt.grad.numpy(), bt.grad.numpy()


def pin_torch_conv_silu_autograd(mod):
    """Forward and every gradient against torch's float64 conv1d + SiLU and its autograd."""
    for silu in (True, False):
        x, w, b, dy = _inputs(seed=3)
        y_ref, dx_ref, dw_ref, db_ref = _torch_ref(x, w, b, dy, silu=silu)
        y, _ = mod.conv_fwd(CU, x, w, b, silu=silu)
        g = mod.conv_bwd(CU, x, w, b, dy, silu=silu)
        np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g["dx"], dx_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g["dweight"], dw_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g["dbias"], db_ref, rtol=1e-12, atol=1e-12)


def pin_finite_differences(mod):
    """Central differences of <dy, y> in float64 on x, weight and bias."""
    x, w, b, dy = _inputs(C=3, W=4, seed=5)
    g = mod.conv_bwd(CU, x, w, b, dy)
    loss = lambda x_, w_, b_: float(np.sum(dy * mod.conv_fwd(CU, x_, w_, b_)[0]))
    h = 1e-6
    for name, arr, grad in (("x", x, g["dx"]), ("w", w, g["dweight"]), ("b", b, g["dbias"])):
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p = {"x": (ap, w, b), "w": (x, ap, b), "b": (x, w, ap)}[name]
            args_m = {"x": (am, w, b), "w": (x, am, b), "b": (x, w, am)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def pin_documents_isolated(mod):
    """A packed run equals the documents run one by one; a document never sees another's tokens."""
    x, w, b, dy = _inputs(seed=7)
    y, _ = mod.conv_fwd(CU, x, w, b)
    g = mod.conv_bwd(CU, x, w, b, dy)
    dw_sum, db_sum = np.zeros_like(w), np.zeros_like(b)
    for n in range(len(CU) - 1):
        s, e = int(CU[n]), int(CU[n + 1])
        cu1 = np.array([0, e - s], dtype=np.int32)
        y1, _ = mod.conv_fwd(cu1, x[s:e], w, b)
        g1 = mod.conv_bwd(cu1, x[s:e], w, b, dy[s:e])
        np.testing.assert_allclose(y[s:e], y1, rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(g["dx"][s:e], g1["dx"], rtol=1e-14, atol=1e-14)
        dw_sum += g1["dweight"]
        db_sum += g1["dbias"]
    np.testing.assert_allclose(g["dweight"], dw_sum, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dbias"], db_sum, rtol=1e-12, atol=1e-12)


def pin_closed_forms(mod):
    """One tap: y = SiLU(w x + b) elementwise. A window that picks its newest tap with no bias and
    no SiLU is the identity; one that picks its oldest is a shift by W - 1 within each document."""
    x, w, b, _ = _inputs(W=1, seed=9)
    y, _ = mod.conv_fwd(CU, x, w, b)
    z = w[:, 0] * x + b
    np.testing.assert_allclose(y, z / (1 + np.exp(-z)), rtol=1e-14, atol=1e-14)
    x, _, _, _ = _inputs(W=4, seed=10)
    C = x.shape[1]
    newest = np.zeros((C, 4))
    newest[:, 3] = 1.0
    np.testing.assert_array_equal(mod.conv_fwd(CU, x, newest, None, silu=False)[0], x)
    oldest = np.zeros((C, 4))
    oldest[:, 0] = 1.0
    y = mod.conv_fwd(CU, x, oldest, None, silu=False)[0]
    for n in range(len(CU) - 1):
        s, e = int(CU[n]), int(CU[n + 1])
        ref = np.zeros((e - s, C))
        if e - s > 3:
            ref[3:] = x[s:e - 3]
        np.testing.assert_array_equal(y[s:e], ref)


ALL_PINS = [pin_numpy_convolve, pin_torch_conv_silu_autograd, pin_finite_differences, pin_documents_isolated,
            pin_closed_forms]
