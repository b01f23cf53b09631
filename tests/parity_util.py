"""Helpers for the GPU-vs-oracle parity tests: tolerances, comparisons, sampled oracle runs."""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle

_GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tolerance.json")
with open(_GOLD) as _f:
    TOL = json.load(_f)
REL_RMS = float(TOL["rel_rms"])
MAX_ABS = float(TOL["max_abs_over_max_ref"])


def to_np(x):
    if x is None:
        return None
    if torch.is_tensor(x):
        return x.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def errors(got, ref):
    """(rel_rms, max_abs / max|ref|) in float64; rel-RMS = ||got - ref|| / ||ref|| over all elements."""
    g, r = to_np(got), to_np(ref)
    d = g - r
    nr = np.sqrt(np.sum(r * r))
    mr = np.max(np.abs(r)) if r.size else 0.0
    rr = np.sqrt(np.sum(d * d)) / nr if nr > 0 else np.sqrt(np.sum(d * d))
    ma = np.max(np.abs(d)) / mr if mr > 0 else (np.max(np.abs(d)) if d.size else 0.0)
    return float(rr), float(ma)


def assert_close(name, got, ref, report=None):
    g = to_np(got)
    assert np.all(np.isfinite(g)), "%s: non-finite values" % name
    r = to_np(ref)
    if r.size and np.max(np.abs(r)) == 0:
        assert np.max(np.abs(g)) <= 1e-6, "%s: reference is zero, got max %g" % (name, np.max(np.abs(g)))
        return
    rr, ma = errors(g, r)
    if report is not None:
        report[name] = (rr, ma)
    assert rr <= REL_RMS and ma <= MAX_ABS, "%s: rel_rms %.3e (<= %.0e), max_abs/max|ref| %.3e (<= %.0e)" % (
        name, rr, REL_RMS, ma, MAX_ABS)


def host_inputs(inp, docs=None, heads=None, G=1):
    """Float32 numpy copies of the inputs, restricted to documents `docs` and q/k heads `heads`
    (with their G value heads each). Returns (arrays, token index, value-head index)."""
    cu = inp["cu_seqlens"].cpu().numpy().astype(np.int64)
    N = cu.shape[0] - 1
    docs = list(range(N)) if docs is None else list(docs)
    H = inp["q"].shape[1]
    heads = list(range(H)) if heads is None else list(heads)
    vheads = [j * G + gi for j in heads for gi in range(G)]
    tok = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in docs]) if docs else np.zeros(0, np.int64)
    lens = [int(cu[n + 1] - cu[n]) for n in docs]
    cu2 = np.zeros(len(docs) + 1, np.int32)
    cu2[1:] = np.cumsum(lens)
    ti = torch.from_numpy(tok).to(inp["q"].device)

    def sl(name, hidx, per_doc=False):
        t = inp.get(name)
        if t is None:
            return None
        if per_doc:
            return t[docs][:, hidx].float().cpu().numpy()
        return t.index_select(0, ti)[:, hidx].float().cpu().numpy()

    out = dict(cu=cu2, q=sl("q", heads), k=sl("k", heads), v=sl("v", vheads), g=sl("g", vheads),
               beta=sl("beta", vheads), dO=sl("dO", vheads), h0=sl("h0", vheads, True),
               dht=sl("dht", vheads, True))
    return out, ti, vheads


def oracle_fwd(h, l2norm):
    return oracle.fwd(h["cu"], h["q"], h["k"], h["v"], h["g"], h["beta"], h["h0"], l2norm=l2norm)


def oracle_bwd(h, l2norm):
    return oracle.bwd(h["cu"], h["q"], h["k"], h["v"], h["g"], h["beta"], h["dO"], h["h0"], h["dht"], l2norm=l2norm)
