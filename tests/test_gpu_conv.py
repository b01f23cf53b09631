"""GPU parity of the causal conv1d + SiLU front-end (through the C ABI) against the FP64 oracle,
with the pages' accuracy budget (rel-RMS <= 1e-2, max-abs <= 2e-2 max|ref| per tensor).

Small and multi-block cases compare every element: ragged and empty documents, documents that
end exactly at a wave's or a workgroup's token boundary, one-token documents, channel groups that
split a wave's channels, every window width 1..4, bf16 and f32, SiLU and bias on and off. The
pages' B23 shape (32,768 tokens, 10,240 channels) runs at full size and is compared on sampled
channels (the convolution never mixes channels), including the groups' edges."""
import numpy as np
import pytest
import torch

import gated_deltanet_fwd_amd as G
import synthetic as syn
from oracle import conv_oracle
from parity_util import assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(w, inp=None):
    if inp is None:
        inp = {k: (v.to(DEV) if torch.is_tensor(v) else [t.to(DEV) for t in v] if isinstance(v, list) else v)
               for k, v in syn.make_conv_inputs(w).items()}
    p = G.ConvProblem(inp["cu_seqlens"].cpu().numpy(), w.groups, width=w.width, dtype=w.torch_dtype, silu=w.silu)
    print("conv case %s: T=%d C=%d W=%d %s silu=%d bias=%d" % (w.name, w.T, w.C, w.width, w.dtype, w.silu,
                                                                  w.bias), flush=True)
    nan = float("nan")
    outs = [torch.full((w.T, c), nan, dtype=w.torch_dtype, device=DEV) for c in w.groups]
    G.gdn_conv_fwd(p, inp["x"], inp["weight"], inp["bias"], inp["cu_seqlens"], outs=outs)
    dx = torch.full_like(inp["x"], nan)
    dw = torch.full_like(inp["weight"], nan)
    db = torch.full_like(inp["bias"], nan) if inp["bias"] is not None else None
    ws = torch.full((G.gdn_conv_workspace_bytes(p),), 255, dtype=torch.uint8, device=DEV)
    gr = G.gdn_conv_bwd(p, inp["x"], inp["weight"], inp["bias"], inp["cu_seqlens"], inp["dy"], dx=dx, dweight=dw,
                        dbias=db, workspace=ws)
    torch.cuda.synchronize()
    return inp, torch.cat(outs, dim=1), gr


def _f64(t):
    return t.detach().double().cpu().numpy()


def _check(w, inp, y, gr, cols=None):
    cols = np.arange(w.C) if cols is None else np.asarray(cols)
    cu = inp["cu_seqlens"].cpu().numpy()
    x = _f64(inp["x"][:, cols])
    wt = _f64(inp["weight"][cols])
    b = _f64(inp["bias"][cols]) if inp["bias"] is not None else None
    dy = _f64(torch.cat(inp["dy"], dim=1)[:, cols])
    y_ref, _ = conv_oracle.conv_fwd(cu, x, wt, b, silu=w.silu)
    ref = conv_oracle.conv_bwd(cu, x, wt, b, dy, silu=w.silu)
    assert_close("y", y[:, cols], y_ref)
    assert_close("dx", gr["dx"][:, cols], ref["dx"])
    assert_close("dweight", gr["dweight"][cols], ref["dweight"])
    if b is not None:
        assert_close("dbias", gr["dbias"][cols], ref["dbias"])


SMALL = [syn.conv_custom("ragged_w%d_%s" % (W, dt), [0, 5, 5, 17, 18, 30, 1], [8, 8, 8], width=W, dtype=dt,
                         seed=40 + W) for W in (1, 2, 3, 4) for dt in ("bf16", "f32")]
SMALL += [syn.conv_custom("no_silu_no_bias", [9, 0, 40], [16, 8], silu=False, bias=False, seed=50),
          syn.conv_custom("single_token_docs", [1, 1, 1, 2, 1], [8], seed=51)]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_conv_small(w):
    inp, y, gr = _run(w)
    _check(w, inp, y, gr)


MULTI = [
    # documents ending at a wave's (128) and a workgroup's (512) token boundary, a one-token
    # document across a boundary, a last partial workgroup; groups split the 256-channel tiles
    syn.conv_custom("blocks_bf16", [1024, 1, 255, 769, 700, 251], [512, 16, 520], seed=52),
    syn.conv_custom("blocks_f32_w3", [300, 1500, 3], [24, 1000], width=3, dtype="f32", seed=53),
]


@pytest.mark.parametrize("w", MULTI, ids=[w.name for w in MULTI])
def test_conv_multi_block(w):
    inp, y, gr = _run(w)
    _check(w, inp, y, gr)


def test_conv_b23_full_size_sampled_and_deterministic():
    w = syn.CONV_WORKLOADS["b23_conv"]
    inp, y, gr = _run(w)
    cols = np.concatenate([np.arange(0, 8), np.arange(2040, 2056), np.arange(4088, 4104), np.arange(5000, 5008),
                           np.arange(10232, 10240)])
    _check(w, inp, y, gr, cols)
    dw1, db1 = gr["dweight"].clone(), gr["dbias"].clone()
    _, _, gr2 = _run(w, inp)
    assert torch.equal(dw1, gr2["dweight"]) and torch.equal(db1, gr2["dbias"])


def test_conv_no_tokens():
    w = syn.conv_custom("empty", [0, 0], [8, 8], seed=54)
    inp, y, gr = _run(w)
    assert torch.equal(gr["dweight"], torch.zeros_like(gr["dweight"]))
    assert torch.equal(gr["dbias"], torch.zeros_like(gr["dbias"]))
