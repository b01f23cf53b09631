"""GPU parity of the segmented walks (problem->segments >= 2): long documents walked as segments
side by side after transfer walks and a carry merge, against the FP64 oracle (o, ht, and the
gradients of a backward that reads the segmented forward's saved set), in the light, full and
kept-tape forms, with h0, ht, dht, ragged and empty documents, d = 64 f32 and d = 128 bf16; the
same bits with and without the auxiliary stream; the 8,192-token document at full size."""
import numpy as np
import pytest
import torch

import gated_deltanet_fwd_amd as G
import oracle
import synthetic as syn
from parity_util import assert_close, host_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = ("o", "ht", "dq", "dk", "dv", "dg", "dbeta", "dh0")


def _dev(inp):
    return {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}


def _run(w, inp, segments, save_mode=G.SAVE_LIGHT, recompute_mode=None, aux=True, bwd=True):
    p = G.problem_for(w, save_mode=save_mode, segments=segments, use_aux_stream=aux)
    print("segments case %s: T=%d segments=%d mode=%d recompute=%s" % (w.name, w.T, segments, save_mode,
                                                                       recompute_mode), flush=True)
    a = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"])
    nan = float("nan")
    o = torch.full_like(inp["v"], nan)
    ht = torch.full((w.N, w.HV, w.d, w.d), nan, dtype=torch.float32, device=DEV) if w.want_ht else None
    ws = torch.full((G.gdn_workspace_bytes(p, G.OP_FWD),), 255, dtype=torch.uint8, device=DEV)
    saved = torch.full((G.gdn_saved_bytes(p),), 255, dtype=torch.uint8, device=DEV)
    o, ht, saved = G.gdn_fwd(p, *a, h0=inp["h0"], o=o, ht=ht, saved=saved, workspace=ws)
    out = dict(o=o, ht=ht, saved=saved)
    pb = p
    if recompute_mode is not None:
        pb = G.problem_for(w, save_mode=recompute_mode, segments=segments, use_aux_stream=aux)
        saved = torch.full((G.gdn_saved_bytes(pb),), 255, dtype=torch.uint8, device=DEV)
        wsr = torch.full((G.gdn_workspace_bytes(pb, G.OP_RECOMPUTE),), 255, dtype=torch.uint8, device=DEV)
        G.gdn_fwd_recompute(pb, *a, h0=inp["h0"], saved=saved, workspace=wsr)
        out["saved_recompute"] = saved
    if bwd:
        gr = G.gdn_bwd(pb, *a, saved, inp["dO"], h0=inp["h0"], dht=inp["dht"])
        out.update(gr)
    torch.cuda.synchronize()
    return out


def _check(w, inp, out, heads=None, bwd=True):
    Gg = w.HV // w.H
    h, ti, vh = host_inputs(inp, None, heads, Gg)
    hq = list(range(w.H)) if heads is None else list(heads)
    o_ref, ht_ref = oracle.fwd(h["cu"], h["q"], h["k"], h["v"], h["g"], h["beta"], h["h0"], l2norm=w.l2norm)
    assert_close("o", out["o"].index_select(0, ti)[:, vh], o_ref)
    if out.get("ht") is not None:
        assert_close("ht", out["ht"][:, vh], ht_ref)
    if not bwd:
        return
    ref = oracle.bwd(h["cu"], h["q"], h["k"], h["v"], h["g"], h["beta"], h["dO"], h["h0"], h["dht"], l2norm=w.l2norm)
    assert_close("dq", out["dq"].index_select(0, ti)[:, hq], ref["dq"])
    assert_close("dk", out["dk"].index_select(0, ti)[:, hq], ref["dk"])
    for k in ("dv", "dg", "dbeta"):
        assert_close(k, out[k].index_select(0, ti)[:, vh], ref[k])
    if out.get("dh0") is not None:
        assert_close("dh0", out["dh0"][:, vh], ref["dh0"])


CASES = [
    # long and short documents side by side, an empty one, h0 / ht / dht
    syn.custom("seg_mixed", [4000, 700, 0, 9000, 130], 2, 6, 128, "bf16", has_h0=True, want_ht=True, has_dht=True,
               seed=61),
    syn.custom("seg_d64_f32", [2500, 70, 1100], 2, 4, 64, "f32", has_h0=True, want_ht=True, has_dht=True, seed=62),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
@pytest.mark.parametrize("segments", [3, 8])
def test_segmented_light(w, segments):
    inp = _dev(syn.make_inputs(w))
    out = _run(w, inp, segments)
    _check(w, inp, out)


@pytest.mark.parametrize("mode", [G.SAVE_FULL, G.SAVE_TAPE])
def test_segmented_full_and_kept_tape(mode):
    """The full / kept-tape forward writes the state tape from the segmented walks; the backward
    reads it (no replay)."""
    w = CASES[0]
    inp = _dev(syn.make_inputs(w))
    out = _run(w, inp, 5, save_mode=mode)
    _check(w, inp, out)
    # the state tape against the chunked oracle's chunk start states
    h, _, _ = host_inputs(inp, None, None, w.HV // w.H)
    ref = oracle.chunked_fwd(h["cu"], h["q"], h["k"], h["v"], h["g"], h["beta"], h["h0"], l2norm=True, chunk=64,
                             full=True)
    NT = sum((L + 63) // 64 for L in w.lengths)
    T, HV, d = w.T, w.HV, w.d
    off = 256
    for n in (T * HV * 64 * 2, T * HV * 4, NT * HV * 4):
        off = (off + n + 255) // 256 * 256
    tape = out["saved"][off:off + NT * HV * d * d * 2].view(torch.bfloat16).reshape(NT, HV, d, d).transpose(2, 3)
    assert_close("h tape", tape, ref["H"])


def test_segmented_kept_tape_checkpoint():
    w = CASES[0]
    inp = _dev(syn.make_inputs(w))
    out = _run(w, inp, 4, save_mode=G.SAVE_LIGHT, recompute_mode=G.SAVE_TAPE)
    _check(w, inp, out)


def test_segmented_light_full_recompute_bitwise():
    """The saved carry plane lets the light backward replay the state tape segment by segment
    from the forward's start states: light, full and checkpointed runs agree bitwise, and the
    light recompute rebuilds the forward's saved set bitwise."""
    w = CASES[0]
    inp = _dev(syn.make_inputs(w))
    light = _run(w, inp, 6)
    full = _run(w, inp, 6, save_mode=G.SAVE_FULL)
    ck = _run(w, inp, 6, recompute_mode=G.SAVE_LIGHT)
    assert torch.equal(ck["saved"], ck["saved_recompute"])
    for k in NAMES:
        assert torch.equal(light[k], full[k]), k
        if k not in ("o", "ht"):
            assert torch.equal(light[k], ck[k]), k


def test_segmented_bitwise_with_and_without_aux_stream():
    w = CASES[0]
    inp = _dev(syn.make_inputs(w))
    for mode in (G.SAVE_LIGHT, G.SAVE_FULL):
        a = _run(w, inp, 6, save_mode=mode, aux=True)
        b = _run(w, inp, 6, save_mode=mode, aux=False)
        assert torch.equal(a["saved"], b["saved"])
        for k in NAMES:
            assert torch.equal(a[k], b[k]), k


def test_single8k_segmented_full_size():
    """The 8,192-token document at (16, 48), d = 128, walked as 8 segments, every head."""
    w = syn.WORKLOADS["single8k"]
    inp = syn.make_inputs(w, device=DEV)
    out = _run(w, inp, 8, bwd=False)
    _check(w, inp, out, bwd=False)


def _regime(inp, kind):
    """Decay regimes outside the pages' distribution: 'strong' (log decays about -4 per token, 10 %
    of tokens at 0 and 5 % at -80: the transfer maps of a segment vanish) or 'none' (g = 0 and
    beta = 1 everywhere: the maps are products of projections, no forgetting)."""
    if kind == "none":
        inp["g"] = torch.zeros_like(inp["g"])
        inp["beta"] = torch.ones_like(inp["beta"])
        return inp
    gen = torch.Generator().manual_seed(172)
    g = torch.nn.functional.logsigmoid(torch.randn(inp["g"].shape, generator=gen) - 4.0)
    pick = torch.rand(inp["g"].shape, generator=gen)
    inp["g"] = torch.where(pick < 0.1, torch.zeros_like(g), torch.where(pick > 0.95, torch.full_like(g, -80.0), g))
    return inp


@pytest.mark.parametrize("kind", ["strong", "none"])
def test_segmented_decay_regimes(kind):
    """Segmented walks (transfer walks, carry merge, segment re-walks, the light backward's replay
    from the carry plane) under vanishing and under absent decay, against the oracle."""
    w = syn.custom("seg_regime", [3000, 200, 1500], 1, 3, 128, "bf16", has_h0=True, want_ht=True, has_dht=True,
                   seed=63)
    inp = _dev(_regime(syn.make_inputs(w), kind))
    out = _run(w, inp, 4)
    _check(w, inp, out)
