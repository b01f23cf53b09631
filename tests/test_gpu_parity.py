"""GPU parity: the HIP path (through the C ABI) against the FP64 oracle, plus bitwise invariants.

Tolerances are the pages' accuracy budget (tests/golden/tolerance.json): rel-RMS <= 1e-2 and
max-abs <= 2e-2 * max|ref| per tensor. Small cases compare every element; the full-size
workloads run on the GPU exactly as the benchmark launches them and compare sampled documents
and q/k-head groups, which the oracle computes independently of the rest.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_fwd_amd as G
import oracle
import synthetic as syn
from parity_util import assert_close, host_inputs, oracle_bwd, oracle_fwd, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dev(inp):
    return {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}


def _run(w, inp, save_mode=G.SAVE_LIGHT, det=None, bwd=True, recompute=False, poison=False, l2norm=None,
         aux=True, recompute_mode=None, dht=True, segments=0):
    """fwd (save_mode), optionally recompute (recompute_mode, default save_mode) into a fresh saved
    buffer, then bwd with the problem of the saved set it reads. segments = 0: the library's plan;
    1: unsegmented walks (the two-part launch plan when one document dominates)."""
    p = G.problem_for(w, save_mode=save_mode, deterministic=det, l2norm=l2norm, use_aux_stream=aux,
                      segments=segments)
    pr = p if recompute_mode is None else G.problem_for(w, save_mode=recompute_mode, deterministic=det,
                                                         l2norm=l2norm, use_aux_stream=aux, segments=segments)
    a = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"])
    fill = float("nan") if poison else 0.0
    o = torch.full_like(inp["v"], fill)
    ht = torch.full((w.N, w.HV, w.d, w.d), fill, dtype=torch.float32, device=DEV) if w.want_ht else None
    saved = torch.full((G.gdn_saved_bytes(p),), 255 if poison else 0, dtype=torch.uint8, device=DEV)
    ws = torch.full((G.gdn_workspace_bytes(p, G.OP_FWD),), 255 if poison else 0, dtype=torch.uint8, device=DEV)
    o, ht, saved = G.gdn_fwd(p, *a, h0=inp["h0"], o=o, ht=ht, saved=saved, workspace=ws)
    out = dict(o=o, ht=ht, saved=saved, p=p)
    pb = p
    if recompute:
        saved2 = torch.full((G.gdn_saved_bytes(pr),), 255 if poison else 0, dtype=torch.uint8, device=DEV)
        ws2 = torch.full((G.gdn_workspace_bytes(pr, G.OP_RECOMPUTE),), 255 if poison else 0, dtype=torch.uint8,
                         device=DEV)
        G.gdn_fwd_recompute(pr, *a, h0=inp["h0"], saved=saved2, workspace=ws2)
        out["saved_recompute"] = saved2
        pb = pr
    if bwd:
        grads = dict(dq=torch.full_like(inp["q"], fill), dk=torch.full_like(inp["k"], fill),
                     dv=torch.full_like(inp["v"], fill), dg=torch.full_like(inp["g"], fill),
                     dbeta=torch.full_like(inp["beta"], fill),
                     dh0=torch.full_like(inp["h0"], fill) if inp["h0"] is not None else None)
        wsb = torch.full((G.gdn_workspace_bytes(pb, G.OP_BWD),), 255 if poison else 0, dtype=torch.uint8,
                         device=DEV)
        G.gdn_bwd(pb, *a, out.get("saved_recompute", saved), inp["dO"], h0=inp["h0"],
                  dht=inp["dht"] if dht else None, grads=grads, workspace=wsb)
        out.update(grads)
        out["status"] = G.gdn_status(pb, G.OP_BWD, wsb)
    torch.cuda.synchronize()
    return out


def _check_all(w, inp, out, docs=None, heads=None, bwd=True, l2norm=None, dht=True):
    """Compare o, ht and the gradients on the sampled documents x q/k heads."""
    l2 = w.l2norm if l2norm is None else l2norm
    Gg = w.HV // w.H
    h, ti, vh = host_inputs(inp, docs, heads, Gg)
    if not dht:
        h["dht"] = None
    if bwd:
        assert out.get("status", G.GDN_OK) == G.GDN_OK
    hq = list(range(w.H)) if heads is None else list(heads)
    dsel = list(range(w.N)) if docs is None else list(docs)
    o_ref, ht_ref = oracle_fwd(h, l2)
    assert_close("o", out["o"].index_select(0, ti)[:, vh], o_ref)
    if out.get("ht") is not None:
        assert_close("ht", out["ht"][dsel][:, vh], ht_ref)
    if not bwd:
        return
    ref = oracle_bwd(h, l2)
    assert_close("dq", out["dq"].index_select(0, ti)[:, hq], ref["dq"])
    assert_close("dk", out["dk"].index_select(0, ti)[:, hq], ref["dk"])
    assert_close("dv", out["dv"].index_select(0, ti)[:, vh], ref["dv"])
    assert_close("dg", out["dg"].index_select(0, ti)[:, vh], ref["dg"])
    assert_close("dbeta", out["dbeta"].index_select(0, ti)[:, vh], ref["dbeta"])
    if out.get("dh0") is not None:
        assert_close("dh0", out["dh0"][dsel][:, vh], ref["dh0"])


# ------------------------------------------------------------------------------------------
# small cases, every element


@pytest.mark.parametrize("det", [True, False])
@pytest.mark.parametrize("mode", [G.SAVE_LIGHT, G.SAVE_FULL])
def test_tiny(det, mode):
    w = syn.WORKLOADS["tiny"]
    inp = _dev(syn.make_inputs(w))
    out = _run(w, inp, save_mode=mode, det=det)
    _check_all(w, inp, out)


@pytest.mark.parametrize("det", [True, False])
@pytest.mark.parametrize("mode", [G.SAVE_LIGHT, G.SAVE_FULL])
def test_strong_decay(det, mode):
    """Log decays far below the pages' distribution: about -4 per token, some tokens at 0 (no
    decay) and some at -80, so the in-chunk cumulative gates reach hundreds and their exponentials
    span the whole f32 range (underflowing to zero) inside the chunk."""
    w = syn.custom("strong_decay", [200, 77, 130], 2, 6, 128, "bf16", has_h0=True, want_ht=True, has_dht=True,
                   seed=17)
    inp = syn.make_inputs(w)
    gen = torch.Generator().manual_seed(171)
    g = torch.nn.functional.logsigmoid(torch.randn(w.T, w.HV, generator=gen) - 4.0)
    pick = torch.rand(w.T, w.HV, generator=gen)
    g = torch.where(pick < 0.1, torch.zeros_like(g), torch.where(pick > 0.95, torch.full_like(g, -80.0), g))
    inp["g"] = g.float()
    inp = _dev(inp)
    out = _run(w, inp, save_mode=mode, det=det)
    _check_all(w, inp, out)


@pytest.mark.parametrize("det", [True, False])
def test_no_decay_full_updates(det):
    """g = 0 and beta = 1 on every token (no forgetting, full delta-rule updates) over a 2,000-token
    document and a short one: the state keeps every chunk's contribution, the longest memory the
    method allows."""
    w = syn.custom("no_decay", [2000, 150], 2, 6, 128, "bf16", has_h0=True, want_ht=True, has_dht=True, seed=19)
    inp = syn.make_inputs(w)
    inp["g"] = torch.zeros_like(inp["g"])
    inp["beta"] = torch.ones_like(inp["beta"])
    inp = _dev(inp)
    out = _run(w, inp, det=det)
    _check_all(w, inp, out)


def test_tiny_prenormalised_without_kernel_norm():
    """q, k L2-normalised on the host (same eps), kernel norm off: matches the oracle with the norm off."""
    w = syn.WORKLOADS["tiny"]
    inp = syn.make_inputs(w)
    for name in ("q", "k"):
        x = inp[name].double()
        inp[name] = (x / torch.sqrt((x * x).sum(-1, keepdim=True) + 1e-6)).float()
    inp = _dev(inp)
    out = _run(w, inp, l2norm=False)
    _check_all(w, inp, out, l2norm=False)


EDGE = [
    syn.custom("edge_tails", [1, 63, 64, 65, 127, 129, 0, 200], 2, 6, 128, "bf16", has_h0=True, want_ht=True,
               has_dht=True),
    syn.custom("edge_d64_f32", [70, 5, 130], 2, 4, 64, "f32", has_h0=True, want_ht=True, has_dht=True, seed=8),
    syn.custom("edge_g1", [64, 64, 1], 3, 3, 128, "bf16", seed=9),
    syn.custom("edge_g4_h0", [100, 33], 1, 4, 64, "bf16", has_h0=True, want_ht=True, seed=10),
    syn.custom("edge_empty_docs", [0, 0, 17, 0], 1, 3, 128, "bf16", has_h0=True, want_ht=True, has_dht=True,
               seed=11),
    # more value heads per q/k head than the deterministic chunk-gradient kernel parks in LDS
    syn.custom("edge_g10", [90, 40], 1, 10, 64, "bf16", seed=12),
    # the longest document (79 chunks) is far longer than the others and sits between them: its
    # intra and walk launches run apart from the others', whose chunk range wraps around it
    syn.custom("split_mid", [700, 5000, 129, 1000], 2, 6, 128, "bf16", has_h0=True, want_ht=True, has_dht=True,
               seed=13),
    # the same two-part plan at d = 64 with f32 inputs, the longest document first
    syn.custom("split_d64_f32", [6000, 700, 65, 1200], 2, 4, 64, "f32", has_h0=True, want_ht=True, has_dht=True,
               seed=14),
]


@pytest.mark.parametrize("w", EDGE, ids=[w.name for w in EDGE])
@pytest.mark.parametrize("det", [True, False])
def test_edge_cases(w, det):
    inp = _dev(syn.make_inputs(w))
    out = _run(w, inp, det=det)
    _check_all(w, inp, out)


# More documents than the chunk tables order by length (above 8,192 they keep the identity order,
# the paired walks alternate their two kinds, and neither the two-part plan nor segments apply):
# 9,000 documents of 0..24 tokens (395 empty), every element compared.
MANY = syn.custom("many_docs", np.random.default_rng(21).integers(0, 25, size=9000).tolist(), 1, 2, 64, "bf16",
                  seed=21)


@pytest.mark.parametrize("det", [True, False])
def test_many_documents_identity_order(det):
    assert MANY.N > 8192
    inp = _dev(syn.make_inputs(MANY))
    out = _run(MANY, inp, det=det)
    _check_all(MANY, inp, out)


def _saved_regions(w, full):
    """Byte offsets of the saved set's regions: a 256-byte tag, then each region aligned to 256."""
    NT = sum((L + 63) // 64 for L in w.lengths)
    T, HV, d = w.T, w.HV, w.d
    sizes = [("A", T * HV * 64 * 2), ("gcum", T * HV * 4), ("gamma", NT * HV * 4)]
    if full:
        sizes += [("H", NT * HV * d * d * 2), ("R", T * HV * d * 2), ("W", T * HV * d * 2), ("U", T * HV * d * 2),
                  ("P", T * HV * 64 * 2)]
    off, out = 256, {}
    for name, n in sizes:
        out[name] = (off, n)
        off = (off + n + 255) // 256 * 256
    return out, NT


@pytest.mark.parametrize("name", ["edge_tails", "edge_d64_f32"])
def test_full_saved_set_against_oracle(name):
    """Every region of the full saved set (A, gcum, gamma; the chunk start states, v_new, w, u and
    the P rows) against the FP64 chunked oracle, with ragged chunks, empty documents and h0."""
    w = [x for x in EDGE if x.name == name][0]
    inp = _dev(syn.make_inputs(w))
    out = _run(w, inp, save_mode=G.SAVE_FULL, bwd=False)
    h, _, _ = host_inputs(inp, None, None, w.HV // w.H)
    ref = oracle.chunked_fwd(h["cu"], h["q"], h["k"], h["v"], h["g"], h["beta"], h["h0"], l2norm=w.l2norm,
                             chunk=64, full=True)
    regions, NT = _saved_regions(w, True)
    raw = out["saved"]

    def view(key, dtype, shape):
        off, n = regions[key]
        return raw[off:off + n].view(dtype).reshape(shape)

    T, HV, d = w.T, w.HV, w.d
    assert_close("A", view("A", torch.bfloat16, (T, HV, 64)), ref["A"])
    assert_close("gcum", view("gcum", torch.float32, (HV, T)).t(), ref["gcum"])
    assert_close("gamma", view("gamma", torch.float32, (NT, HV)), ref["gamma"])
    # the state tape is stored transposed: [chunk][v head][value][key]
    assert_close("h tape", view("H", torch.bfloat16, (NT, HV, d, d)).transpose(2, 3), ref["H"])
    assert_close("v_new", view("R", torch.bfloat16, (T, HV, d)), ref["R"])
    assert_close("w", view("W", torch.bfloat16, (T, HV, d)), ref["W"])
    assert_close("u", view("U", torch.bfloat16, (T, HV, d)), ref["U"])
    assert_close("Aqk", view("P", torch.bfloat16, (T, HV, 64)), ref["P"])


def test_all_documents_empty():
    w = syn.custom("all_empty", [0, 0], 1, 2, 64, "bf16", has_h0=True, want_ht=True, has_dht=True)
    inp = _dev(syn.make_inputs(w))
    out = _run(w, inp)
    assert torch.equal(out["ht"], inp["h0"])
    assert torch.equal(out["dh0"], inp["dht"])


def test_light_equals_full_bitwise():
    w = EDGE[0]
    inp = _dev(syn.make_inputs(w))
    a = _run(w, inp, save_mode=G.SAVE_LIGHT, det=True)
    b = _run(w, inp, save_mode=G.SAVE_FULL, det=True)
    for k in ("o", "ht", "dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert torch.equal(a[k], b[k]), k


def test_split_launch_light_full_recompute_bitwise():
    """With the longest document's work on its own stream: light, full and checkpointed runs agree
    bitwise (the full forward writes the state tape from the split walk, the full backward runs
    the split reverse walk alone)."""
    w = [x for x in EDGE if x.name == "split_mid"][0]
    inp = _dev(syn.make_inputs(w))
    a = _run(w, inp, save_mode=G.SAVE_LIGHT, det=True, segments=1)
    b = _run(w, inp, save_mode=G.SAVE_FULL, det=True, recompute=True, segments=1)
    assert torch.equal(b["saved"], b["saved_recompute"])
    for k in ("o", "ht", "dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("det", [True, False])
def test_split_plan_d64_f32(det):
    """The two-part launch plan (the longest document's intra pass, walks and chunk gradients on the
    caller's stream, the others' on the auxiliary stream, each chunk-gradient part with its own
    work queue) at d = 64 with f32 inputs, against the oracle."""
    w = [x for x in EDGE if x.name == "split_d64_f32"][0]
    inp = _dev(syn.make_inputs(w))
    out = _run(w, inp, det=det, segments=1)
    _check_all(w, inp, out)


def test_split_walk_in_pieces():
    """The longest document (770 chunks) is walked in two pieces that hand the f32 state over
    through the workspace; with h0, ht and dht, against the oracle, and light == full bitwise
    (the full forward's state tape comes from the pieced walk)."""
    w = syn.custom("pieces", [3000, 49252, 700], 1, 2, 64, "bf16", has_h0=True, want_ht=True, has_dht=True,
                   seed=14)
    inp = _dev(syn.make_inputs(w))
    a = _run(w, inp, save_mode=G.SAVE_LIGHT, det=True, segments=1)
    _check_all(w, inp, a)
    b = _run(w, inp, save_mode=G.SAVE_FULL, det=True, segments=1)
    for k in ("o", "ht", "dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert torch.equal(a[k], b[k]), k


def test_concurrent_calls_on_two_streams_bitwise():
    """Two host threads run fwd + bwd at once, each on its own stream and auxiliary stream, on a
    problem whose longest document runs apart on the auxiliary stream: each result equals the
    sequential one bitwise."""
    import threading

    w = [x for x in EDGE if x.name == "split_mid"][0]
    inp = _dev(syn.make_inputs(w))
    ref = _run(w, inp, det=True, segments=1)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    aux_streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [None, None]
    errs = []

    def work(i):
        try:
            with torch.cuda.stream(streams[i]):
                p = G.problem_for(w, deterministic=True, use_aux_stream=aux_streams[i], segments=1)
                a = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"])
                o, ht, saved = G.gdn_fwd(p, *a, h0=inp["h0"], stream=streams[i])
                gr = G.gdn_bwd(p, *a, saved, inp["dO"], h0=inp["h0"], dht=inp["dht"], stream=streams[i])
                streams[i].synchronize()
                outs[i] = dict(o=o, ht=ht, **gr)
        except Exception as e:  # reported below
            errs.append(e)

    torch.cuda.synchronize()
    th = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errs, errs
    for out in outs:
        for k in ("o", "ht", "dq", "dk", "dv", "dg", "dbeta", "dh0"):
            assert torch.equal(out[k], ref[k]), k


def test_recompute_saved_set_bitwise_and_ckpt():
    w = EDGE[0]
    inp = _dev(syn.make_inputs(w))
    a = _run(w, inp, det=True)
    b = _run(w, inp, det=True, recompute=True)
    assert torch.equal(b["saved"], b["saved_recompute"])
    for k in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert torch.equal(a[k], b[k]), k


def test_deterministic_bitwise_repeat_and_nan_poison():
    """Deterministic mode is bitwise reproducible, also when every output, the saved set and the
    workspaces start out NaN-filled (nothing reads a buffer before writing it)."""
    w = EDGE[0]
    inp = _dev(syn.make_inputs(w))
    a = _run(w, inp, det=True)
    b = _run(w, inp, det=True, poison=True)
    for k in ("o", "ht", "dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert torch.isfinite(b[k]).all(), k
        assert torch.equal(a[k], b[k]), k


def test_atomic_close_to_deterministic():
    w = EDGE[0]
    inp = _dev(syn.make_inputs(w))
    a = _run(w, inp, det=True)
    b = _run(w, inp, det=False, poison=True)
    assert torch.equal(a["dh0"], b["dh0"])  # same reverse-walk kernel in both modes
    for k in ("dq", "dk", "dv", "dg", "dbeta"):
        assert_close(k, b[k], a[k])


def _bwd_with(p, inp, saved):
    a = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"])
    ws = torch.zeros((G.gdn_workspace_bytes(p, G.OP_BWD),), dtype=torch.uint8, device=DEV)
    gr = G.gdn_bwd(p, *a, saved, inp["dO"], h0=inp["h0"], dht=inp["dht"], workspace=ws)
    st = G.gdn_status(p, G.OP_BWD, ws)
    return gr, st


def test_saved_tag_checked_on_device():
    """The backward's first kernel compares the saved set's tag with its own problem: a saved set
    written for another save mode, or a buffer whose address now holds other data, yields
    GDN_ESAVED from gdn_status and all-NaN gradients; a copy of a valid saved set at another
    address is accepted and gives the same bits."""
    w = EDGE[0]
    inp = _dev(syn.make_inputs(w))
    ref = _run(w, inp, det=True)
    assert ref["status"] == G.GDN_OK
    # written for the light form, read as the full form
    p_full = G.problem_for(w, save_mode=G.SAVE_FULL, deterministic=True)
    gr, st = _bwd_with(p_full, inp, torch.zeros(G.gdn_saved_bytes(p_full), dtype=torch.uint8, device=DEV))
    assert st == G.GDN_ESAVED
    for k in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert torch.isnan(gr[k]).all(), k
    # a valid saved set copied elsewhere (moved, offloaded and brought back) is accepted
    p = G.problem_for(w, deterministic=True)
    moved = ref["saved"].clone()
    gr, st = _bwd_with(p, inp, moved)
    assert st == G.GDN_OK
    for k in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert torch.equal(gr[k], ref[k]), k
    # the original address now holds other data (as after the buffer was freed and reused)
    ref["saved"].copy_(torch.randint(0, 256, ref["saved"].shape, dtype=torch.uint8, device=DEV))
    gr, st = _bwd_with(p, inp, ref["saved"])
    assert st == G.GDN_ESAVED
    assert all(torch.isnan(gr[k]).all() for k in ("dq", "dk", "dv", "dg", "dbeta", "dh0"))
    # a saved set of another problem (one token fewer in the last document)
    w2 = syn.custom("edge_tails_short", list(w.lengths[:-1]) + [w.lengths[-1] - 1], w.H, w.HV, w.d, w.dtype,
                    has_h0=True, want_ht=True, has_dht=True)
    inp2 = _dev(syn.make_inputs(w2))
    other = _run(w2, inp2, det=True, bwd=False)
    gr, st = _bwd_with(p, inp, torch.cat([other["saved"], torch.zeros(ref["saved"].numel() - other["saved"].numel(),
                                                                      dtype=torch.uint8, device=DEV)]))
    assert st == G.GDN_ESAVED


def test_device_cu_seqlens_mismatch_poisons_outputs():
    """A device cu_seqlens that disagrees with the host copy: the tables kernel sees a different
    chunk count, every kernel skips its work, the outputs are NaN and gdn_status reports it."""
    w = EDGE[0]
    inp = _dev(syn.make_inputs(w))
    p = G.problem_for(w, deterministic=True)
    bad_cu = inp["cu_seqlens"].clone()
    bad_cu[1] = bad_cu[1] + 64  # one chunk more in the first document, one fewer later
    a = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], bad_cu)
    ws = torch.zeros((G.gdn_workspace_bytes(p, G.OP_FWD),), dtype=torch.uint8, device=DEV)
    o, ht, saved = G.gdn_fwd(p, *a, h0=inp["h0"], workspace=ws)
    assert G.gdn_status(p, G.OP_FWD, ws) == G.GDN_EINVAL
    assert torch.isnan(o).all() and torch.isnan(ht).all()
    gr, st = _bwd_with(p, inp, saved)  # the failed forward wrote a zero tag
    assert st == G.GDN_ESAVED


@pytest.mark.parametrize("name", ["split_mid", "pieces"])
def test_single_stream_bitwise(name):
    """Without an auxiliary stream every launch goes to the caller's stream (no split of the launch
    plan): outputs and gradients equal the two-stream run bitwise, in every saved-set form."""
    if name == "pieces":
        w = syn.custom("pieces", [3000, 49252, 700], 1, 2, 64, "bf16", has_h0=True, want_ht=True, has_dht=True,
                       seed=14)
    else:
        w = [x for x in EDGE if x.name == name][0]
    inp = _dev(syn.make_inputs(w))
    for mode in (G.SAVE_LIGHT, G.SAVE_FULL):
        a = _run(w, inp, save_mode=mode, det=True, aux=True, segments=1)
        b = _run(w, inp, save_mode=mode, det=True, aux=False, segments=1)
        assert torch.equal(a["saved"], b["saved"])
        for k in ("o", "ht", "dq", "dk", "dv", "dg", "dbeta", "dh0"):
            assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("name", ["edge_tails", "split_mid"])
def test_kept_tape_checkpoint_bitwise(name):
    """Checkpointed step with kept tapes: fwd (light), recompute (kept-tape form) and bwd (kept-tape
    form, no replay walk) give the gradients of the light fwd + bwd bitwise; fwd and bwd in the
    kept-tape form as well."""
    w = [x for x in EDGE if x.name == name][0]
    inp = _dev(syn.make_inputs(w))
    ref = _run(w, inp, det=True)
    ck = _run(w, inp, det=True, recompute=True, recompute_mode=G.SAVE_TAPE)
    kt = _run(w, inp, save_mode=G.SAVE_TAPE, det=True)
    for k in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert torch.equal(ck[k], ref[k]), k
        assert torch.equal(kt[k], ref[k]), k
    assert torch.equal(kt["o"], ref["o"]) and torch.equal(kt["ht"], ref["ht"])
    # the kept-tape recompute writes the light set bitwise and the tape as the full forward does
    full = _run(w, inp, save_mode=G.SAVE_FULL, det=True, bwd=False)
    regions, _ = _saved_regions(w, True)
    off, n = regions["H"]
    end_light = regions["gamma"][0] + regions["gamma"][1]
    sv = ck["saved_recompute"]
    assert torch.equal(sv[256:end_light], ref["saved"][256:end_light])
    assert torch.equal(sv[off:off + n], full["saved"][off:off + n])


# ------------------------------------------------------------------------------------------
# full-size workloads, sampled


def _big(name):
    w = syn.WORKLOADS[name]
    torch.cuda.empty_cache()
    return w, syn.make_inputs(w, device=DEV)


def test_single8k_fwd():
    w, inp = _big("single8k")
    out = _run(w, inp, bwd=False)
    _check_all(w, inp, out, bwd=False)  # every head


def test_pack262k_fwd_bwd_atomic():
    w, inp = _big("pack262k")
    out = _run(w, inp, det=False)
    for k in ("o", "dq", "dk", "dv", "dg", "dbeta"):
        assert torch.isfinite(out[k]).all(), k
    # the longest document (its own stream, walked in pieces) and the shortest
    _check_all(w, inp, out, docs=[0, 3], heads=[2, 13])


def test_pack262k_deterministic_repeat():
    w, inp = _big("pack262k")
    a = _run(w, inp, det=True)
    dq, dk = a["dq"].clone(), a["dk"].clone()
    del a
    b = _run(w, inp, det=True)
    assert torch.equal(dq, b["dq"]) and torch.equal(dk, b["dk"])
    _check_all(w, inp, b, docs=[0, 3], heads=[5])


def test_pack262k_longest_document_alone_bitwise():
    """The pack's longest document (98,304 tokens) runs apart from the others, its walk in pieces
    that hand the f32 state over; packed twice (two equal documents: no part is the longest, one
    launch per kernel, one walk per chain) it gives the same bits."""
    w, inp = _big("pack262k")
    assert not w.has_h0
    a = _run(w, inp, det=True, segments=1)
    L0 = w.lengths[0]
    w2 = syn.custom("pack_doc0_twice", [L0, L0], w.H, w.HV, w.d, w.dtype, want_ht=True)  # unsegmented below
    two = {k: (torch.cat([v[:L0], v[:L0]]).contiguous() if v is not None and k not in ("cu_seqlens", "h0", "dht")
               else v) for k, v in inp.items()}
    two["cu_seqlens"] = torch.tensor([0, L0, 2 * L0], dtype=torch.int32, device=DEV)
    a_o = a["o"][:L0].clone()
    grads = {k: a[k][:L0].clone() for k in ("dq", "dk", "dv", "dg", "dbeta")}
    del a
    torch.cuda.empty_cache()
    b = _run(w2, two, det=True, segments=1)
    for half in (slice(0, L0), slice(L0, 2 * L0)):
        assert torch.equal(a_o, b["o"][half])
        for k, v in grads.items():
            assert torch.equal(v, b[k][half]), k


@pytest.mark.parametrize("dht", [True, False], ids=["dht", "no_dht"])
def test_cp4share_h0_ht_dh0(dht):
    """Both fragments of the share (the 40,960-token first one runs apart from the second, with h0),
    with the final-state gradient given and absent."""
    w, inp = _big("cp4share")
    out = _run(w, inp, dht=dht)
    _check_all(w, inp, out, docs=[0, 1], heads=[0, 9], dht=dht)


def test_pack262k_ckpt_and_full_saved_set():
    """The packed workload's checkpointed op (fwd, recompute, bwd) against the oracle on sampled
    documents and heads, and its full saved set region by region against the chunked oracle on the
    shortest document for one q/k head group."""
    w, inp = _big("pack262k")
    out = _run(w, inp, det=True, recompute=True)
    assert torch.equal(out["saved"], out["saved_recompute"])
    _check_all(w, inp, out, docs=[0, 3], heads=[7])
    del out
    torch.cuda.empty_cache()
    full = _run(w, inp, save_mode=G.SAVE_FULL, det=True, bwd=False)
    n, j = 3, 11
    Gg = w.HV // w.H
    h, ti, vh = host_inputs(inp, [n], [j], Gg)
    ref = oracle.chunked_fwd(h["cu"], h["q"], h["k"], h["v"], h["g"], h["beta"], None, l2norm=True, chunk=64,
                             full=True)
    regions, NT = _saved_regions(w, True)
    raw = full["saved"]
    T, HV, d = w.T, w.HV, w.d
    c0 = sum(L // 64 for L in w.lengths[:n])
    nc = w.lengths[n] // 64

    def view(key, dtype, shape):
        off, nb = regions[key]
        return raw[off:off + nb].view(dtype).reshape(shape)

    assert_close("A", view("A", torch.bfloat16, (T, HV, 64)).index_select(0, ti)[:, vh], ref["A"])
    assert_close("gcum", view("gcum", torch.float32, (HV, T)).t().index_select(0, ti)[:, vh], ref["gcum"])
    assert_close("gamma", view("gamma", torch.float32, (NT, HV))[c0:c0 + nc][:, vh], ref["gamma"])
    assert_close("h tape", view("H", torch.bfloat16, (NT, HV, d, d))[c0:c0 + nc][:, vh].transpose(2, 3), ref["H"])
    for key, name in (("R", "v_new"), ("W", "w"), ("U", "u")):
        assert_close(name, view(key, torch.bfloat16, (T, HV, d)).index_select(0, ti)[:, vh], ref[key])
    assert_close("Aqk", view("P", torch.bfloat16, (T, HV, 64)).index_select(0, ti)[:, vh], ref["P"])


def test_short512_ckpt_deterministic():
    w, inp = _big("short512")
    out = _run(w, inp, det=True, recompute=True)
    assert torch.equal(out["saved"], out["saved_recompute"])
    lens = np.asarray(w.lengths)
    docs = sorted(set([int(np.argmin(lens)), int(np.argmax(lens))] + list(range(0, w.N, 64))))
    _check_all(w, inp, out, docs=docs, heads=[3, 12])
