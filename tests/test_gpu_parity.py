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


def _run(w, inp, save_mode=G.SAVE_LIGHT, det=None, bwd=True, recompute=False, poison=False, l2norm=None):
    p = G.problem_for(w, save_mode=save_mode, deterministic=det, l2norm=l2norm)
    a = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"])
    fill = float("nan") if poison else 0.0
    o = torch.full_like(inp["v"], fill)
    ht = torch.full((w.N, w.HV, w.d, w.d), fill, dtype=torch.float32, device=DEV) if w.want_ht else None
    saved = torch.full((G.gdn_saved_bytes(p),), 255 if poison else 0, dtype=torch.uint8, device=DEV)
    ws = torch.full((G.gdn_workspace_bytes(p, G.OP_FWD),), 255 if poison else 0, dtype=torch.uint8, device=DEV)
    o, ht, saved = G.gdn_fwd(p, *a, h0=inp["h0"], o=o, ht=ht, saved=saved, workspace=ws)
    out = dict(o=o, ht=ht, saved=saved, p=p)
    if recompute:
        saved2 = torch.full_like(saved, 255 if poison else 0)
        ws2 = torch.full((G.gdn_workspace_bytes(p, G.OP_RECOMPUTE),), 255 if poison else 0, dtype=torch.uint8,
                         device=DEV)
        G.gdn_fwd_recompute(p, *a, h0=inp["h0"], saved=saved2, workspace=ws2)
        out["saved_recompute"] = saved2
    if bwd:
        grads = dict(dq=torch.full_like(inp["q"], fill), dk=torch.full_like(inp["k"], fill),
                     dv=torch.full_like(inp["v"], fill), dg=torch.full_like(inp["g"], fill),
                     dbeta=torch.full_like(inp["beta"], fill),
                     dh0=torch.full_like(inp["h0"], fill) if inp["h0"] is not None else None)
        wsb = torch.full((G.gdn_workspace_bytes(p, G.OP_BWD),), 255 if poison else 0, dtype=torch.uint8, device=DEV)
        G.gdn_bwd(p, *a, out.get("saved_recompute", saved), inp["dO"], h0=inp["h0"], dht=inp["dht"], grads=grads,
                  workspace=wsb)
        out.update(grads)
    torch.cuda.synchronize()
    return out


def _check_all(w, inp, out, docs=None, heads=None, bwd=True, l2norm=None):
    """Compare o, ht and the gradients on the sampled documents x q/k heads."""
    l2 = w.l2norm if l2norm is None else l2norm
    Gg = w.HV // w.H
    h, ti, vh = host_inputs(inp, docs, heads, Gg)
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
]


@pytest.mark.parametrize("w", EDGE, ids=[w.name for w in EDGE])
@pytest.mark.parametrize("det", [True, False])
def test_edge_cases(w, det):
    inp = _dev(syn.make_inputs(w))
    out = _run(w, inp, det=det)
    _check_all(w, inp, out)


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
    a = _run(w, inp, save_mode=G.SAVE_LIGHT, det=True)
    b = _run(w, inp, save_mode=G.SAVE_FULL, det=True, recompute=True)
    assert torch.equal(b["saved"], b["saved_recompute"])
    for k in ("o", "ht", "dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert torch.equal(a[k], b[k]), k


def test_split_walk_in_pieces():
    """The longest document (770 chunks) is walked in two pieces that hand the f32 state over
    through the workspace; with h0, ht and dht, against the oracle, and light == full bitwise
    (the full forward's state tape comes from the pieced walk)."""
    w = syn.custom("pieces", [3000, 49252, 700], 1, 2, 64, "bf16", has_h0=True, want_ht=True, has_dht=True,
                   seed=14)
    inp = _dev(syn.make_inputs(w))
    a = _run(w, inp, save_mode=G.SAVE_LIGHT, det=True)
    _check_all(w, inp, a)
    b = _run(w, inp, save_mode=G.SAVE_FULL, det=True)
    for k in ("o", "ht", "dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert torch.equal(a[k], b[k]), k


def test_concurrent_calls_on_two_streams_bitwise():
    """Two host threads run fwd + bwd at once, each on its own stream, on a problem whose longest
    document runs apart on the library's second stream (shared by both calls): each result equals
    the sequential one bitwise."""
    import threading

    w = [x for x in EDGE if x.name == "split_mid"][0]
    inp = _dev(syn.make_inputs(w))
    ref = _run(w, inp, det=True)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [None, None]
    errs = []

    def work(i):
        try:
            with torch.cuda.stream(streams[i]):
                p = G.problem_for(w, deterministic=True)
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


def test_saved_set_refused_for_other_problem():
    w = EDGE[0]
    inp = _dev(syn.make_inputs(w))
    a = _run(w, inp, bwd=False)
    p2 = G.problem_for(w, save_mode=G.SAVE_FULL)
    with pytest.raises(G.GdnError) as e:
        G.gdn_bwd(p2, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"], a["saved"], inp["dO"],
                  h0=inp["h0"], dht=inp["dht"])
    assert e.value.code == G.GDN_ESAVED


# ------------------------------------------------------------------------------------------
# full-size workloads, sampled


def _big(name):
    w = syn.WORKLOADS[name]
    torch.cuda.empty_cache()
    return w, syn.make_inputs(w, device=DEV)


def test_single8k_fwd():
    w, inp = _big("single8k")
    out = _run(w, inp, bwd=False)
    _check_all(w, inp, out, heads=[0, 15], bwd=False)


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
    a = _run(w, inp, det=True)
    L0 = w.lengths[0]
    w2 = syn.custom("pack_doc0_twice", [L0, L0], w.H, w.HV, w.d, w.dtype, want_ht=True)
    two = {k: (torch.cat([v[:L0], v[:L0]]).contiguous() if v is not None and k not in ("cu_seqlens", "h0", "dht")
               else v) for k, v in inp.items()}
    two["cu_seqlens"] = torch.tensor([0, L0, 2 * L0], dtype=torch.int32, device=DEV)
    a_o = a["o"][:L0].clone()
    grads = {k: a[k][:L0].clone() for k in ("dq", "dk", "dv", "dg", "dbeta")}
    del a
    torch.cuda.empty_cache()
    b = _run(w2, two, det=True)
    for half in (slice(0, L0), slice(L0, 2 * L0)):
        assert torch.equal(a_o, b["o"][half])
        for k, v in grads.items():
            assert torch.equal(v, b[k][half]), k


def test_cp4share_h0_ht_dh0():
    w, inp = _big("cp4share")
    out = _run(w, inp)
    _check_all(w, inp, out, docs=[1], heads=[0, 9])


def test_short512_ckpt_deterministic():
    w, inp = _big("short512")
    out = _run(w, inp, det=True, recompute=True)
    assert torch.equal(out["saved"], out["saved_recompute"])
    lens = np.asarray(w.lengths)
    docs = sorted(set([int(np.argmin(lens)), int(np.argmax(lens))] + list(range(0, w.N, 64))))
    _check_all(w, inp, out, docs=docs, heads=[3, 12])
