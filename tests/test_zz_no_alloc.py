"""The forward entry point that allocates nothing (gdn_fwd_noalloc, through the C ABI): its
workspace is the library's fixed device scratch array. Two calls in a row, the second with a
smaller problem (the array keeps the first call's contents), each equal bitwise to gdn_fwd with a
workspace of its own and within the accuracy budget of the oracle; a problem near the array's
size; and the host-side refusal of a problem whose forward workspace exceeds it."""
import numpy as np
import pytest
import torch

import gated_deltanet_fwd_amd as G
import synthetic as syn
from parity_util import assert_close, host_inputs, oracle_fwd

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dev(inp):
    return {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}


def _both(w, check_oracle=True, segments=0):
    inp = _dev(syn.make_inputs(w))
    p = G.problem_for(w, use_aux_stream=False, segments=segments)
    a = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"])
    # both saved buffers start with the same bytes: the alignment gaps between the saved regions
    # and the tag's unused words are never written
    saved_ref = torch.full((G.gdn_saved_bytes(p),), 255, dtype=torch.uint8, device=DEV)
    o_ref, ht_ref, saved_ref = G.gdn_fwd(p, *a, h0=inp["h0"], saved=saved_ref)
    nan = float("nan")
    o = torch.full_like(o_ref, nan)
    ht = torch.full_like(ht_ref, nan) if ht_ref is not None else None
    saved = torch.full_like(saved_ref, 255)
    print("gdn_fwd_noalloc: %s T=%d (H,HV)=(%d,%d) d=%d, workspace %d bytes" %
          (w.name, w.T, w.H, w.HV, w.d, G.gdn_workspace_bytes(p, G.OP_FWD)), flush=True)
    G.gdn_fwd_noalloc(p, *a, h0=inp["h0"], o=o, ht=ht, saved=saved)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    if ht_ref is not None:
        assert torch.equal(ht, ht_ref)
    assert torch.equal(saved, saved_ref)
    if check_oracle:
        h, ti, vh = host_inputs(inp, None, None, w.HV // w.H)
        o_or, ht_or = oracle_fwd(h, w.l2norm)
        assert_close("o", o.index_select(0, ti)[:, vh], o_or)
        if ht is not None:
            assert_close("ht", ht[:, vh], ht_or)


def test_noalloc_two_calls_second_smaller():
    big = syn.custom("noalloc_big", [700, 129, 1000, 64, 3], 2, 6, 128, "bf16", has_h0=True, want_ht=True, seed=21)
    small = syn.custom("noalloc_small", [65, 200], 1, 3, 64, "bf16", has_h0=True, want_ht=True, seed=22)
    _both(big)
    _both(small)


def test_noalloc_near_the_array_size():
    """The 8,192-token document at (16, 48), d = 128, unsegmented: a forward workspace of about
    55 MiB. (The library's plan walks it in 4 segments, whose transfer matrices take it past the
    array: that call is refused.)"""
    w = syn.WORKLOADS["single8k"]
    p = G.problem_for(w, segments=1)
    assert G.gdn_workspace_bytes(p, G.OP_FWD) > (48 << 20)
    _both(w, check_oracle=False, segments=1)
    assert G.gdn_workspace_bytes(G.problem_for(w), G.OP_FWD) > (64 << 20)


def test_noalloc_refuses_a_problem_beyond_the_array():
    w = syn.custom("noalloc_too_big", [16384], 16, 48, 128, "bf16")
    p = G.problem_for(w)
    assert G.gdn_workspace_bytes(p, G.OP_FWD) > (64 << 20)
    lib = G.load_library()
    rc = lib.gdn_fwd_noalloc(p.ref(), *([None] * 10), None)  # refused before any pointer is read
    assert rc == G.GDN_EWORKSPACE
    assert "scratch" in lib.gdn_last_error().decode()
