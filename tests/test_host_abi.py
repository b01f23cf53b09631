"""Host-side checks of the C ABI that need no GPU: exports, byte queries, validation errors.

No call here reaches a kernel launch: every invalid call is rejected by host validation, which
runs before the first launch.
"""
import ctypes
import json
import os
import re

import numpy as np
import pytest
import torch

import gated_deltanet_fwd_amd as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    return G.load_library()


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "gdn.h")).read()
    declared = set(re.findall(r"^[A-Za-z_][\w \*]*?\b(gdn_\w+)\s*\(", hdr, flags=re.M))
    assert {"gdn_fwd", "gdn_bwd", "gdn_fwd_recompute", "gdn_saved_bytes", "gdn_workspace_bytes"} <= declared
    lib = _lib()
    for name in sorted(declared):
        assert hasattr(lib, name), "libgdn.so does not export %s" % name
    assert lib.gdn_abi_version() == G.ABI_VERSION == 2


def _prob(lengths, H=16, HV=48, d=128, save_mode=G.SAVE_LIGHT, **kw):
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    return G.Problem(cu, H, HV, d, save_mode=save_mode, **kw)


def test_saved_bytes_match_pages():
    """Light and full saved sets at the pages' shape (HV = 48, d = 128, 64-token chunks, all chunks
    full) match the README saved-set table's per-token figures."""
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "saved_set_bytes.json")))
    lengths = [98304, 65536, 57344, 40960]
    T = sum(lengths)
    light = G.gdn_saved_bytes(_prob(lengths, HV=gold["HV"], d=gold["d"]))
    full = G.gdn_saved_bytes(_prob(lengths, HV=gold["HV"], d=gold["d"], save_mode=G.SAVE_FULL))
    assert (light - 256) == gold["light_bytes_per_token"] * T
    assert (full - light) == gold["full_extra_bytes_per_token"] * T


def _align(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("lengths,H,HV,d", [([1, 63, 65, 0, 129], 2, 6, 128), ([70], 1, 1, 64), ([3, 4], 4, 8, 64)])
def test_saved_and_workspace_formula(lengths, H, HV, d):
    T = sum(lengths)
    NT = sum((L + 63) // 64 for L in lengths)
    light = 256 + _align(T * HV * 64 * 2) + _align(T * HV * 4) + _align(NT * HV * 4)
    assert G.gdn_saved_bytes(_prob(lengths, H, HV, d)) == light
    tape = _align(NT * HV * d * d * 2)
    full = light + tape + 3 * _align(T * HV * d * 2) + _align(T * HV * 64 * 2)
    assert G.gdn_saved_bytes(_prob(lengths, H, HV, d, save_mode=G.SAVE_FULL)) == full
    assert G.gdn_saved_bytes(_prob(lengths, H, HV, d, save_mode=G.SAVE_TAPE)) == light + tape
    wf = G.gdn_workspace_bytes(_prob(lengths, H, HV, d), G.OP_FWD)
    wb = G.gdn_workspace_bytes(_prob(lengths, H, HV, d), G.OP_BWD)
    wb_atomic = G.gdn_workspace_bytes(_prob(lengths, H, HV, d, deterministic=False), G.OP_BWD)
    assert wf >= NT * H * 64 * 64 * 2 + HV * d * d * 4  # tables, q.k, norms; the state between walk pieces
    assert wb >= wf - HV * d * d * 4 + 2 * NT * HV * d * d * 2  # the same but that state, plus two tapes
    assert wb_atomic >= wb + 2 * T * H * d * 4
    # the kept-tape and full backwards read the state tape from the saved set: one tape fewer
    for mode in (G.SAVE_FULL, G.SAVE_TAPE):
        assert G.gdn_workspace_bytes(_prob(lengths, H, HV, d, save_mode=mode), G.OP_BWD) == wb - tape


@pytest.mark.parametrize("bad,fragment", [
    (dict(HV=47), "multiple"),
    (dict(d=96), "64 or 128"),
    (dict(lengths=[5, -1]), "decreases"),
    (dict(H=0), "head counts"),
])
def test_invalid_problem_rejected(bad, fragment):
    kw = dict(lengths=[10, 20], H=16, HV=48, d=128)
    kw.update(bad)
    lengths = kw.pop("lengths")
    if min(lengths) < 0:
        cu = np.array([0, 5, 4], np.int32)
        p = G.Problem(cu, kw["H"], kw["HV"], kw["d"])
    else:
        p = _prob(lengths, **kw)
    assert _lib().gdn_saved_bytes(p.ref()) == 0
    assert fragment in _lib().gdn_last_error().decode()


def test_n_tokens_mismatch_rejected():
    p = _prob([10, 20])
    p.st.n_tokens = 31
    assert _lib().gdn_saved_bytes(p.ref()) == 0
    assert "n_tokens" in _lib().gdn_last_error().decode()


class _Fake:
    """Stands in for a device tensor: an aligned address that is never dereferenced."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def _fake(i=1, misalign=0):
    return _Fake(0x100000 * i + misalign)


def _call_fwd(p, q=None, workspace_bytes=None, **over):
    lib = _lib()
    args = dict(q=_fake(1), k=_fake(2), v=_fake(3), g=_fake(4), beta=_fake(5), cu=_fake(6), h0=None, o=_fake(7),
                ht=None, saved=_fake(8), ws=_fake(9))
    args.update(over)
    if q is not None:
        args["q"] = q
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    nbytes = workspace_bytes if workspace_bytes is not None else G.gdn_workspace_bytes(p, G.OP_FWD)
    return lib.gdn_fwd(p.ref(), P(args["q"]), P(args["k"]), P(args["v"]), P(args["g"]), P(args["beta"]),
                       P(args["cu"]), P(args["h0"]), P(args["o"]), P(args["ht"]), P(args["saved"]), P(args["ws"]),
                       nbytes, None)


def test_fwd_rejects_null_and_misaligned_pointers():
    p = _prob([100, 28])
    class Null:
        def data_ptr(self):
            return 0
    assert _call_fwd(p, q=Null()) == G.GDN_EINVAL
    assert "q is NULL" in _lib().gdn_last_error().decode()
    assert _call_fwd(p, q=_fake(1, misalign=4)) == G.GDN_EINVAL
    assert "aligned" in _lib().gdn_last_error().decode()


def test_fwd_rejects_missing_h0_and_ht():
    p = _prob([100], has_h0=True)
    assert _call_fwd(p) == G.GDN_EINVAL and "h0" in _lib().gdn_last_error().decode()
    p = _prob([100], want_ht=True)
    assert _call_fwd(p) == G.GDN_EINVAL and "ht" in _lib().gdn_last_error().decode()


def test_fwd_rejects_small_workspace():
    p = _prob([100, 28])
    need = G.gdn_workspace_bytes(p, G.OP_FWD)
    assert _call_fwd(p, workspace_bytes=need - 1) == G.GDN_EWORKSPACE


def test_reserved_and_segment_fields_validated():
    p = _prob([100, 28])
    p.st.reserved0 = 1
    assert _lib().gdn_saved_bytes(p.ref()) == 0 and "reserved0" in _lib().gdn_last_error().decode()
    p = _prob([100, 28])
    p.st.segments = -1
    assert _lib().gdn_saved_bytes(p.ref()) == 0 and "segments" in _lib().gdn_last_error().decode()
    p = _prob([100, 28])
    p.st.save_mode = 3
    assert _lib().gdn_saved_bytes(p.ref()) == 0 and "save_mode" in _lib().gdn_last_error().decode()


def test_status_rejects_unknown_op():
    p = _prob([100, 28])
    assert _lib().gdn_status(p.ref(), 7, ctypes.c_void_p(_fake(1).data_ptr()), None) == G.GDN_EINVAL
    assert "unknown op" in _lib().gdn_last_error().decode()


def test_binding_refuses_without_library(tmp_path):
    with pytest.raises(OSError):
        G._lib_backup = G._lib
        try:
            G._lib = None
            G.load_library(str(tmp_path / "missing.so"))
        finally:
            G._lib = G._lib_backup


def test_conv_problem_validation_and_workspace():
    lens = [1024, 1, 2000]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    p = G.ConvProblem(cu, [2048, 2048, 6144], width=4)
    blocks = (sum(lens) + 511) // 512  # workgroups of 4 waves x 128 tokens
    assert G.gdn_conv_workspace_bytes(p) == _align(blocks * 10240 * 5 * 4)
    for groups, width, frag in (([2048, 12], 4, "multiple of 8"), ([2048], 5, "width"), ([8, 8, 8, 8, 8], 4, "n_groups")):
        q = G.ConvProblem(cu, groups[:4], width=width)
        if len(groups) > 4:
            q.st.n_groups = 5
        assert _lib().gdn_conv_workspace_bytes(q.ref()) == 0
        assert frag in _lib().gdn_last_error().decode()
    q = G.ConvProblem(cu, [16, 16])
    q.st.channels = 40
    assert _lib().gdn_conv_workspace_bytes(q.ref()) == 0 and "sum of group_channels" in _lib().gdn_last_error().decode()


def test_segmented_workspace_carry_slots():
    """A document of 128 chunks walked as 4 segments keeps 2 transfer matrices and 2 zero-start end
    states (f32 [HV, d, d] each) in the forward and recompute workspaces, and its 3 segment start
    states (the carry plane) at the end of the saved set, in every form; a document shorter than
    two segments' minimum length is not split."""
    HV, d = 6, 128
    base = G.gdn_workspace_bytes(_prob([8192], 2, HV, d, segments=1), G.OP_FWD)
    seg = G.gdn_workspace_bytes(_prob([8192], 2, HV, d, segments=4), G.OP_FWD)
    assert seg - base == _align(4 * HV * d * d * 4)
    for mode in (G.SAVE_LIGHT, G.SAVE_FULL, G.SAVE_TAPE):
        assert G.gdn_saved_bytes(_prob([8192], 2, HV, d, segments=4, save_mode=mode)) == \
            G.gdn_saved_bytes(_prob([8192], 2, HV, d, segments=1, save_mode=mode)) + _align(3 * HV * d * d * 4)
    assert G.gdn_workspace_bytes(_prob([8192], 2, HV, d, segments=4, save_mode=G.SAVE_TAPE), G.OP_RECOMPUTE) > \
        G.gdn_workspace_bytes(_prob([8192], 2, HV, d, segments=1, save_mode=G.SAVE_TAPE), G.OP_RECOMPUTE)
    # 15 chunks: fewer than two segments of 8 chunks, so one segment and no carry slots
    assert G.gdn_workspace_bytes(_prob([960], 2, HV, d, segments=4), G.OP_FWD) == \
        G.gdn_workspace_bytes(_prob([960], 2, HV, d, segments=1), G.OP_FWD)
    # the backward keeps no transfer matrices (it replays from the saved start states)
    assert G.gdn_workspace_bytes(_prob([8192], 2, HV, d, segments=4), G.OP_BWD) == \
        G.gdn_workspace_bytes(_prob([8192], 2, HV, d, segments=1), G.OP_BWD)


def test_library_segment_plan():
    """segments = 0: the library's count from the shape and the CU count (256 without a device):
    the 8,192-token document at (16, 48) is split in 4, the two-fragment share in 3, the 4-document
    pack not at all (its chains already fill the CUs)."""
    HV, d = 48, 128
    extra = lambda lengths, segs: (G.gdn_saved_bytes(_prob(lengths, 16, HV, d, segments=segs)) -
                                   G.gdn_saved_bytes(_prob(lengths, 16, HV, d, segments=1)))
    plane = lambda k: _align(k * HV * d * d * 4)
    assert extra([8192], 0) == plane(3) == extra([8192], 4)
    assert extra([40960, 24576], 0) == plane(4) == extra([40960, 24576], 3)
    assert extra([98304, 65536, 57344, 40960], 0) == 0
