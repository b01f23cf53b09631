"""FP64 CPU oracle for the gated delta rule training kernel (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use this module;
the product path (the HIP library and its binding) never imports it, and it imports
nothing from the product.

Arithmetic lives in ``gdn_oracle.c`` (plain C, double precision); this file only marshals
numpy arrays into it. What it computes, and the reading of the pages it follows, is stated
in the C file's header: the gated delta rule with decay applied before the delta update,
an optional q/k L2 norm, grouped value heads (v head h reads q/k head h // (HV // H)) and
packed documents delimited by ``cu_seqlens`` (flashinfer PR #8172, PR description; README
saved-set table quoted in flashinfer PR #8542).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_liboracle.so")
_CFLAGS = ["-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fPIC", "-shared", "-pthread"]

_lib = None


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc into a shared library and return its path."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *_CFLAGS, src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def load(path: Optional[str] = None):
    """Load (building first if absent) the oracle library; returns the ctypes handle."""
    global _lib
    if path is None:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        path = _LIB_PATH
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    common = [ctypes.c_int64, I, P, I, I, I, I, P, P, P, P, P, P, I, ctypes.c_double]
    lib.gdn_oracle_fwd.argtypes = common + [P, P, I]
    lib.gdn_oracle_fwd.restype = I
    lib.gdn_oracle_bwd.argtypes = common + [P, P, P, P, P, P, P, P, I]
    lib.gdn_oracle_bwd.restype = I
    lib.gdn_oracle_chunked_fwd.argtypes = common + [I, P, P, P, P, P, I]
    lib.gdn_oracle_chunked_fwd.restype = I
    lib.gdn_oracle_chunked_fwd_full.argtypes = common + [I, P, P, P, P, P, P, P, P, P, P, I]
    lib.gdn_oracle_chunked_fwd_full.restype = I
    if path == _LIB_PATH:
        _lib = lib
    return lib


def default_threads() -> int:
    return len(os.sched_getaffinity(0))


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _common(cu_seqlens, q, k, v, g, beta, h0, l2norm, eps):
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    N = cu.shape[0] - 1
    assert k.shape == (T, H, dk) and v.shape == (T, HV, dv)
    assert g.shape == (T, HV) and beta.shape == (T, HV)
    h0 = None if h0 is None else _f32(h0)
    if h0 is not None:
        assert h0.shape == (N, HV, dk, dv)
    keep = (cu, q, k, v, g, beta, h0)
    args = [T, N, _ptr(cu), H, HV, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
            int(bool(l2norm)), float(eps)]
    return keep, args, (T, N, H, HV, dk, dv)


def fwd(cu_seqlens, q, k, v, g, beta, h0=None, l2norm=False, eps=1e-6, threads=None, lib=None,
        want_ht=True):
    """Token-by-token FP64 forward. Returns (o [T,HV,dv], ht [N,HV,dk,dv] or None)."""
    lib = lib or load()
    keep, args, (T, N, H, HV, dk, dv) = _common(cu_seqlens, q, k, v, g, beta, h0, l2norm, eps)
    o = np.zeros((T, HV, dv), np.float64)
    ht = np.zeros((N, HV, dk, dv), np.float64) if want_ht else None
    rc = lib.gdn_oracle_fwd(*args, _ptr(o), _ptr(ht), int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle fwd failed (%d)" % rc)
    del keep
    return o, ht


def bwd(cu_seqlens, q, k, v, g, beta, dO, h0=None, dht=None, l2norm=False, eps=1e-6, threads=None,
        lib=None):
    """Token-by-token FP64 reverse mode. Returns dict dq, dk, dv, dg, dbeta, dh0."""
    lib = lib or load()
    keep, args, (T, N, H, HV, dk, dv) = _common(cu_seqlens, q, k, v, g, beta, h0, l2norm, eps)
    dO = _f32(dO)
    assert dO.shape == (T, HV, dv)
    dht = None if dht is None else _f32(dht)
    out = dict(dq=np.zeros((T, H, dk)), dk=np.zeros((T, H, dk)), dv=np.zeros((T, HV, dv)),
               dg=np.zeros((T, HV)), dbeta=np.zeros((T, HV)), dh0=np.zeros((N, HV, dk, dv)))
    rc = lib.gdn_oracle_bwd(*args, _ptr(dO), _ptr(dht), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                            _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dh0"]),
                            int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle bwd failed (%d)" % rc)
    del keep
    return out


def chunked_fwd(cu_seqlens, q, k, v, g, beta, h0=None, l2norm=False, eps=1e-6, chunk=64, threads=None,
                lib=None, full=False):
    """Chunked FP64 forward. Returns dict o, ht, A [T,HV,chunk], gcum [T,HV], gamma [NT,HV]; with
    full=True also what the full saved set adds: W [T,HV,dk], U and R = v_new [T,HV,dv], the rows of
    P [T,HV,chunk] and the state at the start of each chunk H [NT,HV,dk,dv]."""
    lib = lib or load()
    keep, args, (T, N, H, HV, dk, dv) = _common(cu_seqlens, q, k, v, g, beta, h0, l2norm, eps)
    cu = keep[0]
    NT = int(sum((int(cu[n + 1]) - int(cu[n]) + chunk - 1) // chunk for n in range(N)))
    out = dict(o=np.zeros((T, HV, dv)), ht=np.zeros((N, HV, dk, dv)), A=np.zeros((T, HV, chunk)),
               gcum=np.zeros((T, HV)), gamma=np.zeros((NT, HV)))
    nth = int(threads or default_threads())
    if full:
        out.update(W=np.zeros((T, HV, dk)), U=np.zeros((T, HV, dv)), R=np.zeros((T, HV, dv)),
                   P=np.zeros((T, HV, chunk)), H=np.zeros((NT, HV, dk, dv)))
        rc = lib.gdn_oracle_chunked_fwd_full(*args, int(chunk), *(_ptr(out[x]) for x in
                                                                 ("o", "ht", "A", "gcum", "gamma", "W", "U", "R",
                                                                  "P", "H")), nth)
    else:
        rc = lib.gdn_oracle_chunked_fwd(*args, int(chunk), _ptr(out["o"]), _ptr(out["ht"]), _ptr(out["A"]),
                                        _ptr(out["gcum"]), _ptr(out["gamma"]), nth)
    if rc != 0:
        raise RuntimeError("oracle chunked fwd failed (%d)" % rc)
    del keep
    return out
