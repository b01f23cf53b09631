"""Python binding of the MI355X gated-delta-rule training kernel (libgdn.so, include/gdn.h).

Argument marshalling only: every step of the computation runs in the HIP kernels behind the C
ABI. PyTorch supplies device memory and the current stream. The functions carry the C names:

    gdn_saved_bytes(problem)                      -> int
    gdn_workspace_bytes(problem, op)              -> int
    gdn_fwd(problem, q, k, v, g, beta, cu, ...)   -> (o, ht, saved)
    gdn_fwd_recompute(problem, q, k, v, g, beta, cu, ...) -> saved
    gdn_bwd(problem, q, k, v, g, beta, cu, saved, dO, ...) -> dict of gradients

A missing or unloadable library raises ImportError-like errors at first use; there is no other
code path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_ESAVED, GDN_EWORKSPACE, GDN_EHIP = range(6)
DTYPE_BF16, DTYPE_F32 = 0, 1
SAVE_LIGHT, SAVE_FULL = 0, 1
OP_FWD, OP_RECOMPUTE, OP_BWD = 0, 1, 2

EXPORTS = ("gdn_saved_bytes", "gdn_workspace_bytes", "gdn_fwd", "gdn_fwd_recompute", "gdn_bwd", "gdn_last_error",
           "gdn_abi_version")


class GdnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("gdn error %d: %s" % (code, msg))
        self.code = code


class _Problem(ctypes.Structure):
    _fields_ = [
        ("n_seqs", ctypes.c_int32),
        ("h_qk", ctypes.c_int32),
        ("h_v", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("n_tokens", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("l2norm_qk", ctypes.c_int32),
        ("has_h0", ctypes.c_int32),
        ("want_ht", ctypes.c_int32),
        ("save_mode", ctypes.c_int32),
        ("deterministic", ctypes.c_int32),
        ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libgdn.so once. Raises OSError if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError("libgdn.so not found at %s: build it with `python -m gated_deltanet_fwd_amd.build`" % path)
    lib = ctypes.CDLL(path)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    pp = ctypes.POINTER(_Problem)
    lib.gdn_saved_bytes.argtypes = [pp]
    lib.gdn_saved_bytes.restype = Z
    lib.gdn_workspace_bytes.argtypes = [pp, I]
    lib.gdn_workspace_bytes.restype = Z
    lib.gdn_fwd.argtypes = [pp] + [P] * 11 + [Z, P]
    lib.gdn_fwd.restype = I
    lib.gdn_fwd_recompute.argtypes = [pp] + [P] * 9 + [Z, P]
    lib.gdn_fwd_recompute.restype = I
    lib.gdn_bwd.argtypes = [pp] + [P] * 17 + [Z, P]
    lib.gdn_bwd.restype = I
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_abi_version.argtypes = []
    lib.gdn_abi_version.restype = I
    _lib = lib
    return lib


class Problem:
    """A gdn_problem descriptor plus the host copy of cu_seqlens it points to."""

    def __init__(self, cu_seqlens_host, h_qk: int, h_v: int, d: int, dtype=torch.bfloat16, l2norm: bool = True,
                 has_h0: bool = False, want_ht: bool = False, save_mode: int = SAVE_LIGHT,
                 deterministic: bool = True):
        self.cu = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
        self.dtype = dtype
        self.st = _Problem(
            n_seqs=int(self.cu.shape[0] - 1),
            h_qk=int(h_qk),
            h_v=int(h_v),
            d=int(d),
            n_tokens=int(self.cu[-1]),
            dtype=DTYPE_BF16 if dtype == torch.bfloat16 else DTYPE_F32,
            l2norm_qk=int(bool(l2norm)),
            has_h0=int(bool(has_h0)),
            want_ht=int(bool(want_ht)),
            save_mode=int(save_mode),
            deterministic=int(bool(deterministic)),
            cu_seqlens_host=self.cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        )

    @property
    def T(self) -> int:
        return int(self.st.n_tokens)

    @property
    def N(self) -> int:
        return int(self.st.n_seqs)

    def ref(self):
        return ctypes.byref(self.st)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(rc: int):
    if rc != GDN_OK:
        raise GdnError(rc, load_library().gdn_last_error().decode())


def gdn_saved_bytes(p: Problem) -> int:
    n = load_library().gdn_saved_bytes(p.ref())
    if n == 0:
        raise GdnError(GDN_EINVAL, load_library().gdn_last_error().decode())
    return int(n)


def gdn_workspace_bytes(p: Problem, op: int) -> int:
    n = load_library().gdn_workspace_bytes(p.ref(), int(op))
    if n == 0:
        raise GdnError(GDN_EINVAL, load_library().gdn_last_error().decode())
    return int(n)


def _empty_bytes(n: int, device) -> torch.Tensor:
    return torch.empty(n, dtype=torch.uint8, device=device)


def gdn_fwd(p: Problem, q, k, v, g, beta, cu_seqlens, h0=None, o=None, ht=None, saved=None, workspace=None,
            stream=None):
    """Forward: returns (o, ht or None, saved)."""
    lib = load_library()
    dev = q.device
    T, HV, d = p.T, p.st.h_v, p.st.d
    if o is None:
        o = torch.empty((T, HV, d), dtype=q.dtype, device=dev)
    if p.st.want_ht and ht is None:
        ht = torch.empty((p.N, HV, d, d), dtype=torch.float32, device=dev)
    if saved is None:
        saved = _empty_bytes(gdn_saved_bytes(p), dev)
    if workspace is None:
        workspace = _empty_bytes(gdn_workspace_bytes(p, OP_FWD), dev)
    _check(lib.gdn_fwd(p.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), _ptr(h0), _ptr(o),
                       _ptr(ht), _ptr(saved), _ptr(workspace), workspace.numel(), _stream(stream)))
    return o, ht, saved


def gdn_fwd_recompute(p: Problem, q, k, v, g, beta, cu_seqlens, h0=None, saved=None, workspace=None, stream=None):
    """Checkpoint re-run of the forward: returns the saved set only."""
    lib = load_library()
    dev = q.device
    if saved is None:
        saved = _empty_bytes(gdn_saved_bytes(p), dev)
    if workspace is None:
        workspace = _empty_bytes(gdn_workspace_bytes(p, OP_RECOMPUTE), dev)
    _check(lib.gdn_fwd_recompute(p.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                 _ptr(h0), _ptr(saved), _ptr(workspace), workspace.numel(), _stream(stream)))
    return saved


def gdn_bwd(p: Problem, q, k, v, g, beta, cu_seqlens, saved, dO, h0=None, dht=None, grads=None, workspace=None,
            stream=None) -> Dict[str, torch.Tensor]:
    """Backward: returns dict dq, dk, dv, dg, dbeta, dh0 (dh0 None without h0)."""
    lib = load_library()
    dev = q.device
    if grads is None:
        grads = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                     dg=torch.empty_like(g), dbeta=torch.empty_like(beta),
                     dh0=torch.empty_like(h0) if (p.st.has_h0 and h0 is not None) else None)
    if workspace is None:
        workspace = _empty_bytes(gdn_workspace_bytes(p, OP_BWD), dev)
    _check(lib.gdn_bwd(p.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), _ptr(h0),
                       _ptr(saved), _ptr(dO), _ptr(dht), _ptr(grads["dq"]), _ptr(grads["dk"]), _ptr(grads["dv"]),
                       _ptr(grads["dg"]), _ptr(grads["dbeta"]), _ptr(grads.get("dh0")), _ptr(workspace),
                       workspace.numel(), _stream(stream)))
    return grads


def problem_for(w, save_mode: int = SAVE_LIGHT, deterministic: Optional[bool] = None, l2norm: Optional[bool] = None,
                want_ht: Optional[bool] = None) -> Problem:
    """Problem descriptor for a synthetic workload description (see synthetic.Workload)."""
    cu = np.zeros(w.N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(w.lengths, dtype=np.int64))
    return Problem(cu, w.H, w.HV, w.d, dtype=w.torch_dtype, l2norm=w.l2norm if l2norm is None else l2norm,
                   has_h0=w.has_h0, want_ht=w.want_ht if want_ht is None else want_ht, save_mode=save_mode,
                   deterministic=w.deterministic if deterministic is None else deterministic)
