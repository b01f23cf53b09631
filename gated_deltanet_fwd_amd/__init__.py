"""Python binding of the MI355X gated-delta-rule training kernel (libgdn.so, include/gdn.h).

Argument marshalling only: every step of the computation runs in the HIP kernels behind the C
ABI. PyTorch supplies device memory and streams: the launch stream (torch's current stream unless
one is given) and, for problems whose longest document runs apart from the others, an auxiliary
stream that this module keeps per device and names in the problem descriptor. Buffers that a call
allocates are allocated on its launch stream. The functions carry the C names:

    gdn_saved_bytes(problem)                      -> int
    gdn_workspace_bytes(problem, op)              -> int
    gdn_fwd(problem, q, k, v, g, beta, cu, ...)   -> (o, ht, saved)
    gdn_fwd_recompute(problem, q, k, v, g, beta, cu, ...) -> saved
    gdn_bwd(problem, q, k, v, g, beta, cu, saved, dO, ...) -> dict of gradients
    gdn_status(problem, op, workspace)            -> int (synchronises the stream)
    gdn_conv_fwd(conv_problem, x, weight, bias, cu, ...)      -> list of outputs (one per group)
    gdn_conv_bwd(conv_problem, x, weight, bias, cu, dys, ...) -> dict dx, dweight, dbias

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
SAVE_LIGHT, SAVE_FULL, SAVE_TAPE = 0, 1, 2
OP_FWD, OP_RECOMPUTE, OP_BWD = 0, 1, 2
ABI_VERSION = 2

EXPORTS = ("gdn_saved_bytes", "gdn_workspace_bytes", "gdn_fwd", "gdn_fwd_recompute", "gdn_bwd", "gdn_status",
           "gdn_fwd_noalloc", "gdn_conv_workspace_bytes", "gdn_conv_fwd", "gdn_conv_bwd", "gdn_last_error",
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
        ("aux_stream", ctypes.c_void_p),
        ("segments", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
    ]


class _ConvProblem(ctypes.Structure):
    _fields_ = [
        ("n_seqs", ctypes.c_int32),
        ("channels", ctypes.c_int32),
        ("n_tokens", ctypes.c_int64),
        ("width", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("silu", ctypes.c_int32),
        ("n_groups", ctypes.c_int32),
        ("group_channels", ctypes.c_int32 * 4),
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
    lib.gdn_status.argtypes = [pp, I, P, P]
    lib.gdn_status.restype = I
    lib.gdn_fwd_noalloc.argtypes = [pp] + [P] * 10 + [P]
    lib.gdn_fwd_noalloc.restype = I
    cp = ctypes.POINTER(_ConvProblem)
    lib.gdn_conv_workspace_bytes.argtypes = [cp]
    lib.gdn_conv_workspace_bytes.restype = Z
    lib.gdn_conv_fwd.argtypes = [cp, P, P, P, P, P, P]
    lib.gdn_conv_fwd.restype = I
    lib.gdn_conv_bwd.argtypes = [cp, P, P, P, P, P, P, P, P, P, Z, P]
    lib.gdn_conv_bwd.restype = I
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_abi_version.argtypes = []
    lib.gdn_abi_version.restype = I
    if lib.gdn_abi_version() != ABI_VERSION:
        raise OSError("libgdn.so has ABI version %d, this binding expects %d: rebuild it" %
                      (lib.gdn_abi_version(), ABI_VERSION))
    _lib = lib
    return lib


class Problem:
    """A gdn_problem descriptor plus the host copy of cu_seqlens it points to."""

    def __init__(self, cu_seqlens_host, h_qk: int, h_v: int, d: int, dtype=torch.bfloat16, l2norm: bool = True,
                 has_h0: bool = False, want_ht: bool = False, save_mode: int = SAVE_LIGHT,
                 deterministic: bool = True, use_aux_stream=True, segments: int = 0):
        self.cu = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
        self.dtype = dtype
        # True: the module's auxiliary stream of the device; False: one stream; or a stream object
        self.use_aux_stream = use_aux_stream
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
            aux_stream=None,
            segments=int(segments),
            reserved0=0,
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


def _torch_stream(stream, device) -> torch.cuda.Stream:
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


_aux_streams: Dict[int, torch.cuda.Stream] = {}


def aux_stream(device) -> torch.cuda.Stream:
    """The auxiliary stream this module names in problems on `device` (created on first use, kept
    for the life of the process, default priority)."""
    idx = torch.device(device).index
    idx = torch.cuda.current_device() if idx is None else idx
    if idx not in _aux_streams:
        _aux_streams[idx] = torch.cuda.Stream(device=idx)
    return _aux_streams[idx]


class _Call:
    """Launch context of one call: the launch stream, allocations on it, and the problem's auxiliary
    stream set for the call."""

    def __init__(self, p: "Problem", device, stream):
        self.p = p
        self.device = device
        self.stream = _torch_stream(stream, device)
        u = p.use_aux_stream
        aux = u if isinstance(u, torch.cuda.Stream) else aux_stream(device) if u else None
        p.st.aux_stream = None if aux is None or aux.cuda_stream == self.stream.cuda_stream else aux.cuda_stream

    def empty(self, *shape, dtype):
        with torch.cuda.stream(self.stream):
            return torch.empty(*shape, dtype=dtype, device=self.device)

    def empty_like(self, t):
        with torch.cuda.stream(self.stream):
            return torch.empty_like(t)

    def handle(self) -> ctypes.c_void_p:
        return ctypes.c_void_p(self.stream.cuda_stream)


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


def gdn_fwd(p: Problem, q, k, v, g, beta, cu_seqlens, h0=None, o=None, ht=None, saved=None, workspace=None,
            stream=None):
    """Forward: returns (o, ht or None, saved)."""
    lib = load_library()
    c = _Call(p, q.device, stream)
    T, HV, d = p.T, p.st.h_v, p.st.d
    if o is None:
        o = c.empty((T, HV, d), dtype=q.dtype)
    if p.st.want_ht and ht is None:
        ht = c.empty((p.N, HV, d, d), dtype=torch.float32)
    if saved is None:
        saved = c.empty(gdn_saved_bytes(p), dtype=torch.uint8)
    if workspace is None:
        workspace = c.empty(gdn_workspace_bytes(p, OP_FWD), dtype=torch.uint8)
    _check(lib.gdn_fwd(p.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), _ptr(h0), _ptr(o),
                       _ptr(ht), _ptr(saved), _ptr(workspace), workspace.numel(), c.handle()))
    return o, ht, saved


def gdn_fwd_recompute(p: Problem, q, k, v, g, beta, cu_seqlens, h0=None, saved=None, workspace=None, stream=None):
    """Checkpoint re-run of the forward: returns the saved set only."""
    lib = load_library()
    c = _Call(p, q.device, stream)
    if saved is None:
        saved = c.empty(gdn_saved_bytes(p), dtype=torch.uint8)
    if workspace is None:
        workspace = c.empty(gdn_workspace_bytes(p, OP_RECOMPUTE), dtype=torch.uint8)
    _check(lib.gdn_fwd_recompute(p.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                 _ptr(h0), _ptr(saved), _ptr(workspace), workspace.numel(), c.handle()))
    return saved


def gdn_bwd(p: Problem, q, k, v, g, beta, cu_seqlens, saved, dO, h0=None, dht=None, grads=None, workspace=None,
            stream=None) -> Dict[str, torch.Tensor]:
    """Backward: returns dict dq, dk, dv, dg, dbeta, dh0 (dh0 None without h0)."""
    lib = load_library()
    c = _Call(p, q.device, stream)
    if grads is None:
        grads = dict(dq=c.empty_like(q), dk=c.empty_like(k), dv=c.empty_like(v), dg=c.empty_like(g),
                     dbeta=c.empty_like(beta),
                     dh0=c.empty_like(h0) if (p.st.has_h0 and h0 is not None) else None)
    if workspace is None:
        workspace = c.empty(gdn_workspace_bytes(p, OP_BWD), dtype=torch.uint8)
    _check(lib.gdn_bwd(p.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), _ptr(h0),
                       _ptr(saved), _ptr(dO), _ptr(dht), _ptr(grads["dq"]), _ptr(grads["dk"]), _ptr(grads["dv"]),
                       _ptr(grads["dg"]), _ptr(grads["dbeta"]), _ptr(grads.get("dh0")), _ptr(workspace),
                       workspace.numel(), c.handle()))
    return grads


def gdn_fwd_noalloc(p: Problem, q, k, v, g, beta, cu_seqlens, h0=None, o=None, ht=None, saved=None, stream=None):
    """Forward whose workspace is the library's fixed device scratch array (no workspace
    argument; the library allocates nothing). Returns (o, ht or None, saved); o, ht and saved are
    allocated here when not given."""
    lib = load_library()
    c = _Call(p, q.device, stream)
    T, HV, d = p.T, p.st.h_v, p.st.d
    if o is None:
        o = c.empty((T, HV, d), dtype=q.dtype)
    if p.st.want_ht and ht is None:
        ht = c.empty((p.N, HV, d, d), dtype=torch.float32)
    if saved is None:
        saved = c.empty(gdn_saved_bytes(p), dtype=torch.uint8)
    _check(lib.gdn_fwd_noalloc(p.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), _ptr(h0),
                               _ptr(o), _ptr(ht), _ptr(saved), c.handle()))
    return o, ht, saved


def gdn_status(p: Problem, op: int, workspace, stream=None) -> int:
    """Device-side status of the last call of `op` on this workspace: GDN_OK, GDN_EINVAL or
    GDN_ESAVED (synchronises the launch stream)."""
    c = _Call(p, workspace.device, stream)
    return int(load_library().gdn_status(p.ref(), int(op), _ptr(workspace), c.handle()))


def problem_for(w, save_mode: int = SAVE_LIGHT, deterministic: Optional[bool] = None, l2norm: Optional[bool] = None,
                want_ht: Optional[bool] = None, use_aux_stream=True, segments: int = 0) -> Problem:
    """Problem descriptor for a synthetic workload description (see synthetic.Workload)."""
    cu = np.zeros(w.N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(w.lengths, dtype=np.int64))
    return Problem(cu, w.H, w.HV, w.d, dtype=w.torch_dtype, l2norm=w.l2norm if l2norm is None else l2norm,
                   has_h0=w.has_h0, want_ht=w.want_ht if want_ht is None else want_ht, save_mode=save_mode,
                   deterministic=w.deterministic if deterministic is None else deterministic,
                   use_aux_stream=use_aux_stream, segments=segments)


class ConvProblem:
    """A gdn_conv_problem descriptor: the causal conv1d + SiLU front-end over [T, sum(groups)]
    channels with a `width`-tap window, its output split into the groups' tensors."""

    def __init__(self, cu_seqlens_host, group_channels, width: int = 4, dtype=torch.bfloat16, silu: bool = True):
        self.cu = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
        self.groups = [int(c) for c in group_channels]
        self.dtype = dtype
        gc = (ctypes.c_int32 * 4)(*(self.groups + [0] * (4 - len(self.groups))))
        self.st = _ConvProblem(n_seqs=int(self.cu.shape[0] - 1), channels=int(sum(self.groups)),
                               n_tokens=int(self.cu[-1]), width=int(width),
                               dtype=DTYPE_BF16 if dtype == torch.bfloat16 else DTYPE_F32, silu=int(bool(silu)),
                               n_groups=len(self.groups), group_channels=gc,
                               cu_seqlens_host=self.cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))

    @property
    def T(self) -> int:
        return int(self.st.n_tokens)

    def ref(self):
        return ctypes.byref(self.st)


def _ptr_array(ts):
    return (ctypes.c_void_p * 4)(*([t.data_ptr() for t in ts] + [0] * (4 - len(ts))))


def gdn_conv_workspace_bytes(p: ConvProblem) -> int:
    n = load_library().gdn_conv_workspace_bytes(p.ref())
    if n == 0:
        raise GdnError(GDN_EINVAL, load_library().gdn_last_error().decode())
    return int(n)


def gdn_conv_fwd(p: ConvProblem, x, weight, bias, cu_seqlens, outs=None, stream=None):
    """Forward of the conv front-end: returns the list of output tensors, [T, group_channels[g]]."""
    lib = load_library()
    dev = x.device
    s = _torch_stream(stream, dev)
    if outs is None:
        with torch.cuda.stream(s):
            outs = [torch.empty((p.T, c), dtype=x.dtype, device=dev) for c in p.groups]
    _check(lib.gdn_conv_fwd(p.ref(), _ptr(x), _ptr(weight), _ptr(bias), _ptr(cu_seqlens), _ptr_array(outs),
                            ctypes.c_void_p(s.cuda_stream)))
    return outs


def gdn_conv_bwd(p: ConvProblem, x, weight, bias, cu_seqlens, dys, dx=None, dweight=None, dbias=None,
                 workspace=None, stream=None) -> Dict[str, torch.Tensor]:
    """Backward of the conv front-end: returns dict dx [T, C], dweight [C, W], dbias [C] (None when
    bias is None)."""
    lib = load_library()
    dev = x.device
    s = _torch_stream(stream, dev)
    with torch.cuda.stream(s):
        if dx is None:
            dx = torch.empty_like(x)
        if dweight is None:
            dweight = torch.empty_like(weight)
        if dbias is None and bias is not None:
            dbias = torch.empty_like(bias)
        if workspace is None:
            workspace = torch.empty(gdn_conv_workspace_bytes(p), dtype=torch.uint8, device=dev)
    _check(lib.gdn_conv_bwd(p.ref(), _ptr(x), _ptr(weight), _ptr(bias), _ptr(cu_seqlens), _ptr_array(dys), _ptr(dx),
                            _ptr(dweight), _ptr(dbias), _ptr(workspace), workspace.numel(),
                            ctypes.c_void_p(s.cuda_stream)))
    return dict(dx=dx, dweight=dweight, dbias=dbias)
