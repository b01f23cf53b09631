"""Seeded synthetic inputs for the gated delta rule kernel and its oracle.

This module only draws random numbers; it holds none of the method's arithmetic, and both
the HIP path's tests/benchmark and the FP64 oracle read the tensors it returns.

The workloads follow the shapes the pages measure: (H, HV) = (16, 48) heads with d = 128,
BF16 q/k/v and FP32 g and beta on packed variable-length documents (flashinfer PR #8181
single-GPU table and PR #8172 CP tables; shape A = 4 documents 98304/65536/57344/40960 is
named in the flashinfer PR #8542 "Conventions" section). Value distributions:

  q, k, v ~ N(0, 1)                  drawn in float32, then rounded to the io dtype (RNE)
  beta    = sigmoid(N(0, 1))         float32
  g       = logsigmoid(N(0, 1) + 3)  float32 log decay (always < 0)
  h0, dht ~ N(0, 0.1^2)              float32 (only where the workload has them)
  dO      ~ N(0, 1)                  io dtype

Draw order within one workload: q, k, v, beta, g, h0, dO, dht, from one torch.Generator
seeded with the workload's seed on the device the tensors are made on. Document lengths
are drawn first, with numpy's PCG64 on the host.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    lengths: tuple
    H: int
    HV: int
    d: int
    dtype: str  # "bf16" or "f32"
    l2norm: bool
    has_h0: bool
    want_ht: bool
    has_dht: bool
    deterministic: bool
    ops: tuple  # which passes the workload exercises

    @property
    def T(self) -> int:
        return int(sum(self.lengths))

    @property
    def N(self) -> int:
        return len(self.lengths)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


def short_doc_lengths(seed: int, n_docs: int = 512, total: int = 262144, lo: int = 64, hi: int = 4096,
                      chunk: int = 64) -> List[int]:
    """Log-uniform lengths in [lo, hi], rescaled to sum to `total`, none a multiple of `chunk`.

    Rounding residue is spread by +-1 steps in index order, skipping a step that would make a
    length a multiple of `chunk` (or zero).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    raw = np.exp(rng.uniform(np.log(lo), np.log(hi), size=n_docs))
    lens = np.maximum(1, np.rint(raw * (total / raw.sum())).astype(np.int64))
    lens[lens % chunk == 0] += 1
    resid = int(total - lens.sum())
    i = 0
    while resid != 0:
        step = 1 if resid > 0 else -1
        cand = lens[i % n_docs] + step
        if cand >= 1 and cand % chunk != 0:
            lens[i % n_docs] = cand
            resid -= step
        i += 1
    assert int(lens.sum()) == total and not np.any(lens % chunk == 0)
    return [int(x) for x in lens]


def _workloads() -> Dict[str, Workload]:
    w = {}
    w["tiny"] = Workload("tiny", 1001, (256,), 2, 2, 64, "f32", True, False, False, False, True,
                         ("fwd", "bwd"))
    w["single8k"] = Workload("single8k", 1002, (8192,), 16, 48, 128, "bf16", True, False, False, False, True,
                             ("fwd",))
    w["pack262k"] = Workload("pack262k", 1003, (98304, 65536, 57344, 40960), 16, 48, 128, "bf16", True,
                             False, False, False, False, ("fwd", "bwd", "ckpt"))
    w["cp4share"] = Workload("cp4share", 1004, (40960, 24576), 16, 48, 128, "bf16", True, True, True, True,
                             False, ("fwd", "bwd"))
    w["short512"] = Workload("short512", 1005, tuple(short_doc_lengths(1005)), 16, 48, 128, "bf16", True,
                             False, False, False, True, ("ckpt",))
    return w


WORKLOADS: Dict[str, Workload] = _workloads()
ORDER = ["tiny", "single8k", "pack262k", "cp4share", "short512"]


def custom(name: str, lengths, H: int, HV: int, d: int, dtype: str = "bf16", l2norm: bool = True,
           has_h0: bool = False, want_ht: bool = False, has_dht: bool = False, deterministic: bool = True,
           seed: int = 7) -> Workload:
    """A workload of any shape, drawn with the same distributions (for edge-case tests)."""
    return Workload(name, seed, tuple(int(x) for x in lengths), H, HV, d, dtype, l2norm, has_h0, want_ht,
                    has_dht, deterministic, ("fwd", "bwd"))


def make_inputs(w: Workload, device="cpu", with_grads: bool = True) -> Dict[str, Optional[torch.Tensor]]:
    """Draw the workload's tensors on `device` (io tensors in the io dtype, the rest float32)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    T, N, H, HV, d = w.T, w.N, w.H, w.HV, w.d
    dt = w.torch_dtype

    def normal(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    out: Dict[str, Optional[torch.Tensor]] = {}
    out["q"] = normal(T, H, d).to(dt)
    out["k"] = normal(T, H, d).to(dt)
    out["v"] = normal(T, HV, d).to(dt)
    out["beta"] = torch.sigmoid(normal(T, HV))
    out["g"] = torch.nn.functional.logsigmoid(normal(T, HV) + 3.0)
    out["h0"] = (0.1 * normal(N, HV, d, d)) if w.has_h0 else None
    if with_grads:
        out["dO"] = normal(T, HV, d).to(dt)
        out["dht"] = (0.1 * normal(N, HV, d, d)) if w.has_dht else None
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(w.lengths, dtype=np.int64))
    out["cu_seqlens"] = torch.from_numpy(cu).to(device)
    return out


# ----------------------------------------------------------------------------------------------
# The short causal conv1d + SiLU front-end over the packed q/k/v channels (the pages' shape B23:
# 4 documents 12288/8192/7168/5120 = 32768 tokens, (H, HV) = (16, 48), d = 128, so 2048 + 2048 +
# 6144 = 10240 channels; flashinfer PR #8542 "Conventions"). Distributions:
#   x      ~ N(0, 1)              [T, C], rounded to the io dtype (RNE)
#   weight ~ N(0, 1) / sqrt(W)    [C, W] float32
#   bias   ~ N(0, 0.1^2)          [C] float32
#   dy     ~ N(0, 1)              one [T, C_g] tensor per output group, io dtype
# drawn in that order from one torch.Generator seeded with the workload's seed.


@dataclasses.dataclass(frozen=True)
class ConvWorkload:
    name: str
    seed: int
    lengths: tuple
    groups: tuple  # channels of each output group
    width: int
    dtype: str
    silu: bool = True
    bias: bool = True

    @property
    def T(self) -> int:
        return int(sum(self.lengths))

    @property
    def C(self) -> int:
        return int(sum(self.groups))

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


CONV_WORKLOADS: Dict[str, ConvWorkload] = {
    "b23_conv": ConvWorkload("b23_conv", 1006, (12288, 8192, 7168, 5120), (2048, 2048, 6144), 4, "bf16"),
}

# the gated delta rule layer of shape B23, fed by the conv front-end's q, k, v
WORKLOADS["b23"] = Workload("b23", 1007, (12288, 8192, 7168, 5120), 16, 48, 128, "bf16", True, False, False, False,
                            False, ("fwd", "bwd", "ckpt"))


def make_conv_inputs(w: ConvWorkload, device="cpu") -> Dict[str, Optional[torch.Tensor]]:
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)

    def normal(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = normal(w.T, w.C).to(w.torch_dtype)
    out["weight"] = normal(w.C, w.width) / float(np.sqrt(w.width))
    b = 0.1 * normal(w.C)
    out["bias"] = b if w.bias else None
    out["dy"] = [normal(w.T, c).to(w.torch_dtype) for c in w.groups]
    cu = np.zeros(len(w.lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(w.lengths, dtype=np.int64))
    out["cu_seqlens"] = torch.from_numpy(cu).to(device)
    return out


def conv_custom(name, lengths, groups, width=4, dtype="bf16", silu=True, bias=True, seed=31) -> ConvWorkload:
    return ConvWorkload(name, seed, tuple(int(x) for x in lengths), tuple(int(c) for c in groups), int(width), dtype,
                        silu, bias)
