#!/usr/bin/env python3
"""Benchmark of the MI355X gated-delta-rule training kernel (one GPU).

One step = one pass of the whole hot path over one batch: gdn_fwd then gdn_bwd (light saved
set) on the packed workload of 4 documents 98304/65536/57344/40960 = 262144 tokens,
(H, HV) = (16, 48), d = 128, bf16 inputs with the in-kernel q/k L2 norm (the pages' "shape A").
Inputs are drawn once on the GPU and are resident in HBM before timing starts.

Prints one JSON line: tokens/s of the fwd+bwd step (the headline), plus fwd-only and
checkpointed (fwd + recompute + bwd) rates, the roofline of the dominant kernel with its
per-launch duration measured by HIP events on the launch stream during the timed region, and
the FP64 CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload pack262k] [--deterministic]
                    [--no-cpu-baseline] [--gpus 1]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12           # bytes/s, MI355X HBM3E
PEAK_BF16 = 2.5e15          # flop/s, MI355X dense bf16 MFMA
CHUNK = 64
METRIC = "tokens/s fwd+bwd (and fwd, ckpt) at (H,HV)=(16,48), d=128, 262144 tok"


def kernel_models(T, NT, N, H, HV, D, io, has_h0=False):
    """Algorithmic (compulsory) bytes and MFMA flops of one launch of each kernel.

    Bytes: every operand of the kernel read once and every result written once. Flops: the
    contractions of the chunked method the kernel performs, 2 flops per multiply-add.
    """
    C = CHUNK
    f4 = 4
    qk_ws = NT * H * C * C * 2
    akk = T * HV * C * 2
    scal_v = T * HV * f4
    scal_q = T * H * f4
    tape = NT * HV * D * D * 2
    qkin = T * H * D * io
    vin = T * HV * D * io
    states = N * HV * D * D * f4
    m = {}
    m["gdn_intra"] = (2 * qkin + 2 * scal_v + 2 * scal_q + qk_ws + akk + scal_v + NT * HV * f4,
                      NT * H * 2 * (2 * C * C * D) + NT * HV * (2 * C ** 3 // 3))
    m["gdn_intra_bwd"] = (2 * qkin + 2 * scal_q + qk_ws, NT * H * 2 * (2 * C * C * D))
    m["gdn_walk_fwd"] = (2 * qkin + vin + akk + qk_ws + 2 * scal_v + 2 * scal_q + NT * HV * f4 + vin
                         + (states if has_h0 else 0), T * HV * (6 * D * D + 4 * C * D))
    m["gdn_walk_tape"] = (qkin + vin + akk + 2 * scal_v + scal_q + NT * HV * f4 + tape,
                          T * HV * (4 * D * D + 2 * C * D))
    m["gdn_walk_bwd"] = (2 * qkin + vin + akk + qk_ws + 2 * scal_v + 2 * scal_q + NT * HV * f4 + tape,
                         T * HV * (6 * D * D + 4 * C * D))
    m["gdn_chunk_grad"] = (2 * tape + 2 * qkin + 2 * vin + akk + 2 * scal_v + 2 * scal_q + NT * HV * f4
                           + 2 * qkin + vin + 2 * scal_v,
                           T * HV * 2 * (5 * D * D + 8 * C * D + 2 * C * C) + NT * H * 2 * (2 * C * C * D))
    m["gdn_finalize_qk"] = (2 * T * H * D * f4 + 2 * qkin + 2 * scal_q + 2 * qkin, 0)
    m["gdn_fill_zero"] = (T * H * D * f4, 0)
    return m


def step_roofline(T, HV, D, io_bytes):
    """Op-level algorithmic work (inputs, outputs and the light saved set; tapes excluded) per token."""
    C = CHUNK
    G = 3
    fl_f = 6 * D * D + 6 * C * D + 4 * C * D / G + 2 * C * C / 3
    fl_b = 16 * D * D + (12 + 2 / G) * 2 * C * D + 4 * C * C / 3
    fl_r = 2 * C * D / G + 2 * C * C / 3
    inputs = 2 * 16 * D * io_bytes + HV * D * io_bytes + 2 * HV * 4
    saved = HV * C * 2 + HV * 4 + HV * 4 / C
    b_f = inputs + HV * D * io_bytes + saved
    b_b = inputs + HV * D * io_bytes + saved + 2 * 16 * D * io_bytes + HV * D * io_bytes + 2 * HV * 4
    b_r = 16 * D * io_bytes + 2 * HV * 4 + saved
    out = {}
    for name, fl, by in (("fwd", fl_f, b_f), ("fwdbwd", fl_f + fl_b, b_f + b_b),
                         ("ckpt", fl_f + fl_r + fl_b, b_f + b_r + b_b)):
        t = max(fl * HV * T / PEAK_BF16, by * T / PEAK_HBM)
        out[name] = {"flops_per_token": fl * HV, "bytes_per_token": by, "roofline_s": t}
    return out


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(kernel, workload):
    """HBM traffic per launch from committed rocprofv3 counter runs, if the kernel is unchanged."""
    path = os.path.join(ROOT, "profiles", "pmc_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, "gated_deltanet_fwd_amd", "csrc", rec.get("source", ""))
    if not os.path.exists(src) or source_sha(src) != rec.get("source_sha"):
        return None
    return float(rec["bytes_per_launch"])


def cpu_baseline(w, inputs_dev):
    """Time the FP64 oracle (fwd + bwd) on the shortest document of the workload, all heads."""
    import numpy as np
    import oracle

    cu = inputs_dev["cu_seqlens"].cpu().numpy()
    lens = np.diff(cu)
    n = int(np.argmin(lens))
    s, e = int(cu[n]), int(cu[n + 1])
    f = lambda t: None if t is None else t[s:e].float().cpu().numpy()
    q, k, v, g, b, dO = (f(inputs_dev[x]) for x in ("q", "k", "v", "g", "beta", "dO"))
    cu1 = np.array([0, e - s], np.int32)
    threads = oracle.default_threads()
    used = min(threads, w.H)  # the oracle splits work over (document, q/k head) items
    t0 = time.time()
    oracle.fwd(cu1, q, k, v, g, b, None, l2norm=w.l2norm, threads=threads)
    oracle.bwd(cu1, q, k, v, g, b, dO, None, None, l2norm=w.l2norm, threads=threads)
    dt = time.time() - t0
    return {"value": (e - s) / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": "fwd+bwd of document %d (%d tokens, all %d q/k and %d v heads, d=%d) of the same pack, "
                      "FP64 token recurrence, %.1f s" % (n, e - s, w.H, w.HV, w.d, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="pack262k")
    ap.add_argument("--deterministic", action="store_true", help="deterministic dq/dk reduction")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the fwd-only and ckpt timings")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (it would shard the "
              "q/k-head groups or the sequence across GPUs; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_fwd_amd as G
    import synthetic as syn

    lib = G.load_library()
    w = syn.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    inp = syn.make_inputs(w, device=dev)
    det = bool(args.deterministic)
    p = G.problem_for(w, save_mode=G.SAVE_LIGHT, deterministic=det)
    saved = torch.empty(G.gdn_saved_bytes(p), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(G.gdn_workspace_bytes(p, G.OP_FWD), dtype=torch.uint8, device=dev)
    ws_r = torch.empty(G.gdn_workspace_bytes(p, G.OP_RECOMPUTE), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(G.gdn_workspace_bytes(p, G.OP_BWD), dtype=torch.uint8, device=dev)
    o = torch.empty_like(inp["v"])
    ht = torch.empty((w.N, w.HV, w.d, w.d), dtype=torch.float32, device=dev) if w.want_ht else None
    grads = dict(dq=torch.empty_like(inp["q"]), dk=torch.empty_like(inp["k"]), dv=torch.empty_like(inp["v"]),
                 dg=torch.empty_like(inp["g"]), dbeta=torch.empty_like(inp["beta"]),
                 dh0=torch.empty_like(inp["h0"]) if inp["h0"] is not None else None)
    stream = torch.cuda.current_stream()
    a = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"])

    def fwd():
        G.gdn_fwd(p, *a, h0=inp["h0"], o=o, ht=ht, saved=saved, workspace=ws_f, stream=stream)

    def recompute():
        G.gdn_fwd_recompute(p, *a, h0=inp["h0"], saved=saved, workspace=ws_r, stream=stream)

    def bwd():
        G.gdn_bwd(p, *a, saved, inp["dO"], h0=inp["h0"], dht=inp["dht"], grads=grads, workspace=ws_b,
                  stream=stream)

    def timed(fn, steps, warmup, kernel_timing=False):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        if kernel_timing:
            lib.gdn_timing_reset()
            lib.gdn_timing_enable(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.time()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.time() - t0
        if kernel_timing:
            lib.gdn_timing_enable(0)
        return e0.elapsed_time(e1) / 1e3, wall

    step = lambda: (fwd(), bwd())
    t_fb, wall_fb = timed(step, args.steps, args.warmup, kernel_timing=True)
    # per-kernel totals over the timed region
    names = (ctypes.c_char_p * 32)()
    tot = (ctypes.c_double * 32)()
    cnt = (ctypes.c_int * 32)()
    lib.gdn_timing_collect.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    nk = lib.gdn_timing_collect(32, names, tot, cnt)
    kernels = {names[i].decode(): {"total_ms": tot[i], "launches": cnt[i], "avg_ms": tot[i] / max(1, cnt[i])}
               for i in range(min(nk, 32))}
    lib.gdn_timing_reset()

    extra = {}
    if not args.no_extra:
        ksteps = max(3, args.steps // 2)
        t_f, _ = timed(fwd, ksteps, 1)
        t_c, _ = timed(lambda: (fwd(), recompute(), bwd()), ksteps, 1)
        extra["fwd"] = {"tokens_per_s": w.T * ksteps / t_f, "ms": 1e3 * t_f / ksteps}
        extra["ckpt"] = {"tokens_per_s": w.T * ksteps / t_c, "ms": 1e3 * t_c / ksteps}

    ms = 1e3 * t_fb / args.steps
    value = w.T * args.steps / t_fb
    io = 2 if w.dtype == "bf16" else 4
    NT = int(sum((L + CHUNK - 1) // CHUNK for L in w.lengths))
    models = kernel_models(w.T, NT, w.N, w.H, w.HV, w.d, io, has_h0=w.has_h0)
    # dominant kernel = largest share of the timed step
    dom = max((k for k in kernels if k in models), key=lambda k: kernels[k]["total_ms"])
    by, fl = models[dom]
    avg_s = kernels[dom]["avg_ms"] / 1e3
    t_hbm, t_mfma = by / PEAK_HBM, fl / PEAK_BF16
    if t_mfma > t_hbm:
        roof = {"bound": "mfma", "achieved": fl / avg_s / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": by / avg_s / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = load_traffic(dom, args.workload)
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = by
    roof["algorithmic_flops"] = fl
    roof["avg_launch_ms"] = kernels[dom]["avg_ms"]

    sr = step_roofline(w.T, w.HV, w.d, io)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": "%s: %d docs %s, %d tokens, (H,HV)=(%d,%d), d=%d, l2norm=%d, light saved set, "
                               "%s dq/dk reduction" % (w.name, w.N, "/".join(str(x) for x in w.lengths[:4]) +
                                                       ("/..." if w.N > 4 else ""), w.T, w.H, w.HV, w.d,
                                                       int(w.l2norm), "deterministic" if det else "atomic"),
                   "global_batch": w.T, "seq_len": max(w.lengths), "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "step_roofline": {"op": "fwdbwd", "roofline_ms": 1e3 * sr["fwdbwd"]["roofline_s"],
                          "frac": sr["fwdbwd"]["roofline_s"] / (ms / 1e3)},
        "kernels_ms_per_step": {k: v["total_ms"] / args.steps for k, v in sorted(kernels.items())},
        "wall_s": wall_fb,
    }
    for k, v in extra.items():
        out[k] = dict(v, roofline_frac=sr[k]["roofline_s"] / (v["ms"] / 1e3))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
