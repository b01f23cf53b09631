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

    python bench.py [--steps K] [--warmup W] [--workload pack262k] [--atomic]
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


def kernel_models(T, NT, N, H, HV, D, io, has_h0=False, det=False, full=False):
    """Algorithmic (compulsory) bytes and MFMA flops of one launch of each kernel.

    Bytes: every operand of the kernel read once and every result written once (a q/k tile read by
    the G value heads of its group counts once). Flops: the contractions of the chunked method the
    kernel performs, 2 flops per multiply-add.
    """
    C = CHUNK
    f4 = 4
    pv = NT * HV * C * C * 2       # decayed masked q.k per value head (P or P^T), bf16
    akk = T * HV * C * 2           # A rows, bf16
    scal_v = T * HV * f4           # one f32 per token and value head
    scal_q = T * H * f4            # one f32 per token and q/k head
    gam = NT * HV * f4
    tape = NT * HV * D * D * 2     # one bf16 state per chunk and value head
    qkin = T * H * D * io
    vin = T * HV * D * io
    states = N * HV * D * D * f4
    acc = T * H * D * f4           # f32 dq or dk accumulator (atomic reduction)
    m = {}
    m["gdn_intra"] = (2 * qkin + 2 * scal_v + 2 * scal_q + pv + akk + scal_v + gam,
                      NT * H * 2 * (2 * C * C * D) + NT * HV * (2 * C ** 3 // 3))
    m["gdn_intra_bwd"] = (2 * qkin + scal_v + 2 * scal_q + pv, NT * H * 2 * (2 * C * C * D))
    m["gdn_walk_fwd"] = (2 * qkin + vin + akk + pv + 2 * scal_v + 2 * scal_q + vin + (2 * states if has_h0 else 0),
                         T * HV * (6 * D * D + 4 * C * D))
    m["gdn_walk_tape"] = (qkin + vin + akk + 2 * scal_v + scal_q + tape + (states if has_h0 else 0),
                          T * HV * (4 * D * D + 2 * C * D))
    m["gdn_walk_bwd"] = (2 * qkin + vin + akk + pv + 2 * scal_v + 2 * scal_q + tape + (2 * states if has_h0 else 0),
                         T * HV * (6 * D * D + 4 * C * D))
    m["gdn_walk_pair"] = tuple(x + y for x, y in zip(m["gdn_walk_tape"], m["gdn_walk_bwd"]))
    if full:
        # the full saved set: the forward walk also writes the state tape and v_new (bf16); w, u
        # and the P rows are formed and copied by k_wy_full
        fw = m["gdn_walk_fwd"]
        m["gdn_walk_fwd"] = (fw[0] + tape + T * HV * D * 2, fw[1])
        m["gdn_wy_full"] = (akk + qkin + vin + pv + 2 * scal_v + scal_q + 2 * T * HV * D * 2 + akk,
                            T * HV * 2 * (2 * C * D))
    out_qk = 2 * qkin if det else 2 * acc
    m["gdn_chunk_grad"] = (2 * tape + 2 * qkin + 2 * vin + akk + pv + 2 * scal_v + 2 * scal_q + gam
                           + vin + 2 * scal_v + out_qk,
                           T * HV * 2 * (5 * D * D + 8 * C * D + 2 * C * C) + NT * H * 2 * (2 * C * C * D))
    m["gdn_finalize_qk"] = (2 * acc + 2 * qkin + 2 * scal_q + 2 * qkin, 0)
    m["gdn_fill_zero"] = (acc, 0)
    return m


def step_roofline(T, HV, D, io_bytes, full=False):
    """Op-level algorithmic work (inputs, outputs and the saved set; tapes excluded) per token. The
    full saved set adds a bf16 state per chunk and v_new, w, u and the q.k tiles per token."""
    C = CHUNK
    G = 3
    fl_f = 6 * D * D + 6 * C * D + 4 * C * D / G + 2 * C * C / 3
    fl_b = 16 * D * D + (12 + 2 / G) * 2 * C * D + 4 * C * C / 3
    fl_r = 2 * C * D / G + 2 * C * C / 3
    inputs = 2 * 16 * D * io_bytes + HV * D * io_bytes + 2 * HV * 4
    saved = HV * C * 2 + HV * 4 + HV * 4 / C
    if full:
        saved += HV * D * D * 2 / C + 3 * HV * D * 2 + HV * C * 2
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
    """Hash of a kernel source file and every header beside it (the kernels include them)."""
    import glob
    h = hashlib.sha256()
    for p in [path] + sorted(glob.glob(os.path.join(os.path.dirname(path), "*.h"))):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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
    """Time the FP64 oracle (fwd + bwd, all heads) on the two shortest documents of the workload."""
    import numpy as np
    import oracle

    cu = inputs_dev["cu_seqlens"].cpu().numpy()
    lens = np.diff(cu)
    docs = sorted(np.argsort(lens, kind="stable")[:2].tolist())
    tok = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in docs])
    ti = __import__("torch").from_numpy(tok).to(inputs_dev["q"].device)
    f = lambda t: None if t is None else t.index_select(0, ti).float().cpu().numpy()
    q, k, v, g, b, dO = (f(inputs_dev[x]) for x in ("q", "k", "v", "g", "beta", "dO"))
    cu1 = np.zeros(len(docs) + 1, np.int32)
    cu1[1:] = np.cumsum(lens[docs])
    threads = oracle.default_threads()
    used = min(threads, len(docs) * w.H)  # the oracle splits work over (document, q/k head) items
    t0 = time.time()
    oracle.fwd(cu1, q, k, v, g, b, None, l2norm=w.l2norm, threads=threads)
    oracle.bwd(cu1, q, k, v, g, b, dO, None, None, l2norm=w.l2norm, threads=threads)
    dt = time.time() - t0
    ntok = int(len(tok))
    return {"value": ntok / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": "fwd+bwd of documents %s (%d tokens, all %d q/k and %d v heads, d=%d) of the same pack, "
                      "FP64 token recurrence, %.1f s" % ("/".join(str(int(lens[n])) for n in docs), ntok, w.H,
                                                          w.HV, w.d, dt)}


COPY_BYTES = 1 << 30  # bytes read (and written) by the calibration copy

# Library kernels in launch order within one fwd + bwd step (light, D = 128). rocprofv3 prints some
# template instances mangled and some garbled, so two instances of one template are told apart by
# the order in which their kernel ids first appear: the forward call runs before the backward.
KERNEL_ORDER = {"k_tables": ["gdn_tables"], "k_intra": ["gdn_intra", "gdn_intra_bwd"],
                "k_walk_fwd": ["gdn_walk_fwd", "gdn_walk_tape"], "k_write_tag": ["gdn_write_tag"],
                "k_walk_pair": ["gdn_walk_pair"], "k_walk_bwd": ["gdn_walk_bwd"], "k_fill_zero": ["gdn_fill_zero"],
                "k_chunk_grad": ["gdn_chunk_grad"], "k_finalize_qk": ["gdn_finalize_qk"]}
KERNEL_SOURCE = {"gdn_tables": "gdn_fwd.hip", "gdn_intra": "gdn_fwd.hip", "gdn_intra_bwd": "gdn_fwd.hip",
                 "gdn_walk_fwd": "gdn_fwd.hip", "gdn_walk_tape": "gdn_fwd.hip", "gdn_write_tag": "gdn_bwd.hip",
                 "gdn_walk_bwd": "gdn_bwd.hip", "gdn_walk_pair": "gdn_bwd.hip", "gdn_fill_zero": "gdn_bwd.hip", "gdn_chunk_grad": "gdn_bwd.hip",
                 "gdn_finalize_qk": "gdn_bwd.hip"}


def _csv_rows(d, suffix):
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


def _kernel_names(rows):
    """Kernel_Id -> library kernel name (or None), by template and first appearance."""
    first = {}
    for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
        first.setdefault(r["Kernel_Id"], (int(r["Dispatch_Id"]), r["Kernel_Name"]))
    seen = {}
    out = {}
    for kid, (_, name) in sorted(first.items(), key=lambda x: x[1][0]):
        tmpl = next((t for t in KERNEL_ORDER if t in name), None)
        if tmpl is None:
            out[kid] = None
            continue
        i = seen.get(tmpl, 0)
        seen[tmpl] = i + 1
        out[kid] = KERNEL_ORDER[tmpl][min(i, len(KERNEL_ORDER[tmpl]) - 1)]
    return out


def summarize_pmc(fetch_dir, write_dir, out_dir, workload):
    """Per-launch HBM bytes of each library kernel: FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    each scaled by bytes / reading of the same counter on the calibration copy (COPY_BYTES read and
    written by one copy kernel, the run's last torch elementwise kernel). Writes
    pmc_<kernel>_<workload>.json per kernel into out_dir and prints a table."""
    res, scales = {}, {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _csv_rows(d, "counter_collection.csv") if r["Counter_Name"] == counter]
        if not rows:
            raise SystemExit("no %s rows in %s" % (counter, d))
        names = _kernel_names(rows)
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        copies = [float(r["Counter_Value"]) for r in rows
                  if names[r["Kernel_Id"]] is None and ("copy" in r["Kernel_Name"].lower()
                                                        or "elementwise" in r["Kernel_Name"].lower())]
        scales[counter] = COPY_BYTES / copies[-1]
        for r in rows:
            n = names[r["Kernel_Id"]]
            if n:
                res.setdefault(n, {}).setdefault(counter, []).append(float(r["Counter_Value"]) * scales[counter])
    os.makedirs(out_dir, exist_ok=True)
    # a kernel may run as two launches per call (one per part of a split launch plan): traffic is
    # summed per fwd+bwd step (gdn_tables runs once per call, twice per step)
    n_steps = max(1, len(res.get("gdn_tables", {}).get("FETCH_SIZE", [])) // 2)
    lines = ["| kernel | launches/step | FETCH bytes/step | WRITE bytes/step | HBM GB/step |",
             "|---|---|---|---|---|"]
    for name, c in sorted(res.items()):
        if "FETCH_SIZE" not in c or "WRITE_SIZE" not in c:
            continue
        fb, wb = sum(c["FETCH_SIZE"]) / n_steps, sum(c["WRITE_SIZE"]) / n_steps
        per_step = len(c["FETCH_SIZE"]) / n_steps
        src = KERNEL_SOURCE[name]
        rec = {"kernel": name, "workload": workload, "fetch_bytes_per_step": fb, "write_bytes_per_step": wb,
               "bytes_per_step": fb + wb, "launches_per_step": per_step, "bytes_per_launch": (fb + wb) / per_step,
               "source": src,
               "source_sha": source_sha(os.path.join(ROOT, "gated_deltanet_fwd_amd", "csrc", src)),
               "copy_scale_bytes_per_unit": scales}
        with open(os.path.join(out_dir, "pmc_%s_%s.json" % (name, workload)), "w") as f:
            json.dump(rec, f, indent=1)
        lines.append("| `%s` | %g | %.4e | %.4e | %.3f |" % (name, per_step, fb, wb, (fb + wb) / 1e9))
    print("\n".join(lines))
    print("\ncalibration: bytes per counter unit %s (copy of %d bytes read and written)" % (scales, COPY_BYTES))


def summarize_mfma(pmc_dir, command):
    """MFMA work and utilisation per library kernel from one rocprofv3 --pmc run of this script with
    the derived counters MfmaUtil (MFMA-busy SIMD cycles / (GPU-active cycles x SIMDs), per cent),
    MfmaFlopsBF16 and MfmaFlopsF32 (MFMA operations x 512). Durations are the dispatch timestamps of
    the same run (the profiler runs dispatches one at a time). Prints a markdown table per step."""
    rows = _csv_rows(pmc_dir, "counter_collection.csv")
    names = _kernel_names(rows)
    disp = {}
    for r in rows:
        n = names[r["Kernel_Id"]]
        if not n:
            continue
        d = disp.setdefault(int(r["Dispatch_Id"]), {"name": n, "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    n_steps = max(1, sum(1 for d in disp.values() if d["name"] == "gdn_tables") // 2)
    agg = {}
    for d in disp.values():
        a = agg.setdefault(d["name"], {"n": 0, "ns": 0.0, "bf16": 0.0, "f32": 0.0, "util_ns": 0.0})
        a["n"] += 1
        a["ns"] += d["ns"]
        a["bf16"] += d.get("MfmaFlopsBF16", 0.0)
        a["f32"] += d.get("MfmaFlopsF32", 0.0)
        a["util_ns"] += d.get("MfmaUtil", 0.0) * d["ns"]
    lines = ["Command (from the repository root on one MI355X):", "", "```", command, "```", "",
             "| kernel | launches/step | ms/step (profiled) | bf16 MFMA TFLOP/step | f32 MFMA TFLOP/step "
             "| MFMA busy (% of SIMD cycles) | bf16 MFMA TFLOP/s | of 2.5 PFLOP/s |",
             "|---|---|---|---|---|---|---|---|"]
    for n, a in sorted(agg.items(), key=lambda x: -x[1]["ns"]):
        if a["bf16"] == 0 and a["f32"] == 0:
            continue
        sec = a["ns"] * 1e-9
        lines.append("| `%s` | %g | %.3f | %.3f | %.3f | %.1f | %.1f | %.3f |" % (
            n, a["n"] / n_steps, 1e3 * sec / n_steps, a["bf16"] / n_steps / 1e12, a["f32"] / n_steps / 1e12,
            a["util_ns"] / a["ns"], a["bf16"] / sec / 1e12, a["bf16"] / sec / PEAK_BF16))
    print("\n".join(lines))


def summarize_trace(trace_dir, command):
    """Per-kernel count, total and average duration from a rocprofv3 --kernel-trace CSV."""
    import statistics
    rows = _csv_rows(trace_dir, "kernel_trace.csv")
    names = _kernel_names(rows)
    agg = {}
    for r in rows:
        n = names[r["Kernel_Id"]] or r["Kernel_Name"][:60]
        agg.setdefault(n, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6)
    total = sum(sum(v) for v in agg.values())
    lines = ["Command (from the repository root on one MI355X):", "", "```", command, "```", "",
             "| kernel | calls | total ms | avg ms | median ms | % of GPU time |", "|---|---|---|---|---|---|"]
    for n, v in sorted(agg.items(), key=lambda x: -sum(x[1])):
        lines.append("| `%s` | %d | %.3f | %.3f | %.3f | %.1f |" % (n, len(v), sum(v), sum(v) / len(v),
                                                                  statistics.median(v), 100 * sum(v) / total))
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="pack262k")
    ap.add_argument("--atomic", action="store_true",
                    help="float-atomic dq/dk reduction (default: the deterministic fixed-order reduction)")
    ap.add_argument("--full", action="store_true",
                    help="full saved set: the forward also saves the states, v_new, w, u and the q.k tiles, "
                         "and the backward does not replay the states (default: the light saved set)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the fwd-only and ckpt timings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run a plain device copy of %d MiB (counter calibration)" %
                    (COPY_BYTES >> 20))
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script with "
                         "--copy-calibration into per-kernel HBM traffic records; no GPU is used")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_DIR", "COMMAND"),
                    help="MFMA utilisation and work per kernel from a rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 "
                         "MfmaFlopsF32 run of this script; no GPU")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "COMMAND"),
                    help="per-kernel durations from a rocprofv3 --kernel-trace run of this script; no GPU")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, workload=args.workload)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (it would shard the "
              "q/k-head groups or the sequence across GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_fwd_amd as G
    import synthetic as syn

    lib = G.load_library()
    w = syn.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    inp = syn.make_inputs(w, device=dev)
    det = not args.atomic
    p = G.problem_for(w, save_mode=G.SAVE_FULL if args.full else G.SAVE_LIGHT, deterministic=det)
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
    models = kernel_models(w.T, NT, w.N, w.H, w.HV, w.d, io, has_h0=w.has_h0, det=det, full=args.full)
    # dominant kernel = largest share of the timed step (summed launch time). A kernel may run as
    # several launches per step (the longest document's and the others'); its per-launch
    # algorithmic work is then the step's divided by the launches, so that achieved = the step's
    # work / the step's summed launch time (a lower bound when the launches overlap in time).
    dom = max((k for k in kernels if k in models), key=lambda k: kernels[k]["total_ms"])
    per_step = kernels[dom]["launches"] / args.steps
    by, fl = (x / per_step for x in models[dom])
    avg_s = kernels[dom]["avg_ms"] / 1e3
    t_hbm, t_mfma = by / PEAK_HBM, fl / PEAK_BF16
    if t_mfma > t_hbm:
        roof = {"bound": "mfma", "achieved": fl / avg_s / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": by / avg_s / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # the committed counters are of the default step (light saved set, deterministic reduction)
    default_kernel = not args.full and not (args.atomic and dom in ("gdn_chunk_grad", "gdn_fill_zero",
                                                                    "gdn_finalize_qk"))
    roof["traffic"] = load_traffic(dom, args.workload) if default_kernel else None
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = by
    roof["algorithmic_flops"] = fl
    roof["avg_launch_ms"] = kernels[dom]["avg_ms"]
    roof["launches_per_step"] = per_step

    sr = step_roofline(w.T, w.HV, w.d, io, full=args.full)
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
        "config": {"workload": "%s: %d docs %s, %d tokens, (H,HV)=(%d,%d), d=%d, l2norm=%d, %s saved set, "
                               "%s dq/dk reduction" % (w.name, w.N, "/".join(str(x) for x in w.lengths[:4]) +
                                                       ("/..." if w.N > 4 else ""), w.T, w.H, w.HV, w.d,
                                                       int(w.l2norm), "full" if args.full else "light",
                                                       "deterministic" if det else "atomic"),
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
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
