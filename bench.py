#!/usr/bin/env python3
"""Benchmark of the MI355X gated-delta-rule training kernel (one GPU).

One step = one pass of the whole hot path over one batch: gdn_fwd then gdn_bwd (light saved
set, deterministic dq/dk reduction) on the packed workload of 4 documents
98304/65536/57344/40960 = 262144 tokens, (H, HV) = (16, 48), d = 128, bf16 inputs with the
in-kernel q/k L2 norm (the pages' "shape A"). Inputs are drawn once on the GPU and are resident
in HBM before timing starts.

Prints one JSON line:
  value / ms_per_step   fwd+bwd tokens/s over exactly --steps back-to-back steps, bracketed by
                        synchronisations (no per-kernel instrumentation in that loop)
  protocol              fwd, fwd+bwd and checkpointed (fwd + recompute + bwd, also with the
                        recompute's kept tape) under the pages' timing protocol: a >= 512 MiB
                        buffer written before every timed call, 5 groups x 12 calls, median and
                        per-group drift
  configs               the other workloads (8,192-token document fwd, CP4 share fwd+bwd with h0,
                        512 short documents checkpointed, and the pages' shape B23: the causal
                        conv1d + SiLU front-end over 10,240 packed q/k/v channels with the layer),
                        same protocol, each with its op roofline fraction
  roofline              the kernel with the longest span on the step's critical path: its
                        algorithmic bytes (inputs, outputs, saved set) or flops per step over its
                        span per step (first launch's start to last launch's end, HIP events
                        recorded on the stream each launch goes to, in a separate pass; with one
                        launch per step, that launch's duration); `traffic` is the committed HBM
                        counter figure for that kernel per step when its source is unchanged
  cpu_baseline          the FP64 oracle on the host cores on a bounded sample of the same workload
                        (every document, a few q/k-head groups), fwd+bwd, fwd and checkpointed

    python bench.py [--steps K] [--warmup W] [--workload pack262k] [--atomic] [--full]
                    [--no-cpu-baseline] [--no-extra] [--gpus 1]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12           # bytes/s, MI355X HBM3E
PEAK_BF16 = 2.5e15          # flop/s, MI355X dense bf16 MFMA
CHUNK = 64
FLUSH_BYTES = 512 << 20     # written before every timed call of the protocol (L2 and MALL)
METRIC = "tokens/s fwd+bwd (and fwd, ckpt) at (H,HV)=(16,48), d=128, 262144 tok"


def kernel_models(T, NT, N, H, HV, D, io, has_h0=False, has_dht=False, want_ht=False, det=True, save_mode="light"):
    """Per kernel, over one fwd + bwd step: (algorithmic bytes, MFMA flops, intermediate bytes).

    Algorithmic bytes are the op roofline's: the inputs, outputs, saved set and states that the
    kernel reads or writes, each tensor counted once per kernel (a q/k tile read by the G value
    heads of its group counts once). Intermediates the implementation moves (the replayed state
    tape and the end-state-gradient tape, the per-value-head q.k tiles, the inverse norms, FP32
    dq/dk accumulators) are not algorithmic and are reported apart. In the full and kept-tape forms
    the state tape (and, full, v_new, w, u, the q.k rows) belong to the saved set, so their writes
    and reads are algorithmic. Flops: the contractions of the chunked method the kernel performs,
    2 flops per multiply-add.
    """
    C = CHUNK
    f4 = 4
    full, kept = save_mode == "full", save_mode in ("full", "tape")
    pv = NT * HV * C * C * 2       # decayed masked q.k per value head (P or P^T), bf16
    akk = T * HV * C * 2           # A rows, bf16 (saved)
    gb = T * HV * f4               # g or beta (input), gcum (saved), dg or dbeta (output)
    gam = NT * HV * f4             # gamma (saved)
    nrm = T * H * f4               # inverse norms of q or k rows (workspace)
    tape = NT * HV * D * D * 2     # one bf16 state per chunk and value head
    qk = T * H * D * io            # q or k (input), dq or dk (output)
    vv = T * HV * D * io           # v, dO (inputs), o, dv (outputs)
    wuv = T * HV * D * 2           # w, u or v_new rows, bf16
    st = N * HV * D * D * f4       # one state tensor
    acc = T * H * D * f4           # f32 dq or dk accumulator (atomic reduction)
    h0 = st if has_h0 else 0
    m = {}
    # name: (algorithmic bytes, flops, intermediate bytes)
    m["gdn_intra"] = (2 * qk + 2 * gb + akk + gb + gam,
                      NT * H * 2 * (2 * C * C * D) + NT * HV * (2 * C ** 3 // 3), pv + 2 * nrm)
    m["gdn_walk_fwd"] = (2 * qk + vv + akk + 2 * gb + h0 + vv + (st if want_ht else 0)
                         + (tape if kept else 0) + (wuv if full else 0),
                         T * HV * (6 * D * D + 4 * C * D), pv + 2 * nrm)
    if full:
        m["gdn_wy_full"] = (akk + qk + vv + 2 * gb + 2 * wuv + akk, T * HV * 2 * (2 * C * D), pv + nrm)
    m["gdn_intra_bwd"] = (2 * qk + gb, NT * H * 2 * (2 * C * C * D), pv + 2 * nrm)
    rev = (2 * qk + vv + akk + 2 * gb + (st if has_dht else 0) + h0, T * HV * (6 * D * D + 4 * C * D),
           pv + 2 * nrm + tape)
    if kept:
        m["gdn_walk_bwd"] = rev
    else:
        tw = (qk + vv + akk + 2 * gb + h0, T * HV * (4 * D * D + 2 * C * D), nrm + tape)
        m["gdn_walk_pair"] = tuple(x + y for x, y in zip(tw, rev))
    grad_alg = 2 * qk + 2 * vv + akk + 2 * gb + vv + 2 * gb + (2 * qk if det else 0) + (tape if kept else 0)
    grad_int = (tape if kept else 2 * tape) + pv + 2 * nrm + (0 if det else 2 * acc)
    m["gdn_chunk_grad"] = (grad_alg, T * HV * 2 * (5 * D * D + 8 * C * D + 2 * C * C) + NT * H * 2 * (2 * C * C * D),
                           grad_int)
    if not det:
        m["gdn_finalize_qk"] = (2 * qk + 2 * qk, 0, 2 * acc + 2 * nrm)
        m["gdn_fill_zero"] = (0, 0, acc)
    return m


def step_roofline(T, HV, D, io_bytes, H=16, NT=None, N=1, has_h0=False, want_ht=False, has_dht=False,
                  save_mode="light"):
    """Op-level algorithmic work per token: MFMA flops of the chunked method and HBM bytes of the
    inputs, outputs and the saved set (written by fwd and recompute, read by bwd), plus the states
    a workload passes (h0 and dht read, ht and dh0 written). Tapes and other intermediates are not
    counted. The full saved set adds a bf16 state per chunk and v_new, w, u and the q.k rows per
    token; the kept-tape form adds the state only. Returns fwd, fwdbwd and ckpt (fwd + recompute +
    bwd) records with the roofline time max(flops / MFMA peak, bytes / HBM peak)."""
    C = CHUNK
    G = HV // H
    NT = T / C if NT is None else NT
    fl_f = 6 * D * D + 6 * C * D + 4 * C * D / G + 2 * C * C / 3
    fl_b = 16 * D * D + (12 + 2 / G) * 2 * C * D + 4 * C * C / 3
    fl_r = 2 * C * D / G + 2 * C * C / 3
    inputs = 2 * H * D * io_bytes + HV * D * io_bytes + 2 * HV * 4
    saved = HV * C * 2 + HV * 4 + HV * 4 * NT / T
    if save_mode in ("full", "tape"):
        saved += HV * D * D * 2 * NT / T
    if save_mode == "full":
        saved += 3 * HV * D * 2 + HV * C * 2
    state = N * HV * D * D * 4 / T if T else 0.0
    b_f = inputs + HV * D * io_bytes + saved + state * (has_h0 + want_ht)
    b_b = (inputs + HV * D * io_bytes + saved + 2 * H * D * io_bytes + HV * D * io_bytes + 2 * HV * 4
           + state * (has_h0 + has_dht + has_h0))
    # the recompute reads k, g, beta; its state walk (kept-tape and full forms) also v, and the full
    # form's q.k rows q
    b_r = (H * D * io_bytes + 2 * HV * 4 + saved + (HV * D * io_bytes if save_mode != "light" else 0)
           + (H * D * io_bytes if save_mode == "full" else 0))
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
    """HBM bytes per step from committed rocprofv3 counter runs, if the kernel is unchanged."""
    path = os.path.join(ROOT, "profiles", "pmc_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, "gated_deltanet_fwd_amd", "csrc", rec.get("source", ""))
    if not os.path.exists(src) or source_sha(src) != rec.get("source_sha"):
        return None
    return float(rec["bytes_per_step"])


def _oracle_sample(w, inputs_dev, heads, ops=("fwd", "bwd")):
    """Times the FP64 oracle on every document of the workload for q/k heads [0, heads) with their
    value heads. Returns (seconds per op, threads used, value heads sampled)."""
    import oracle

    threads = oracle.default_threads()
    Gg = w.HV // w.H
    vh = [j * Gg + gi for j in range(heads) for gi in range(Gg)]
    f = lambda name, idx: inputs_dev[name][:, idx].float().cpu().numpy()
    q, k = f("q", list(range(heads))), f("k", list(range(heads)))
    v, g, b, dO = (f(x, vh) for x in ("v", "g", "beta", "dO"))
    h0 = inputs_dev["h0"][:, vh].float().cpu().numpy() if inputs_dev.get("h0") is not None else None
    dht = inputs_dev["dht"][:, vh].float().cpu().numpy() if inputs_dev.get("dht") is not None else None
    cu = inputs_dev["cu_seqlens"].cpu().numpy()
    used = min(threads, w.N * heads)  # the oracle splits work over (document, q/k head) items
    t = {}
    if "fwd" in ops:
        t0 = time.time()
        oracle.fwd(cu, q, k, v, g, b, h0, l2norm=w.l2norm, threads=threads)
        t["fwd"] = time.time() - t0
    if "bwd" in ops:
        t0 = time.time()
        oracle.bwd(cu, q, k, v, g, b, dO, h0, dht, l2norm=w.l2norm, threads=threads)
        t["bwd"] = time.time() - t0
    return t, used, len(vh)


def cpu_baseline(w, inputs_dev):
    """Time the FP64 oracle on a bounded sample of the workload: every document in full, for the
    first few q/k heads (with their value heads), enough (document, head) items to occupy the host
    cores. The oracle's cost per token and head is the same everywhere, so the whole workload's
    rate is the sample's tokens x H / sampled heads over its time. Times fwd and bwd (the oracle's
    reverse mode recomputes its forward) separately; fwd+bwd = both, ckpt = 2 fwd + bwd."""
    import oracle

    threads = oracle.default_threads()
    heads = max(1, min(w.H, math.ceil(threads / max(1, w.N))))
    t, used, nvh = _oracle_sample(w, inputs_dev, heads)
    t_f, t_b = t["fwd"], t["bwd"]
    scale = w.H / heads  # whole-workload time = sample time x this
    rate = lambda t: w.T / (t * scale)
    return {"value": rate(t_f + t_b), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": "fwd+bwd of all %d documents (%d tokens) for q/k heads 0..%d of %d with their %d value heads, "
                      "d=%d, FP64 token recurrence: fwd %.1f s + bwd %.1f s; tokens/s scaled by %d/%d heads"
                      % (w.N, w.T, heads - 1, w.H, nvh, w.d, t_f, t_b, w.H, heads),
            "fwd_tokens_per_s": rate(t_f), "ckpt_tokens_per_s": rate(2 * t_f + t_b), "threads": threads}


# The other workloads' oracle rates: q/k heads sampled per workload so that each takes a few
# seconds of host time (the oracle's cost is per token and value head).
CPU_CONFIG_HEADS = {"tiny": 2, "single8k": 16, "cp4share": 8, "short512": 2}


def cpu_configs(dev):
    """The FP64 oracle's fwd, fwd+bwd and ckpt (2 fwd + bwd) rates on each other workload, on a
    bounded sample (all documents, the first q/k heads), scaled to the whole workload."""
    import synthetic as syn

    out = {}
    for name, heads in CPU_CONFIG_HEADS.items():
        w = syn.WORKLOADS[name]
        heads = min(heads, w.H)
        inp = syn.make_inputs(w, device=dev)
        t, used, nvh = _oracle_sample(w, inp, heads)
        del inp
        scale = w.H / heads
        rate = lambda x: w.T / (x * scale)
        out[name] = {"fwd_tokens_per_s": rate(t["fwd"]), "fwdbwd_tokens_per_s": rate(t["fwd"] + t["bwd"]),
                     "ckpt_tokens_per_s": rate(2 * t["fwd"] + t["bwd"]), "cores": used,
                     "sample": "all %d documents (%d tokens), q/k heads 0..%d of %d (%d value heads): fwd %.2f s, "
                               "bwd %.2f s; scaled by %d/%d heads" % (w.N, w.T, heads - 1, w.H, nvh, t["fwd"],
                                                                     t["bwd"], w.H, heads)}
    return out


COPY_BYTES = 1 << 30  # bytes read (and written) by the calibration copy

# Library kernels in launch order within one fwd + bwd step (light, D = 128). rocprofv3 prints some
# template instances mangled and some garbled, so two instances of one template are told apart by
# the order in which their kernel ids first appear: the forward call runs before the backward.
KERNEL_ORDER = {"k_tables": ["gdn_tables"], "k_intra": ["gdn_intra", "gdn_intra_bwd"],
                "k_walk_fwd": ["gdn_walk_fwd", "gdn_walk_tape"], "k_write_tag": ["gdn_write_tag"],
                "k_walk_pair": ["gdn_walk_pair"], "k_walk_bwd": ["gdn_walk_bwd"], "k_fill_zero": ["gdn_fill_zero"],
                "k_chunk_grad": ["gdn_chunk_grad"], "k_finalize_qk": ["gdn_finalize_qk"],
                "k_poison": ["gdn_poison"]}
KERNEL_SOURCE = {"gdn_tables": "gdn_fwd.hip", "gdn_intra": "gdn_fwd.hip", "gdn_intra_bwd": "gdn_fwd.hip",
                 "gdn_walk_fwd": "gdn_fwd.hip", "gdn_walk_tape": "gdn_fwd.hip", "gdn_write_tag": "gdn_bwd.hip",
                 "gdn_walk_bwd": "gdn_bwd.hip", "gdn_walk_pair": "gdn_bwd.hip", "gdn_fill_zero": "gdn_bwd.hip", "gdn_chunk_grad": "gdn_bwd.hip",
                 "gdn_finalize_qk": "gdn_bwd.hip", "gdn_poison": "gdn_bwd.hip"}


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
    """Per-kernel count, total and average duration from a rocprofv3 --kernel-trace CSV, and the
    mean span per fwd+bwd step (first start to last end of the kernel's launches between the
    starts of consecutive forward calls; gdn_tables opens every call, the forward's first)."""
    import statistics
    rows = _csv_rows(trace_dir, "kernel_trace.csv")
    names = _kernel_names(rows)
    agg, iv = {}, []
    for r in rows:
        n = names[r["Kernel_Id"]] or r["Kernel_Name"][:60]
        s, e = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        agg.setdefault(n, []).append((e - s) * 1e-6)
        iv.append((s, e, n))
    iv.sort()
    opens = [s for s, _, n in iv if n == "gdn_tables"][::2]  # forward calls
    spans = {}
    for a, b in zip(opens, opens[1:] + [float("inf")]):
        step = {}
        for s, e, n in iv:
            if a <= s < b:
                lo, hi = step.get(n, (s, e))
                step[n] = (min(lo, s), max(hi, e))
        for n, (lo, hi) in step.items():
            spans.setdefault(n, []).append((hi - lo) * 1e-6)
    total = sum(sum(v) for v in agg.values())
    lines = ["Command (from the repository root on one MI355X):", "", "```", command, "```", "",
             "| kernel | calls | total ms | avg ms | median ms | span ms/step | % of GPU time |",
             "|---|---|---|---|---|---|---|"]
    for n, v in sorted(agg.items(), key=lambda x: -sum(x[1])):
        sp = "%.3f" % statistics.mean(spans[n]) if n in spans and n.startswith("gdn_") else ""
        lines.append("| `%s` | %d | %.3f | %.3f | %.3f | %s | %.1f |" % (n, len(v), sum(v), sum(v) / len(v),
                                                                       statistics.median(v), sp,
                                                                       100 * sum(v) / total))
    print("\n".join(lines))


def _nt(w):
    return int(sum((L + CHUNK - 1) // CHUNK for L in w.lengths))


def _workload_desc(w, save_mode, det):
    lens = "/".join(str(x) for x in w.lengths[:4]) + ("/..." if w.N > 4 else "")
    return ("%s: %d docs %s, %d tokens, (H,HV)=(%d,%d), d=%d, l2norm=%d%s, %s saved set, %s dq/dk reduction"
            % (w.name, w.N, lens, w.T, w.H, w.HV, w.d, int(w.l2norm), ", h0, ht, dht" if w.has_h0 else "",
               save_mode, "deterministic" if det else "atomic"))


class Runner:
    """Buffers and calls of one workload on the GPU (inputs resident in HBM)."""

    def __init__(self, G, syn, w, dev, save_mode="light", det=True, segments=0):
        import torch
        self.G, self.w, self.dev = G, w, dev
        modes = {"light": G.SAVE_LIGHT, "full": G.SAVE_FULL, "tape": G.SAVE_TAPE}
        self.inp = syn.make_inputs(w, device=dev)
        self.p = G.problem_for(w, save_mode=modes[save_mode], deterministic=det, segments=segments)
        self.pt = G.problem_for(w, save_mode=G.SAVE_TAPE, deterministic=det, segments=segments)  # kept-tape ckpt
        e = lambda n: torch.empty(n, dtype=torch.uint8, device=dev)
        self.saved = e(G.gdn_saved_bytes(self.p))
        self.saved_t = e(G.gdn_saved_bytes(self.pt))
        self.ws_f = e(G.gdn_workspace_bytes(self.p, G.OP_FWD))
        self.ws_r = e(G.gdn_workspace_bytes(self.p, G.OP_RECOMPUTE))
        self.ws_rt = e(G.gdn_workspace_bytes(self.pt, G.OP_RECOMPUTE))
        self.ws_b = e(G.gdn_workspace_bytes(self.p, G.OP_BWD))
        self.ws_bt = e(G.gdn_workspace_bytes(self.pt, G.OP_BWD))
        inp = self.inp
        self.o = torch.empty_like(inp["v"])
        self.ht = torch.empty((w.N, w.HV, w.d, w.d), dtype=torch.float32, device=dev) if w.want_ht else None
        self.grads = dict(dq=torch.empty_like(inp["q"]), dk=torch.empty_like(inp["k"]), dv=torch.empty_like(inp["v"]),
                          dg=torch.empty_like(inp["g"]), dbeta=torch.empty_like(inp["beta"]),
                          dh0=torch.empty_like(inp["h0"]) if inp["h0"] is not None else None)
        self.stream = torch.cuda.current_stream()
        self.a = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"])

    def fwd(self):
        self.G.gdn_fwd(self.p, *self.a, h0=self.inp["h0"], o=self.o, ht=self.ht, saved=self.saved,
                       workspace=self.ws_f, stream=self.stream)

    def recompute(self, kept=False):
        p, sv, ws = (self.pt, self.saved_t, self.ws_rt) if kept else (self.p, self.saved, self.ws_r)
        self.G.gdn_fwd_recompute(p, *self.a, h0=self.inp["h0"], saved=sv, workspace=ws, stream=self.stream)

    def bwd(self, kept=False):
        p, sv, ws = (self.pt, self.saved_t, self.ws_bt) if kept else (self.p, self.saved, self.ws_b)
        self.G.gdn_bwd(p, *self.a, sv, self.inp["dO"], h0=self.inp["h0"], dht=self.inp["dht"], grads=self.grads,
                       workspace=ws, stream=self.stream)

    def op(self, name):
        return {"fwd": self.fwd,
                "fwdbwd": lambda: (self.fwd(), self.bwd()),
                "ckpt": lambda: (self.fwd(), self.recompute(), self.bwd()),
                "ckpt_kept_tape": lambda: (self.fwd(), self.recompute(kept=True), self.bwd(kept=True))}[name]


class B23Runner:
    """The pages' shape B23 layer: the causal conv1d + SiLU front-end over the 10,240 packed q/k/v
    channels, writing q, k and v, then the gated delta rule on them (backward: the rule's backward,
    then the front-end's with dq, dk, dv as its upstream gradients)."""

    def __init__(self, G, syn, dev):
        import torch
        self.G = G
        self.wc = syn.CONV_WORKLOADS["b23_conv"]
        self.w = syn.WORKLOADS["b23"]
        ci = syn.make_conv_inputs(self.wc, device=dev)
        self.x, self.weight, self.bias = ci["x"], ci["weight"], ci["bias"]
        self.cp = G.ConvProblem(ci["cu_seqlens"].cpu().numpy(), self.wc.groups, width=self.wc.width)
        gi = syn.make_inputs(self.w, device=dev)
        self.cu, self.g, self.beta, self.dO = gi["cu_seqlens"], gi["g"], gi["beta"], gi["dO"]
        T, H, HV, d = self.w.T, self.w.H, self.w.HV, self.w.d
        self.q = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
        self.k = torch.empty_like(self.q)
        self.v = torch.empty((T, HV, d), dtype=torch.bfloat16, device=dev)
        self.outs = [self.q.view(T, H * d), self.k.view(T, H * d), self.v.view(T, HV * d)]
        self.p = G.problem_for(self.w)
        e = lambda n: torch.empty(n, dtype=torch.uint8, device=dev)
        self.saved = e(G.gdn_saved_bytes(self.p))
        self.ws_f = e(G.gdn_workspace_bytes(self.p, G.OP_FWD))
        self.ws_r = e(G.gdn_workspace_bytes(self.p, G.OP_RECOMPUTE))
        self.ws_b = e(G.gdn_workspace_bytes(self.p, G.OP_BWD))
        self.ws_c = e(G.gdn_conv_workspace_bytes(self.cp))
        self.o = torch.empty_like(self.v)
        self.grads = dict(dq=torch.empty_like(self.q), dk=torch.empty_like(self.k), dv=torch.empty_like(self.v),
                          dg=torch.empty_like(self.g), dbeta=torch.empty_like(self.beta), dh0=None)
        self.dys = [self.grads["dq"].view(T, H * d), self.grads["dk"].view(T, H * d), self.grads["dv"].view(T, HV * d)]
        self.dx, self.dweight, self.dbias = torch.empty_like(self.x), torch.empty_like(self.weight), torch.empty_like(self.bias)
        self.stream = torch.cuda.current_stream()

    def conv_fwd(self):
        self.G.gdn_conv_fwd(self.cp, self.x, self.weight, self.bias, self.cu, outs=self.outs, stream=self.stream)

    def conv_bwd(self):
        self.G.gdn_conv_bwd(self.cp, self.x, self.weight, self.bias, self.cu, self.dys, dx=self.dx,
                            dweight=self.dweight, dbias=self.dbias, workspace=self.ws_c, stream=self.stream)

    def gdn_fwd(self):
        self.G.gdn_fwd(self.p, self.q, self.k, self.v, self.g, self.beta, self.cu, o=self.o, saved=self.saved,
                       workspace=self.ws_f, stream=self.stream)

    def gdn_recompute(self):
        self.G.gdn_fwd_recompute(self.p, self.q, self.k, self.v, self.g, self.beta, self.cu, saved=self.saved,
                                 workspace=self.ws_r, stream=self.stream)

    def gdn_bwd(self):
        self.G.gdn_bwd(self.p, self.q, self.k, self.v, self.g, self.beta, self.cu, self.saved, self.dO,
                       grads=self.grads, workspace=self.ws_b, stream=self.stream)

    def op(self, name):
        return {"conv_fwd": self.conv_fwd, "conv_bwd": self.conv_bwd,
                "fwd": lambda: (self.conv_fwd(), self.gdn_fwd()),
                "fwdbwd": lambda: (self.conv_fwd(), self.gdn_fwd(), self.gdn_bwd(), self.conv_bwd()),
                "ckpt": lambda: (self.conv_fwd(), self.gdn_fwd(), self.conv_fwd(), self.gdn_recompute(),
                                 self.gdn_bwd(), self.conv_bwd())}[name]


def protocol_time(fn, flush, stream, warmup=10, groups=5, per_group=12):
    """The pages' timing protocol, adapted: `warmup` untimed calls, then `groups` x `per_group`
    timed calls; before each, `flush` (>= 512 MiB) is written and the stream synchronised, and HIP
    events bracket the call alone. Returns the median (ms), the per-group medians and their drift
    (max / min - 1)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    per = []
    for _ in range(groups):
        evs = []
        for _ in range(per_group):
            flush.fill_(1.0)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        per.append([a.elapsed_time(b) for a, b in evs])
    allv = [x for g in per for x in g]
    med_g = [statistics.median(g) for g in per]
    drift = max(med_g) / min(med_g) - 1.0
    return {"median_ms": statistics.median(allv), "group_medians_ms": med_g, "drift": drift,
            "drift_flag": drift > 0.02, "calls": len(allv)}


def kernel_pass(lib, fn, steps):
    """Per-kernel launch times over `steps` calls of fn, each timed alone (every launch bracketed
    by HIP events on its own stream; a synchronisation between calls). Per kernel: launches per
    call, summed launch time per call, span per call (first start to last end of its launches)
    and mean launch duration (ms)."""
    import torch
    names = (ctypes.c_char_p * 256)()
    st = (ctypes.c_double * 256)()
    en = (ctypes.c_double * 256)()
    lib.gdn_timing_launches.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    agg = {}
    wall = []
    for _ in range(steps):
        lib.gdn_timing_reset()
        lib.gdn_timing_enable(1)
        fn()
        torch.cuda.synchronize()
        lib.gdn_timing_enable(0)
        n = min(256, lib.gdn_timing_launches(256, names, st, en))
        per = {}
        for i in range(n):
            per.setdefault(names[i].decode(), []).append((st[i], en[i]))
        wall.append(max(en[i] for i in range(n)) - min(st[i] for i in range(n)))
        for k, iv in per.items():
            a = agg.setdefault(k, {"launches": 0, "sum_ms": 0.0, "span_ms": 0.0})
            a["launches"] += len(iv)
            a["sum_ms"] += sum(e - s for s, e in iv)
            a["span_ms"] += max(e for _, e in iv) - min(s for s, _ in iv)
    lib.gdn_timing_reset()
    out = {}
    for k, a in agg.items():
        out[k] = {"launches_per_step": a["launches"] / steps, "sum_ms_per_step": a["sum_ms"] / steps,
                  "span_ms_per_step": a["span_ms"] / steps, "avg_launch_ms": a["sum_ms"] / a["launches"]}
    return out, statistics.median(wall)


def roofline_of(kernels, models, workload_name, default_step):
    """The kernel with the longest span per step (the largest block of the step's critical path):
    its algorithmic bytes or flops per step over its span per step, against the MI355X peak that
    bounds it (the larger of the HBM and MFMA times at peak). With one launch per step the span is
    that launch's duration; the launches of the two parts of a split plan overlap (and differ in
    size), so their mean duration would misstate the time the kernel holds the step."""
    dom = max((k for k in kernels if k in models), key=lambda k: kernels[k]["span_ms_per_step"])
    kt = kernels[dom]
    per = kt["launches_per_step"]
    by, fl, inter = models[dom]
    avg_s = kt["span_ms_per_step"] / 1e3
    t_hbm, t_mfma = by / PEAK_HBM, fl / PEAK_BF16
    if t_mfma > t_hbm:
        roof = {"bound": "mfma", "achieved": fl / avg_s / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": by / avg_s / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    traffic = load_traffic(dom, workload_name) if default_step else None
    roof["traffic"] = traffic
    roof.update({"kernel": dom, "algorithmic_bytes": by, "algorithmic_flops": fl, "intermediate_bytes": inter,
                 "traffic_ratio": (traffic / by) if traffic else None, "per": "step",
                 "avg_launch_ms": kt["avg_launch_ms"], "launches_per_step": per,
                 "span_ms_per_step": kt["span_ms_per_step"],
                 "mfma_frac": fl / avg_s / PEAK_BF16, "hbm_frac": by / avg_s / PEAK_HBM})
    return roof


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
    ap.add_argument("--no-extra", action="store_true",
                    help="only the headline loop and the kernel pass (no protocol timings, no other workloads)")
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
        print("bench.py measures one GPU only: the library has no multi-GPU path (it would shard the "
              "q/k-head groups or the sequence across GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_fwd_amd as G
    import synthetic as syn

    lib = G.load_library()
    w = syn.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    det = not args.atomic
    mode = "full" if args.full else "light"
    r = Runner(G, syn, w, dev, save_mode=mode, det=det)
    stream = r.stream
    step = r.op("fwdbwd")

    # ---- headline: exactly --steps steps back to back, synchronised on both sides
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.time()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.time() - t0
    t_fb = e0.elapsed_time(e1) / 1e3
    ms = 1e3 * t_fb / args.steps
    value = w.T * args.steps / t_fb

    # ---- per-kernel pass (separate from the headline loop)
    kernels, step_wall_ms = kernel_pass(lib, step, max(3, min(args.steps, 10)))
    io = 2 if w.dtype == "bf16" else 4
    NT = _nt(w)
    models = kernel_models(w.T, NT, w.N, w.H, w.HV, w.d, io, has_h0=w.has_h0, has_dht=w.has_dht,
                           want_ht=w.want_ht, det=det, save_mode=mode)
    default_step = mode == "light" and det
    roof = roofline_of(kernels, models, args.workload, default_step)
    kern_out = {}
    for k, v in sorted(kernels.items()):
        d = dict(v)
        if k in models:
            d.update(algorithmic_bytes_per_step=models[k][0], flops_per_step=models[k][1],
                     intermediate_bytes_per_step=models[k][2])
            tr = load_traffic(k, args.workload) if default_step else None
            if tr:
                d.update(traffic_bytes_per_step=tr, traffic_ratio=tr / models[k][0])
        kern_out[k] = d

    sr = step_roofline(w.T, w.HV, w.d, io, H=w.H, NT=NT, N=w.N, has_h0=w.has_h0, want_ht=w.want_ht,
                       has_dht=w.has_dht, save_mode=mode)
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
        "config": {"workload": _workload_desc(w, mode, det), "global_batch": w.T, "seq_len": max(w.lengths),
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "step_roofline": {"op": "fwdbwd", "roofline_ms": 1e3 * sr["fwdbwd"]["roofline_s"],
                          "frac": sr["fwdbwd"]["roofline_s"] / (ms / 1e3),
                          "bytes_per_token": sr["fwdbwd"]["bytes_per_token"],
                          "flops_per_token": sr["fwdbwd"]["flops_per_token"]},
        "kernels": kern_out,
        "kernel_pass_step_ms": step_wall_ms,
        "wall_s": wall,
    }

    if not args.no_extra:
        flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        prot = {}
        for op in ("fwd", "fwdbwd", "ckpt", "ckpt_kept_tape"):
            t = protocol_time(r.op(op), flush, stream)
            sr_op = sr["ckpt" if op.startswith("ckpt") else op]
            if op == "ckpt_kept_tape":
                sr_op = step_roofline(w.T, w.HV, w.d, io, H=w.H, NT=NT, N=w.N, has_h0=w.has_h0, want_ht=w.want_ht,
                                      has_dht=w.has_dht, save_mode="tape")["ckpt"]
            t.update(tokens_per_s=w.T / (t["median_ms"] / 1e3), roofline_ms=1e3 * sr_op["roofline_s"],
                     roofline_frac=sr_op["roofline_s"] / (t["median_ms"] / 1e3))
            prot[op] = t
        out["protocol"] = prot
        del r
        torch.cuda.empty_cache()
        cfgs = {}
        # segments: 0 = the library's plan (the 8k document in 4 segments, the CP share in 3, the
        # pack and the short documents unsegmented), 1 = unsegmented, 3 = forced
        for key, name, op, segs in (("single8k", "single8k", "fwd", 0), ("single8k_unsegmented", "single8k", "fwd", 1),
                                    ("cp4share", "cp4share", "fwdbwd", 0),
                                    ("cp4share_unsegmented", "cp4share", "fwdbwd", 1),
                                    ("pack262k_fwd_3_segments", "pack262k", "fwd", 3),
                                    ("short512", "short512", "ckpt", 0)):
            wc = syn.WORKLOADS[name]
            rc = Runner(G, syn, wc, dev, save_mode="light", det=wc.deterministic or det, segments=segs)
            t = protocol_time(rc.op(op), flush, stream)
            ioc = 2 if wc.dtype == "bf16" else 4
            src = step_roofline(wc.T, wc.HV, wc.d, ioc, H=wc.H, NT=_nt(wc), N=wc.N, has_h0=wc.has_h0,
                                want_ht=wc.want_ht, has_dht=wc.has_dht)[op]
            t.update(op=op, segments=segs, workload=_workload_desc(wc, "light", wc.deterministic or det),
                     tokens_per_s=wc.T / (t["median_ms"] / 1e3), roofline_ms=1e3 * src["roofline_s"],
                     roofline_frac=src["roofline_s"] / (t["median_ms"] / 1e3))
            cfgs[key] = t
            del rc
            torch.cuda.empty_cache()
        # the pages' shape B23: conv front-end + gated delta rule layer
        b23 = B23Runner(G, syn, dev)
        wc, wb = b23.wc, b23.w
        conv_bytes = {"conv_fwd": 2 * wc.T * wc.C * 2, "conv_bwd": 3 * wc.T * wc.C * 2}
        rec = {"workload": "b23: 4 docs %s, %d tokens, conv over %d channels (%s), width %d, SiLU, then (H,HV)=(%d,%d), "
                           "d=%d, l2norm=1, light saved set" % ("/".join(str(x) for x in wc.lengths), wc.T, wc.C,
                                                               "+".join(str(c) for c in wc.groups), wc.width, wb.H,
                                                               wb.HV, wb.d)}
        srb = step_roofline(wb.T, wb.HV, wb.d, 2, H=wb.H, NT=_nt(wb), N=wb.N)
        for op in ("conv_fwd", "conv_bwd", "fwd", "fwdbwd", "ckpt"):
            t = protocol_time(b23.op(op), flush, stream)
            if op.startswith("conv"):
                t.update(gb_per_s=conv_bytes[op] / (t["median_ms"] / 1e3) / 1e9,
                         roofline_ms=1e3 * conv_bytes[op] / PEAK_HBM,
                         roofline_frac=conv_bytes[op] / PEAK_HBM / (t["median_ms"] / 1e3))
            else:
                extra_bytes = {"fwd": conv_bytes["conv_fwd"], "fwdbwd": sum(conv_bytes.values()),
                               "ckpt": 2 * conv_bytes["conv_fwd"] + conv_bytes["conv_bwd"]}[op]
                r_s = max(srb[op]["roofline_s"], (srb[op]["bytes_per_token"] * wb.T + extra_bytes) / PEAK_HBM)
                t.update(tokens_per_s=wb.T / (t["median_ms"] / 1e3), roofline_ms=1e3 * r_s,
                         roofline_frac=r_s / (t["median_ms"] / 1e3))
            rec[op] = t
        cfgs["b23"] = rec
        del b23
        torch.cuda.empty_cache()
        out["configs"] = cfgs
        del flush
        r = None
    if not args.no_cpu_baseline:
        inp = syn.make_inputs(w, device=dev)
        out["cpu_baseline"] = cpu_baseline(w, inp)
        del inp
        if not args.no_extra:
            out["cpu_baseline"]["configs"] = cpu_configs(dev)
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
