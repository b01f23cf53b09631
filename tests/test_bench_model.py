"""The benchmark's op-level roofline model at the pages' shape: per-token bytes built from the
saved-set table's figures and the tensor sizes, and the chunked method's MFMA work per token."""
import json
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_step_roofline_bytes_and_flops():
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "saved_set_bytes.json")))
    HV, d, C, H = gold["HV"], gold["d"], gold["chunk"], 16
    T = 262144
    io = 2
    inputs = 2 * H * d * io + HV * d * io + 2 * HV * 4          # q, k, v, g, beta
    light, full_extra = gold["light_bytes_per_token"], gold["full_extra_bytes_per_token"]
    fwd = inputs + HV * d * io + light                          # + o, saved set written
    bwd = inputs + HV * d * io + light + 2 * H * d * io + HV * d * io + 2 * HV * 4  # dO, saved read; dq, dk, dv, dg, dbeta
    rec = H * d * io + 2 * HV * 4 + light                       # k, g, beta read; saved written
    tape_extra = HV * d * d * 2 // C                            # the kept-tape form's state per chunk
    # the full and kept-tape recomputes walk the states (v read); the full one also forms the q.k rows (q read)
    for mode, extra, rec_extra in (("light", 0, 0), ("full", full_extra, HV * d * io + H * d * io),
                                   ("tape", tape_extra, HV * d * io)):
        m = bench.step_roofline(T, HV, d, io, H=H, save_mode=mode)
        assert abs(m["fwd"]["bytes_per_token"] - (fwd + extra)) < 1e-6
        assert abs(m["fwdbwd"]["bytes_per_token"] - (fwd + bwd + 2 * extra)) < 1e-6
        assert abs(m["ckpt"]["bytes_per_token"] - (fwd + rec + rec_extra + bwd + 3 * extra)) < 1e-6
    m = bench.step_roofline(T, HV, d, io, H=H)
    assert round(m["fwd"]["bytes_per_token"]) == 39491
    assert round(m["fwdbwd"]["bytes_per_token"]) == 99846
    # MFMA work per v head and token: fwd 6d^2 + 6Cd + 4Cd/G + 2C^2/3, bwd 16d^2 + (12 + 2/G) 2Cd + 4C^2/3
    G = HV // H
    f_fwd = 6 * d * d + 6 * C * d + 4 * C * d / G + 2 * C * C / 3
    f_bwd = 16 * d * d + (12 + 2 / G) * 2 * C * d + 4 * C * C / 3
    assert abs(m["fwd"]["flops_per_token"] - HV * f_fwd) < 1e-3
    assert abs(m["fwdbwd"]["flops_per_token"] - HV * (f_fwd + f_bwd)) < 1e-3
    assert round(f_fwd) == 161109 and round(f_bwd) == 475136
    # fwd + bwd at the packed workload: HBM and MFMA terms within a few percent, 3.27 ms
    assert abs(m["fwdbwd"]["roofline_s"] - 3.2718e-3) < 2e-6


def test_kernel_models_count_no_intermediates_as_algorithmic():
    """Per-kernel algorithmic bytes of the default step (light, deterministic) add up to the op's
    compulsory tensors as each kernel reads or writes them, and contain no tape or q.k-tile bytes:
    those are reported as intermediates."""
    T, NT, N, H, HV, d, io = 262144, 4096, 4, 16, 48, 128, 2
    m = bench.kernel_models(T, NT, N, H, HV, d, io)
    tape = NT * HV * d * d * 2
    pv = NT * HV * 64 * 64 * 2
    qk, vv, akk, gb = T * H * d * io, T * HV * d * io, T * HV * 64 * 2, T * HV * 4
    # the chunk-gradient kernel: reads q, k, v, dO, A, gcum, beta; writes dq, dk, dv, dg, dbeta
    assert m["gdn_chunk_grad"][0] == 2 * qk + 2 * vv + akk + 2 * gb + 2 * qk + vv + 2 * gb
    assert m["gdn_chunk_grad"][2] >= 2 * tape + pv
    # the paired walks: q, k, v, dO, A, gcum, beta (k, v, A, gcum, beta once per walk kind)
    assert m["gdn_walk_pair"][0] == (qk + vv + akk + 2 * gb) + (2 * qk + vv + akk + 2 * gb)
    assert m["gdn_walk_pair"][2] >= 2 * tape + pv
    # the forward walk: q, k, v, A, gcum, beta read and o written; the q.k tiles and norms are not algorithmic
    assert m["gdn_walk_fwd"][0] == 2 * qk + vv + akk + 2 * gb + vv
    # in the kept-tape form the chunk-gradient kernel's read of the state tape is a saved-set read
    mt = bench.kernel_models(T, NT, N, H, HV, d, io, save_mode="tape")
    assert mt["gdn_chunk_grad"][0] == m["gdn_chunk_grad"][0] + tape


def test_roofline_is_bytes_per_step_over_span():
    """The dominant kernel is the one with the longest span per step; its achieved rate is its
    algorithmic bytes per step over that span, whether it ran as one launch or as two overlapping
    launches of different sizes (whose mean duration would misstate the time it holds the step)."""
    models = {"gdn_chunk_grad": (15.77e9, 4.05e12, 14.5e9), "gdn_walk_pair": (13.09e9, 2.68e12, 14.5e9)}
    two = {"gdn_chunk_grad": {"launches_per_step": 2.0, "sum_ms_per_step": 14.7, "span_ms_per_step": 10.5,
                              "avg_launch_ms": 7.35},
           "gdn_walk_pair": {"launches_per_step": 2.0, "sum_ms_per_step": 13.9, "span_ms_per_step": 7.4,
                             "avg_launch_ms": 6.95}}
    r = bench.roofline_of(two, models, "no-such-workload", False)
    assert r["kernel"] == "gdn_chunk_grad" and r["bound"] == "hbm" and r["per"] == "step"
    assert abs(r["achieved"] - 15.77e9 / 10.5e-3 / 1e9) < 1e-6
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-12
    assert r["traffic"] is None and r["traffic_ratio"] is None
    one = {"gdn_chunk_grad": {"launches_per_step": 1.0, "sum_ms_per_step": 10.5, "span_ms_per_step": 10.5,
                              "avg_launch_ms": 10.5}}
    assert abs(bench.roofline_of(one, models, "no-such-workload", False)["achieved"] - r["achieved"]) < 1e-9


def test_cpu_config_rates_on_the_tiny_workload(monkeypatch):
    """The per-workload oracle rates: every op's rate is the workload's tokens over the scaled sample
    time, so ckpt (2 fwd + bwd) < fwd+bwd < fwd, and the sample covers the heads asked for."""
    monkeypatch.setattr(bench, "CPU_CONFIG_HEADS", {"tiny": 1})
    out = bench.cpu_configs("cpu")
    r = out["tiny"]
    assert set(r) >= {"fwd_tokens_per_s", "fwdbwd_tokens_per_s", "ckpt_tokens_per_s", "cores", "sample"}
    assert 0 < r["ckpt_tokens_per_s"] < r["fwdbwd_tokens_per_s"] < r["fwd_tokens_per_s"]
    assert "q/k heads 0..0 of 2 (1 value heads)" in r["sample"] and "scaled by 2/1 heads" in r["sample"]
