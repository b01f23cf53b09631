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
    for full, extra in ((False, 0), (True, full_extra)):
        m = bench.step_roofline(T, HV, d, io, full=full)
        assert abs(m["fwd"]["bytes_per_token"] - (fwd + extra)) < 1e-6
        assert abs(m["fwdbwd"]["bytes_per_token"] - (fwd + bwd + 2 * extra)) < 1e-6
        assert abs(m["ckpt"]["bytes_per_token"] - (fwd + rec + bwd + 3 * extra)) < 1e-6
    m = bench.step_roofline(T, HV, d, io)
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
