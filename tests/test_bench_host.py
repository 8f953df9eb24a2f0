"""Host-side pieces of bench.py (CPU): the algorithmic work per launch that the
roofline entries divide by, checked against the sizes the workload fixes, and
the reader of the committed HBM-traffic summary."""
import json
import os
import re

import numpy as np

import bench
import workloads
from oracle import layout as olayout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_work_of_the_bench_workload():
    w = workloads.get("ep8_2048x8_h7168")
    ids, _ = workloads.routing(w)
    ref = olayout.route_layout(ids, w.S, w.Ts, w.k, w.e0, w.L)
    R, U = (int(v) for v in ref["totals"])
    Rc = w.T * w.k
    a = bench.algorithmic(w, R, U, Rc)
    H, N = w.H, w.N
    # quant: the landed rows read once as bf16 (+ their slot ids), written once as fp8 + scales
    assert a["quant"] == U * 4 + U * H * 2 + U * H + U * (H // 128) * 4
    assert abs(a["quant"] / 1e6 - 235.8) < 0.5                       # ~10.85k landed rows
    # GEMM1: 2 R H N flop; ~16.4k rows
    assert a["gemm1_flop"] == 2 * R * H * N and abs(a["gemm1_flop"] / 1e9 - 960.5) < 1
    # combine over all T*k contributions at width H
    assert a["combine"] == Rc * H * 2 + w.T * w.k * 8 + w.T * H * 2 and abs(a["combine"] / 1e9 - 2.115) < 0.001
    # stage2 with I = N/2: act reads 2I bf16 and writes I fp8 + I/32 bytes of scales a row
    I = N // 2
    assert a["silu_mul_quant"] == 8 + R * (4 * I + I + (I // 128) * 4)
    assert a["gemm2_flop"] == 2 * R * I * H
    # expected counts: R ~ T*k*L/E, U = landed tokens
    assert abs(R - w.T * w.k * w.L / w.E) < 0.02 * R
    assert 0.6 < U / w.T < 0.72


def test_committed_traffic_summary_parses():
    path = os.path.join(ROOT, "profiles", "hbm_traffic_step_ep8_2048x8_h7168.md")
    text = open(path).read()
    block = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
    ent = block["entries"]
    for key in ("layout_local", "quant", "gemm1", "combine", "silu_mul_quant", "gemm2"):
        assert key in ent and ent[key]["bytes"] > 0 and len(ent[key]["source_sha256"]) == 64
    # bench.py fills an entry only while its source still hashes to what was profiled
    got = bench.measured_traffic("ep8_2048x8_h7168")
    assert set(got) <= set(ent)
    assert all(isinstance(v, int) and v > 0 for v in got.values())
    assert bench.measured_traffic("tiny_t64_h256_e8") == {}


def test_gemm_roofline_bound_follows_arithmetic_intensity():
    # 2048 tokens per source: ~830 FLOP/B, above the 625 FLOP/B ridge -> MFMA-bound
    e = bench.gemm_entry(960.5e9, 1.154e9, 500.0, None)
    assert e["bound"] == "mfma" and e["unit"] == "TFLOP/s"
    assert abs(e["achieved"] - 960.5e9 / 500e-6 / 1e12) < 0.1
    assert abs(e["frac"] - e["achieved"] / bench.FP8_PEAK_TFLOPS) < 1e-4
    # 256 tokens per source: the weights dominate (~120 FLOP/B) -> HBM-bound
    e = bench.gemm_entry(120e9, 0.967e9, 180.0, 123)
    assert e["bound"] == "hbm" and e["unit"] == "GB/s" and e["traffic"] == 123
    assert abs(e["achieved"] - 0.967e9 / 180e-6 / 1e9) < 0.1
    assert e["algorithmic_flop"] == int(120e9) and e["algorithmic_bytes"] == int(0.967e9)
