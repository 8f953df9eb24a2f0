"""Benchmark of the MoE expert-dispatch hot path on one MI355X.

One step = the whole path over one batch of synthetic input already resident
in HBM:
  layout (local experts) -> quant + dispatch -> grouped GEMM1
  -> layout (all experts, the combine's row map) -> combine.
Every kernel is timed with HIP events recorded on the stream it is launched
on (torch's current stream, which the binding passes to the library).

Prints ONE JSON line.  `value` is stage1 = layout + quant + GEMM1 in
microseconds (lower is better): the median of `steps` replays of stage1
captured in one HIP graph, each replay preceded by a 1 GiB read (ordinary
loads) that evicts the 256 MB last-level cache without leaving dirty lines
behind, and interleaved with an eager stage1 step (the chip's clock drifts over
a run, so only interleaved numbers compare).  The
median eager stage1 of the first timed loop is reported beside it.  The line
also carries the dispatch / combine HBM GB/s, the GEMM1 fp8 TFLOP/s, a
roofline entry per kernel (rates over the kernels' average launch durations in
the first timed loop), the measured HBM read-stream and MFMA-loop ceilings,
and the CPU oracle timed in full on the same workload.  After the timed
steps, the MX-style variant of stage1 (e8m0 scales per 32 K elements: layout
-> moe_quant_dispatch_mx -> moe_grouped_gemm1_mx) is timed on the same inputs
in a separate A/B loop that alternates one fp32-scale stage1 step with one MX
step (the clock drifts over a run, so only interleaved numbers compare), and
reported under "mx".  Stage2 on GEMM1's output (silu(gate) * up with its fp8
quant -> grouped GEMM2 with the routing weights -> combine of the local rows)
is timed after that and reported under "stage2", with its MX variant timed
against it in an A/B loop of the same kind under "stage2.mx".

Each timed loop starts with `warmup` untimed steps (20 by default): after the
chip has idled, the first back-to-back calls of the GEMMs run through a clock
transient (fast for two or three calls, then up to ≈30 % slower for a few,
settling after ≈15), which the timed steps should not sample.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline] [--copy-calib]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "stage1 µs (layout+quant+GEMM1), dispatch/combine HBM GB/s, GEMM1 fp8 TFLOP/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_step_ep8_2048x8_h7168.md")


def measured_traffic(workload: str) -> dict:
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE counter summary, per
    bench entry, for entries whose kernel source still hashes to what was profiled."""
    import re
    if workload != "ep8_2048x8_h7168" or not os.path.exists(TRAFFIC_PROFILE):
        return {}
    m = re.search(r"```json\n(.*?)\n```", open(TRAFFIC_PROFILE).read(), re.S)
    if not m:
        return {}
    out = {}
    for name, e in json.loads(m.group(1))["entries"].items():
        if source_sha256(e["source"]) == e["source_sha256"]:
            out[name] = int(e["bytes"])
    return out


def source_sha256(source: str) -> str:
    """SHA-256 over every header of the kernel sources (sorted by name), then the
    kernel's own file: a change to any code the kernel is built from changes it."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "combine_expert_histogram_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(csrc, "*.h"))) + [os.path.join(csrc, os.path.basename(source))]:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="ep8_2048x8_h7168")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calib", action="store_true",
                   help="also run a plain 1 GiB device copy (counter calibration)")
    return p.parse_args()


def gemm_entry(flop, byts, us, traffic_v):
    """Roofline entry of one GEMM launch, against whichever peak sets the longer
    floor for its algorithmic work: the fp8 MFMA peak for its FLOP or the HBM
    peak for its bytes (arithmetic intensity above or below 625 FLOP/B).  At
    2048 tokens per source GEMM1 is MFMA-bound (≈830 FLOP/B); at 256 tokens per
    source its weights dominate and it is HBM-bound (≈120 FLOP/B)."""
    if flop / (FP8_PEAK_TFLOPS * 1e12) >= byts / (HBM_PEAK_GBS * 1e9):
        a = flop / (us * 1e-6) / 1e12
        e = {"bound": "mfma", "achieved": round(a, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(a / FP8_PEAK_TFLOPS, 4)}
    else:
        a = byts / (us * 1e-6) / 1e9
        e = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(a / HBM_PEAK_GBS, 4)}
    e.update({"traffic": traffic_v, "algorithmic_flop": int(flop), "algorithmic_bytes": int(byts)})
    return e


def algorithmic(w, R, U, Rc):
    """Bytes (or flops) each kernel must move at minimum, per launch."""
    T, k, H, N, L, E = w.T, w.k, w.H, w.N, w.L, w.E
    width = w.combine_width
    lay_local = T * k * 4 + (R * 8 + T * k * 4 + T * 4 + U * 4)
    lay_full = T * k * 4 + (Rc * 8 + T * k * 4 + T * 4 + T * 4)
    quant = U * 4 + U * H * 2 + U * H + U * (H // 128) * 4
    gemm_flop = 2 * R * H * N
    gemm_bytes = U * (H + H // 32) + L * N * H + L * N * H // (128 * 128) * 4 + R * N * 2
    # MX: the same payloads; one packed dword of e8m0 codes per 128 K elements on
    # both operands (activations: as the fp32 scale; weights: per column)
    gemm_mx_bytes = U * (H + H // 32) + L * N * H + L * N * (H // 128) * 4 + R * N * 2
    combine = Rc * width * 2 + T * k * 8 + T * width * 2
    # stage2: I = N/2; act reads [R, 2I] bf16, writes [R, I] fp8 + scales; GEMM2 reads
    # h + its scales, W2 [L, H, I] + block scales and the row weights, writes [R, H]
    I = N // 2
    act = 8 + R * (2 * I * 2 + I + (I // 128) * 4)
    gemm2_flop = 2 * R * I * H
    gemm2_bytes = R * (I + I // 32) + L * H * I + L * (H // 128) * (I // 128) * 4 + R * 8 + R * H * 2
    combine_local = R * H * 2 + T * k * 8 + T * H * 2
    return dict(layout_local=lay_local, quant=quant, gemm1_flop=gemm_flop, gemm1_bytes=gemm_bytes,
                layout_full=lay_full, combine=combine, quant_mx=quant, gemm1_mx_bytes=gemm_mx_bytes,
                silu_mul_quant=act, gemm2_flop=gemm2_flop, gemm2_bytes=gemm2_bytes, combine_local=combine_local,
                silu_mul_quant_mx=act,
                gemm2_mx_bytes=R * (I + I // 32) + L * H * I + L * (I // 128) * H * 4 + R * 8 + R * H * 2)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only: --gpus must be 1"}))
        sys.exit(2)

    import torch
    import workloads
    import combine_expert_histogram_amd as moe

    w = workloads.get(args.workload)
    d_loc = moe.Dims(S=w.S, Ts=w.Ts, k=w.k, E=w.E, e0=w.e0, L=w.L, H=w.H)
    d_all = moe.Dims(S=w.S, Ts=w.Ts, k=w.k, E=w.E, e0=0, L=w.E, H=w.H)
    width = w.combine_width
    log(f"[bench] workload {w.name}: T={w.T} H={w.H} E={w.E} L={w.L} k={w.k} N={w.N}")

    t0 = time.time()
    ids, wts = workloads.routing(w)
    x = workloads.activations(w)
    wq, ws = workloads.weights(w)
    Y = workloads.expert_outputs(w)
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s")

    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ids_d = dev(ids.reshape(-1))
    wts_d = dev(wts.reshape(-1))
    x_d = dev(x.view(np.int16))
    wq_d = dev(wq)
    ws_d = dev(ws)
    Y_d = dev(Y.view(np.int16)).view(torch.bfloat16)
    del x, wq, Y
    lay = moe.alloc_layout(d_loc)
    lay_all = moe.alloc_layout(d_all)
    q = torch.empty((w.T, w.H), dtype=torch.uint8, device="cuda")
    qs = torch.empty((w.T, w.H // 128), dtype=torch.float32, device="cuda")
    y1 = torch.empty((w.T * w.k, w.N), dtype=torch.bfloat16, device="cuda")
    g_ws = moe.alloc_gemm1_workspace(d_loc, w.N)
    out = torch.empty((w.T, width), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    names = ["layout_local", "quant", "gemm1", "layout_full", "combine"]

    def step(ev=None):
        if ev: ev[0].record(stream)
        moe.route_layout(d_loc, ids_d, lay)
        if ev: ev[1].record(stream)
        moe.quant_dispatch(d_loc, x_d, lay, q, qs)
        if ev: ev[2].record(stream)
        moe.grouped_gemm1(d_loc, w.N, q, qs, lay, wq_d, ws_d, y1, g_ws)
        if ev: ev[3].record(stream)
        moe.route_layout(d_all, ids_d, lay_all)
        if ev: ev[4].record(stream)
        moe.combine(d_all, width, Y_d, lay_all["assign_row"], wts_d, out)
        if ev: ev[5].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    R, U = (int(v) for v in lay["totals"].cpu())
    Rc = int(lay_all["totals"][0].cpu())
    log(f"[bench] R={R} U={U} Rc={Rc}; timing {args.steps} steps")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    per = {n: [] for n in names}
    for e in evs:
        for j, n in enumerate(names):
            per[n].append(e[j].elapsed_time(e[j + 1]) * 1e3)        # us
    med = {n: float(np.median(v)) for n, v in per.items()}
    mean = {n: float(np.mean(v)) for n, v in per.items()}
    log("[bench] per-kernel median us: " + ", ".join(f"{n}={med[n]:.1f}" for n in names))

    alg = algorithmic(w, R, U, Rc)
    stage1 = float(np.median([sum(per[n][i] for n in ("layout_local", "quant", "gemm1"))
                              for i in range(args.steps)]))
    hbm_names = ("layout_local", "quant", "layout_full", "combine")
    hbm_bytes = sum(alg[n] for n in hbm_names)
    # rates (roofline `achieved`, the GB/s and TFLOP/s figures) divide the
    # algorithmic work by the kernel's average launch duration over the timed steps
    hbm_time = sum(mean[n] for n in hbm_names)
    hbm_gbs = hbm_bytes / (hbm_time * 1e-6) / 1e9
    gemm_tflops = alg["gemm1_flop"] / (mean["gemm1"] * 1e-6) / 1e12

    def hbm_entry(n):
        a = alg[n] / (mean[n] * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4), "traffic": traffic.get(n), "us": round(mean[n], 2),
                "us_median": round(med[n], 2), "algorithmic_bytes": int(alg[n])}

    traffic = measured_traffic(args.workload)
    kernels = {n: hbm_entry(n) for n in hbm_names}
    kernels["gemm1"] = gemm_entry(alg["gemm1_flop"], alg["gemm1_bytes"], mean["gemm1"], traffic.get("gemm1"))
    kernels["gemm1"]["us"] = round(mean["gemm1"], 2)
    kernels["gemm1"]["us_median"] = round(med["gemm1"], 2)
    dominant = max(names, key=lambda n: mean[n])
    roof = {k: v for k, v in kernels[dominant].items() if k in ("bound", "achieved", "peak", "unit", "frac",
                                                                "traffic")}
    roof["kernel"] = dominant

    pct = lambda v, p: float(np.percentile(v, p))
    stage1_all = [sum(per[n][i] for n in ("layout_local", "quant", "gemm1")) for i in range(args.steps)]
    spread = {n: {"p10": round(pct(per[n], 10), 2), "p90": round(pct(per[n], 90), 2)} for n in names}
    spread["stage1"] = {"p10": round(pct(stage1_all, 10), 2), "p90": round(pct(stage1_all, 90), 2)}

    # stage1 (layout -> quant -> GEMM1) captured once in a graph and replayed beside
    # eager steps; the calls read their counts on the device, so the capture needs
    # no host sync
    graph = stage1_graph(torch, moe, d_loc, ids_d, x_d, wq_d, ws_d, lay, q, qs, y1, g_ws, w, R, U, args.steps)
    mx = mx_stage1(torch, moe, w, d_loc, ids_d, x_d, lay, g_ws, alg, traffic, args,
                   fp32_step=lambda: (moe.quant_dispatch(d_loc, x_d, lay, q, qs),
                                      moe.grouped_gemm1(d_loc, w.N, q, qs, lay, wq_d, ws_d, y1, g_ws)))
    s2 = stage2(torch, moe, w, d_loc, lay, y1, wts_d, alg, traffic, args)
    ceil = ceilings(torch, moe, args.copy_calib, (U * w.H, w.T * width * 2, R * (w.N // 2)))

    vendor = vendor_gemm(torch, w, R)
    rec = {
        "metric": METRIC, "value": graph["us_median"], "unit": "µs", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": w.name, "sources": w.S, "tokens_per_source": w.Ts, "hidden": w.H,
                   "experts": w.E, "local_experts": w.L, "top_k": w.k, "gemm1_n": w.N,
                   "combine_width": width, "rows": R, "slots": U, "combine_rows": Rc},
        "stage1_eager_us_median": round(stage1, 2),
        "dispatch_combine_hbm_gbs": round(hbm_gbs, 1),
        "gemm1_fp8_tflops": round(gemm_tflops, 1),
        "kernels_us_median": {n: round(med[n], 2) for n in names},
        "kernels_us_mean": {n: round(mean[n], 2) for n in names},
        "kernels": kernels,
        "roofline": roof,
        "percentiles_us": spread,
        "stage1_graph": graph,
        "mx": mx,
        "stage2": s2,
        "ceilings": ceil,
        "vendor_fp8_gemm": vendor,
        "fraction_of_measured_ceilings": {
            "gemm1_vs_mfma_loop": round(gemm_tflops / ceil["mfma_fp8_tflops"], 4),
            "gemm1_mx_vs_mfma_scaled_loop": round(mx["kernels"]["gemm1_mx"]["achieved"] / ceil["mfma_fp8_scaled_tflops"],
                                                  4),
            "dispatch_combine_vs_read_stream": round(hbm_gbs / ceil["read_stream_gbs"], 4),
            "combine_vs_read_stream": round(kernels["combine"]["achieved"] / ceil["read_stream_gbs"], 4),
            "quant_vs_rw21_stream": round(kernels["quant"]["achieved"] / ceil["rw21_stream_gbs"], 4),
            "combine_vs_rw81_stream": round(kernels["combine"]["achieved"] / ceil["rw81_stream_gbs"], 4),
            "act_vs_rw41_stream": round(s2["kernels"]["silu_mul_quant"]["achieved"] / ceil["rw41_stream_gbs"], 4),
            "gemm1_vs_vendor_dense": round(gemm_tflops / vendor["dense_tflops"], 4) if "dense_tflops" in vendor else None,
            "gemm1_vs_vendor_per_expert": (round(gemm_tflops / vendor["per_expert_tflops"], 4)
                                           if "per_expert_tflops" in vendor else None)},
    }

    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, ids, lay, q, qs, y1, R, U, graph["us_median"])

    print(json.dumps(rec), flush=True)


def mx_stage1(torch, moe, w, d, ids_d, x_d, lay, g_ws, alg, traffic, args, fp32_step):
    """The MX-style stage1 (layout -> quant_mx -> GEMM1 MX) on the same inputs:
    `warmup` untimed, then `steps` A/B pairs, each an fp32-scale stage1 step
    followed by an MX step, HIP events between the calls."""
    import workloads
    t0 = time.time()
    wq, ws = workloads.weights_mx(w)
    log(f"[bench] MX weights generated in {time.time() - t0:.1f}s")
    wq_d = torch.from_numpy(wq).cuda()
    ws_d = torch.from_numpy(ws.view(np.int32)).cuda()
    del wq, ws
    q = torch.empty((w.T, w.H), dtype=torch.uint8, device="cuda")
    qs = torch.empty((w.T, w.H // 128), dtype=torch.int32, device="cuda")
    y = torch.empty((w.T * w.k, w.N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    names = ["layout_local", "quant_mx", "gemm1_mx"]

    def step(ev=None):
        if ev: ev[0].record(stream)
        moe.route_layout(d, ids_d, lay)
        if ev: ev[1].record(stream)
        moe.quant_dispatch_mx(d, x_d, lay, q, qs)
        if ev: ev[2].record(stream)
        moe.grouped_gemm1_mx(d, w.N, q, qs, lay, wq_d, ws_d, y, g_ws)
        if ev: ev[3].record(stream)

    def step_fp32(ev):
        ev[0].record(stream)
        moe.route_layout(d, ids_d, lay)
        fp32_step()
        ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    evf = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step_fp32(evf[i])
        step(evs[i])
    torch.cuda.synchronize()
    per = {n: [e[j].elapsed_time(e[j + 1]) * 1e3 for e in evs] for j, n in enumerate(names)}
    med = {n: float(np.median(v)) for n, v in per.items()}
    mean = {n: float(np.mean(v)) for n, v in per.items()}
    stage1 = [sum(per[n][i] for n in names) for i in range(args.steps)]
    stage1_fp32 = [e[0].elapsed_time(e[1]) * 1e3 for e in evf]
    qa = alg["quant_mx"] / (mean["quant_mx"] * 1e-6) / 1e9
    del wq_d, ws_d, q, qs, y
    return {"stage1_us": round(float(np.median(stage1)), 2),
            "stage1_p10_p90_us": [round(float(np.percentile(stage1, 10)), 2),
                                  round(float(np.percentile(stage1, 90)), 2)],
            "fp32_scale_stage1_us_same_loop": round(float(np.median(stage1_fp32)), 2),
            "mx_over_fp32_stage1": round(float(np.median(stage1)) / float(np.median(stage1_fp32)), 4),
            "kernels_us_median": {n: round(med[n], 2) for n in names},
            "kernels_us_mean": {n: round(mean[n], 2) for n in names},
            "kernels": {
                "quant_mx": {"bound": "hbm", "achieved": round(qa, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(qa / HBM_PEAK_GBS, 4), "traffic": traffic.get("quant_mx"),
                             "algorithmic_bytes": int(alg["quant_mx"])},
                "gemm1_mx": gemm_entry(alg["gemm1_flop"], alg["gemm1_mx_bytes"], mean["gemm1_mx"],
                                       traffic.get("gemm1_mx"))}}


def stage2(torch, moe, w, d, lay, y1, wts_d, alg, traffic, args):
    """Stage2 on GEMM1's output y1: silu_mul_quant -> GEMM2 (routing weights
    applied) -> combine of the local rows with unit weights; `warmup` untimed
    then `steps` timed, HIP events between the calls."""
    import workloads
    t0 = time.time()
    w2, w2s = workloads.weights2(w)
    log(f"[bench] GEMM2 weights generated in {time.time() - t0:.1f}s")
    w2_d, w2s_d = torch.from_numpy(w2).cuda(), torch.from_numpy(w2s).cuda()
    del w2, w2s
    I = w.N // 2
    rows_cap = w.T * w.k
    h = torch.empty((rows_cap, I), dtype=torch.uint8, device="cuda")
    hs = torch.empty((rows_cap, I // 128), dtype=torch.float32, device="cuda")
    y2 = torch.empty((rows_cap, w.H), dtype=torch.bfloat16, device="cuda")
    g2_ws = moe.alloc_gemm2_workspace(d, I)
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    ones = torch.ones(rows_cap, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    names = ["silu_mul_quant", "gemm2", "combine_local"]

    def step(ev=None):
        if ev: ev[0].record(stream)
        moe.silu_mul_quant(d, I, y1, lay, h, hs)
        if ev: ev[1].record(stream)
        moe.grouped_gemm2(d, I, h, hs, lay, wts_d, w2_d, w2s_d, y2, g2_ws)
        if ev: ev[2].record(stream)
        moe.combine(d, w.H, y2, lay["assign_row"], ones, out)
        if ev: ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    per = {n: [e[j].elapsed_time(e[j + 1]) * 1e3 for e in evs] for j, n in enumerate(names)}
    med = {n: float(np.median(v)) for n, v in per.items()}
    mean = {n: float(np.mean(v)) for n, v in per.items()}
    tot = [sum(per[n][i] for n in names) for i in range(args.steps)]

    def hbm(n, key):
        a = alg[key] / (mean[n] * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4), "traffic": traffic.get(n), "algorithmic_bytes": int(alg[key])}


    # MX variant, A/B against the fp32-scale stage2 on the same GEMM1 output
    t0 = time.time()
    m2, m2s = workloads.weights2_mx(w)
    log(f"[bench] MX GEMM2 weights generated in {time.time() - t0:.1f}s")
    m2_d, m2s_d = torch.from_numpy(m2).cuda(), torch.from_numpy(m2s.view(np.int32)).cuda()
    del m2, m2s
    hm = torch.empty((rows_cap, I), dtype=torch.uint8, device="cuda")
    hms = torch.empty((rows_cap, I // 128), dtype=torch.int32, device="cuda")
    mx_names = ["silu_mul_quant_mx", "gemm2_mx", "combine_local"]

    def step_mx(ev=None):
        if ev: ev[0].record(stream)
        moe.silu_mul_quant_mx(d, I, y1, lay, hm, hms)
        if ev: ev[1].record(stream)
        moe.grouped_gemm2_mx(d, I, hm, hms, lay, wts_d, m2_d, m2s_d, y2, g2_ws)
        if ev: ev[2].record(stream)
        moe.combine(d, w.H, y2, lay["assign_row"], ones, out)
        if ev: ev[3].record(stream)

    for _ in range(args.warmup):
        step_mx()
    evm = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    evf = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evf[i])
        step_mx(evm[i])
    torch.cuda.synchronize()
    perm = {n: [e[j].elapsed_time(e[j + 1]) * 1e3 for e in evm] for j, n in enumerate(mx_names)}
    medm = {n: float(np.median(v)) for n, v in perm.items()}
    meanm = {n: float(np.mean(v)) for n, v in perm.items()}
    totm = [sum(perm[n][i] for n in mx_names) for i in range(args.steps)]
    totf = [e[0].elapsed_time(e[3]) * 1e3 for e in evf]
    qam = alg["silu_mul_quant_mx"] / (meanm["silu_mul_quant_mx"] * 1e-6) / 1e9
    del w2_d, w2s_d, m2_d, m2s_d, h, hs, hm, hms, y2, out
    mx = {"us_median": round(float(np.median(totm)), 2),
          "fp32_scale_us_same_loop": round(float(np.median(totf)), 2),
          "mx_over_fp32": round(float(np.median(totm)) / float(np.median(totf)), 4),
          "kernels_us_median": {n: round(medm[n], 2) for n in mx_names},
          "kernels_us_mean": {n: round(meanm[n], 2) for n in mx_names},
          "kernels": {"silu_mul_quant_mx": {"bound": "hbm", "achieved": round(qam, 1), "peak": HBM_PEAK_GBS,
                                            "unit": "GB/s", "frac": round(qam / HBM_PEAK_GBS, 4),
                                            "traffic": traffic.get("silu_mul_quant_mx"),
                                            "algorithmic_bytes": int(alg["silu_mul_quant_mx"])},
                      "gemm2_mx": gemm_entry(alg["gemm2_flop"], alg["gemm2_mx_bytes"], meanm["gemm2_mx"],
                                             traffic.get("gemm2_mx"))}}
    return {"us_median": round(float(np.median(tot)), 2),
            "us_p10_p90": [round(float(np.percentile(tot, 10)), 2), round(float(np.percentile(tot, 90)), 2)],
            "inter": I, "kernels_us_median": {n: round(med[n], 2) for n in names},
            "kernels_us_mean": {n: round(mean[n], 2) for n in names},
            "kernels": {"silu_mul_quant": hbm("silu_mul_quant", "silu_mul_quant"),
                        "gemm2": gemm_entry(alg["gemm2_flop"], alg["gemm2_bytes"], mean["gemm2"],
                                            traffic.get("gemm2")),
                        "combine_local": hbm("combine_local", "combine_local")},
            "mx": mx}


def ceiling_lib():
    """libmoe_ceiling.so: the read-stream and MFMA-loop measurement kernels."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "combine_expert_histogram_amd", "libmoe_ceiling.so"))
    lib.moe_ceiling_read_stream.restype = ctypes.c_int
    lib.moe_ceiling_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_void_p]
    for f in (lib.moe_ceiling_mfma_fp8, lib.moe_ceiling_mfma_fp8_scaled):
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.moe_ceiling_rw_stream.restype = ctypes.c_int
    lib.moe_ceiling_rw_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_void_p]
    return lib


class ReadFlush:
    """Evicts the caches by reading a 1 GiB buffer with ordinary loads: the
    256 MB last-level cache then holds only clean lines of this buffer.  (A
    write flush would make the next kernel pay for writing its dirty lines
    back: measured +33 us on the quant and +41 us on stage1.)"""

    def __init__(self, torch, nbytes=1 << 30):
        import ctypes
        self.torch, self.ctypes, self.nbytes = torch, ctypes, nbytes
        self.lib = ceiling_lib()
        self.buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        self.grid = torch.cuda.get_device_properties(0).multi_processor_count * 2
        self.out = torch.empty(self.grid * 256, dtype=torch.int32, device="cuda")

    def __call__(self, stream):
        c = self.ctypes
        if self.lib.moe_ceiling_read_stream(c.c_void_p(self.buf.data_ptr()), self.nbytes, self.grid, 1,
                                            c.c_void_p(self.out.data_ptr()), c.c_void_p(stream.cuda_stream)):
            raise RuntimeError("flush launch failed")


def stage1_graph(torch, moe, d, ids_d, x_d, wq_d, ws_d, lay, q, qs, y1, g_ws, w, R, U, steps):
    """Captures layout -> quant -> GEMM1 into one graph (all buffers preallocated),
    checks the graph's outputs against the eager step's, then times `steps`
    pairs of one eager stage1 step and one replay, alternating on the same
    stream (the clock drifts over a run, so only interleaved numbers compare).
    Before each timed step a 1 GiB buffer is read with ordinary loads, which
    evicts the 256 MB last-level cache (the step's own inputs are then read
    from HBM) and leaves no dirty lines; the read is outside the events.  A second loop of back-to-back replays without the
    write gives the warm figure."""
    ref_lay = {k: v.clone() for k, v in lay.items() if k != "ws"}
    ref_q, ref_qs, ref_y = q[:U].clone(), qs[:U].clone(), y1[:R].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()

    def eager():
        moe.route_layout(d, ids_d, lay)
        moe.quant_dispatch(d, x_d, lay, q, qs)
        moe.grouped_gemm1(d, w.N, q, qs, lay, wq_d, ws_d, y1, g_ws)

    with torch.cuda.stream(s):
        eager()                                              # warm the stream before capture
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            eager()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    same = (all(torch.equal(lay[k], v) for k, v in ref_lay.items()) and torch.equal(q[:U], ref_q)
            and torch.equal(qs[:U], ref_qs) and torch.equal(y1[:R], ref_y))
    flush = ReadFlush(torch)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    with torch.cuda.stream(s):
        for i in range(steps):
            flush(s)
            ev[i][0].record(s)
            eager()
            ev[i][1].record(s)
            flush(s)
            ev[i][2].record(s)
            g.replay()
            ev[i][3].record(s)
    torch.cuda.synchronize()
    t_e = [e[0].elapsed_time(e[1]) * 1e3 for e in ev]
    t_g = [e[2].elapsed_time(e[3]) * 1e3 for e in ev]
    warm = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    with torch.cuda.stream(s):
        warm[0].record(s)
        for i in range(steps):
            g.replay()
            warm[i + 1].record(s)
    torch.cuda.synchronize()
    t_w = [warm[i].elapsed_time(warm[i + 1]) * 1e3 for i in range(steps)]
    del flush
    med = lambda v: round(float(np.median(v)), 2)
    return {"us_median": med(t_g), "us_p10": round(float(np.percentile(t_g, 10)), 2),
            "us_p90": round(float(np.percentile(t_g, 90)), 2), "eager_us_median_same_loop": med(t_e),
            "graph_over_eager": round(float(np.median(t_g)) / float(np.median(t_e)), 4),
            "warm_us_median": med(t_w), "replays": steps, "flush_bytes_read_before_each": 1 << 30,
            "matches_eager": bool(same)}


def vendor_gemm(torch, w, R):
    """Context, not part of the path: the vendor library's fp8 GEMM (hipBLASLt
    through torch._scaled_mm, per-tensor scales, bf16 out) on GEMM1's shapes, in
    the same run: one dense GEMM of all R rows against one [N, H] weight
    matrix, and one GEMM per local expert (R / L rows each) against its own
    weights.  Neither has the block scales, the row gather or the fold of the
    grouped GEMM1; the dense one also streams 1/L of its weight bytes."""
    f8 = torch.float8_e4m3fn
    one = torch.tensor(1.0, device="cuda")

    def rand(m, k):
        return (torch.randn(m, k, device="cuda") * 0.5).to(f8)

    def med(fn, iters):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(iters):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    flop = 2.0 * R * w.N * w.H
    out = {"flop": flop}
    try:
        a, b = rand(R, w.H), rand(w.N, w.H)
        us = med(lambda: torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16), 10)
        out["dense_us"] = round(us, 1)
        out["dense_tflops"] = round(flop / (us * 1e-6) / 1e12, 1)
        del a, b
        rows = [R // w.L + (1 if i < R % w.L else 0) for i in range(w.L)]
        a_s = [rand(r, w.H) for r in rows]
        b_s = [rand(w.N, w.H) for _ in range(w.L)]

        def per_expert():
            for a_, b_ in zip(a_s, b_s):
                torch._scaled_mm(a_, b_.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        us = med(per_expert, 5)
        out["per_expert_us"] = round(us, 1)
        out["per_expert_tflops"] = round(flop / (us * 1e-6) / 1e12, 1)
        del a_s, b_s
    except Exception as ex:                       # the library GEMM is optional context
        out["error"] = str(ex)[:200]
    return out


def ceilings(torch, moe, copy_calib, rw_out_bytes):
    """What this GPU sustains in the same run: one pass of non-temporal 16 B
    loads over 2 GiB, each workgroup reading one contiguous chunk (the HBM read
    rate; the hot path's HBM-bound kernels mostly read), streams reading two,
    eight and four bytes per byte written (the quant's, the combine's and
    stage2's act mixes) at those kernels' own sizes (`rw_out_bytes` = bytes each
    writes, in that order), timed cold after the same read flush as stage1, a
    1 GiB device-to-device copy (bytes read + written per second; its counter
    reading also calibrates the traffic summary) and loops of independent fp8
    MFMAs, plain and with e8m0 scales."""
    import ctypes
    lib = ceiling_lib()
    st = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rbytes = 2 << 30
    rbuf = torch.ones(rbytes, dtype=torch.uint8, device="cuda")
    rgrid = cus * 2
    rout = torch.empty(rgrid * 256, dtype=torch.int32, device="cuda")

    def read_pass():
        if lib.moe_ceiling_read_stream(ctypes.c_void_p(rbuf.data_ptr()), rbytes, rgrid, 0,
                                       ctypes.c_void_p(rout.data_ptr()), ctypes.c_void_p(st.cuda_stream)):
            raise RuntimeError("read-stream launch failed")
    read_pass()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for i in range(5):
        e[i].record(st)
        read_pass()
    e[5].record(st)
    torch.cuda.synchronize()
    read_us = float(np.median([e[i].elapsed_time(e[i + 1]) * 1e3 for i in range(5)]))
    del rbuf, rout
    flush = ReadFlush(torch)
    rw = {}
    for ratio, out_bytes in ((2, rw_out_bytes[0]), (4, rw_out_bytes[2]), (8, rw_out_bytes[1])):
        wbytes = (int(out_bytes) + 4095) // 4096 * 4096
        src = torch.ones(ratio * wbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty(wbytes, dtype=torch.uint8, device="cuda")
        times = []
        for i in range(7):
            flush(st)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            if lib.moe_ceiling_rw_stream(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), wbytes,
                                         ratio, ctypes.c_void_p(st.cuda_stream)):
                raise RuntimeError("read/write-stream launch failed")
            e1.record(st)
            e1.synchronize()
            if i >= 2:
                times.append(e0.elapsed_time(e1) * 1e3)
        us = float(np.median(times))
        rw[ratio] = (us, (ratio + 1) * wbytes)
        del src, dst
    del flush
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    reps = 3 if copy_calib else 5
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    for i in range(reps):
        e[i].record(); b.copy_(a)
    e[reps].record(); torch.cuda.synchronize()
    copy_us = float(np.median([e[i].elapsed_time(e[i + 1]) * 1e3 for i in range(reps)]))
    del a, b
    grid = cus
    out = torch.empty(grid * 512, dtype=torch.float32, device="cuda")
    iters = 4000
    if lib.moe_ceiling_mfma_fp8(grid, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(st.cuda_stream)):
        raise RuntimeError("MFMA ceiling launch failed")
    torch.cuda.synchronize()
    # the plain and the scaled (nonzero e8m0 operands, the MX GEMM1's form) loops alternate
    t_mfma = {False: [], True: []}
    for i in range(6):
        scaled = bool(i % 2)
        fn = lib.moe_ceiling_mfma_fp8_scaled if scaled else lib.moe_ceiling_mfma_fp8
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        if fn(grid, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(st.cuda_stream)):
            raise RuntimeError("MFMA ceiling launch failed")
        e1.record(st)
        torch.cuda.synchronize()
        t_mfma[scaled].append(e0.elapsed_time(e1) * 1e3)
    mfma_us = float(np.median(t_mfma[False]))
    mfma_scaled_us = float(np.median(t_mfma[True]))
    flop = grid * 8 * iters * 16 * 65536
    return {"read_stream_gbs": round(rbytes / (read_us * 1e-6) / 1e9, 1),
            "read_stream_frac_of_peak": round(rbytes / (read_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "rw21_stream_gbs": round(rw[2][1] / (rw[2][0] * 1e-6) / 1e9, 1),
            "rw21_stream_us": round(rw[2][0], 2),
            "rw21_stream_bytes": rw[2][1],
            "rw41_stream_gbs": round(rw[4][1] / (rw[4][0] * 1e-6) / 1e9, 1),
            "rw41_stream_us": round(rw[4][0], 2),
            "rw41_stream_bytes": rw[4][1],
            "rw81_stream_gbs": round(rw[8][1] / (rw[8][0] * 1e-6) / 1e9, 1),
            "rw81_stream_us": round(rw[8][0], 2),
            "rw81_stream_bytes": rw[8][1],
            "copy_gbs": round(2 * (1 << 30) / (copy_us * 1e-6) / 1e9, 1),
            "mfma_fp8_tflops": round(flop / (mfma_us * 1e-6) / 1e12, 1),
            "mfma_fp8_frac_of_peak": round(flop / (mfma_us * 1e-6) / 1e12 / FP8_PEAK_TFLOPS, 4),
            "mfma_fp8_scaled_tflops": round(flop / (mfma_scaled_us * 1e-6) / 1e12, 1)}


def cpu_baseline(w, ids, lay, q, qs, y1, R, U, gpu_stage1_us):
    """The oracle, as it stands, timed in full on this host on the same workload
    (layout of every assignment, quant of every landed slot, GEMM1 of every row
    of every local expert; each step once, with perf_counter), in microseconds
    of stage1.  Its outputs are then checked against the GPU's: layout and quant
    bit for bit, GEMM1 by rel-L2 over every row."""
    import torch
    import workloads
    from oracle import gemm1 as og, layout as ol, quant as oq

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    x = workloads.activations(w)
    wq, ws = workloads.weights(w)

    t = time.perf_counter()
    ref = ol.route_layout(ids, w.S, w.Ts, w.k, w.e0, w.L)
    t_layout = time.perf_counter() - t
    t = time.perf_counter()
    rq, rs = oq.quant_dispatch(x, ref["slot_tok"])
    t_quant = time.perf_counter() - t
    t = time.perf_counter()
    yref = og.grouped_gemm1(rq, rs, ref["row_slot"], ref["expert_offsets"], wq, ws)
    t_gemm = time.perf_counter() - t
    del wq

    ok_layout = all(np.array_equal(lay[k][: len(ref[k])].cpu().numpy(), ref[k])
                    for k in ("expert_counts", "expert_offsets", "row_slot", "row_assign", "slot_tok",
                              "tok_slot", "src_slot_offsets", "totals"))
    ok_quant = bool(np.array_equal(q[:U].cpu().numpy(), rq) and np.array_equal(qs[:U].cpu().numpy(), rs))
    g = y1[:R].float().cpu().numpy().astype(np.float64)
    r64 = yref.astype(np.float64)
    rel = float(np.linalg.norm(g - r64) / np.linalg.norm(r64))
    total_us = (t_layout + t_quant + t_gemm) * 1e6
    return {"value": round(total_us, 1), "unit": "µs", "cores": int(min(cores, blas_threads)),
            "host_cores": cores, "blas_threads": int(blas_threads), "kind": "oracle",
            "sample": f"full: layout of all {w.T * w.k} assignments, quant of all {U} slots, "
                      f"GEMM1 of all {R} rows x {w.N} columns (32-expert numpy fp32 matmul)",
            "steps_s": {"layout": round(t_layout, 3), "quant": round(t_quant, 3), "gemm1": round(t_gemm, 3)},
            "gpu_speedup": round(total_us / gpu_stage1_us, 1),
            "parity_full": {"layout_bit_exact": bool(ok_layout), "quant_bit_exact": ok_quant,
                            "gemm1_rel_l2": rel}}


if __name__ == "__main__":
    main()
