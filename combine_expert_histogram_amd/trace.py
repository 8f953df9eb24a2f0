"""Clock-stamp trace of the hot path's kernels (measurement aid).

Loads libmoe_hotpath_trace.so (the library's sources built with MOE_TRACE=1 by
`python -m combine_expert_histogram_amd.build`), runs warm-up steps of a
workload (layout of the local experts -> quant -> GEMM1 -> layout of all
experts -> combine, then stage2's act -> GEMM2), and then traces each call of
`--steps` more steps on its own: a device buffer is attached before the call
and read back after it.  Every kernel stamps its workgroups (the layouts, the
GEMM pre-pass, the combine), wavefronts (quant, act) or GEMM tiles with the
chip's constant 100 MHz clock (csrc/trace.h).  Printed per call, from the
first stamp of the call: how many units recorded, the spread of their starts,
their durations, and when the last one ended; for the grouped GEMMs also the
tiles' durations and, per XCD (workgroup b runs on XCD b % 8), when its
workgroups' compute wavefronts finished.

  python -m combine_expert_histogram_amd.trace [--workload NAME] [--steps K] [--json FILE]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

import numpy as np

from . import build as _build

TICK_US = 0.01                 # s_memrealtime: 100 MHz
KERNELS = {1: "layout_count", 2: "layout_place", 3: "quant", 4: "quant_mx", 5: "gemm_prep",
           6: "gemm_loader", 7: "gemm_compute", 8: "gemm_tile", 9: "combine", 10: "act"}
REC = np.dtype([("t0", "<u8"), ("t1", "<u8"), ("kernel", "<u4"), ("block", "<u4"), ("item", "<u4"),
                ("aux", "<u4")])
HDR_BYTES = 16
N_KERNEL_IDS = 16


class Tracer:
    """The traced library, loaded in place of the product one, with a device
    buffer of `region` records for each of the 16 kernel ids."""

    def __init__(self, torch, region: int = 1 << 17):
        from . import binding as B
        if not os.path.exists(_build.TRACE_LIB):
            raise RuntimeError(f"{_build.TRACE_LIB} is missing: build it with "
                               "`python -m combine_expert_histogram_amd.build`")
        self._B, self._saved = B, (B.LIB_PATH, B._lib)
        B.LIB_PATH = _build.TRACE_LIB
        B._lib = None
        self.lib = B.lib()
        self.lib.moe_trace_attach.restype = ctypes.c_int
        self.lib.moe_trace_attach.argtypes = [ctypes.c_void_p, ctypes.c_uint64]
        self.lib.moe_trace_detach.restype = ctypes.c_int
        self.torch = torch
        self.region = region
        self.buf = torch.zeros(HDR_BYTES + N_KERNEL_IDS * region * REC.itemsize, dtype=torch.uint8, device="cuda")

    def close(self):
        """Detaches the buffer and puts the product library back in the binding."""
        self.lib.moe_trace_detach()
        self._B.LIB_PATH, self._B._lib = self._saved

    def run(self, fn) -> np.ndarray:
        """Records of the kernels `fn` launches (synchronised before and after)."""
        torch = self.torch
        torch.cuda.synchronize()
        if self.lib.moe_trace_attach(ctypes.c_void_p(self.buf.data_ptr()), self.buf.numel()) != 0:
            raise RuntimeError("moe_trace_attach failed")
        fn()
        torch.cuda.synchronize()
        if self.lib.moe_trace_detach() != 0:
            raise RuntimeError("moe_trace_detach failed")
        # written slots only (the attach zeroed the buffer: kernel ids start at 1)
        words = self.buf[HDR_BYTES:].view(torch.int64).view(-1, REC.itemsize // 8)
        used = words[(words[:, 2] & 0xFFFFFFFF) != 0]
        return used.cpu().numpy().view(REC).reshape(-1)


def summarise(rec: np.ndarray) -> dict:
    """Per kernel id: units, start spread, durations, end (µs from the first stamp)."""
    if rec.size == 0:
        return {}
    origin = int(rec["t0"].min())
    out = {}
    for kid in sorted(set(int(k) for k in rec["kernel"])):
        r = rec[rec["kernel"] == kid]
        t0 = (r["t0"].astype(np.int64) - origin) * TICK_US
        t1 = (r["t1"].astype(np.int64) - origin) * TICK_US
        dur = t1 - t0
        e = {"units": int(r.size), "start_first": round(float(t0.min()), 2),
             "start_spread": round(float(t0.max() - t0.min()), 2),
             "dur_mean": round(float(dur.mean()), 2), "dur_min": round(float(dur.min()), 2),
             "dur_max": round(float(dur.max()), 2), "end_first": round(float(t1.min()), 2),
             "end_last": round(float(t1.max()), 2)}
        if KERNELS.get(kid) == "gemm_compute":
            xcd = r["block"] % 8
            e["end_by_xcd"] = {int(x): {"mean": round(float(t1[xcd == x].mean()), 2),
                                        "max": round(float(t1[xcd == x].max()), 2)}
                               for x in sorted(set(int(v) for v in xcd))}
        if KERNELS.get(kid) == "gemm_tile":
            e["tiles_per_workgroup_max"] = int(r["aux"].max()) + 1
            e["dur_by_position"] = {int(p): round(float(dur[r["aux"] == p].mean()), 2)
                                    for p in sorted(set(int(v) for v in r["aux"]))}
        out[KERNELS.get(kid, str(kid))] = e
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="ep8_2048x8_h7168")
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--json", default=None, help="also write the summaries to this file")
    args = ap.parse_args()

    import torch
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import workloads
    tr = Tracer(torch)
    import combine_expert_histogram_amd as moe

    w = workloads.get(args.workload)
    d_loc = moe.Dims(S=w.S, Ts=w.Ts, k=w.k, E=w.E, e0=w.e0, L=w.L, H=w.H)
    d_all = moe.Dims(S=w.S, Ts=w.Ts, k=w.k, E=w.E, e0=0, L=w.E, H=w.H)
    ids, wts = workloads.routing(w)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ids_d, wts_d = dev(ids.reshape(-1)), dev(wts.reshape(-1))
    x_d = dev(workloads.activations(w).view(np.int16))
    wq, ws = workloads.weights(w)
    wq_d, ws_d = dev(wq), dev(ws)
    del wq
    w2q, w2s = workloads.weights2(w)
    w2q_d, w2s_d = dev(w2q), dev(w2s)
    del w2q
    Y_d = dev(workloads.expert_outputs(w).view(np.int16)).view(torch.bfloat16)
    lay, lay_all = moe.alloc_layout(d_loc), moe.alloc_layout(d_all)
    q = torch.empty((w.T, w.H), dtype=torch.uint8, device="cuda")
    qs = torch.empty((w.T, w.H // 128), dtype=torch.float32, device="cuda")
    y1 = torch.empty((w.T * w.k, w.N), dtype=torch.bfloat16, device="cuda")
    g_ws = moe.alloc_gemm1_workspace(d_loc, w.N)
    out = torch.empty((w.T, w.combine_width), dtype=torch.bfloat16, device="cuda")
    inter = w.N // 2
    h = torch.empty((w.T * w.k, inter), dtype=torch.uint8, device="cuda")
    hs = torch.empty((w.T * w.k, inter // 128), dtype=torch.float32, device="cuda")
    y2 = torch.empty((w.T * w.k, w.H), dtype=torch.bfloat16, device="cuda")
    g2_ws = moe.alloc_gemm2_workspace(d_loc, inter)

    calls = [
        ("layout_local", lambda: moe.route_layout(d_loc, ids_d, lay)),
        ("quant", lambda: moe.quant_dispatch(d_loc, x_d, lay, q, qs)),
        ("gemm1", lambda: moe.grouped_gemm1(d_loc, w.N, q, qs, lay, wq_d, ws_d, y1, g_ws)),
        ("layout_full", lambda: moe.route_layout(d_all, ids_d, lay_all)),
        ("combine", lambda: moe.combine(d_all, w.combine_width, Y_d, lay_all["assign_row"], wts_d, out)),
        ("act", lambda: moe.silu_mul_quant(d_loc, inter, y1, lay, h, hs)),
        ("gemm2", lambda: moe.grouped_gemm2(d_loc, inter, h, hs, lay, wts_d, w2q_d, w2s_d, y2, g2_ws)),
    ]
    for _ in range(args.warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()
    result = {"workload": w.name, "steps": args.steps, "calls": {}}
    for step in range(args.steps):
        for name, fn in calls:
            result["calls"].setdefault(name, []).append(summarise(tr.run(fn)))
    for name, runs in result["calls"].items():
        print(f"== {name} ({len(runs)} calls; µs from the call's first stamp)")
        for kname in runs[0]:
            vals = [r[kname] for r in runs if kname in r]
            pick = lambda key: "/".join(f"{v[key]:.1f}" for v in vals)
            print(f"  {kname:13s} units {vals[0]['units']:7d}  start spread {pick('start_spread')}  "
                  f"dur mean {pick('dur_mean')} (min {pick('dur_min')}, max {pick('dur_max')})  "
                  f"end {pick('end_first')} .. {pick('end_last')}")
            if "end_by_xcd" in vals[0]:
                for x, v in vals[0]["end_by_xcd"].items():
                    print(f"      XCD {x}: compute end mean {v['mean']:.1f}, max {v['max']:.1f}")
            if "dur_by_position" in vals[0]:
                pos = vals[0]["dur_by_position"]
                print("      tile duration by position: " + ", ".join(f"{p}: {v:.1f}" for p, v in pos.items()))
    if args.json:
        with open(args.json, "w") as f:
            json.dump(result, f, indent=1)


if __name__ == "__main__":
    main()
