"""The clock-stamp trace (a measurement aid: csrc/trace.h, the traced library
libmoe_hotpath_trace.so and combine_expert_histogram_amd/trace.py): the
summaries' arithmetic on the host, the trace calls present only in the traced
library, and on the GPU a traced step that records every kernel and computes
the same bytes as the product library."""
import ctypes
import os

import numpy as np
import pytest

from combine_expert_histogram_amd import build as cbuild
from combine_expert_histogram_amd import trace as ctrace


def _recs(rows):
    r = np.zeros(len(rows), dtype=ctrace.REC)
    for i, (t0, t1, k, b, item, aux) in enumerate(rows):
        r[i] = (t0, t1, k, b, item, aux)
    return r


def test_summarise_spreads_durations_and_xcds():
    # two GEMM workgroups (blocks 0 and 9: XCDs 0 and 1), three tiles, one quant wave
    rec = _recs([
        (1000, 1500, 7, 0, 0, 0), (1010, 1800, 7, 9, 0, 0),
        (1000, 1200, 8, 0, 0, 0), (1200, 1500, 8, 0, 256, 1), (1010, 1800, 8, 9, 9, 0),
        (1100, 1150, 3, 4, 2, 0),
    ])
    s = ctrace.summarise(rec)
    c = s["gemm_compute"]
    assert c["units"] == 2 and c["start_spread"] == pytest.approx(0.1)
    assert c["end_last"] == pytest.approx(8.0) and c["dur_max"] == pytest.approx(7.9)
    assert c["end_by_xcd"] == {0: {"mean": 5.0, "max": 5.0}, 1: {"mean": 8.0, "max": 8.0}}
    t = s["gemm_tile"]
    assert t["units"] == 3 and t["tiles_per_workgroup_max"] == 2
    assert t["dur_by_position"] == {0: pytest.approx((2.0 + 7.9) / 2), 1: pytest.approx(3.0)}
    q = s["quant"]
    assert q["start_first"] == pytest.approx(1.0) and q["dur_mean"] == pytest.approx(0.5)
    assert ctrace.summarise(rec[:0]) == {}


def test_trace_calls_only_in_the_traced_library():
    if not (os.path.exists(cbuild.LIB) and os.path.exists(cbuild.TRACE_LIB)):
        pytest.skip("libraries not built")
    prod = ctypes.CDLL(cbuild.LIB)
    traced = ctypes.CDLL(cbuild.TRACE_LIB)
    assert not hasattr(prod, "moe_trace_attach") and not hasattr(prod, "moe_trace_detach")
    assert hasattr(traced, "moe_trace_attach") and hasattr(traced, "moe_trace_detach")
    # the traced library is the same ABI plus the two trace calls
    from combine_expert_histogram_amd import binding
    for name in binding.EXPORTS:
        assert hasattr(traced, name), name


@pytest.mark.gpu
def test_traced_step_records_every_kernel_and_matches_the_product():
    import torch

    import combine_expert_histogram_amd as moe
    import workloads
    from gpu_helpers import require_gpu, say
    require_gpu()
    w = workloads.get("ep8_256x8_h7168")
    d = moe.Dims(S=w.S, Ts=w.Ts, k=w.k, E=w.E, e0=w.e0, L=w.L, H=w.H)
    ids, wts = workloads.routing(w)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ids_d, wts_d = dev(ids.reshape(-1)), dev(wts.reshape(-1))
    x_d = dev(workloads.activations(w).view(np.int16))
    wq, ws = workloads.weights(w)
    wq_d, ws_d = dev(wq), dev(ws)

    def step():
        lay = moe.route_layout(d, ids_d)
        q, qs = moe.quant_dispatch(d, x_d, lay)
        y = moe.grouped_gemm1(d, w.N, q, qs, lay, wq_d, ws_d)
        torch.cuda.synchronize()
        return lay, q, qs, y

    lay_p, q_p, qs_p, y_p = step()                       # product library
    R, U = (int(v) for v in lay_p["totals"].cpu())
    tr = ctrace.Tracer(torch, region=1 << 14)
    try:
        recs = {}
        out = {}
        recs["layout"] = tr.run(lambda: out.__setitem__("lay", moe.route_layout(d, ids_d)))
        recs["quant"] = tr.run(lambda: out.__setitem__("q", moe.quant_dispatch(d, x_d, out["lay"])))
        recs["gemm1"] = tr.run(lambda: out.__setitem__(
            "y", moe.grouped_gemm1(d, w.N, out["q"][0], out["q"][1], out["lay"], wq_d, ws_d)))
    finally:
        tr.close()
    for name, r in recs.items():
        say(f"trace {name}: {r.size} records")
        assert r.size > 0 and (r["t1"] >= r["t0"]).all(), name
    kinds = lambda r: set(int(k) for k in r["kernel"])
    assert kinds(recs["layout"]) == {1, 2}
    assert kinds(recs["quant"]) == {3}
    assert kinds(recs["gemm1"]) == {5, 6, 7, 8}
    g = recs["gemm1"]
    offs = out["lay"]["expert_offsets"].cpu().numpy()
    tiles = int(sum(-(-int(c) // 128) for c in np.diff(offs))) * (w.N // 256)
    slots = g["item"][g["kernel"] == 8]
    assert slots.size == tiles and np.unique(slots).size == tiles     # one record per tile, by schedule slot
    assert (g["kernel"] == 6).sum() == (g["kernel"] == 7).sum() > 0
    # the traced library computes the same bytes
    assert torch.equal(out["lay"]["row_slot"][:R], lay_p["row_slot"][:R])
    assert torch.equal(out["q"][0][:U], q_p[:U]) and torch.equal(out["q"][1][:U], qs_p[:U])
    assert torch.equal(out["y"][:R], y_p[:R])
    # the product library is back in the binding
    from combine_expert_histogram_amd import binding
    assert binding.LIB_PATH == cbuild.LIB
