"""GPU: the calls read their counts on the device, so a whole step can be
captured once in a graph and replayed.  Each replay (with eager work and
synchronisations in between) must reproduce the eager step bit for bit:
layout tables, fp8 payloads and scales, the GEMM and act outputs and the combine."""
import numpy as np
import pytest
import torch

import combine_expert_histogram_amd as moe
import workloads
from gpu_helpers import activations, dev, dims, require_gpu, routing, say, weights

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny_t64_h256_e8", "ep8_256x8_h7168"])
def test_step_graph_replays_match_eager(name):
    require_gpu()
    w = workloads.get(name)
    say(f"graph replay: {name}")
    d = dims(w)
    ids, wts = routing(name)
    x = activations(name)
    wq, ws = weights(name)
    ids_d, wts_d, x_d = dev(ids.reshape(-1)), dev(wts.reshape(-1)), dev(x.view(np.int16))
    wq_d, ws_d = dev(wq), dev(ws)
    lay = moe.alloc_layout(d)
    q = torch.empty((w.T, w.H), dtype=torch.uint8, device="cuda")
    qs = torch.empty((w.T, w.H // 128), dtype=torch.float32, device="cuda")
    y1 = torch.zeros((w.T * w.k, w.N), dtype=torch.bfloat16, device="cuda")
    g_ws = moe.alloc_gemm1_workspace(d, w.N)
    out = torch.zeros((w.T, w.N), dtype=torch.bfloat16, device="cuda")

    def step():
        moe.route_layout(d, ids_d, lay)
        moe.quant_dispatch(d, x_d, lay, q, qs)
        moe.grouped_gemm1(d, w.N, q, qs, lay, wq_d, ws_d, y1, g_ws)
        # combine of GEMM1's own rows (local experts only): exercises the fourth call
        moe.combine(d, w.N, y1, lay["assign_row"], wts_d, out)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    R, U = (int(v) for v in lay["totals"].cpu())
    ref = {k: v.clone() for k, v in lay.items() if k != "ws"}
    ref_q, ref_qs, ref_y, ref_out = q[:U].clone(), qs[:U].clone(), y1[:R].clone(), out.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: wipe every output the graph writes
        for k, v in lay.items():
            if k != "ws":
                v.fill_(-7)
        q.fill_(0xAB)
        qs.fill_(-1.0)
        y1.fill_(3.0)
        out.fill_(5.0)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            if k in ("row_slot", "row_assign"):
                assert torch.equal(lay[k][:R], v[:R]), (rep, k)
            elif k == "slot_tok":
                assert torch.equal(lay[k][:U], v[:U]), (rep, k)
            else:
                assert torch.equal(lay[k], v), (rep, k)
        assert torch.equal(q[:U], ref_q) and torch.equal(qs[:U], ref_qs), rep
        assert torch.equal(y1[:R], ref_y), rep
        assert torch.equal(out, ref_out), rep
        say(f"  replay {rep}: bit-identical (R={R}, U={U})")


@pytest.mark.parametrize("name", ["tiny_t64_h256_e8", "ep8_256x8_h7168"])
def test_mx_and_stage2_graph_replays_match_eager(name):
    """The other entry points captured in one graph: layout -> MX quant -> MX
    GEMM1, then stage2 on the fp32-scale GEMM1's output (act -> GEMM2 ->
    combine of the local rows) and its MX form (act -> GEMM2).  Three replays
    with the outputs wiped in between must each reproduce the eager pass bit
    for bit."""
    require_gpu()
    w = workloads.get(name)
    say(f"graph replay, MX and stage2: {name}")
    d = dims(w)
    I = w.N // 2
    ids, wts = routing(name)
    x = activations(name)
    wq, ws = weights(name)
    wmq, wms = workloads.weights_mx(w)
    w2q, w2s = workloads.weights2(w)
    w2mq, w2ms = workloads.weights2_mx(w)
    ids_d, wts_d, x_d = dev(ids.reshape(-1)), dev(wts.reshape(-1)), dev(x.view(np.int16))
    wq_d, ws_d, wmq_d, wms_d = dev(wq), dev(ws), dev(wmq), dev(wms.view(np.int32))
    w2q_d, w2s_d, w2mq_d, w2ms_d = dev(w2q), dev(w2s), dev(w2mq), dev(w2ms.view(np.int32))
    rows = w.T * w.k
    lay = moe.alloc_layout(d)
    q = torch.empty((w.T, w.H), dtype=torch.uint8, device="cuda")
    qs = torch.empty((w.T, w.H // 128), dtype=torch.float32, device="cuda")
    qm = torch.empty((w.T, w.H), dtype=torch.uint8, device="cuda")
    qms = torch.empty((w.T, w.H // 128), dtype=torch.int32, device="cuda")
    y1 = torch.zeros((rows, w.N), dtype=torch.bfloat16, device="cuda")
    ym = torch.zeros((rows, w.N), dtype=torch.bfloat16, device="cuda")
    h = torch.empty((rows, I), dtype=torch.uint8, device="cuda")
    hs = torch.empty((rows, I // 128), dtype=torch.float32, device="cuda")
    hm = torch.empty((rows, I), dtype=torch.uint8, device="cuda")
    hms = torch.empty((rows, I // 128), dtype=torch.int32, device="cuda")
    y2 = torch.zeros((rows, w.H), dtype=torch.bfloat16, device="cuda")
    y2m = torch.zeros((rows, w.H), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    ones = torch.ones(w.T * w.k, dtype=torch.float32, device="cuda")
    g1_ws = moe.alloc_gemm1_workspace(d, w.N)
    g1m_ws = moe.alloc_gemm1_workspace(d, w.N)
    g2_ws = moe.alloc_gemm2_workspace(d, I)
    g2m_ws = moe.alloc_gemm2_workspace(d, I)

    def step():
        moe.route_layout(d, ids_d, lay)
        moe.quant_dispatch(d, x_d, lay, q, qs)
        moe.grouped_gemm1(d, w.N, q, qs, lay, wq_d, ws_d, y1, g1_ws)
        moe.quant_dispatch_mx(d, x_d, lay, qm, qms)
        moe.grouped_gemm1_mx(d, w.N, qm, qms, lay, wmq_d, wms_d, ym, g1m_ws)
        moe.silu_mul_quant(d, I, y1, lay, h, hs)
        moe.grouped_gemm2(d, I, h, hs, lay, wts_d, w2q_d, w2s_d, y2, g2_ws)
        moe.combine(d, w.H, y2, lay["assign_row"], ones, out)
        moe.silu_mul_quant_mx(d, I, y1, lay, hm, hms)
        moe.grouped_gemm2_mx(d, I, hm, hms, lay, wts_d, w2mq_d, w2ms_d, y2m, g2m_ws)

    outputs = {"q": q, "qs": qs, "qm": qm, "qms": qms, "y1": y1, "ym": ym, "h": h, "hs": hs, "hm": hm,
               "hms": hms, "y2": y2, "y2m": y2m, "out": out}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    R, U = (int(v) for v in lay["totals"].cpu())
    valid = {"q": U, "qs": U, "qm": U, "qms": U, "y1": R, "ym": R, "h": R, "hs": R, "hm": R, "hms": R, "y2": R,
             "y2m": R, "out": w.T}
    ref = {k: v[:valid[k]].clone() for k, v in outputs.items()}

    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        for k, v in outputs.items():          # eager work between replays
            v.view(torch.uint8).fill_(0x5A)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(outputs[k][:valid[k]].view(torch.uint8), v.view(torch.uint8)), (rep, k)
        say(f"  replay {rep}: bit-identical (R={R}, U={U})")
