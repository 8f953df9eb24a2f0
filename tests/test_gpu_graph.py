"""GPU: the four calls read their counts on the device, so a whole step can be
captured once in a graph and replayed.  Each replay (with eager work and
synchronisations in between) must reproduce the eager step bit for bit:
layout tables, fp8 payloads and scales, GEMM1 output and the combine."""
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
