"""The grouped GEMM's tile schedule, read back from the workspace after a call
(the pre-pass writes it there: a count, then one 16 B descriptor {expert,
column tile, first row, valid rows | row tile << 9} per slot, slot it * G + w
being tile it of workgroup w).  Checked against the tiles derived here from
the layout's expert offsets, independently of the pre-pass:
  * every tile of every local expert is scheduled exactly once, and nothing
    else but idle slots (zero valid rows);
  * a workgroup's idle slots come after all of its tiles (the kernel stops at
    the first one, so a tile behind it would never run);
  * K loops under 32 steps, and tables of more tiles than the planner holds,
    keep the natural order (slot s = tile s);
  * with the balanced schedule (K loops of 32 steps and more) each round gives
    each XCD exactly the natural tiles [r G + x G/8, + G/8) of the plain
    round-robin, only permuted among the XCD's workgroups (the row tiles that
    share a weight slab stay on one XCD in one round), and in every round but
    the last the partial tiles (an expert's last rows) rotate through the XCD's
    workgroups, so their counts per workgroup differ by at most one.
The operand values do not enter the schedule: zero weights and codes."""
import numpy as np
import pytest
import torch

import combine_expert_histogram_amd as moe
from gpu_helpers import dims, require_gpu, routing, say

pytestmark = pytest.mark.gpu

BM, BN, KMAXGRID, XCDS = 128, 256, 1024, 8
PLAN_MAX_TILES = 12288       # the planner keeps every tile's expert in LDS up to this many tiles


def _natural(offs, L, NT):
    """Tiles in the natural order: experts in order, column tiles outer, row
    tiles inner, as (expert, column tile, first row, valid rows, row tile)."""
    out = []
    for e in range(L):
        c = int(offs[e + 1] - offs[e])
        mt = (c + BM - 1) // BM
        for nt in range(NT):
            for m in range(mt):
                r0 = int(offs[e]) + BM * m
                out.append((e, nt, r0, min(BM, c - BM * m), m))
    return out


def _table(d, n, ws):
    rows_cap = d.T * d.k
    KB = d.H // 128
    scale_ld = ((rows_cap + 256) + 63) & ~63
    table_bytes = (KB * scale_ld * 4 + 255) & ~255
    tiles_cap = (rows_cap // BM + d.L) * ((n + BN - 1) // BN)
    raw = ws.view(torch.uint8)[table_bytes:table_bytes + 16 * (1 + tiles_cap + KMAXGRID)].cpu().numpy()
    return raw.view(np.int32).reshape(-1, 4)


def _run(d, n, ids):
    lay = moe.route_layout(d, torch.from_numpy(np.ascontiguousarray(ids.reshape(-1))).cuda())
    q = torch.zeros((d.T, d.H), dtype=torch.uint8, device="cuda")
    qs = torch.ones((d.T, d.H // 128), dtype=torch.float32, device="cuda")
    w = torch.zeros((d.L, n, d.H), dtype=torch.uint8, device="cuda")
    wsc = torch.ones((d.L, n // 128, d.H // 128), dtype=torch.float32, device="cuda")
    ws = moe.alloc_gemm1_workspace(d, n)
    moe.grouped_gemm1(d, n, q, qs, lay, w, wsc, None, ws)
    torch.cuda.synchronize()
    return lay["expert_offsets"].cpu().numpy(), _table(d, n, ws)


def _check(d, n, ids):
    offs, tab = _run(d, n, ids)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    G = (cus + XCDS - 1) // XCDS * XCDS
    NT = (n + BN - 1) // BN
    nat = _natural(offs, d.L, NT)
    total = len(nat)
    slots = int(tab[0, 0])
    desc = [tuple(int(v) for v in tab[1 + s]) for s in range(slots)]
    balanced = d.H // 128 >= 32 and total <= PLAN_MAX_TILES
    say(f"  tiles {total}, slots {slots}, grid {G}, balanced {balanced}")
    # every tile once, the rest idle
    as_tile = lambda t: (t[0], t[1], t[2], t[3] | (t[4] << 9))
    real = [x for x in desc if (x[3] & 511) != 0]
    assert sorted(real) == sorted(as_tile(t) for t in nat)
    assert all(x == (0, 0, 0, 0) for x in desc if (x[3] & 511) == 0)
    # a workgroup's idle slots come last
    for wg in range(G):
        seq = [(desc[s][3] & 511) != 0 for s in range(wg, slots, G)]
        assert seq == sorted(seq, reverse=True), f"workgroup {wg}: a tile after an idle slot"
    if not balanced:
        assert slots == total and desc == [as_tile(t) for t in nat]
        return
    R = (total + G - 1) // G
    assert slots == R * G
    nx = G // XCDS
    for r in range(R):
        for x in range(XCDS):
            c0 = r * G + x * nx
            got = sorted(d_ for d_ in desc[c0:c0 + nx] if (d_[3] & 511) != 0)
            want = sorted(as_tile(t) for t in nat[c0:min(total, c0 + nx)])
            assert got == want, f"round {r}, XCD {x}"
    for x in range(XCDS):
        parts = np.zeros(nx, np.int64)
        for r in range(R - 1):
            for w_ in range(nx):
                t = desc[r * G + x * nx + w_]
                parts[w_] += int((t[3] & 511) != 0 and (t[3] & 511) < BM)
        assert parts.max() - parts.min() <= 1, f"XCD {x}: partial tiles per workgroup {parts}"


@pytest.mark.parametrize("name", ["ep8_2048x8_h7168", "ep8_2048x8_h4096", "ep8_256x8_h7168"])
def test_schedule_of_the_workloads(name):
    require_gpu()
    import workloads
    w = workloads.get(name)
    say(f"schedule {name}")
    ids, _ = routing(name)
    _check(dims(w), w.N, ids)


@pytest.mark.parametrize("S,Ts,k,E,e0,L,H,n,skew", [
    (4, 500, 4, 32, 0, 16, 4096, 512, None),      # one round, mostly idle slots, balanced
    (2, 3000, 8, 64, 8, 32, 4096, 1024, 0.15),    # skewed, empty experts, several rounds
    (2, 700, 2, 16, 0, 16, 512, 384, None),       # short K loop: natural order, half column tile
    (8, 2048, 8, 32, 0, 32, 4096, 4096, None),    # more tiles than the planner holds: natural order
])
def test_schedule_small_shapes(S, Ts, k, E, e0, L, H, n, skew):
    require_gpu()
    rng = np.random.default_rng(11)
    T = S * Ts
    if skew is None:
        ids = rng.integers(0, E, (T, k)).astype(np.int32)
    else:
        p = np.exp2(-skew * np.arange(E))
        ids = rng.choice(E, (T, k), p=p / p.sum()).astype(np.int32)
    say(f"schedule T={T} L={L} H={H} n={n}")
    _check(moe.Dims(S=S, Ts=Ts, k=k, E=E, e0=e0, L=L, H=H), n, ids)
