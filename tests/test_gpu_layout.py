"""GPU parity: moe_route_layout vs the oracle, bit-exact, on every workload
(local share and the full-expert layout the combine uses) and edge cases."""
import numpy as np
import pytest
import torch

import combine_expert_histogram_amd as moe
import workloads
from gpu_helpers import check_layout, dims, poisoned_layout, require_gpu, routing, say

pytestmark = pytest.mark.gpu

NAMES = list(workloads.WORKLOADS)


@pytest.mark.parametrize("full", [False, True], ids=["local", "all_experts"])
@pytest.mark.parametrize("name", NAMES)
def test_layout_workloads(name, full):
    require_gpu()
    w = workloads.get(name)
    d = dims(w, full)
    say(f"layout {name} full={full} T={d.T} L={d.L}")
    ids, _ = routing(name)
    check_layout(d, ids)


def _edge(seed, S, Ts, k, E, e0, L, lo=None, hi=None, const=None):
    rng = np.random.default_rng(seed)
    T = S * Ts
    if const is not None:
        ids = np.full((T, k), const, np.int32)
    else:
        ids = rng.integers(0 if lo is None else lo, E if hi is None else hi, (T, k)).astype(np.int32)
    return moe.Dims(S=S, Ts=Ts, k=k, E=E, e0=e0, L=L), ids


EDGES = {
    "empty": dict(S=2, Ts=0, k=2, E=8, e0=0, L=8),
    "one_expert_all_rows": dict(S=2, Ts=300, k=4, E=16, e0=4, L=6, const=5),
    "out_of_range_and_negative": dict(S=3, Ts=1000, k=3, E=40, e0=7, L=13, lo=-5, hi=45),
    "single_local_expert": dict(S=8, Ts=257, k=8, E=64, e0=63, L=1),
    "k1": dict(S=4, Ts=999, k=1, E=32, e0=0, L=32),
    "ragged_sources": dict(S=3, Ts=17, k=5, E=12, e0=2, L=7),
    "wide_L1024": dict(S=8, Ts=512, k=8, E=1024, e0=0, L=1024),
    "no_local_assignment": dict(S=2, Ts=100, k=2, E=16, e0=8, L=8, lo=0, hi=8),
    "duplicates_in_row": dict(S=1, Ts=4096, k=6, E=6, e0=1, L=3),
    "many_chunks": dict(S=8, Ts=8192, k=2, E=64, e0=0, L=8),
}


@pytest.mark.parametrize("case", list(EDGES))
def test_layout_edge_cases(case):
    require_gpu()
    say(f"layout edge {case}")
    d, ids = _edge(11, **EDGES[case])
    check_layout(d, ids)


def test_layout_is_deterministic_and_reusable():
    """Same inputs twice into the same buffers: identical bytes (no order races)."""
    require_gpu()
    name = "ep8_2048x8_h7168"
    d = dims(workloads.get(name), full=True)
    ids, _ = routing(name)
    lay = check_layout(d, ids)
    first = {k: v.clone() for k, v in lay.items() if k != "ws"}
    for _ in range(3):
        moe.route_layout(d, torch.from_numpy(ids.reshape(-1)).cuda(), lay)
    torch.cuda.synchronize()
    for k, v in first.items():
        assert torch.equal(v, lay[k]), k


def test_layout_rejects_short_buffers():
    require_gpu()
    d = moe.Dims(S=1, Ts=64, k=2, E=8, e0=0, L=8)
    lay = poisoned_layout(d)
    lay["row_slot"] = lay["row_slot"][:10]
    with pytest.raises(ValueError):
        moe.route_layout(d, torch.zeros(128, dtype=torch.int32, device="cuda"), lay)
