"""The allocation-free layout (moe_route_layout_noalloc, its workspace in a
static device array) against moe_route_layout with a caller workspace: every
output table bit for bit, on two calls in a row on the same GPU, the second
with a smaller input (so a stale histogram from the first call would show)."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from combine_expert_histogram_amd import binding as b

pytestmark = pytest.mark.gpu


def _layout(d, ids, noalloc):
    out = b.alloc_layout(d)
    for k in b.LAYOUT_KEYS:                       # poison: unwritten entries must match too
        out[k].fill_(-7)
    args = [out[k] for k in b.LAYOUT_KEYS]
    if noalloc:
        b.moe_route_layout_noalloc(d, ids, *args)
    else:
        b.moe_route_layout(d, ids, *args, out["ws"])
    return out


def _check(d, ids_np):
    ids = torch.from_numpy(np.ascontiguousarray(ids_np.reshape(-1))).cuda()
    ref = _layout(d, ids, noalloc=False)
    got = _layout(d, ids, noalloc=True)
    torch.cuda.synchronize()
    for k in b.LAYOUT_KEYS:
        assert torch.equal(ref[k], got[k]), (d, k)
    return int(ref["totals"][0]), int(ref["totals"][1])


@pytest.mark.parametrize("name", ["ep8_2048x8_h7168", "ep8_256x8_h7168"])
def test_noalloc_matches_workspace_layout_two_calls(name):
    w = workloads.get(name)
    ids, _ = workloads.routing(w)
    print(f"[noalloc] {name} T={w.T}", flush=True)
    # all-expert layout (the largest histogram: 256 experts), then the local one
    # (32 experts), then a much smaller input on the same GPU
    for L in (w.E, w.L):
        d = b.Dims(S=w.S, Ts=w.Ts, k=w.k, E=w.E, e0=0, L=L, H=w.H)
        R, U = _check(d, ids)
        assert R > 0 and U > 0
    small = ids[: w.T // 8]
    d = b.Dims(S=1, Ts=w.T // 8, k=w.k, E=w.E, e0=0, L=w.L, H=w.H)
    _check(d, small)


def test_noalloc_edge_cases():
    rng = np.random.default_rng(11)
    # empty input, a single token, ids outside the local range, duplicates
    for S, Ts, k, E, e0, L in ((2, 0, 2, 8, 0, 8), (1, 1, 4, 16, 4, 8), (3, 17, 4, 16, 2, 5)):
        d = b.Dims(S=S, Ts=Ts, k=k, E=E, e0=e0, L=L, H=128)
        ids = rng.integers(-2, E + 2, size=(max(S * Ts, 1), k)).astype(np.int32)[: S * Ts]
        if S * Ts:
            ids[0, :] = e0                         # a duplicate id inside one token
        print(f"[noalloc] edge S={S} Ts={Ts} k={k} E={E} e0={e0} L={L}", flush=True)
        _check(d, ids if S * Ts else np.zeros((1, k), np.int32))


def test_noalloc_rejects_oversized_plan():
    d = b.Dims(S=8, Ts=1 << 17, k=8, E=1024, e0=0, L=1024)
    P = ctypes.c_void_p(4096)
    assert b.lib().moe_route_layout_noalloc(ctypes.byref(d.c()), *([P] * 10), None) == -2
