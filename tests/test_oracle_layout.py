"""Pins for the oracle's layout step (CPU only): brute-force loops on tiny
inputs, invariants of the stable counting sort, and closed-form statistics of
the routing draw."""
import math

import numpy as np
import pytest

import workloads
from oracle import layout


def brute_force_layout(ids, S, Ts, k, e0, L):
    """Walk the assignments in (g, j) order and append each local one to its
    expert's list; number rows expert by expert."""
    T = S * Ts
    per_expert = [[] for _ in range(L)]
    landed = []
    for g in range(T):
        any_local = False
        for j in range(k):
            le = int(ids[g][j]) - e0
            if 0 <= le < L:
                per_expert[le].append(g * k + j)
                any_local = True
        if any_local:
            landed.append(g)
    tok_slot = [-1] * T
    for u, g in enumerate(landed):
        tok_slot[g] = u
    row_assign, offsets = [], [0]
    for le in range(L):
        row_assign += per_expert[le]
        offsets.append(len(row_assign))
    assign_row = [-1] * (T * k)
    for r, a in enumerate(row_assign):
        assign_row[a] = r
    src = [sum(1 for g in landed if g < s * Ts) for s in range(S + 1)]
    return dict(
        expert_counts=[len(p) for p in per_expert], expert_offsets=offsets,
        row_slot=[tok_slot[a // k] for a in row_assign], row_assign=row_assign,
        assign_row=assign_row, tok_slot=tok_slot, slot_tok=landed,
        src_slot_offsets=src, totals=[len(row_assign), len(landed)],
    )


def _random_case(rng):
    S = int(rng.choice([1, 2, 3]))
    Ts = int(rng.integers(0, 18))
    E = int(rng.integers(1, 17))
    k = int(rng.integers(1, 5))
    L = int(rng.integers(1, E + 1))
    e0 = int(rng.integers(0, E - L + 1))
    mode = rng.integers(0, 4)
    T = S * Ts
    if mode == 0:      # uniform ids, duplicates allowed
        ids = rng.integers(0, E, (T, k))
    elif mode == 1:    # everything on one expert
        ids = np.full((T, k), int(rng.integers(0, E)))
    elif mode == 2:    # out-of-range and negative ids mixed in
        ids = rng.integers(-3, E + 3, (T, k))
    else:              # distinct ids per token when possible
        ids = np.stack([rng.permutation(max(E, k))[:k] for _ in range(T)]) if T else np.zeros((0, k))
    return S, Ts, k, e0, L, ids.astype(np.int32).reshape(T, k)


@pytest.mark.parametrize("seed", range(60))
def test_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    S, Ts, k, e0, L, ids = _random_case(rng)
    got = layout.route_layout(ids, S, Ts, k, e0, L)
    exp = brute_force_layout(ids, S, Ts, k, e0, L)
    for key, val in exp.items():
        np.testing.assert_array_equal(got[key], np.asarray(val, dtype=np.int32), err_msg=key)


def check_invariants(lay, ids, S, Ts, k, e0, L):
    T = S * Ts
    R, U = (int(v) for v in lay["totals"])
    ra, ar = lay["row_assign"].astype(np.int64), lay["assign_row"].astype(np.int64)
    offs = lay["expert_offsets"].astype(np.int64)
    flat = np.asarray(ids, np.int64).reshape(-1)
    # bijection between rows and local assignments
    assert ra.size == R and (ar >= 0).sum() == R
    np.testing.assert_array_equal(ar[ra], np.arange(R))
    # each row's expert equals its segment; segments contiguous and stable
    assert offs[0] == 0 and offs[-1] == R and (np.diff(offs) == lay["expert_counts"]).all()
    for le in range(L):
        seg = ra[offs[le]:offs[le + 1]]
        assert (flat[seg] - e0 == le).all()
        assert (np.diff(seg) > 0).all()
    # slots: inverse maps, increasing, landed == has a local assignment
    st, ts = lay["slot_tok"].astype(np.int64), lay["tok_slot"].astype(np.int64)
    assert st.size == U and (np.diff(st) > 0).all()
    np.testing.assert_array_equal(ts[st], np.arange(U))
    assert (ts >= 0).sum() == U
    np.testing.assert_array_equal(lay["row_slot"], ts[ra // k])
    src = lay["src_slot_offsets"]
    assert src[0] == 0 and src[-1] == U and (np.diff(src) >= 0).all()
    assert T == S * Ts


@pytest.mark.parametrize("seed", range(20))
def test_invariants_random(seed):
    rng = np.random.default_rng(1000 + seed)
    S, Ts, k, e0, L, ids = _random_case(rng)
    lay = layout.route_layout(ids, S, Ts, k, e0, L)
    check_invariants(lay, ids, S, Ts, k, e0, L)


def test_tiny_workload_invariants():
    w = workloads.get("tiny_t64_h256_e8")
    ids, wts = workloads.routing(w)
    lay = layout.route_layout(ids, w.S, w.Ts, w.k, w.e0, w.L)
    check_invariants(lay, ids, w.S, w.Ts, w.k, w.e0, w.L)
    # all 8 experts local and top-2 distinct: every assignment is a row, every token lands
    assert tuple(lay["totals"]) == (w.T * w.k, w.T)


def test_empty_input():
    lay = layout.route_layout(np.zeros((0, 4), np.int32), 3, 0, 4, 0, 5)
    assert tuple(lay["totals"]) == (0, 0)
    assert (lay["expert_offsets"] == 0).all() and (lay["src_slot_offsets"] == 0).all()


def test_ep8_share_statistics():
    """Closed forms for uniform top-8 of 256 with 32 local experts:
    E[R] = T*k*L/E and P(landed) = 1 - C(224,8)/C(256,8)."""
    w = workloads.get("ep8_256x8_h7168")
    ids, wts = workloads.routing(w)
    lay = layout.route_layout(ids, w.S, w.Ts, w.k, w.e0, w.L)
    R, U = (int(v) for v in lay["totals"])
    exp_R = w.T * w.k * w.L / w.E
    p_land = 1 - math.comb(w.E - w.L, w.k) / math.comb(w.E, w.k)
    assert abs(R - exp_R) < 5 * math.sqrt(exp_R)
    assert abs(U - p_land * w.T) < 5 * math.sqrt(w.T * p_land * (1 - p_land))
    # ids distinct per token, weights renormalised
    assert all(len(set(r)) == w.k for r in ids[:256].tolist())
    assert np.abs(wts.astype(np.float64).sum(1) - 1.0).max() < 2.0 ** -20
