"""GPU parity: moe_grouped_gemm1 vs the oracle (fp32 on the same dequantised
operands) within rel-L2 <= 1e-2 and max-abs <= 2e-2 * rms; bit-exact in the
single-term special cases (identity and permutation weights)."""
import numpy as np
import pytest
import torch

import combine_expert_histogram_amd as moe
import workloads
from gpu_helpers import (activations, dev, dims, host_u16, poisoned_layout, require_gpu, routing,
                         say, tolerance, weights)
from oracle import bf16 as obf16
from oracle import gemm1 as ogemm1
from oracle import layout as olayout
from oracle import quant as oquant

pytestmark = pytest.mark.gpu

Y_POISON = 0x7FC1      # a bf16 NaN pattern the kernel never writes


def _gpu_chain(d, n, ids, x_bits, wq, ws):
    lay = moe.route_layout(d, dev(ids.reshape(-1)), poisoned_layout(d))
    q, qs = moe.quant_dispatch(d, dev(x_bits.view(np.int16)), lay)
    y = torch.full((d.T * d.k, n), Y_POISON, dtype=torch.int16, device="cuda")
    yb = y.view(torch.bfloat16)
    moe.grouped_gemm1(d, n, q, qs, lay, dev(wq), dev(ws), yb)
    torch.cuda.synchronize()
    return lay, q, qs, y


def _sample_rows(offs, R, extra, seed):
    rng = np.random.default_rng(seed)
    rows = set()
    for le in range(len(offs) - 1):
        if offs[le + 1] > offs[le]:
            rows.update({int(offs[le]), int(offs[le + 1]) - 1, int(min(offs[le] + 127, offs[le + 1] - 1)),
                         int(min(offs[le] + 128, offs[le + 1] - 1))})
    rows.update(int(r) for r in rng.choice(R, min(extra, R), replace=False))
    return np.array(sorted(rows))


def _check(d, n, ids, x, wq, ws, sample=None):
    ref = olayout.route_layout(ids, d.S, d.Ts, d.k, d.e0, d.L)
    R = int(ref["totals"][0])
    lay, q, qs, y = _gpu_chain(d, n, ids, x, wq, ws)
    rows = np.arange(R) if sample is None else _sample_rows(ref["expert_offsets"], R, sample, 3)
    slots = ref["row_slot"][rows]
    uslots, inv = np.unique(slots, return_inverse=True)
    rq, rs = oquant.quant_dispatch(x, ref["slot_tok"], slots=uslots)
    # the oracle's operands: its own quant of the needed slots, scattered into
    # a compact table indexed by position in uslots
    row_slot_compact = np.zeros(R, np.int64)
    row_slot_compact[rows] = inv
    yref = ogemm1.grouped_gemm1(rq, rs, row_slot_compact, ref["expert_offsets"], wq, ws, rows=rows)
    got = host_u16(y[torch.from_numpy(rows).cuda()]) if rows.size else np.zeros((0, n), np.uint16)
    t = tolerance(got, yref)
    say(f"  rows={rows.size} {t}")
    assert t.ok, str(t)
    # rows past R untouched
    assert bool((y[R:] == Y_POISON).all())
    return ref, y


@pytest.mark.parametrize("name,sample", [
    ("tiny_t64_h256_e8", None), ("ep8_256x8_h7168", None), ("ep8_2048x8_h7168", None),
    ("ep8_2048x8_h4096", None), ("ep8_8192x8_h7168_zipf", 384),
])
def test_gemm1_workloads(name, sample):
    require_gpu()
    w = workloads.get(name)
    d = dims(w)
    say(f"gemm1 {name} T={d.T} H={d.H} N={w.N}")
    ids, _ = routing(name)
    x = activations(name)
    wq, ws = weights(name)
    _check(d, w.N, ids, x, wq, ws, sample)


def _small(seed, S, Ts, k, E, e0, L, H, n, skew=None):
    rng = np.random.default_rng(seed)
    T = S * Ts
    if skew is not None:
        p = np.exp2(-skew * np.arange(E)); p /= p.sum()
        ids = rng.choice(E, (T, k), p=p).astype(np.int32)
    else:
        ids = rng.integers(0, E, (T, k)).astype(np.int32)
    x = obf16.from_f32(rng.standard_normal((T, H)).astype(np.float32))
    wf = (rng.standard_normal((L, n, H)) * 0.02).astype(np.float32)
    wsc = np.abs(wf).reshape(L, n // 128, 128, H // 128, 128).max(axis=(2, 4)) / np.float32(448)
    wsc = wsc.astype(np.float32)
    v = wf / np.repeat(np.repeat(wsc, 128, axis=1), 128, axis=2)
    wq = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return moe.Dims(S=S, Ts=Ts, k=k, E=E, e0=e0, L=L, H=H), ids, x, wq, wsc


SMALL = {
    "h128_n128": dict(S=2, Ts=100, k=2, E=8, e0=0, L=8, H=128, n=128),
    "ragged_rows_offset_experts": dict(S=3, Ts=211, k=3, E=20, e0=5, L=9, H=384, n=256),
    "skewed_empty_experts": dict(S=4, Ts=500, k=4, E=32, e0=0, L=16, H=512, n=384, skew=0.6),
    "one_row_experts": dict(S=1, Ts=7, k=1, E=8, e0=0, L=8, H=256, n=128),
}


@pytest.mark.parametrize("case", list(SMALL))
def test_gemm1_small_shapes(case):
    require_gpu()
    say(f"gemm1 small {case}")
    d, ids, x, wq, ws = _small(21, **SMALL[case])
    _check(d, SMALL[case]["n"], ids, x, wq, ws)


def test_gemm1_identity_weights_bit_exact():
    """N = H and W = I (byte 0x38 = 1.0, scale 1): every output is one exact
    product, so y = bf16(dequantised A row) bit for bit."""
    require_gpu()
    w = workloads.get("tiny_t64_h256_e8")
    d = dims(w)
    ids, _ = routing(w.name)
    x = activations(w.name)
    H = w.H
    eye = np.where(np.eye(H, dtype=bool), np.uint8(0x38), np.uint8(0))
    wq = np.broadcast_to(eye, (w.L, H, H)).copy()
    ws = np.ones((w.L, H // 128, H // 128), np.float32)
    ref = olayout.route_layout(ids, d.S, d.Ts, d.k, d.e0, d.L)
    lay, q, qs, y = _gpu_chain(d, H, ids, x, wq, ws)
    rq, rs = oquant.quant_dispatch(x, ref["slot_tok"])
    A = ogemm1.dequant_rows(rq, rs)[ref["row_slot"]]
    R = int(ref["totals"][0])
    # a sum of products is +0 where the lone nonzero term is -0 (the other terms add +0)
    np.testing.assert_array_equal(host_u16(y[:R]), obf16.from_f32(A + np.float32(0)))


def test_gemm1_permutation_weights_bit_exact():
    """W = 2 * P (byte 0x40) with scale 0.5: y = bf16(A[:, perm]) exactly;
    checks the column and K-block mapping of every sub-tile."""
    require_gpu()
    d, ids, x, _, _ = _small(8, S=2, Ts=150, k=2, E=6, e0=0, L=6, H=512, n=512)
    rng = np.random.default_rng(1)
    perms = [rng.permutation(512) for _ in range(6)]
    wq = np.zeros((6, 512, 512), np.uint8)
    for le in range(6):
        wq[le, np.arange(512), perms[le]] = 0x40
    ws = np.full((6, 4, 4), 0.5, np.float32)
    ref = olayout.route_layout(ids, d.S, d.Ts, d.k, d.e0, d.L)
    lay, q, qs, y = _gpu_chain(d, 512, ids, x, wq, ws)
    rq, rs = oquant.quant_dispatch(x, ref["slot_tok"])
    A = ogemm1.dequant_rows(rq, rs)
    offs = ref["expert_offsets"]
    got = host_u16(y)
    for le in range(6):
        for r in range(offs[le], offs[le + 1]):
            np.testing.assert_array_equal(got[r], obf16.from_f32(A[ref["row_slot"][r]][perms[le]] + np.float32(0)))


def test_gemm1_most_local_experts():
    """L = 1024 local experts (the most the call accepts) with a K loop of 32
    steps (so the balanced schedule's planner runs, with ≈1000 experts of a few
    rows each, nearly every tile partial) and one column tile.  Weights are
    random e4m3 codes (no NaN patterns) with random block scales; every row
    within the tolerance."""
    require_gpu()
    rng = np.random.default_rng(23)
    S, Ts, k, E, L, H, n = 1, 512, 8, 1024, 1024, 4096, 128
    T = S * Ts
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = obf16.from_f32((rng.standard_normal((T, H)) * np.exp2(rng.uniform(-3, 3, (T, 1)))).astype(np.float32))
    codes = rng.integers(0, 256, (L, n, H), dtype=np.uint8)
    wq = np.where((codes & 0x7F) == 0x7F, codes ^ 0x01, codes).astype(np.uint8)      # 0x7F / 0xFF are NaN
    ws = np.exp2(rng.uniform(-12, -6, (L, n // 128, H // 128))).astype(np.float32)
    d = moe.Dims(S=S, Ts=Ts, k=k, E=E, e0=0, L=L, H=H)
    say(f"gemm1 L={L} T={T} H={H} n={n}")
    _check(d, n, ids, x, wq, ws)
