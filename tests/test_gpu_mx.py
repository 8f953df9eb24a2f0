"""GPU parity of the MX-style variants (e8m0 scales per 32 K elements):
moe_quant_dispatch_mx bit-exact against the oracle (payloads and packed scale
codes) on the workloads and on crafted groups; moe_grouped_gemm1_mx within
rel-L2 <= 1e-2 and max-abs <= 2e-2 * rms of the oracle's fp32 product, and bit
for bit in the single-term cases (identity weights; permutation weights with a
different power-of-two scale for every column and K group)."""
import functools

import numpy as np
import pytest
import torch

import combine_expert_histogram_amd as moe
import workloads
from gpu_helpers import (activations, dev, dims, host_u16, poisoned_layout, require_gpu, routing, say,
                         tolerance)
from oracle import bf16 as obf16
from oracle import layout as olayout
from oracle import mx as omx

pytestmark = pytest.mark.gpu

Q_POISON = 0xA5
S_POISON = 0x5A5A5A5A
Y_POISON = 0x7FC1      # a bf16 NaN pattern the kernel never writes


@functools.lru_cache(maxsize=1)
def weights_mx(name):
    return workloads.weights_mx(workloads.get(name))


def _quant(d, ids, x_bits):
    lay = moe.route_layout(d, dev(ids.reshape(-1)), poisoned_layout(d))
    q = torch.full((d.T, d.H), Q_POISON, dtype=torch.uint8, device="cuda")
    qs = torch.full((d.T, d.H // 128), S_POISON, dtype=torch.int32, device="cuda")
    moe.quant_dispatch_mx(d, dev(x_bits.view(np.int16)), lay, q, qs)
    torch.cuda.synchronize()
    return lay, q, qs


def _compare_quant(ref_lay, q, qs, x_bits, slots):
    rq, rs = omx.quant_dispatch(x_bits, ref_lay["slot_tok"], slots=slots)
    sl = torch.from_numpy(np.asarray(slots, dtype=np.int64)).cuda()
    gq = q[sl].cpu().numpy()
    gs = qs[sl].cpu().numpy().view(np.uint32)
    bad = np.nonzero((gq != rq).any(axis=1))[0]
    assert bad.size == 0, f"payload mismatch in {bad.size} slots, first slot {slots[bad[0]]}"
    np.testing.assert_array_equal(gs, rs)


@pytest.mark.parametrize("name,sample", [
    ("tiny_t64_h256_e8", None), ("ep8_256x8_h7168", None), ("ep8_2048x8_h7168", None),
    ("ep8_2048x8_h4096", None), ("ep8_8192x8_h7168_zipf", 512),
])
def test_quant_mx_workloads(name, sample):
    require_gpu()
    w = workloads.get(name)
    d = dims(w)
    say(f"quant_mx {name} T={d.T} H={d.H}")
    ids, _ = routing(name)
    x = activations(name)
    ref_lay = olayout.route_layout(ids, d.S, d.Ts, d.k, d.e0, d.L)
    U = int(ref_lay["totals"][1])
    lay, q, qs = _quant(d, ids, x)
    if sample is None:
        slots = np.arange(U)
    else:
        rng = np.random.default_rng(19)
        slots = np.unique(np.concatenate([[0, U - 1], rng.choice(U, sample, replace=False)]))
    _compare_quant(ref_lay, q, qs, x, slots)
    assert (q[U:] == Q_POISON).all() and (qs[U:] == S_POISON).all()


def _crafted_rows(H, rng):
    """Rows whose 32-element groups hit the scale rule's edges: all-zero groups
    (negative zeros too), amax = 448 * 2^j exactly and one bf16 step above it,
    bf16 subnormals, the largest bf16 magnitudes, wide in-group dynamic range
    (elements that round to zero or into e4m3 subnormals), e4m3 rounding ties."""
    rows = []
    g = H // 32

    def group(kind):
        v = (rng.standard_normal(32) * np.exp2(rng.uniform(-8, 8))).astype(np.float32)
        if kind == 0:
            return np.zeros(32, np.float32)
        if kind == 1:
            return np.where(rng.random(32) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        if kind == 2:
            v = np.clip(v, -400, 400)
            v[rng.integers(32)] = np.float32(448.0 * 2.0 ** rng.integers(-40, 40))
            return v
        if kind == 3:
            top = np.float32(448.0 * 2.0 ** rng.integers(-40, 40))
            v = v / np.abs(v).max() * top * np.float32(0.5)
            v[rng.integers(32)] = np.nextafter(top, np.float32(np.inf)) * np.float32(1 + 2 ** -7)
            return v
        if kind == 4:
            return (rng.standard_normal(32) * np.float32(2.0 ** -128)).astype(np.float32)
        if kind == 5:
            return (rng.standard_normal(32) * np.float32(2.0 ** 125)).astype(np.float32)
        if kind == 6:
            return (v * np.exp2(rng.uniform(-30, 0, 32))).astype(np.float32)
        # e4m3 ties after the exact scaling: amax 448 (E = 0), values on half steps
        v = (rng.integers(-64, 64, 32) * 0.5 + 0.25).astype(np.float32) * np.float32(2.0 ** rng.integers(-3, 3))
        v[0] = 448.0
        return v

    for r in range(24):
        rows.append(np.concatenate([group((r + j) % 8) for j in range(g)]))
    return np.stack(rows).astype(np.float32)


def test_quant_mx_crafted_groups():
    require_gpu()
    H = 512
    rng = np.random.default_rng(23)
    xf = _crafted_rows(H, rng)
    x = obf16.from_f32(xf)
    # bf16 rounding may push an element of a "tie" group off its tie; the rule is
    # checked on whatever the bf16 bits are
    T = x.shape[0]
    d = moe.Dims(S=2, Ts=T // 2, k=1, E=2, e0=0, L=2, H=H)
    ids = (np.arange(T) % 2).astype(np.int32).reshape(T, 1)
    ref_lay = olayout.route_layout(ids, d.S, d.Ts, d.k, d.e0, d.L)
    U = int(ref_lay["totals"][1])
    assert U == T
    lay, q, qs = _quant(d, ids, x)
    _compare_quant(ref_lay, q, qs, x, np.arange(U))


def _gemm_chain(d, n, ids, x_bits, wq, ws):
    lay = moe.route_layout(d, dev(ids.reshape(-1)), poisoned_layout(d))
    q, qs = moe.quant_dispatch_mx(d, dev(x_bits.view(np.int16)), lay)
    y = torch.full((d.T * d.k, n), Y_POISON, dtype=torch.int16, device="cuda")
    moe.grouped_gemm1_mx(d, n, q, qs, lay, dev(wq), dev(ws.view(np.int32)), y.view(torch.bfloat16))
    torch.cuda.synchronize()
    return lay, y


def _sample_rows(offs, R, extra, seed):
    rng = np.random.default_rng(seed)
    rows = set()
    for le in range(len(offs) - 1):
        if offs[le + 1] > offs[le]:
            rows.update({int(offs[le]), int(offs[le + 1]) - 1, int(min(offs[le] + 127, offs[le + 1] - 1)),
                         int(min(offs[le] + 128, offs[le + 1] - 1))})
    rows.update(int(r) for r in rng.choice(R, min(extra, R), replace=False))
    return np.array(sorted(rows))


def _check_gemm(d, n, ids, x, wq, ws, sample=None):
    ref = olayout.route_layout(ids, d.S, d.Ts, d.k, d.e0, d.L)
    R = int(ref["totals"][0])
    lay, y = _gemm_chain(d, n, ids, x, wq, ws)
    rows = np.arange(R) if sample is None else _sample_rows(ref["expert_offsets"], R, sample, 5)
    slots = ref["row_slot"][rows]
    uslots, inv = np.unique(slots, return_inverse=True)
    rq, rs = omx.quant_dispatch(x, ref["slot_tok"], slots=uslots)
    row_slot_compact = np.zeros(R, np.int64)
    row_slot_compact[rows] = inv
    yref = omx.grouped_gemm1(rq, rs, row_slot_compact, ref["expert_offsets"], wq, ws, rows=rows)
    got = host_u16(y[torch.from_numpy(rows).cuda()]) if rows.size else np.zeros((0, n), np.uint16)
    t = tolerance(got, yref)
    say(f"  rows={rows.size} {t}")
    assert t.ok, str(t)
    assert bool((y[R:] == Y_POISON).all())


@pytest.mark.parametrize("name,sample", [
    ("tiny_t64_h256_e8", None), ("ep8_256x8_h7168", None), ("ep8_2048x8_h7168", None),
    ("ep8_2048x8_h4096", None), ("ep8_8192x8_h7168_zipf", 384),
])
def test_gemm1_mx_workloads(name, sample):
    require_gpu()
    w = workloads.get(name)
    d = dims(w)
    say(f"gemm1_mx {name} T={d.T} H={d.H} N={w.N}")
    ids, _ = routing(name)
    x = activations(name)
    wq, ws = weights_mx(name)
    _check_gemm(d, w.N, ids, x, wq, ws, sample)


def _small(seed, S, Ts, k, E, e0, L, H, n, skew=None):
    rng = np.random.default_rng(seed)
    T = S * Ts
    if skew is not None:
        p = np.exp2(-skew * np.arange(E)); p /= p.sum()
        ids = rng.choice(E, (T, k), p=p).astype(np.int32)
    else:
        ids = rng.integers(0, E, (T, k)).astype(np.int32)
    # per-group magnitudes spread over 2^-6 .. 2^6 so the scales differ
    x = (rng.standard_normal((T, H)) * np.exp2(rng.uniform(-6, 6, (T, H // 32))).repeat(32, 1))
    x = obf16.from_f32(x.astype(np.float32))
    wf = (rng.standard_normal((L * n, H)) * 0.02 * np.exp2(rng.uniform(-3, 3, (L * n, H // 32))).repeat(32, 1))
    wq, wsc = omx.quantise_rows(obf16.to_f32(obf16.from_f32(wf.astype(np.float32))))
    wq = wq.reshape(L, n, H)
    ws = np.ascontiguousarray(wsc.reshape(L, n, H // 128).transpose(0, 2, 1))
    return moe.Dims(S=S, Ts=Ts, k=k, E=E, e0=e0, L=L, H=H), ids, x, wq, ws


SMALL = {
    "h128_n128": dict(S=2, Ts=100, k=2, E=8, e0=0, L=8, H=128, n=128),
    "ragged_rows_offset_experts": dict(S=3, Ts=211, k=3, E=20, e0=5, L=9, H=384, n=256),
    "skewed_empty_experts": dict(S=4, Ts=500, k=4, E=32, e0=0, L=16, H=512, n=384, skew=0.6),
    "one_row_experts": dict(S=1, Ts=7, k=1, E=8, e0=0, L=8, H=256, n=128),
}


@pytest.mark.parametrize("case", list(SMALL))
def test_gemm1_mx_small_shapes(case):
    require_gpu()
    say(f"gemm1_mx small {case}")
    d, ids, x, wq, ws = _small(31, **SMALL[case])
    _check_gemm(d, SMALL[case]["n"], ids, x, wq, ws)


def test_gemm1_mx_identity_weights_bit_exact():
    """N = H, W = I (byte 0x38 = 1.0, every code 127): each output is one exact
    product, so y = bf16(dequantised A row) bit for bit; checks which e8m0 code
    scales which K group of A."""
    require_gpu()
    w = workloads.get("tiny_t64_h256_e8")
    d = dims(w)
    ids, _ = routing(w.name)
    rng = np.random.default_rng(4)
    H = w.H
    x = obf16.from_f32((rng.standard_normal((d.T, H)) *
                        np.exp2(rng.uniform(-20, 20, (d.T, H // 32))).repeat(32, 1)).astype(np.float32))
    eye = np.where(np.eye(H, dtype=bool), np.uint8(0x38), np.uint8(0))
    wq = np.broadcast_to(eye, (w.L, H, H)).copy()
    ws = np.full((w.L, H // 128, H), 0x7F7F7F7F, np.uint32)
    ref = olayout.route_layout(ids, d.S, d.Ts, d.k, d.e0, d.L)
    lay, y = _gemm_chain(d, H, ids, x, wq, ws)
    rq, rs = omx.quant_dispatch(x, ref["slot_tok"])
    A = omx.dequant_rows(rq, rs)[ref["row_slot"]]
    R = int(ref["totals"][0])
    # a sum of products is +0 where the lone nonzero term is -0 (the other terms add +0)
    np.testing.assert_array_equal(host_u16(y[:R]), obf16.from_f32(A + np.float32(0)))


def test_gemm1_mx_permutation_weights_bit_exact():
    """W[le, c, perm(c)] = 1.0 (byte 0x38) and every (column, K group) code drawn
    from [117, 137]: y[r, c] = bf16(A[r, perm(c)] * 2^(code(c, perm(c)/32) - 127))
    exactly; checks the column mapping and which code scales which K group of B."""
    require_gpu()
    L, H, n = 6, 512, 512
    rng = np.random.default_rng(2)
    T = 300
    d = moe.Dims(S=2, Ts=T // 2, k=2, E=6, e0=0, L=L, H=H)
    ids = np.stack([rng.permutation(6)[:2] for _ in range(T)]).astype(np.int32)
    x = obf16.from_f32(rng.standard_normal((T, H)).astype(np.float32))
    perms = [rng.permutation(H) for _ in range(L)]
    wq = np.zeros((L, n, H), np.uint8)
    for le in range(L):
        wq[le, np.arange(n), perms[le]] = 0x38
    codes = rng.integers(117, 138, (L, n, H // 32)).astype(np.uint8)
    ws = np.ascontiguousarray(omx.pack_codes(codes).transpose(0, 2, 1))       # [L, H/128, n]
    ref = olayout.route_layout(ids, d.S, d.Ts, d.k, d.e0, d.L)
    lay, y = _gemm_chain(d, n, ids, x, wq, ws)
    rq, rs = omx.quant_dispatch(x, ref["slot_tok"])
    A = omx.dequant_rows(rq, rs).astype(np.float64)
    offs = ref["expert_offsets"]
    got = host_u16(y)
    for le in range(L):
        cols = np.arange(n)
        shift = codes[le, cols, perms[le] // 32].astype(np.int64) - 127
        for r in range(offs[le], offs[le + 1]):
            want = A[ref["row_slot"][r]][perms[le]] * np.ldexp(1.0, shift)
            np.testing.assert_array_equal(got[r], obf16.from_f32(want.astype(np.float32) + np.float32(0)))
