"""GPU parity of the MX stage2 variants: moe_silu_mul_quant_mx against the
oracle's silu * up and e8m0 group rule (the kernel's h is within a few fp32
ulps of the oracle's, so a group's exponent may differ by one only where
max|h| / 448 sits at a power of two, and every code is within half an e4m3
step of the oracle's h under the kernel's own exponent), and
moe_grouped_gemm2_mx on the oracle's own operands within rel-L2 <= 1e-2 and
max-abs <= 2e-2 * rms (bit-exact for identity weights with power-of-two
routing weights)."""
import functools

import numpy as np
import pytest
import torch

import combine_expert_histogram_amd as moe
import workloads
from gpu_helpers import dev, dims, host_u16, poisoned_layout, require_gpu, routing, say, tolerance
from oracle import bf16 as obf16
from oracle import fp8 as ofp8
from oracle import layout as olayout
from oracle import mx as omx
from oracle import stage2 as ostage2

pytestmark = pytest.mark.gpu

Q_POISON = 0xA5
S_POISON = 0x5A5A5A5A
Y_POISON = 0x7FC1


@functools.lru_cache(maxsize=1)
def weights2_mx(name):
    return workloads.weights2_mx(workloads.get(name))


@functools.lru_cache(maxsize=1)
def stage2_inputs(name):
    return workloads.stage2_inputs(workloads.get(name))


def _half_step(v):
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.exp2(e - 4)


def _check_act_mx(h_ref, q, s, rows):
    n, I = h_ref.shape
    q_ref, s_ref = omx.quantise_rows(h_ref)
    E = omx.unpack_codes(s).astype(np.int64) - 127                       # [n, I/32]
    E_ref = omx.unpack_codes(s_ref).astype(np.int64) - 127
    amax = np.abs(h_ref.reshape(n, I // 32, 32)).max(axis=2).astype(np.float64)
    t = amax / 448.0
    at_pow2 = np.abs(t / np.exp2(np.round(np.log2(np.maximum(t, 1e-300)))) - 1) <= 2.0 ** -20
    diff = E != E_ref
    assert not (np.abs(E - E_ref) > 1).any(), "group exponent off by more than one"
    assert not (diff & ~at_pow2).any(), f"{(diff & ~at_pow2).sum()} exponents differ away from a power of two"
    sc = np.exp2(np.repeat(E, 32, axis=1).astype(np.float64))
    deq = ofp8.decode(q).astype(np.float64) * sc
    bound = _half_step(h_ref / sc) * sc * (1 + 1e-5) + 1e-6 * np.abs(h_ref)
    bad = np.abs(deq - h_ref) > bound
    assert not bad.any(), f"{bad.sum()} codes off by more than half a step, first row {rows[np.nonzero(bad)[0][0]]}"
    same = float((q == q_ref).mean())
    say(f"  act_mx rows={n} identical codes {same:.6f} exponents {1 - diff.mean():.6f}")
    assert same >= 0.9999 and diff.mean() <= 1e-4


def _layout(d, ids):
    lay = moe.route_layout(d, dev(ids.reshape(-1)), poisoned_layout(d))
    ref = olayout.route_layout(ids, d.S, d.Ts, d.k, d.e0, d.L)
    return lay, ref


@pytest.mark.parametrize("name,sample", [
    ("tiny_t64_h256_e8", None), ("ep8_256x8_h7168", None), ("ep8_2048x8_h7168", 512),
])
def test_silu_mul_quant_mx_workloads(name, sample):
    require_gpu()
    w = workloads.get(name)
    d = dims(w)
    I = w.N // 2
    say(f"silu_mul_quant_mx {name} I={I}")
    ids, _ = routing(name)
    lay, ref = _layout(d, ids)
    R = int(ref["totals"][0])
    y1 = stage2_inputs(name)
    rows_cap = d.T * d.k
    h = torch.full((rows_cap, I), Q_POISON, dtype=torch.uint8, device="cuda")
    hs = torch.full((rows_cap, I // 128), S_POISON, dtype=torch.int32, device="cuda")
    moe.silu_mul_quant_mx(d, I, dev(y1.view(np.int16)), lay, h, hs)
    torch.cuda.synchronize()
    if sample is None:
        rows = np.arange(R)
    else:
        rng = np.random.default_rng(21)
        rows = np.unique(np.concatenate([[0, R - 1], rng.choice(R, sample, replace=False)]))
    sel = torch.from_numpy(rows).cuda()
    _check_act_mx(ostage2.silu_mul(obf16.to_f32(y1[rows])), h[sel].cpu().numpy(),
                  hs[sel].cpu().numpy().view(np.uint32), rows)
    assert (h[R:] == Q_POISON).all() and (hs[R:] == S_POISON).all()


def test_silu_mul_quant_mx_special_values():
    """Zero and negative-zero groups, the gate's far tails, and groups whose
    amax spans large and tiny magnitudes."""
    require_gpu()
    I, rows = 256, 16
    rng = np.random.default_rng(22)
    g = (rng.standard_normal((rows, I)) * 3).astype(np.float32)
    u = rng.standard_normal((rows, I)).astype(np.float32)
    g[0] = 0.0
    g[1, :64] = -120.0
    g[2] = 95.0
    u[3, 32:96] = 0.0
    u[4] *= 2.0 ** 60
    u[5] *= 2.0 ** -60
    u[6] *= np.exp2(rng.uniform(-30, 0, I)).astype(np.float32)
    y1 = obf16.from_f32(np.concatenate([g, u], axis=1))
    d = moe.Dims(S=1, Ts=rows, k=1, E=1, e0=0, L=1, H=128)
    lay, ref = _layout(d, np.zeros((rows, 1), np.int32))
    h = torch.full((rows, I), Q_POISON, dtype=torch.uint8, device="cuda")
    hs = torch.full((rows, I // 128), S_POISON, dtype=torch.int32, device="cuda")
    moe.silu_mul_quant_mx(d, I, dev(y1.view(np.int16)), lay, h, hs)
    torch.cuda.synchronize()
    hq, hsc = h.cpu().numpy(), hs.cpu().numpy().view(np.uint32)
    _check_act_mx(ostage2.silu_mul(obf16.to_f32(y1)), hq, hsc, np.arange(rows))
    codes = omx.unpack_codes(hsc)
    assert not hq[0].any() and not codes[0].any()            # all-zero groups: code 0, zero bytes
    assert not codes[1, :2].any() and not (hq[1, :64] & 0x7F).any()
    assert not codes[3, 1:3].any() and not hq[3, 32:96].any()


def _check_gemm2_mx(d, I, ids, wts, q2, s2, w2, w2s, sample=None, seed=23):
    lay, ref = _layout(d, ids)
    R = int(ref["totals"][0])
    rows_cap = d.T * d.k
    y2 = torch.full((rows_cap, d.H), Y_POISON, dtype=torch.int16, device="cuda")
    moe.grouped_gemm2_mx(d, I, dev(q2), dev(s2.view(np.int32)), lay, dev(wts.reshape(-1)), dev(w2),
                         dev(w2s.view(np.int32)), y2.view(torch.bfloat16))
    torch.cuda.synchronize()
    if sample is None:
        rows = np.arange(R)
    else:
        rng = np.random.default_rng(seed)
        offs = ref["expert_offsets"]
        ends = [int(v) for le in range(d.L) if offs[le + 1] > offs[le] for v in (offs[le], offs[le + 1] - 1)]
        rows = np.unique(np.concatenate([ends, rng.choice(R, min(sample, R), replace=False)]).astype(np.int64))
    yref = ostage2.grouped_gemm2_mx(q2[rows], s2[rows], ref["expert_offsets"], ref["row_assign"], wts, w2, w2s,
                                    rows=rows, q_index=np.arange(rows.size))
    got = host_u16(y2[torch.from_numpy(rows).cuda()]) if rows.size else np.zeros((0, d.H), np.uint16)
    t = tolerance(got, yref)
    say(f"  gemm2_mx rows={rows.size} {t}")
    assert t.ok, str(t)
    assert bool((y2[R:] == Y_POISON).all())


@pytest.mark.parametrize("name,sample", [
    ("tiny_t64_h256_e8", None), ("ep8_256x8_h7168", None), ("ep8_2048x8_h7168", 384),
])
def test_gemm2_mx_workloads(name, sample):
    require_gpu()
    w = workloads.get(name)
    d = dims(w)
    I = w.N // 2
    say(f"gemm2_mx {name} I={I} H={d.H}")
    ids, wts = routing(name)
    q2, s2 = ostage2.act_quant_mx(stage2_inputs(name))
    w2, w2s = weights2_mx(name)
    _check_gemm2_mx(d, I, ids, wts, q2, s2, w2, w2s, sample)


@pytest.mark.parametrize("case", [
    dict(S=3, Ts=211, k=3, E=20, e0=5, L=9, H=384, I=256),
    dict(S=1, Ts=7, k=1, E=8, e0=0, L=8, H=256, I=128),
], ids=["ragged_rows_offset_experts", "one_row_experts"])
def test_gemm2_mx_small_shapes(case):
    require_gpu()
    p = dict(case)
    I = p.pop("I")
    rng = np.random.default_rng(24)
    T = p["S"] * p["Ts"]
    ids = np.stack([rng.permutation(p["E"])[:p["k"]] for _ in range(T)]).astype(np.int32)
    wts = rng.uniform(0.01, 1.0, (T, p["k"])).astype(np.float32)
    d = moe.Dims(**p)
    y1 = obf16.from_f32((rng.standard_normal((T * p["k"], 2 * I)) * 1.7).astype(np.float32))
    q2, s2 = ostage2.act_quant_mx(y1)
    wf = obf16.to_f32(obf16.from_f32((rng.standard_normal((p["L"] * p["H"], I)) * 0.02).astype(np.float32)))
    wq, wsc = omx.quantise_rows(wf)
    w2 = wq.reshape(p["L"], p["H"], I)
    w2s = np.ascontiguousarray(wsc.reshape(p["L"], p["H"], I // 128).transpose(0, 2, 1))
    _check_gemm2_mx(d, I, ids, wts, q2, s2, w2, w2s)


def test_gemm2_mx_identity_weights_bit_exact():
    """I = H, W2 = I with every code 127, power-of-two routing weights: each
    output is one exact product, y2 = bf16(w_r * dequantised h row)."""
    require_gpu()
    rng = np.random.default_rng(25)
    S, Ts, k, E, L, H = 2, 96, 2, 8, 8, 256
    T = S * Ts
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    wts = np.exp2(-rng.integers(0, 6, (T, k))).astype(np.float32)
    d = moe.Dims(S=S, Ts=Ts, k=k, E=E, e0=0, L=L, H=H)
    y1 = (rng.standard_normal((T * k, 2 * H)) * np.exp2(rng.uniform(-8, 8, (T * k, 1)))).astype(np.float32)
    q2, s2 = ostage2.act_quant_mx(obf16.from_f32(y1))
    eye = np.where(np.eye(H, dtype=bool), np.uint8(0x38), np.uint8(0))
    w2 = np.broadcast_to(eye, (L, H, H)).copy()
    w2s = np.full((L, H // 128, H), 0x7F7F7F7F, np.uint32)
    lay, ref = _layout(d, ids)
    R = int(ref["totals"][0])
    y2 = torch.full((T * k, H), Y_POISON, dtype=torch.int16, device="cuda")
    moe.grouped_gemm2_mx(d, H, dev(q2), dev(s2.view(np.int32)), lay, dev(wts.reshape(-1)), dev(w2),
                         dev(w2s.view(np.int32)), y2.view(torch.bfloat16))
    torch.cuda.synchronize()
    A = omx.dequant_rows(q2[:R], s2[:R])
    want = A * ostage2.row_weights(ref["row_assign"], wts)[:, None]
    # a sum of products is +0 where the lone nonzero term is -0 (the other terms add +0)
    np.testing.assert_array_equal(host_u16(y2[:R]), obf16.from_f32(want + np.float32(0)))
