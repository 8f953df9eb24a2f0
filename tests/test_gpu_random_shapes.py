"""GPU parity over seeded random shapes.

Sixteen small configurations drawn from one generator: sources, tokens per
source, top-k, the expert count and the local expert window, the hidden size,
GEMM1's width and stage2's intermediate size (multiples of 128, so half
column tiles and single K blocks occur), uniform or skewed routing with
distinct experts per token.  Each configuration runs the whole chain and checks
every output against the oracle to the same bar as the fixed-shape tests:
  * layout (local window) and quant: bit for bit, every slot;
  * GEMM1 with fp32 scales and with e8m0 (MX) scales: every row within the
    tolerance, rows past R untouched;
  * GEMM2 on the oracle's quantised activations, with fp32 and with e8m0
    scales: every row within the tolerance, rows past R untouched;
  * combine over the all-expert layout: every token within the tolerance.
"""
import numpy as np
import pytest
import torch

import combine_expert_histogram_amd as moe
from gpu_helpers import check_layout, dev, host_u16, poisoned_layout, require_gpu, say, tolerance
from oracle import bf16 as obf16
from oracle import combine as ocombine
from oracle import gemm1 as ogemm1
from oracle import layout as olayout
from oracle import mx as omx
from oracle import quant as oquant
from oracle import stage2 as ostage2

pytestmark = pytest.mark.gpu

Y_POISON = 0x7FC1      # a bf16 NaN pattern the kernels never write
SEEDS = list(range(16))


def _shape(seed):
    rng = np.random.default_rng(7000 + seed)
    S = int(rng.integers(1, 5))
    Ts = int(rng.integers(1, 321))
    k = int(rng.integers(1, 9))
    E = int(rng.integers(max(k, 2), 65))
    L = int(rng.integers(1, E + 1))
    e0 = int(rng.integers(0, E - L + 1))
    H = 128 * int(rng.integers(1, 9))
    n = 128 * int(rng.integers(1, 7))
    inter = 128 * int(rng.integers(1, 5))
    skew = [None, 0.15, 0.6][int(rng.integers(0, 3))]
    return dict(S=S, Ts=Ts, k=k, E=E, L=L, e0=e0, H=H, n=n, inter=inter, skew=skew), rng


def _routing(rng, T, E, k, skew):
    """k distinct experts per token (Gumbel top-k over the expert weights
    2^(-skew * e), uniform when skew is None), routing weights in [0.01, 1)."""
    logp = np.zeros(E) if skew is None else -skew * np.arange(E) * np.log(2.0)
    keys = logp[None, :] + rng.gumbel(size=(T, E))
    ids = np.argsort(-keys, axis=1)[:, :k].astype(np.int32)
    wts = rng.uniform(0.01, 1.0, (T, k)).astype(np.float32)
    return ids, wts


def _block_scaled_fp8(wf, L, rows, cols):
    """fp8 e4m3 codes of wf [L, rows, cols] with one fp32 scale per 128 x 128 block."""
    sc = np.abs(wf).reshape(L, rows // 128, 128, cols // 128, 128).max(axis=(2, 4)) / np.float32(448)
    sc = np.maximum(sc, np.float32(1e-30)).astype(np.float32)
    v = wf / np.repeat(np.repeat(sc, 128, axis=1), 128, axis=2)
    q = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q, sc


def _rows_check(y, R, ref_f32, what):
    if R:
        t = tolerance(host_u16(y[:R]), ref_f32)
        say(f"  {what} rows={R} {t}")
        assert t.ok, f"{what}: {t}"
    assert bool((y[R:] == Y_POISON).all()), f"{what} wrote past R"


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape_chain(seed):
    require_gpu()
    p, rng = _shape(seed)
    S, Ts, k, E, L, e0, H, n, inter = (p[x] for x in ("S", "Ts", "k", "E", "L", "e0", "H", "n", "inter"))
    T = S * Ts
    say(f"random shape seed={seed}: {p}")
    ids, wts = _routing(rng, T, E, k, p["skew"])
    # activations with per-block magnitudes 2^-4 .. 2^4, so the block scales differ
    mag = np.exp2(rng.uniform(-4, 4, (T, H // 32))).repeat(32, axis=1)
    x = obf16.from_f32((rng.standard_normal((T, H)) * mag).astype(np.float32))
    d = moe.Dims(S=S, Ts=Ts, k=k, E=E, e0=e0, L=L, H=H)
    rows_cap = T * k

    # layout (bit for bit, poisoned tails untouched) and quant (bit for bit, every slot)
    lay = check_layout(d, ids)
    ref = olayout.route_layout(ids, S, Ts, k, e0, L)
    R, U = (int(v) for v in ref["totals"])
    x_d = dev(x.view(np.int16))
    q = torch.full((T, H), 0xA5, dtype=torch.uint8, device="cuda")
    qs = torch.full((T, H // 128), -7.0, dtype=torch.float32, device="cuda")
    moe.quant_dispatch(d, x_d, lay, q, qs)
    torch.cuda.synchronize()
    rq, rs = oquant.quant_dispatch(x, ref["slot_tok"])
    np.testing.assert_array_equal(q[:U].cpu().numpy(), rq, err_msg="quant payload")
    np.testing.assert_array_equal(qs[:U].cpu().numpy().view(np.uint32), rs.view(np.uint32), err_msg="quant scales")

    # GEMM1, fp32 block scales
    w1, w1s = _block_scaled_fp8((rng.standard_normal((L, n, H)) * 0.02).astype(np.float32), L, n, H)
    y1 = torch.full((rows_cap, n), Y_POISON, dtype=torch.int16, device="cuda")
    moe.grouped_gemm1(d, n, q, qs, lay, dev(w1), dev(w1s), y1.view(torch.bfloat16))
    torch.cuda.synchronize()
    ref1 = ogemm1.grouped_gemm1(rq, rs, ref["row_slot"], ref["expert_offsets"], w1, w1s) if R else None
    _rows_check(y1, R, ref1, "gemm1")

    # MX quant (bit for bit) and MX GEMM1
    qm, qms = moe.quant_dispatch_mx(d, x_d, lay)
    torch.cuda.synchronize()
    rqm, rsm = omx.quant_dispatch(x, ref["slot_tok"])
    np.testing.assert_array_equal(qm[:U].cpu().numpy(), rqm, err_msg="mx quant payload")
    np.testing.assert_array_equal(qms[:U].cpu().numpy().view(np.uint32), rsm.view(np.uint32),
                                  err_msg="mx quant scales")
    wf = rng.standard_normal((L * n, H)) * 0.02 * np.exp2(rng.uniform(-3, 3, (L * n, H // 32))).repeat(32, axis=1)
    wm, wmc = omx.quantise_rows(obf16.to_f32(obf16.from_f32(wf.astype(np.float32))))
    wm = wm.reshape(L, n, H)
    wms = np.ascontiguousarray(wmc.reshape(L, n, H // 128).transpose(0, 2, 1))
    ym = torch.full((rows_cap, n), Y_POISON, dtype=torch.int16, device="cuda")
    moe.grouped_gemm1_mx(d, n, qm, qms, lay, dev(wm), dev(wms.view(np.int32)), ym.view(torch.bfloat16))
    torch.cuda.synchronize()
    refm = omx.grouped_gemm1(rqm, rsm, ref["row_slot"], ref["expert_offsets"], wm, wms) if R else None
    _rows_check(ym, R, refm, "gemm1_mx")

    # GEMM2 on the oracle's quantised activations of synthetic GEMM1 rows
    g1 = obf16.from_f32((rng.standard_normal((rows_cap, 2 * inter)) * 1.7).astype(np.float32))
    q2, s2 = ostage2.act_quant(g1)
    w2, w2s = _block_scaled_fp8((rng.standard_normal((L, H, inter)) * 0.02).astype(np.float32), L, H, inter)
    y2 = torch.full((rows_cap, H), Y_POISON, dtype=torch.int16, device="cuda")
    moe.grouped_gemm2(d, inter, dev(q2), dev(s2), lay, dev(wts.reshape(-1)), dev(w2), dev(w2s),
                      y2.view(torch.bfloat16))
    torch.cuda.synchronize()
    ref2 = (ostage2.grouped_gemm2(q2, s2, ref["expert_offsets"], ref["row_assign"], wts, w2, w2s)
            if R else None)
    _rows_check(y2, R, ref2, "gemm2")

    # MX GEMM2 on the oracle's MX-quantised activations of the same rows
    q2m, s2m = ostage2.act_quant_mx(g1)
    wf2 = (rng.standard_normal((L * H, inter)) * 0.02
           * np.exp2(rng.uniform(-3, 3, (L * H, inter // 32))).repeat(32, axis=1))
    w2m, w2mc = omx.quantise_rows(obf16.to_f32(obf16.from_f32(wf2.astype(np.float32))))
    w2m = w2m.reshape(L, H, inter)
    w2ms = np.ascontiguousarray(w2mc.reshape(L, H, inter // 128).transpose(0, 2, 1))
    y2m = torch.full((rows_cap, H), Y_POISON, dtype=torch.int16, device="cuda")
    moe.grouped_gemm2_mx(d, inter, dev(q2m), dev(s2m.view(np.int32)), lay, dev(wts.reshape(-1)), dev(w2m),
                         dev(w2ms.view(np.int32)), y2m.view(torch.bfloat16))
    torch.cuda.synchronize()
    ref2m = (ostage2.grouped_gemm2_mx(q2m, s2m, ref["expert_offsets"], ref["row_assign"], wts, w2m, w2ms)
             if R else None)
    _rows_check(y2m, R, ref2m, "gemm2_mx")

    # combine over the all-expert layout (every assignment is a row)
    da = moe.Dims(S=S, Ts=Ts, k=k, E=E, e0=0, L=E, H=H)
    lay_a = moe.route_layout(da, dev(ids.reshape(-1)), poisoned_layout(da))
    ref_a = olayout.route_layout(ids, S, Ts, k, 0, E)
    Y = obf16.from_f32((rng.standard_normal((rows_cap, H)) * 0.5).astype(np.float32))
    out = moe.combine(da, H, dev(Y.view(np.int16)), lay_a["assign_row"], dev(wts.reshape(-1)))
    torch.cuda.synchronize()
    acc, _ = ocombine.combine(Y, ref_a["assign_row"], wts, T, k)
    t = tolerance(host_u16(out[:T]), acc)
    say(f"  combine tokens={T} {t}")
    assert t.ok, f"combine: {t}"
