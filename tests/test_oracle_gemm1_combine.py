"""Pins for the oracle's GEMM1 and combine steps (CPU only): float64 brute
force, identity/permutation weights, identity experts, k=1 gathers and
linearity."""
import numpy as np
import pytest

import workloads
from oracle import bf16, combine, fp8, gemm1, layout, quant


def _tiny_chain():
    w = workloads.get("tiny_t64_h256_e8")
    ids, wts = workloads.routing(w)
    x = workloads.activations(w)
    wq, ws = workloads.weights(w)
    lay = layout.route_layout(ids, w.S, w.Ts, w.k, w.e0, w.L)
    q, qs = quant.quant_dispatch(x, lay["slot_tok"])
    return w, ids, wts, x, wq, ws, lay, q, qs


def rel_l2(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def test_gemm1_matches_float64_triple_loop():
    w, ids, wts, x, wq, ws, lay, q, qs = _tiny_chain()
    y = gemm1.grouped_gemm1(q, qs, lay["row_slot"], lay["expert_offsets"], wq, ws)
    offs = lay["expert_offsets"]
    rng = np.random.default_rng(0)
    for r in rng.choice(int(lay["totals"][0]), 12, replace=False):
        le = int(np.searchsorted(offs, r, side="right") - 1)
        u = lay["row_slot"][r]
        for n in rng.choice(w.N, 6, replace=False):
            acc = 0.0
            for h in range(w.H):
                a = float(fp8.decode(q[u, h])) * float(qs[u, h // 128])
                b = float(fp8.decode(wq[le, n, h])) * float(ws[le, n // 128, h // 128])
                acc += a * b
            assert abs(acc - y[r, n]) <= 1e-5 * (abs(acc) + 1e-3)


def test_gemm1_identity_weights_give_the_dequantised_rows():
    # N = H, w = identity (0x38 = 1.0), scale 1: y[r] = A[row_slot[r]] exactly.
    w, ids, wts, x, wq, ws, lay, q, qs = _tiny_chain()
    L, H = w.L, w.H
    eye = np.where(np.eye(H, dtype=bool), np.uint8(0x38), np.uint8(0))
    wid = np.broadcast_to(eye, (L, H, H)).copy()
    sid = np.ones((L, H // 128, H // 128), np.float32)
    y = gemm1.grouped_gemm1(q, qs, lay["row_slot"], lay["expert_offsets"], wid, sid)
    A = gemm1.dequant_rows(q, qs)[lay["row_slot"]]
    np.testing.assert_array_equal(y, A)


def test_gemm1_permutation_weights_permute_columns():
    w, ids, wts, x, wq, ws, lay, q, qs = _tiny_chain()
    L, H = w.L, w.H
    rng = np.random.default_rng(5)
    perms = [rng.permutation(H) for _ in range(L)]
    wp = np.zeros((L, H, H), np.uint8)
    for le in range(L):
        wp[le, np.arange(H), perms[le]] = 0x40          # 2.0 at (n, perm[n])
    sp = np.full((L, H // 128, H // 128), 0.5, np.float32)   # 2.0 * 0.5 = 1
    y = gemm1.grouped_gemm1(q, qs, lay["row_slot"], lay["expert_offsets"], wp, sp)
    A = gemm1.dequant_rows(q, qs)
    offs = lay["expert_offsets"]
    for le in range(L):
        for r in range(offs[le], offs[le + 1]):
            np.testing.assert_array_equal(y[r], A[lay["row_slot"][r]][perms[le]])


def test_gemm1_sampled_rows_equal_full():
    w, ids, wts, x, wq, ws, lay, q, qs = _tiny_chain()
    y = gemm1.grouped_gemm1(q, qs, lay["row_slot"], lay["expert_offsets"], wq, ws)
    rows = [0, 5, 127, 64]
    ys = gemm1.grouped_gemm1(q, qs, lay["row_slot"], lay["expert_offsets"], wq, ws, rows=rows)
    # same sums; BLAS may block a row subset differently, so compare to fp32 rounding
    np.testing.assert_allclose(ys, y[rows], rtol=1e-5, atol=1e-6)


def test_combine_identity_experts_reproduce_input():
    """Y[r] = x[token of r], every expert in the layout, weights summing to 1:
    the fp32 result is x*(1 +- ~2^-20) and rounds back to x in bf16."""
    w = workloads.get("ep8_256x8_h7168")
    ids, wts = workloads.routing(w)
    T, k = 512, w.k
    ids, wts = ids[:T], wts[:T]
    rng = np.random.default_rng(2)
    x = bf16.from_f32(rng.standard_normal((T, 256)).astype(np.float32))
    lay = layout.route_layout(ids, 1, T, k, 0, w.E)
    Y = x[lay["row_assign"] // k]
    acc, out = combine.combine(Y, lay["assign_row"], wts, T, k)
    np.testing.assert_array_equal(out, x)


def test_combine_k1_is_a_gather_and_brute_force():
    rng = np.random.default_rng(4)
    T, k, R, width = 40, 3, 90, 64
    Y = bf16.from_f32(rng.standard_normal((R, width)).astype(np.float32))
    ar = rng.integers(-1, R, T * k).astype(np.int32)
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    acc, out = combine.combine(Y, ar, w, T, k)
    Yf = bf16.to_f32(Y).astype(np.float64)
    for g in range(T):
        ref = np.zeros(width)
        for j in range(k):
            r = ar[g * k + j]
            if r >= 0:
                ref = ref + float(w[g, j]) * Yf[r]
        np.testing.assert_allclose(acc[g], ref, rtol=1e-6, atol=1e-6)
    # k = 1, w = 1: exact gather; -1 gives +0
    ar1 = rng.integers(-1, R, T).astype(np.int32)
    acc1, out1 = combine.combine(Y, ar1, np.ones((T, 1), np.float32), T, 1)
    for g in range(T):
        if ar1[g] >= 0:
            np.testing.assert_array_equal(out1[g], Y[ar1[g]])
        else:
            assert (out1[g] == 0).all()


def test_combine_linear_in_weights():
    rng = np.random.default_rng(9)
    T, k, R, width = 16, 4, 50, 32
    Y = bf16.from_f32(rng.standard_normal((R, width)).astype(np.float32))
    ar = rng.integers(0, R, T * k).astype(np.int32)
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    a1, _ = combine.combine(Y, ar, w, T, k)
    a2, _ = combine.combine(Y, ar, 2 * w, T, k)                  # exact scaling by 2
    np.testing.assert_array_equal(a2, 2 * a1)
    wz = w.copy(); wz[:, 1:] = 0
    a3, _ = combine.combine(Y, ar, wz, T, k)
    np.testing.assert_array_equal(a3, bf16.to_f32(Y[ar.reshape(T, k)[:, 0]]) * w[:, :1])


def test_tiny_chain_tolerance_vs_float64():
    """The full tiny chain: GEMM1 then combine in float64 vs the oracle's fp32."""
    w, ids, wts, x, wq, ws, lay, q, qs = _tiny_chain()
    y = gemm1.grouped_gemm1(q, qs, lay["row_slot"], lay["expert_offsets"], wq, ws)
    A = gemm1.dequant_rows(q, qs).astype(np.float64)[lay["row_slot"]]
    offs = lay["expert_offsets"]
    y64 = np.zeros_like(y, dtype=np.float64)
    for le in range(w.L):
        B = gemm1.dequant_weight(wq[le], ws[le]).astype(np.float64)
        y64[offs[le]:offs[le + 1]] = A[offs[le]:offs[le + 1]] @ B.T
    assert rel_l2(y, y64) < 1e-6
