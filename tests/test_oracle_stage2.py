"""Pins for the oracle's stage2 (CPU only): silu checked against closed forms
of the logistic function and torch's own silu, the gate/up halves, the
composition with the quant rule, GEMM2 against a float64 triple loop and its
identity / routing-weight special cases, and the unit-weight combine against
a brute-force per-token sum."""
import math

import numpy as np
import pytest
import torch

from oracle import bf16, fp8, mx, quant, stage2


def test_silu_closed_forms_and_halves():
    # sigma(ln a) = a / (1 + a), so silu(ln a) = ln(a) * a / (1 + a); first half
    # is the gate, second half the up factor
    a = np.array([0.25, 1.0, 3.0, 9.0, 1e3])
    gate = np.log(a)
    up = np.array([2.0, -1.5, 0.5, 1.0, 4.0])
    y = np.concatenate([gate, up])[None, :].astype(np.float32)
    h = stage2.silu_mul(y)[0].astype(np.float64)
    g32 = gate.astype(np.float32).astype(np.float64)
    want = g32 * (np.exp(g32) / (1 + np.exp(g32))) * up          # sigma via e^x/(1+e^x)
    np.testing.assert_allclose(h, want, rtol=2 ** -23)
    assert h[1] == 0.0                                            # ln 1 = 0
    # large |x|: silu -> x and -> -0
    h2 = stage2.silu_mul(np.array([[200.0, -200.0, 1.0, 1.0]], np.float32))[0]
    assert h2[0] == np.float32(200.0) and h2[1] == 0.0 and np.signbit(h2[1])


def test_silu_odd_part_and_torch():
    rng = np.random.default_rng(5)
    g = (rng.standard_normal((16, 256)) * 4).astype(np.float32)
    u = np.ones_like(g)
    h = stage2.silu_mul(np.concatenate([g, u], 1)).astype(np.float64)
    hn = stage2.silu_mul(np.concatenate([-g, u], 1)).astype(np.float64)
    # silu(x) - silu(-x) = x (sigma(x) + sigma(-x) = 1), up to the two fp32 roundings
    np.testing.assert_allclose(h - hn, g.astype(np.float64), rtol=0, atol=4 * 2 ** -24 * 16)
    t = torch.nn.functional.silu(torch.from_numpy(g.astype(np.float64))).numpy()
    np.testing.assert_allclose(h, t, rtol=2 ** -23, atol=1e-30)


def test_act_quant_is_quant_of_silu_mul():
    rng = np.random.default_rng(6)
    y = bf16.from_f32((rng.standard_normal((9, 512)) * 1.7).astype(np.float32))
    q2, s2 = stage2.act_quant(y)
    h = stage2.silu_mul(bf16.to_f32(y))
    q, s = quant.quantise_rows(h)
    assert np.array_equal(q2, q) and np.array_equal(s2.view(np.uint32), s.view(np.uint32))
    # every block's amax element codes to +-448 (the quant rule's invariant)
    dec = np.abs(fp8.decode(q2).astype(np.float64)).reshape(9, 2, 128)
    assert np.all(dec.max(axis=2) == 448.0)


def _weights(rng, L, H, I):
    wf = (rng.standard_normal((L, H, I)) * 0.05).astype(np.float32)
    sc = (np.abs(wf).reshape(L, H // 128, 128, I // 128, 128).max(axis=(2, 4)) / np.float32(448)).astype(np.float32)
    v = wf / np.repeat(np.repeat(sc, 128, 1), 128, 2)
    wq = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return wq, sc


def test_gemm2_matches_float64_triple_loop():
    rng = np.random.default_rng(7)
    L, H, I, R = 2, 128, 128, 6
    offs = np.array([0, 2, 6])
    y1 = bf16.from_f32((rng.standard_normal((R, 2 * I)) * 1.7).astype(np.float32))
    q2, s2 = stage2.act_quant(y1)
    w2, w2s = _weights(rng, L, H, I)
    T, k = 4, 2
    topk_w = rng.uniform(0.05, 1.0, (T, k)).astype(np.float32)
    row_assign = np.array([3, 0, 6, 1, 5, 2])
    y2 = stage2.grouped_gemm2(q2, s2, offs, row_assign, topk_w, w2, w2s)
    for r in range(R):
        le = 0 if r < 2 else 1
        wr = float(topk_w.reshape(-1)[row_assign[r]])
        for c in range(0, H, 7):
            acc = 0.0
            for i in range(I):
                a = float(fp8.decode(q2[r, i])) * float(s2[r, i // 128])
                b = float(fp8.decode(w2[le, c, i])) * float(w2s[le, c // 128, i // 128])
                acc += a * b
            assert math.isclose(y2[r, c], wr * acc, rel_tol=1e-5, abs_tol=1e-6 * max(1.0, abs(acc)))


def test_gemm2_identity_weights_and_routing_weight():
    rng = np.random.default_rng(8)
    I = H = 256
    R = 5
    y1 = bf16.from_f32((rng.standard_normal((R, 2 * I)) * 2).astype(np.float32))
    q2, s2 = stage2.act_quant(y1)
    w2 = np.where(np.eye(H, dtype=bool), np.uint8(0x38), np.uint8(0))[None]
    w2s = np.ones((1, H // 128, I // 128), np.float32)
    topk_w = np.array([0.5, 0.25, 1.0, 2.0 ** -5, 0.125], np.float32)
    y2 = stage2.grouped_gemm2(q2, s2, np.array([0, R]), np.arange(R), topk_w, w2, w2s)
    from oracle import gemm1
    A = gemm1.dequant_rows(q2, s2)
    assert np.array_equal(y2, A * topk_w[:, None])              # powers of two: exact


def test_gemm2_sampled_rows_with_compact_operands():
    rng = np.random.default_rng(9)
    L, H, I = 3, 128, 256
    offs = np.array([0, 4, 4, 9])
    y1 = bf16.from_f32(rng.standard_normal((9, 2 * I)).astype(np.float32))
    q2, s2 = stage2.act_quant(y1)
    w2, w2s = _weights(rng, L, H, I)
    tw = rng.uniform(0, 1, 20).astype(np.float32)
    ra = rng.permutation(20)[:9]
    full = stage2.grouped_gemm2(q2, s2, offs, ra, tw, w2, w2s)
    rows = np.array([1, 5, 8])
    part = stage2.grouped_gemm2(q2[rows], s2[rows], offs, ra, tw, w2, w2s, rows=rows, q_index=np.arange(3))
    # the same sums; BLAS may block a row subset differently, so compare to fp32 rounding
    np.testing.assert_allclose(part, full[rows], rtol=1e-5, atol=1e-6)


def test_combine_rows_is_the_unweighted_sum_brute_force():
    rng = np.random.default_rng(10)
    T, k, H = 7, 3, 128
    y2 = bf16.from_f32(rng.standard_normal((12, H)).astype(np.float32))
    ar = np.full(T * k, -1, np.int64)
    ar[rng.permutation(T * k)[:12]] = np.arange(12)
    acc, out = stage2.combine_rows(y2, ar, T, k)
    for g in range(T):
        want = np.zeros(H, np.float64)
        for j in range(k):
            r = ar[g * k + j]
            if r >= 0:
                want += bf16.to_f32(y2[r]).astype(np.float64)
        np.testing.assert_allclose(acc[g], want, rtol=1e-6, atol=1e-6)


def test_act_quant_mx_is_mx_quant_of_silu_mul():
    rng = np.random.default_rng(11)
    y = bf16.from_f32((rng.standard_normal((7, 256)) * 1.7).astype(np.float32))
    q2, s2 = stage2.act_quant_mx(y)
    q, s = mx.quantise_rows(stage2.silu_mul(bf16.to_f32(y)))
    assert np.array_equal(q2, q) and np.array_equal(s2, s)
    assert s2.dtype == np.uint32 and s2.shape == (7, 1)          # I = 128: one packed dword a row


def test_gemm2_mx_matches_float64_triple_loop():
    rng = np.random.default_rng(12)
    L, H, I, R = 2, 128, 128, 5
    offs = np.array([0, 3, 5])
    y1 = bf16.from_f32((rng.standard_normal((R, 2 * I)) * 1.7).astype(np.float32))
    q2, s2 = stage2.act_quant_mx(y1)
    wf = bf16.to_f32(bf16.from_f32((rng.standard_normal((L * H, I)) * 0.02).astype(np.float32)))
    wq, wsc = mx.quantise_rows(wf)
    w2 = wq.reshape(L, H, I)
    w2s = np.ascontiguousarray(wsc.reshape(L, H, I // 128).transpose(0, 2, 1))
    T, k = 3, 2
    topk_w = rng.uniform(0.05, 1.0, (T, k)).astype(np.float32)
    row_assign = np.array([5, 2, 0, 4, 1])
    y2 = stage2.grouped_gemm2_mx(q2, s2, offs, row_assign, topk_w, w2, w2s)
    codes_a = mx.unpack_codes(s2).astype(int) - 127
    for r in range(R):
        le = 0 if r < 3 else 1
        wr = float(topk_w.reshape(-1)[row_assign[r]])
        codes_b = mx.unpack_codes(w2s[le].T).astype(int) - 127          # [H, I/32]
        for c in range(0, H, 9):
            acc = 0.0
            for i in range(I):
                a = float(fp8.decode(q2[r, i])) * 2.0 ** codes_a[r, i // 32]
                b = float(fp8.decode(w2[le, c, i])) * 2.0 ** codes_b[c, i // 32]
                acc += a * b
            assert math.isclose(y2[r, c], wr * acc, rel_tol=1e-5, abs_tol=1e-6 * max(1.0, abs(acc)))


def test_generated_gemm2_weights_follow_the_rules():
    """workloads.weights2 (fp32 block scales) and weights2_mx (e8m0 groups) against
    the oracle's own quantisers applied to the same bf16 draws."""
    import workloads
    w = workloads.get("tiny_t64_h256_e8")
    I = w.N // 2
    wq, ws = workloads.weights2(w, experts=range(2))
    mq, ms = workloads.weights2_mx(w, experts=range(2))
    for i in range(2):
        g = np.random.default_rng(np.random.SeedSequence(w.seed).spawn(6)[4].spawn(w.L)[i])
        wf = g.standard_normal(size=(w.H, I), dtype=np.float32) * np.float32(0.02)
        wf = bf16.to_f32(bf16.from_f32(wf))
        q, sc = mx.quantise_rows(wf)
        assert np.array_equal(mq[i], q) and np.array_equal(ms[i], sc.T)
        # fp32 128x128 block scales: scale = block |max| / 448, payload decodes within half a step
        blk = np.abs(wf).reshape(w.H // 128, 128, I // 128, 128).max(axis=(1, 3)) / np.float32(448)
        assert np.array_equal(ws[i], blk.astype(np.float32))
        deq = fp8.decode(wq[i]).astype(np.float64) * np.repeat(np.repeat(ws[i], 128, 0), 128, 1)
        assert np.all(np.abs(deq - wf) <= np.abs(wf) * 2.0 ** -4 + np.repeat(np.repeat(ws[i], 128, 0), 128, 1) * 2.0 ** -10)
