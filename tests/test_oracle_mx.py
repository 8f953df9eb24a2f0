"""Pins for the oracle's MX-style quant and GEMM1 (CPU only): a scalar brute
force that finds each group's power of two by search (not by reading the
exponent), the bracketing invariant of the scale, exact round trips, the
packing order, special values, and a float64 triple loop for the GEMM."""
import math
import struct

import numpy as np
import pytest

import workloads
from oracle import bf16, fp8, mx


def f32(x: float) -> float:
    return struct.unpack("f", struct.pack("f", x))[0]


def brute_group(xs):
    """One group of 32 values -> (codes, e8m0 code) with scalar Python floats."""
    a = max(abs(v) for v in xs)
    if a == 0.0:
        return [0] * len(xs), 0
    t = f32(a / 448.0)
    E = -127
    while E < 127 and 2.0 ** E < t:          # smallest power of two >= t
        E += 1
    return [int(fp8.encode(np.float64(v * 2.0 ** -E))) for v in xs], E + 127


@pytest.mark.parametrize("seed", range(6))
def test_matches_scalar_brute_force(seed):
    rng = np.random.default_rng(seed)
    n, H = 3, 256
    x = (rng.standard_normal((n, H)) * np.exp2(rng.uniform(-30, 20, (n, H // 32)).repeat(32, 1))).astype(np.float32)
    x = bf16.to_f32(bf16.from_f32(x))
    x[1, 32:64] = 0.0                                  # a zero group
    x[2, 64:96] = -np.abs(x[2, 64:96])
    q, sc = mx.quantise_rows(x)
    codes = mx.unpack_codes(sc)
    for r in range(n):
        for g in range(H // 32):
            bq, bc = brute_group([float(v) for v in x[r, 32 * g:32 * g + 32]])
            assert codes[r, g] == bc, (r, g)
            assert list(q[r, 32 * g:32 * g + 32]) == bq, (r, g)


def test_scale_is_the_smallest_power_of_two_at_or_above_amax_over_448():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 128)) * np.exp2(rng.uniform(-40, 40, (64, 4)).repeat(32, 1))).astype(np.float32)
    x = bf16.to_f32(bf16.from_f32(x))
    q, sc = mx.quantise_rows(x)
    E = mx.unpack_codes(sc).astype(np.int64) - 127
    a = np.abs(x.reshape(64, 4, 32)).max(axis=2).astype(np.float64)
    t = np.array([[f32(v / 448.0) for v in row] for row in a])
    assert np.all(np.ldexp(1.0, E) >= t) and np.all(np.ldexp(1.0, E - 1) < t)
    # nothing saturates: every payload decodes to at most 448, and the group's
    # amax element keeps at least 224 (the scale was rounded up by < 2x)
    dec = np.abs(fp8.decode(q).astype(np.float64)).reshape(64, 4, 32)
    assert dec.max() <= 448.0
    assert np.all(dec.max(axis=2) >= 224.0)


def test_round_trip_within_half_an_e4m3_ulp():
    rng = np.random.default_rng(8)
    x = bf16.to_f32(bf16.from_f32(rng.standard_normal((16, 256)).astype(np.float32)))
    q, sc = mx.quantise_rows(x)
    back = mx.dequant_rows(q, sc).astype(np.float64)
    E = (mx.unpack_codes(sc).astype(np.int64) - 127).repeat(32, 1)
    v = np.abs(x.astype(np.float64)) * np.ldexp(1.0, -E)
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
    half_ulp = np.ldexp(1.0, (e - 4).astype(np.int64)) * np.ldexp(1.0, E)   # 3 mantissa bits
    assert np.all(np.abs(back - x) <= half_ulp * (1 + 1e-12))


def test_special_values_and_packing():
    x = np.zeros((1, 128), np.float32)
    x[0, :32] = 448.0            # t = 1 exactly -> E = 0, payload 0x7E
    x[0, 32] = 449.0             # t just above 1 -> E = 1 (449/2 = 224.5 -> 224)
    x[0, 33] = -1.0
    x[0, 64:96] = 0.0            # zero group -> code 0
    x[0, 96] = 2.0 ** -100       # tiny group: E = ceil(log2(2^-100 / 448)) = -108
    q, sc = mx.quantise_rows(x)
    codes = mx.unpack_codes(sc)[0]
    assert list(codes) == [127, 128, 0, 127 - 108]
    assert q[0, 0] == 0x7E and q[0, 32] == fp8.encode(np.float64(224.0))
    assert q[0, 33] == fp8.encode(np.float64(-0.5))
    assert not q[0, 64:96].any()
    assert int(sc[0, 0]) == (127 | 128 << 8 | 0 << 16 | 19 << 24)
    assert np.array_equal(mx.unpack_codes(mx.pack_codes(codes[None])), codes[None])


def test_generated_mx_weights_follow_the_rule():
    w = workloads.get("tiny_t64_h256_e8")
    wq, ws = workloads.weights_mx(w, experts=range(2))
    # the same bf16 weights through the oracle's quantiser, per column (rows of [N, H])
    for i in range(2):
        g = np.random.default_rng(np.random.SeedSequence(w.seed).spawn(4)[2].spawn(w.L)[i])
        wf = g.standard_normal(size=(w.N, w.H), dtype=np.float32) * np.float32(0.02)
        wf = bf16.to_f32(bf16.from_f32(wf))
        q, sc = mx.quantise_rows(wf)
        assert np.array_equal(wq[i], q)
        assert np.array_equal(ws[i], sc.T)            # stored K-block-major [H/128, N]


def test_gemm1_matches_float64_triple_loop():
    rng = np.random.default_rng(9)
    L, N, H, S = 2, 8, 128, 5
    x = bf16.to_f32(bf16.from_f32((rng.standard_normal((S, H)) * 3).astype(np.float32)))
    q, qs = mx.quantise_rows(x)
    wq = np.stack([mx.quantise_rows(bf16.to_f32(bf16.from_f32(rng.standard_normal((N, H)).astype(np.float32))))[0]
                   for _ in range(L)])
    wsc = np.stack([mx.quantise_rows(bf16.to_f32(bf16.from_f32(rng.standard_normal((N, H)).astype(np.float32))))[1].T
                    for _ in range(L)])
    offs = np.array([0, 3, 7])
    row_slot = np.array([4, 0, 2, 1, 1, 3, 0])
    y = mx.grouped_gemm1(q, qs, row_slot, offs, wq, wsc)
    for r in range(7):
        le = 0 if r < 3 else 1
        s = row_slot[r]
        ea = mx.unpack_codes(qs[s]).astype(int) - 127
        eb = mx.unpack_codes(wsc[le].T).astype(int) - 127
        for n in range(N):
            acc = 0.0
            for h in range(H):
                acc += (float(fp8.decode(q[s, h])) * 2.0 ** ea[h // 32]) * \
                       (float(fp8.decode(wq[le, n, h])) * 2.0 ** eb[n, h // 32])
            assert math.isclose(y[r, n], acc, rel_tol=1e-5, abs_tol=1e-6 * max(1.0, abs(acc)))


def test_gemm1_identity_weights_give_the_dequantised_rows():
    rng = np.random.default_rng(10)
    H = 128
    x = bf16.to_f32(bf16.from_f32(rng.standard_normal((4, H)).astype(np.float32)))
    q, qs = mx.quantise_rows(x)
    wq = np.zeros((1, H, H), np.uint8)
    wq[0][np.arange(H), np.arange(H)] = 0x38              # 1.0
    wsc = np.full((1, 1, H), 127 | 127 << 8 | 127 << 16 | 127 << 24, np.uint32)
    y = mx.grouped_gemm1(q, qs, np.arange(4), np.array([0, 4]), wq, wsc)
    assert np.array_equal(y, mx.dequant_rows(q, qs))
