"""Pins for the oracle's quant step (CPU only): an element-by-element brute
force using Python floats, invariants of amax/448 block scaling, and the
half-ulp round-trip bound."""
import struct

import numpy as np
import pytest

import workloads
from oracle import bf16, fp8, layout, quant


def f32(x: float) -> float:
    """Round a Python float (fp64) to the nearest fp32 (ties to even)."""
    return struct.unpack("f", struct.pack("f", x))[0]


def brute_force_block(xs):
    """One block of 128 fp32 values -> (codes, scale) with scalar Python floats.
    fp32 division = fp32(fp64 quotient): double rounding is harmless for a
    quotient when the wide format has >= 2p+2 bits (53 >= 50)."""
    a = max(abs(v) for v in xs)
    s = f32(a / 448.0)
    if a == 0.0:
        return [0] * len(xs), 0.0
    codes = []
    for v in xs:
        q = f32(v / s)
        codes.append(int(fp8.encode(np.float64(q))))
    return codes, s


@pytest.mark.parametrize("seed", range(6))
def test_matches_scalar_brute_force(seed):
    rng = np.random.default_rng(seed)
    n, H = 3, 256
    x = (rng.standard_normal((n, H)) * np.exp2(rng.uniform(-20, 10, (n, 1)))).astype(np.float32)
    x = bf16.to_f32(bf16.from_f32(x))
    x[1, 128:] = 0.0                                  # a zero block
    x[2, :128] = -x[2, :128]
    q, s = quant.quantise_rows(x)
    for i in range(n):
        for b in range(H // 128):
            codes, sc = brute_force_block([float(v) for v in x[i, 128 * b:128 * (b + 1)]])
            assert np.float32(sc) == s[i, b]
            assert list(q[i, 128 * b:128 * (b + 1)]) == codes


def test_amax_element_encodes_to_448_and_bound():
    rng = np.random.default_rng(3)
    x = bf16.to_f32(bf16.from_f32(rng.standard_normal((64, 1024)).astype(np.float32)))
    q, s = quant.quantise_rows(x)
    blocks = x.reshape(64, 8, 128)
    qb = q.reshape(64, 8, 128)
    am = np.abs(blocks).argmax(axis=2)
    top = np.take_along_axis(qb, am[:, :, None], axis=2)[..., 0]
    sgn = np.take_along_axis(blocks, am[:, :, None], axis=2)[..., 0] < 0
    np.testing.assert_array_equal(top, np.where(sgn, 0xFE, 0x7E))
    # |q| <= 448 and no NaN code
    assert not np.isin(q, [0x7F, 0xFF]).any()
    # half-ulp bound: |f32(q)*s - x| <= 0.5*ulp_e4m3(v)*s*(1+2^-20)
    v = fp8.decode(q).astype(np.float64).reshape(64, 8, 128)
    sd = s.astype(np.float64)[:, :, None]
    xv = blocks.astype(np.float64) / sd
    e = np.floor(np.log2(np.maximum(np.abs(xv), 2.0 ** -6)))
    ulp = np.exp2(e - 3)
    err = np.abs(v * sd - blocks)
    assert (err <= 0.5 * ulp * sd * (1 + 2.0 ** -20)).all()


def test_zero_and_tiny_blocks():
    x = np.zeros((2, 256), np.float32)
    x[1, 5] = -2.0 ** -100                 # one tiny element: amax scale still normal fp32
    q, s = quant.quantise_rows(x)
    assert (q[0] == 0).all() and (s[0] == 0).all()
    assert q[1, 5] == 0xFE and (np.delete(q[1, :128], 5) == 0x00).all()
    assert s[1, 1] == 0 and (q[1, 128:] == 0).all()


def test_dispatch_reads_only_landed_tokens():
    w = workloads.get("tiny_t64_h256_e8")
    ids, _ = workloads.routing(w)
    x = workloads.activations(w)
    lay = layout.route_layout(ids, w.S, w.Ts, w.k, w.e0, w.L)
    q, s = quant.quant_dispatch(x, lay["slot_tok"])
    q2, s2 = quant.quantise_rows(bf16.to_f32(x[lay["slot_tok"]]))
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(s, s2)
    # sampled slot subset equals the rows of the full result
    qs, ss = quant.quant_dispatch(x, lay["slot_tok"], slots=[3, 0, 17])
    np.testing.assert_array_equal(qs, q[[3, 0, 17]])
