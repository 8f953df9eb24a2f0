"""Host checks of the arithmetic identities the fp8 block encoder of the HIP
path relies on to reach the IEEE-division definition of the block scale
without dividing (the kernels' own bytes are compared with the oracle by the
GPU tests; these tests pin the identities themselves, on the CPU).

Identity 1: for c = fl32(1/448), s0 = fl32(a * c), rem = a - 448 * s0 (exact in
fp32) and s = fl32(rem * c + s0) (one rounding, as a fused multiply-add),
s equals the IEEE quotient fl32(a / 448) for every normal a >= 2^-100.

Identity 2: r_hi = fl32(r * (1 + 2^-20)) and r_lo = fl32(r * (1 - 2^-20))
bracket 1/s whenever r is within 2^-22 of 1/s relatively.
"""
from fractions import Fraction

import numpy as np

C = np.float32(1.0) / np.float32(448.0)


def _rn32(fr: Fraction) -> np.float32:
    """Round a rational to the nearest float32, ties to even (normal range)."""
    x = np.float32(float(fr))
    best = None
    for v in (np.nextafter(x, np.float32(-np.inf)), x, np.nextafter(x, np.float32(np.inf))):
        key = (abs(Fraction(float(v)) - fr), int(np.array(v).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return best[1]


def _fma_div448_f64(a: np.ndarray) -> np.ndarray:
    s0 = (a * C).astype(np.float32)
    rem64 = a.astype(np.float64) - s0.astype(np.float64) * 448.0      # exact in float64
    rem = rem64.astype(np.float32)
    assert np.array_equal(rem.astype(np.float64), rem64), "residual not exact in fp32"
    t = rem.astype(np.float64) * np.float64(C) + s0.astype(np.float64)
    return s0, rem, t


def test_fma_corrected_division_by_448_every_mantissa():
    """Every fp32 mantissa of the binade [1, 2): the quotient's rounding depends
    only on the mantissa while no intermediate is subnormal, so this covers
    every binade down to 2^-100."""
    m = np.arange(1 << 23, 1 << 24, dtype=np.uint32)
    a = (m.astype(np.float64) * 2.0 ** -23).astype(np.float32)
    q = a / np.float32(448.0)                                            # IEEE float32 division
    s0, rem, t = _fma_div448_f64(a)
    # t = rem*c + s0 in float64 may itself be rounded; where it lies near an fp32
    # rounding midpoint, redo the single rounding exactly
    low = t.view(np.uint64) & np.uint64((1 << 29) - 1)
    near = np.abs(low.astype(np.int64) - (1 << 28)) <= 4
    s = t.astype(np.float32)
    for i in np.nonzero(near)[0]:
        s[i] = _rn32(Fraction(float(rem[i])) * Fraction(float(C)) + Fraction(float(s0[i])))
    assert np.array_equal(s, q)
    # the plain product alone would not do
    assert not np.array_equal((a * C).astype(np.float32), q)


def test_fma_corrected_division_by_448_every_bf16_amax_exactly():
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint32) << 16
    a_all = bits.view(np.float32)
    a_all = a_all[a_all >= np.float32(2.0 ** -100)]
    q = a_all / np.float32(448.0)
    for a, want in zip(a_all[::7], q[::7]):                              # every 7th, exactly
        A = Fraction(float(a))
        s0 = np.float32(a * C)
        rem = _rn32(A - Fraction(float(s0)) * 448) if A != Fraction(float(s0)) * 448 else np.float32(0)
        assert Fraction(float(rem)) == A - Fraction(float(s0)) * 448      # the residual is exact
        assert _rn32(Fraction(float(rem)) * Fraction(float(C)) + Fraction(float(s0))) == want
    s0, rem, t = _fma_div448_f64(a_all)                                 # and all of them in float64
    assert np.array_equal(t.astype(np.float32), q)


def test_reciprocal_bracket_holds_for_a_few_ulps_of_error():
    rng = np.random.default_rng(5)
    s = (rng.uniform(1.0, 2.0, 200_000) * 2.0 ** rng.integers(-100, 100, 200_000)).astype(np.float32)
    inv = 1.0 / s.astype(np.float64)
    for rel in (-2.0 ** -22, -2.0 ** -23, 0.0, 2.0 ** -23, 2.0 ** -22):
        r = (inv * (1.0 + rel)).astype(np.float32)
        r_hi = (r * np.float32(1.0 + 2.0 ** -20)).astype(np.float32)
        r_lo = (r * np.float32(1.0 - 2.0 ** -20)).astype(np.float32)
        assert np.all(r_lo.astype(np.float64) <= inv) and np.all(r_hi.astype(np.float64) >= inv)
