"""Host checks of the arithmetic identities the fp8 block encoder of the HIP
path relies on to reach the IEEE-division definitions of the block scale and
of the scaled values without dividing (the kernels' own bytes are compared
with the oracle by the GPU tests; these tests pin the identities themselves,
on the CPU).

Identity 1: for c = fl32(1/448), s0 = fl32(a * c), rem = a - 448 * s0 (exact in
fp32) and s = fl32(rem * c + s0) (one rounding, as a fused multiply-add),
s equals the IEEE quotient fl32(a / 448) for every normal a >= 2^-100.

Identity 2: two fp64 Newton steps R <- fma(R, fma(-s, R, 1), R) from an fp32
reciprocal within 2^-20 of 1/s leave |R s - 1| <= 2^-51.

Identity 3: for such R, fl32(fl64(x * R)) is the IEEE quotient fl32(x / s) for
every fp32 x whose quotient is a normal fp32 number (x / s never lies within
2^-49 of an fp32 rounding midpoint there), and both have the same e4m3 code for
every x (quotients below 2^-126 encode to a zero of x's sign either way).
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


def _fma64(a: float, b: float, c: float) -> float:
    """fp64 fused multiply-add: one rounding of the exact a*b + c (Python's
    int / int true division, which Fraction uses, is correctly rounded)."""
    return float(Fraction(a) * Fraction(b) + Fraction(c))


def test_two_fp64_newton_steps_reach_2_pow_minus_51():
    rng = np.random.default_rng(5)
    s = (rng.uniform(1.0, 2.0, 3000) * 2.0 ** rng.integers(-108, 100, 3000)).astype(np.float32)
    worst = Fraction(0)
    for si in s:
        S = Fraction(float(si))
        for rel in (-2.0 ** -20, -2.0 ** -23, 0.0, 2.0 ** -23, 2.0 ** -20):
            r = float(np.float32(float(1 / S) * (1.0 + rel)))          # the fp32 starting value
            R = r
            for _ in range(2):
                R = _fma64(R, _fma64(-float(si), R, 1.0), R)
            worst = max(worst, abs(Fraction(R) * S - 1))
    assert worst <= Fraction(1, 2 ** 51), float(worst)


def _check_quotients(x: np.ndarray, s: np.float32):
    """fl32(fl64(x * R)) == fl32(x / s) where the quotient is a normal fp32
    number, and equal e4m3 codes everywhere, for R = fl64(1/s) moved by up to
    4 ulps (|R s - 1| up to about 2^-51) in both directions."""
    from oracle import fp8
    want = x / s                                                           # IEEE float32 division
    normal = np.abs(want) >= np.float32(2.0 ** -126)
    want_code = fp8.encode(want)
    x64 = x.astype(np.float64)
    R = np.float64(1.0) / np.float64(s)
    for k in (-4, -1, 0, 1, 4):
        Rk = R
        for _ in range(abs(k)):
            Rk = np.nextafter(Rk, np.inf if k > 0 else -np.inf)
        got = (x64 * Rk).astype(np.float32)
        assert np.array_equal(got[normal].view(np.uint32), want[normal].view(np.uint32)), (float(s), k)
        assert np.array_equal(fp8.encode(got), want_code), (float(s), k)


def test_fp64_product_gives_the_ieee_quotient_every_bf16_value():
    """Every finite bf16 x against block maxima of all 128 bf16 mantissas in
    several binades (quotients from 448 down through the fp32 subnormals)."""
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    xs = bits.view(np.float32)
    xs = xs[np.isfinite(xs)]
    for e in (-100, -37, 0, 1, 40, 100, 127):
        for m in range(128):
            amax = np.float32((1.0 + m / 128.0) * 2.0 ** e)
            if not np.isfinite(amax):
                continue
            s = amax / np.float32(448.0)
            _check_quotients(xs[np.abs(xs) <= amax], s)


def test_fp64_product_gives_the_ieee_quotient_random_fp32():
    """fp32 x with full 24-bit significands (stage2's h values)."""
    rng = np.random.default_rng(11)
    for e in (-90, -3, 0, 17, 100):
        amax = np.float32(rng.uniform(1.0, 2.0) * 2.0 ** e)
        x = (rng.uniform(-1.0, 1.0, 400_000) * float(amax)).astype(np.float32)
        x = x[np.abs(x) <= amax]
        _check_quotients(x, amax / np.float32(448.0))


def test_bf16_quotients_often_fall_near_e4m3_midpoints():
    """Why the encoder computes the quotient to fp64 precision instead of
    bracketing it in fp32: with bf16 inputs, x / s lands within 2^-19
    (relative) of an e4m3 rounding midpoint far more often than random fp32
    values would (about 2^-15)."""
    from oracle import fp8
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((4000, 128))).astype(np.float32)
    x = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)       # bf16 values
    amax = np.abs(x).max(axis=1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    q = (x.astype(np.float64) / s.astype(np.float64)[:, None])
    hi = fp8.encode((q * (1 + 2.0 ** -20)).astype(np.float32))
    lo = fp8.encode((q * (1 - 2.0 ** -20)).astype(np.float32))
    assert (hi != lo).mean() > 2.0 ** -10
