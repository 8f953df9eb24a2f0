"""OCP FP8 E4M3 ("fn": finite, no infinities) encode / decode.

TEST INFRASTRUCTURE (see the package docstring).

The pages quantise activations and weights to fp8 ("poc(cco): MegaMoE stage1
dispatch over SDMA", commit 1: GEMM1 reads its fp8 A rows and block scales
through a rowmap).  The format itself is the OCP 8-bit floating point E4M3
variant: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
field 0 holds subnormals m * 2^-9; exponent field 15 with mantissa 7 is NaN and
there are no infinities, so the largest finite magnitude is 1.75 * 2^8 = 448.

Readings taken where the pages are silent: rounding is to nearest, ties to
even, on the 3-bit mantissa (also across the subnormal/normal boundary); a
rounded magnitude above 448 saturates to 448; the sign is kept for results
that round to zero (so -0 and tiny negatives give 0x80).  Inputs are finite.

Everything is evaluated in float64, where every step below is exact.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6


def encode(v) -> np.ndarray:
    """fp32 (or fp64) finite values -> e4m3 bytes (uint8)."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v)
    a = np.abs(v)
    code = np.zeros(a.shape, dtype=np.int64)

    # normal range: a = mant * 2^e with mant in [1, 2); keep 3 fraction bits.
    nrm = a >= _MIN_NORMAL
    m, ex = np.frexp(np.where(nrm, a, 1.0))        # a = m * 2^ex, m in [0.5, 1)
    e = ex.astype(np.int64) - 1
    r = np.rint(m * 16.0)                          # = mant * 8 in [8, 16], ties to even
    carry = r >= 16.0
    r = np.where(carry, 8.0, r)
    e = np.where(carry, e + 1, e)
    mag = ((e + 7) << 3) | (r.astype(np.int64) - 8)
    mag = np.where((e > 8) | ((e == 8) & (r >= 15.0)), 0x7E, mag)   # saturate at 448
    code = np.where(nrm, mag, code)

    # subnormal range: a < 2^-6, multiples of 2^-9; a count of 8 is 2^-6 = 0x08.
    sub = ~nrm
    q = np.rint(np.where(sub, a, 0.0) * 512.0).astype(np.int64)
    code = np.where(sub, q, code)

    code = code | np.where(sign, 0x80, 0)
    return code.astype(np.uint8)


def _decode_formula(c) -> np.ndarray:
    c = np.asarray(c, dtype=np.int64)
    s = np.where((c & 0x80) != 0, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    val = np.where(ef == 0, mf * 2.0 ** -9, (1.0 + mf / 8.0) * np.exp2(ef - 7.0))
    val = np.where((ef == 15) & (mf == 7), np.nan, val)
    return (s * val).astype(np.float32)


_TABLE = _decode_formula(np.arange(256))   # the formula above, evaluated once per code


def decode(c) -> np.ndarray:
    """e4m3 bytes -> float32 values (0x7F / 0xFF decode to NaN)."""
    c = np.asarray(c)
    if c.dtype == np.uint8:
        return _TABLE[c]
    return _decode_formula(c)
