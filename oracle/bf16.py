"""bf16 <-> fp32.

TEST INFRASTRUCTURE (see the package docstring).

bf16 is fp32 with the low 16 bits of the encoding dropped.  fp32 -> bf16 rounds
to the nearest bf16 value, ties to the one whose last kept bit is 0 (even).
Written as the plain definition: take the two neighbouring bf16 values and pick
the nearer, in float64 (exact for these operands).  Inputs are finite and do
not overflow.
"""
from __future__ import annotations

import numpy as np


def to_f32(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def from_f32(x) -> np.ndarray:
    """float32 -> bf16 bits (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lo_bits = u & np.uint32(0xFFFF0000)                 # truncation toward zero
    lo = lo_bits.view(np.float32).astype(np.float64)
    hi_bits = lo_bits + np.uint32(0x10000)              # next bf16 away from zero
    hi = hi_bits.view(np.float32).astype(np.float64)
    xd = x.astype(np.float64)
    d_lo = np.abs(xd - lo)
    d_hi = np.abs(hi - xd)
    lo_even = ((lo_bits >> np.uint32(16)) & np.uint32(1)) == 0
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~lo_even)
    pick_hi &= d_lo != 0                                # exactly representable: keep it
    out = np.where(pick_hi, hi_bits, lo_bits) >> np.uint32(16)
    return out.astype(np.uint16)
