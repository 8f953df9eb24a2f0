"""Pins for the oracle's OCP E4M3 encoder/decoder (CPU only).

The expected values come from the format's definition (1 sign, 4 exponent
bits with bias 7, 3 mantissa bits, subnormals m*2^-9, 0x7F/0xFF NaN, largest
finite 448) and from torch's float8_e4m3fn casts, an implementation that shares
nothing with the oracle.
"""
import numpy as np
import pytest
import torch

from oracle import fp8

# (value, code) pairs derived by hand from the format definition.
KNOWN = [
    (0.0, 0x00), (-0.0, 0x80),
    (1.0, 0x38),                    # exponent field 7, mantissa 0
    (0.5, 0x30), (2.0, 0x40),
    (448.0, 0x7E), (-448.0, 0xFE),  # 1.75 * 2^8, the largest finite
    (240.0, 0x77),                  # 1.875 * 2^7
    (2.0 ** -6, 0x08),              # smallest normal
    (2.0 ** -9, 0x01),              # smallest subnormal
    (7 * 2.0 ** -9, 0x07),          # largest subnormal
    (2.0 ** -10, 0x00),             # tie between 0 and 2^-9 -> even (0)
    (-(2.0 ** -10), 0x80),          # ... keeps its sign
    (3 * 2.0 ** -10, 0x02),         # tie between 1 and 2 (x 2^-9) -> even (2)
    (15 * 2.0 ** -10, 0x08),        # tie between 7*2^-9 and 2^-6 -> even (2^-6)
    (1.0625, 0x38),                 # tie between 1.0 (m=0) and 1.125 (m=1) -> m=0
    (1.1875, 0x3A),                 # tie between 1.125 (m=1) and 1.25 (m=2) -> m=2
    (1.9375, 0x40),                 # tie between 1.875 (m=7) and 2.0 -> 2.0 (carry)
    (0.1, 0x1D),                    # 1.6 * 2^-4 -> 1.625 * 2^-4
    (3.3, 0x45),                    # 1.65 * 2 -> 1.625 * 2
    (464.0, 0x7E),                  # tie between 448 and 480 (not finite) -> 448
    (465.0, 0x7E), (1e30, 0x7E), (-1e30, 0xFE),   # saturation
    (-1e-30, 0x80),                 # rounds to zero, sign kept
]


@pytest.mark.parametrize("v,code", KNOWN)
def test_known_values(v, code):
    assert int(fp8.encode(np.float32(v))) == code


def _torch_encode(v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(v32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_every_bf16_pattern_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    v = bits.view(np.float32)
    ok = np.isfinite(v) & (np.abs(v) < 464.0)
    v = v[ok]
    np.testing.assert_array_equal(fp8.encode(v), _torch_encode(v))


def _midpoints() -> np.ndarray:
    finite = fp8.decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)   # 0 .. 448
    mids = (finite[:-1] + finite[1:]) / 2.0
    return np.concatenate([mids, -mids]).astype(np.float32)


def test_midpoints_and_neighbours_match_torch():
    m = _midpoints()
    below = np.nextafter(m, np.float32(0.0))
    above = np.nextafter(m, np.float32(np.copysign(np.inf, 1.0)) * np.sign(m))
    v = np.concatenate([m, below, above]).astype(np.float32)
    v = v[np.abs(v) < 464.0]
    np.testing.assert_array_equal(fp8.encode(v), _torch_encode(v))


def test_random_fp32_matches_torch():
    rng = np.random.default_rng(1234)
    v = (rng.standard_normal(200_000) * np.exp2(rng.uniform(-14, 8.8, 200_000))).astype(np.float32)
    v = v[np.abs(v) < 464.0]
    np.testing.assert_array_equal(fp8.encode(v), _torch_encode(v))


def test_saturation_above_464():
    v = np.array([464.0001, 479.9, 480.0, 481.0, 1e4, 3.0e38], dtype=np.float32)
    assert (fp8.encode(v) == 0x7E).all()
    assert (fp8.encode(-v) == 0xFE).all()


def test_decode_matches_torch_and_round_trips():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[fin], ref[fin])
    # every finite code is its own encoding (including 0x80 = -0)
    np.testing.assert_array_equal(fp8.encode(ours[fin]), codes[fin])
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
