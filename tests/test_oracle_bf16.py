"""Pins for the oracle's bf16 rounding (CPU only): torch's bf16 cast is an
independent round-to-nearest-even implementation."""
import numpy as np
import torch

from oracle import bf16


def _torch_bits(x):
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_known_values():
    x = np.array([1.0, -2.0, 0.0, -0.0, 1.0 + 2**-7, 1.0 + 2**-8, 1.0 + 3 * 2**-8,
                  1.0 + 2**-8 + 2**-20, 1.0 + 2**-9], dtype=np.float32)
    # bf16 keeps 7 fraction bits: 1+2^-7 is a bf16 value; 1+2^-8 ties to 1.0 (even);
    # 1+3*2^-8 ties up to 1+2^-6 (even); just above a tie rounds up; 1+2^-9 rounds down.
    exp = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3F81, 0x3F80, 0x3F82, 0x3F81, 0x3F80],
                   np.uint16)
    np.testing.assert_array_equal(bf16.from_f32(x), exp)


def test_random_matches_torch():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(300_000) * np.exp2(rng.uniform(-60, 60, 300_000))).astype(np.float32)
    # ties: values exactly halfway between bf16 neighbours
    base = rng.integers(0, 1 << 15, 50_000).astype(np.uint32) << np.uint32(16)
    ties = (base | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    x = x[np.isfinite(x) & (np.abs(x) < 3e38)]
    np.testing.assert_array_equal(bf16.from_f32(x), _torch_bits(x))


def test_to_f32_round_trip():
    bits = np.arange(1 << 16, dtype=np.uint16)
    f = bf16.to_f32(bits)
    fin = np.isfinite(f)
    np.testing.assert_array_equal(bf16.from_f32(f[fin]), bits[fin])
