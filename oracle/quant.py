"""Quant step: per-landed-token fp8 e4m3 quantisation with 1x128 block scales.

TEST INFRASTRUCTURE (see the package docstring).

"poc(cco): MegaMoE stage1 dispatch over SDMA", commit 2: each token's bf16 row
is read and quantised once and stored to every place it is needed; "How it
works now" (prepare): the quant writes each row once.  Here that place is the
token's compact slot in the receive layout (the layout step's slot_tok).

Block format (the pages' own runs use e8m0 scales; this library uses the
stated fp32 form): blocks of 128 consecutive hidden elements of one row; for
block b of slot u, holding token g = slot_tok[u]:
  a = max_i |x[g, 128b+i]|            (fp32; exact, bf16 is a subset of fp32)
  s = a / 448                          (IEEE fp32 division, round to nearest even)
  a == 0: s = 0 and the 128 bytes are 0x00
  else:   q[u, 128b+i] = e4m3(fl32(x / s)), x / s an IEEE fp32 division
q_scale[u, b] = s.  The plain reading of "scale = amax / 448" is a true
division, not a multiply by a reciprocal.
"""
from __future__ import annotations

import numpy as np

from . import bf16, fp8

BLOCK = 128


def quantise_rows(x_f32: np.ndarray):
    """x_f32 [n, H] float32 -> (q uint8 [n, H], scale float32 [n, H/128])."""
    x = np.asarray(x_f32, dtype=np.float32)
    n, H = x.shape
    assert H % BLOCK == 0
    blocks = x.reshape(n, H // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=2) if n else np.zeros((0, H // BLOCK), np.float32)
    s = (amax / np.float32(448.0)).astype(np.float32)
    nz = s != 0
    safe = np.where(nz, s, np.float32(1.0)).astype(np.float32)
    v = (blocks / safe[:, :, None]).astype(np.float32)
    q = fp8.encode(v)
    q = np.where(nz[:, :, None], q, np.uint8(0)).astype(np.uint8)
    return q.reshape(n, H), s


def quant_dispatch(x_bf16_bits, slot_tok, slots=None):
    """Quantise the landed tokens' rows into their slots.

    x_bf16_bits: uint16 [T, H]; slot_tok: int32 [U].  ``slots`` optionally
    restricts the work to a subset of slot indices (for sampled checks).
    Returns (q uint8 [n, H], q_scale float32 [n, H/128]) for the slots taken.
    """
    slot_tok = np.asarray(slot_tok)
    idx = np.arange(slot_tok.size) if slots is None else np.asarray(slots)
    rows = np.asarray(x_bf16_bits)[slot_tok[idx]]
    return quantise_rows(bf16.to_f32(rows))
