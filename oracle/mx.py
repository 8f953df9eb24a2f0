"""MX-style quant and GEMM1: fp8 e4m3 payloads with power-of-two (e8m0) scales
per group of 32 consecutive K elements.

TEST INFRASTRUCTURE (see the package docstring).

"poc(cco): MegaMoE stage1 dispatch over SDMA": the pages' own stage1 runs use
e8m0 block scales ("Where we stand"), packed four per dword (commit
"ready-first / quant-lds-store"), i.e. four 32-element groups per dword.  The
pages fix neither the group's scale rule nor its packing order; the readings
taken here:
  * group = 32 consecutive hidden (K) elements of one row; a 128-element K
    block holds groups 4kb .. 4kb+3, and their four e8m0 codes are packed into
    one uint32, group 4kb+g in byte g (little-endian);
  * a = max |x| over the group (fp32; exact for bf16 inputs);
    a == 0: code 0 (2^-127, the smallest e8m0 value) and payload 0x00;
    else:   t = a / 448 (IEEE fp32 division) and E = ceil(log2 t), read off t's
            binary exponent exactly, clamped to [-127, 127]; code = E + 127;
            payload = e4m3(x * 2^-E): the scaling by a power of two is exact,
            |x| * 2^-E <= a * 2^-E <= 448, so the only rounding is the e4m3
            encode itself (round to nearest even) and nothing saturates.
    This is the scale that the block's amax needs, rounded up to a power of
    two (the fp32 path's amax/448 rounded up), so no element is clipped.
Dequantised value = f32(e4m3(payload)) * 2^E, exact in float32.

GEMM1 definition (same as the fp32-scale path with these operands): for local
expert le, row r and column n,
  y[r, n] = sum_h A[r, h] * B[le, n, h]
  A[r, h] = dequant(q[row_slot[r], h]),   B[le, n, h] = dequant(w[le, n, h]),
a float32 matmul per expert on the dequantised operands.  Weight scales are
per column n and K group, stored K-block-major: w_scale[le, kb, n] (uint32,
four packed codes, byte g = group 4kb+g of column n).
"""
from __future__ import annotations

import numpy as np

from . import bf16, fp8

GROUP = 32
KBLOCK = 128


def group_exponent(amax: np.ndarray) -> np.ndarray:
    """E = ceil(log2(amax / 448)) per group (int64), the fp32 quotient's exact
    binary exponent, clamped to [-127, 127]; amax == 0 gives -127."""
    a = np.asarray(amax, dtype=np.float32)
    t = (a / np.float32(448.0)).astype(np.float32)
    m, e = np.frexp(t.astype(np.float64))          # t = m * 2^e, m in [0.5, 1)
    E = np.where(m == 0.5, e - 1, e).astype(np.int64)   # a power of two: log2 t = e - 1
    E = np.where(a == 0, -127, E)
    return np.clip(E, -127, 127)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """codes uint8 [..., H/32] -> uint32 [..., H/128], group 4kb+g in byte g."""
    c = np.asarray(codes, dtype=np.uint32)
    c = c.reshape(*c.shape[:-1], c.shape[-1] // 4, 4)
    return (c[..., 0] | (c[..., 1] << 8) | (c[..., 2] << 16) | (c[..., 3] << 24)).astype(np.uint32)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """uint32 [..., H/128] -> codes uint8 [..., H/32]."""
    p = np.asarray(packed, dtype=np.uint32)
    c = np.stack([(p >> np.uint32(8 * g)) & np.uint32(0xFF) for g in range(4)], axis=-1)
    return c.reshape(*p.shape[:-1], p.shape[-1] * 4).astype(np.uint8)


def quantise_rows(x_f32: np.ndarray):
    """x_f32 [n, H] float32 -> (q uint8 [n, H], packed scale codes uint32 [n, H/128])."""
    x = np.asarray(x_f32, dtype=np.float32)
    n, H = x.shape
    assert H % KBLOCK == 0
    g = x.reshape(n, H // GROUP, GROUP)
    amax = np.abs(g).max(axis=2) if n else np.zeros((0, H // GROUP), np.float32)
    E = group_exponent(amax)                                   # [n, H/32]
    v = (g.astype(np.float64) * np.ldexp(1.0, -E)[:, :, None]).astype(np.float32)   # exact
    q = fp8.encode(v).reshape(n, H)
    q = np.where((amax == 0)[:, :, None].repeat(GROUP, 2).reshape(n, H), np.uint8(0), q).astype(np.uint8)
    return q, pack_codes((E + 127).astype(np.uint8))


def quant_dispatch(x_bf16_bits, slot_tok, slots=None):
    """MX quant of the landed tokens' rows into their slots (as quant.quant_dispatch)."""
    slot_tok = np.asarray(slot_tok)
    idx = np.arange(slot_tok.size) if slots is None else np.asarray(slots)
    rows = np.asarray(x_bf16_bits)[slot_tok[idx]]
    return quantise_rows(bf16.to_f32(rows))


def dequant_rows(q: np.ndarray, packed: np.ndarray) -> np.ndarray:
    """q uint8 [n, H], packed uint32 [n, H/128] -> float32 [n, H] (exact)."""
    v = fp8.decode(q).astype(np.float64)
    n, H = v.shape
    E = unpack_codes(packed).astype(np.int64) - 127
    return (v.reshape(n, H // GROUP, GROUP) * np.ldexp(1.0, E)[:, :, None]).reshape(n, H).astype(np.float32)


def dequant_weight(w_e: np.ndarray, w_scale_e: np.ndarray) -> np.ndarray:
    """One expert: uint8 [N, H] + packed uint32 [H/128, N] (K-block-major) -> float32 [N, H]."""
    return dequant_rows(w_e, np.ascontiguousarray(np.asarray(w_scale_e).T))


def grouped_gemm1(q, q_scale, row_slot, expert_offsets, w, w_scale, rows=None):
    """MX GEMM1 over the rows named (all rows when ``rows`` is None).

    q uint8 [S, H], q_scale uint32 [S, H/128]; row_slot [R] indexes q's rows;
    w uint8 [L, N, H], w_scale uint32 [L, H/128, N].  Returns float32 [len(rows), N].
    """
    offs = np.asarray(expert_offsets, dtype=np.int64)
    R = int(offs[-1])
    rows = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    N = w.shape[1]
    out = np.zeros((rows.size, N), np.float32)
    le_of = np.searchsorted(offs, rows, side="right") - 1
    for le in np.unique(le_of):
        sel = np.nonzero(le_of == le)[0]
        slots = np.asarray(row_slot)[rows[sel]]
        A = dequant_rows(np.asarray(q)[slots], np.asarray(q_scale)[slots])
        B = dequant_weight(w[le], w_scale[le])
        out[sel] = A @ B.T
    return out
