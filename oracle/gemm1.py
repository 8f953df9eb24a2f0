"""GEMM1 step: grouped GEMM over the local experts, A rows read through the rowmap.

TEST INFRASTRUCTURE (see the package docstring).

"poc(cco): MegaMoE stage1 dispatch over SDMA", "What": GEMM1 reads its A rows
in place through a rowmap; commit 1: it reads the fp8 rows and their block
scales through the rowmap; "Where we stand": block-scaled fp8 tiles of one
expert at a time (do_tile).

Definition, for local expert le, expert-major row r in
[expert_offsets[le], expert_offsets[le+1]) and output column n < N:
  A[r, h]  = f32(e4m3(q[row_slot[r], h])) * q_scale[row_slot[r], h/128]
  B[le,n,h] = f32(e4m3(w[le, n, h]))      * w_scale[le, n/128, h/128]
  y[r, n]  = sum_h A[r, h] * B[le, n, h]
Dequantisation is a float32 product; the sum is a float32 matmul per expert
(a library primitive).  The result stays float32; the HIP path stores bf16 and
is compared within tolerance.
"""
from __future__ import annotations

import numpy as np

from . import fp8

BLOCK = 128


def dequant_rows(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """q uint8 [n, H], scale float32 [n, H/128] -> float32 [n, H]."""
    v = fp8.decode(q)
    n, H = v.shape
    return (v.reshape(n, H // BLOCK, BLOCK) * scale[:, :, None].astype(np.float32)).reshape(n, H)


def dequant_weight(w_e: np.ndarray, w_scale_e: np.ndarray) -> np.ndarray:
    """One expert's weight, uint8 [N, H] + float32 [N/128, H/128] -> float32 [N, H]."""
    v = fp8.decode(w_e)
    N, H = v.shape
    blk = v.reshape(N // BLOCK, BLOCK, H // BLOCK, BLOCK)
    return (blk * w_scale_e[:, None, :, None].astype(np.float32)).reshape(N, H)


def grouped_gemm1(q, q_scale, row_slot, expert_offsets, w, w_scale, rows=None) -> np.ndarray:
    """y float32 [R, N] (or [len(rows), N] for the listed expert-major rows).

    w: uint8 [L, N, H] (or a callable le -> (w_e, w_scale_e) so that callers can
    generate one expert at a time); w_scale: float32 [L, N/128, H/128].
    """
    offs = np.asarray(expert_offsets, dtype=np.int64)
    L = offs.size - 1
    R = int(offs[-1])
    rows = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    row_expert = np.searchsorted(offs, rows, side="right") - 1
    get_w = w if callable(w) else (lambda le: (w[le], w_scale[le]))
    out = None
    for le in range(L):
        sel = np.nonzero(row_expert == le)[0]
        if sel.size == 0:
            continue
        w_e, s_e = get_w(le)
        B = dequant_weight(np.asarray(w_e), np.asarray(s_e))
        slots = np.asarray(row_slot)[rows[sel]]
        A = dequant_rows(np.asarray(q)[slots], np.asarray(q_scale)[slots])
        y = A @ B.T                                     # float32 matmul
        if out is None:
            out = np.zeros((rows.size, B.shape[0]), dtype=np.float32)
        out[sel] = y
    if out is None:
        N = (w(0)[0].shape[0] if callable(w) else np.asarray(w).shape[1]) if L else 0
        out = np.zeros((rows.size, N), dtype=np.float32)
    return out
