"""Stage2: SiLU(gate) * up on GEMM1's output, fp8 quantisation of the product,
the grouped down-projection GEMM2 with each row's routing weight, and the
combine of the weighted expert outputs.

TEST INFRASTRUCTURE (see the package docstring).

"poc(cco): MegaMoE stage1 dispatch over SDMA", "What": stage1 (quant,
dispatch, GEMM1) hands its expert-major output to an unchanged stage2 +
combine; commit "recv_layout": the receiver's layout also writes each row's
routing weight (its wts_em table) for stage2.  The pages do not state stage2's
arithmetic.  The readings taken (plain gated-MLP expert):
  * GEMM1's width is N = 2*I: columns [0, I) are the gate, [I, 2I) the up
    projection of the same row.
  * h[r, i] = silu(gate[r, i]) * up[r, i], silu(x) = x / (1 + exp(-x)), from
    the bf16 values of GEMM1's output; exact in real arithmetic, here in
    float64 and rounded once to float32 (the precision the kernels keep h in).
  * h is quantised with GEMM1's activation rule (oracle.quant: blocks of 128
    along I, fp32 scale = amax / 448, e4m3 of the IEEE quotient).
  * GEMM2 of local expert le: logical weight [I, H], stored K-contiguous as
    [L, H, I] bytes with one fp32 scale per 128(H) x 128(I) block;
      y2[r, c] = w_r * sum_i deq(q2[r, i]) * deq(w2[le, c, i]),  c < H,
    w_r = topk_w.flat[row_assign[r]] (the row's routing weight); float32.
  * MX variant (the pages' own e8m0 format, as oracle.mx): h quantised with
    power-of-two scales per 32 elements (oracle.mx.quantise_rows); GEMM2's
    weights likewise per column and group, codes stored [L, I/128, H]; the
    routing weight multiplies the float32 sum (it is not a power of two, so it
    cannot ride in an e8m0 code).
  * The combine then sums the weighted rows back per token:
      out[g, c] = sum_j y2[assign_row[g*k + j], c]  (local rows only),
    i.e. oracle.combine with unit weights: the share of each token's output
    that this GPU's experts produce, which an expert rank would send back.
"""
from __future__ import annotations

import numpy as np

from . import bf16, combine, gemm1, mx, quant


def silu_mul(y1_f32: np.ndarray) -> np.ndarray:
    """y1 float32 [n, 2I] -> h float32 [n, I] = silu(gate) * up."""
    y = np.asarray(y1_f32, dtype=np.float64)
    n, N = y.shape
    assert N % 2 == 0
    I = N // 2
    gate, up = y[:, :I], y[:, I:]
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-gate))          # exp overflow -> inf -> sigma 0
    return (gate * sig * up).astype(np.float32)


def act_quant(y1_bf16_bits: np.ndarray):
    """GEMM1 output rows (bf16 bits [n, 2I]) -> (q2 uint8 [n, I], s2 float32 [n, I/128])."""
    return quant.quantise_rows(silu_mul(bf16.to_f32(np.asarray(y1_bf16_bits))))


def row_weights(row_assign: np.ndarray, topk_w: np.ndarray) -> np.ndarray:
    """w_r = topk_w.flat[row_assign[r]] (the layout's per-row routing weight)."""
    return np.asarray(topk_w, dtype=np.float32).reshape(-1)[np.asarray(row_assign, dtype=np.int64)]


def grouped_gemm2(q2, s2, expert_offsets, row_assign, topk_w, w2, w2_scale, rows=None,
                  q_index=None) -> np.ndarray:
    """y2 float32 [R, H] (or [len(rows), H]): per local expert, the weighted
    down projection of the rows' quantised h.  Row r's h is q2[r] (or
    q2[q_index[i]] for the i-th listed row, for callers that quantised only the
    listed rows); w2 uint8 [L, H, I] or a callable le -> (w2_e, w2_scale_e);
    w2_scale float32 [L, H/128, I/128]."""
    offs = np.asarray(expert_offsets, dtype=np.int64)
    R = int(offs[-1])
    rows = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    rowmap = np.arange(max(R, 1))
    if q_index is not None:
        rowmap[rows] = np.asarray(q_index, dtype=np.int64)
    # GEMM1's definition with the identity rowmap: the same per-expert float32 matmul
    y = gemm1.grouped_gemm1(q2, s2, rowmap, offs, w2, w2_scale, rows=rows)
    w = row_weights(np.asarray(row_assign)[rows], topk_w) if rows.size else np.zeros(0, np.float32)
    return (y * w[:, None]).astype(np.float32)


def combine_rows(y2_bf16_bits: np.ndarray, assign_row: np.ndarray, T: int, k: int, tokens=None):
    """(acc float32, out bf16 bits) [n, H]: per token, the sum of its local rows
    of y2 (the weights were applied in GEMM2), i.e. the combine with unit weights."""
    return combine.combine(y2_bf16_bits, assign_row, np.ones(T * k, np.float32), T, k, tokens=tokens)


def act_quant_mx(y1_bf16_bits: np.ndarray):
    """MX variant: (q2 uint8 [n, I], packed e8m0 codes uint32 [n, I/128])."""
    return mx.quantise_rows(silu_mul(bf16.to_f32(np.asarray(y1_bf16_bits))))


def grouped_gemm2_mx(q2, s2, expert_offsets, row_assign, topk_w, w2, w2_scale, rows=None,
                     q_index=None) -> np.ndarray:
    """MX GEMM2: as grouped_gemm2 with e8m0 group scales (oracle.mx's GEMM1
    definition on the expert-major rows): s2 uint32 [., I/128], w2 uint8
    [L, H, I], w2_scale uint32 [L, I/128, H].  Float32 [len(rows), H]."""
    offs = np.asarray(expert_offsets, dtype=np.int64)
    R = int(offs[-1])
    rows = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    rowmap = np.arange(max(R, 1))
    if q_index is not None:
        rowmap[rows] = np.asarray(q_index, dtype=np.int64)
    y = mx.grouped_gemm1(q2, s2, rowmap, offs, w2, w2_scale, rows=rows)
    w = row_weights(np.asarray(row_assign)[rows], topk_w) if rows.size else np.zeros(0, np.float32)
    return (y * w[:, None]).astype(np.float32)
