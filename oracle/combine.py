"""Combine step: top-k weighted gather-sum of expert outputs back to token order.

TEST INFRASTRUCTURE (see the package docstring).

TilePipe, "Communication Kernels": the combine pushes expert outputs back to
the token owners; "poc(cco): MegaMoE stage1 dispatch over SDMA", "What":
stage2 + combine produce the layer output from the expert-major tables.  The
pages do not spell out the arithmetic; the plain reading is the routing-weighted
sum over a token's k assignments.

Definition, for token g and column c:
  acc = +0.0 (fp32)
  for j = 0 .. k-1 (ascending): if assign_row[g*k+j] >= 0:
      acc += topk_w[g, j] * f32(Y[assign_row[g*k+j], c])      (fp32)
  out[g, c] = bf16_rne(acc)
Tokens with no row give +0.  The fp32 sum is returned as well; the HIP path is
compared to it within tolerance, and bit-exactly in the exact special cases.
"""
from __future__ import annotations

import numpy as np

from . import bf16


def combine(y_bf16_bits, assign_row, topk_w, T: int, k: int, tokens=None):
    """Returns (acc float32 [n, width], out bf16 bits uint16 [n, width]) for the
    tokens listed (default all T)."""
    Y = np.asarray(y_bf16_bits)
    ar = np.asarray(assign_row, dtype=np.int64).reshape(T, k)
    wt = np.asarray(topk_w, dtype=np.float32).reshape(T, k)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    width = Y.shape[1]
    acc = np.zeros((toks.size, width), dtype=np.float32)
    for j in range(k):
        r = ar[toks, j]
        ok = r >= 0
        if not ok.any():
            continue
        contrib = bf16.to_f32(Y[r[ok]]) * wt[toks[ok], j][:, None]     # fp32 product
        acc[ok] = (acc[ok] + contrib).astype(np.float32)                # fp32 sum
    return acc, bf16.from_f32(acc)
