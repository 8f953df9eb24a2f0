"""Layout step: stable counting sort of routed assignments into expert-major rows.

TEST INFRASTRUCTURE (see the package docstring).

What the pages say the step computes:
* "poc(cco): MegaMoE stage1 dispatch over SDMA", commit "recv_layout": the
  receiver counts the routes per expert and writes the rowmap (expert-major row
  -> where the token's quantised row sits) and srcmap (expert-major row ->
  source token) tables that GEMM1 and stage2 read.
* same page, "What" / "How it works now": GEMM1 reads its A rows in place
  through the rowmap; each landed token's row sits once in the receive region
  of its source.
* "EPDispatchKernel", wait_for_arrivals_and_compute_offsets: per-local-expert
  output offsets; copy_received_tokens_to_output: the rows of one expert, from
  several source ranks, are one contiguous range.

Readings taken (the pages leave these open):
* Rows within an expert are in ascending (global token g, top-k slot j), with
  g = s*Ts + t (source-major): a stable sort, so the result is unique.
* No padding of experts to a tile multiple: offsets are dense.
* Ids outside [e0, e0+L) (negative ones too) are not local and are skipped;
  a token that names the same expert twice gets two rows, in j order.
* A token has landed iff it has at least one local assignment; landed tokens
  get compact slots in ascending g; src_slot_offsets[s] counts landed tokens
  with g < s*Ts.
"""
from __future__ import annotations

import numpy as np


def route_layout(topk_ids, S: int, Ts: int, k: int, e0: int, L: int) -> dict:
    """Returns a dict of int32 arrays:

    expert_counts[L], expert_offsets[L+1], row_slot[R], row_assign[R],
    assign_row[T*k] (-1 for non-local), tok_slot[T] (-1 if not landed),
    slot_tok[U], src_slot_offsets[S+1], totals[2] = (R, U).
    """
    T = S * Ts
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(T, k)
    le = ids - e0
    local = (le >= 0) & (le < L)

    flat_le = le.reshape(-1)
    flat_local = local.reshape(-1)
    a_idx = np.nonzero(flat_local)[0]          # local assignments, ascending (g, j)
    keys = flat_le[a_idx]
    order = np.argsort(keys, kind="stable")    # stable: equal keys keep (g, j) order
    row_assign = a_idx[order]
    R = row_assign.size

    counts = np.bincount(keys, minlength=L)[:L] if R else np.zeros(L, np.int64)
    offsets = np.zeros(L + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)

    assign_row = np.full(T * k, -1, dtype=np.int64)
    assign_row[row_assign] = np.arange(R)

    landed = local.any(axis=1) if T else np.zeros(0, bool)
    slot_tok = np.nonzero(landed)[0]
    U = slot_tok.size
    tok_slot = np.full(T, -1, dtype=np.int64)
    tok_slot[slot_tok] = np.arange(U)
    src = np.zeros(S + 1, dtype=np.int64)
    for s in range(1, S + 1):
        src[s] = int(landed[: s * Ts].sum())

    row_slot = tok_slot[row_assign // k] if R else np.zeros(0, np.int64)

    i32 = lambda a: np.ascontiguousarray(a, dtype=np.int32)
    return dict(
        expert_counts=i32(counts), expert_offsets=i32(offsets), row_slot=i32(row_slot),
        row_assign=i32(row_assign), assign_row=i32(assign_row), tok_slot=i32(tok_slot),
        slot_tok=i32(slot_tok), src_slot_offsets=i32(src), totals=i32([R, U]),
    )
