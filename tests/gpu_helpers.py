"""Shared helpers for the GPU parity tests: seeded inputs (cached per
workload), device copies, the oracle-vs-HIP comparisons and the tolerance."""
from __future__ import annotations

import functools
import sys
from typing import NamedTuple

import numpy as np
import torch

import combine_expert_histogram_amd as moe
import workloads
from oracle import bf16 as obf16
from oracle import layout as olayout

POISON = -123456789
REL_L2_TOL = 1e-2          # GEMM1 / combine: rel-L2 <= 1e-2
MAX_ABS_TOL = 2e-2         # ... and max |err| <= 2e-2 * rms(reference)


def require_gpu():
    assert torch.cuda.is_available(), "the GPU parity tests need an MI355X"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@functools.lru_cache(maxsize=None)
def routing(name):
    return workloads.routing(workloads.get(name))


@functools.lru_cache(maxsize=2)
def activations(name):
    return workloads.activations(workloads.get(name))


@functools.lru_cache(maxsize=1)
def weights(name):
    return workloads.weights(workloads.get(name))


def dims(w: workloads.Workload, full: bool = False) -> moe.Dims:
    if full:
        return moe.Dims(S=w.S, Ts=w.Ts, k=w.k, E=w.E, e0=0, L=w.E, H=w.H)
    return moe.Dims(S=w.S, Ts=w.Ts, k=w.k, E=w.E, e0=w.e0, L=w.L, H=w.H)


def poisoned_layout(d: moe.Dims) -> dict:
    lay = moe.alloc_layout(d)
    for k, v in lay.items():
        if k != "ws":
            v.fill_(POISON)
    return lay


def check_layout(d: moe.Dims, ids: np.ndarray, lay: dict | None = None) -> dict:
    """Runs the HIP layout on poisoned outputs and asserts bit-exact equality
    with the oracle; entries past R / U must still hold the poison."""
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(d.T, d.k)
    ref = olayout.route_layout(ids, d.S, d.Ts, d.k, d.e0, d.L)
    lay = poisoned_layout(d) if lay is None else lay
    moe.route_layout(d, dev(ids.reshape(-1) if d.T else np.zeros(1, np.int32)), lay)
    torch.cuda.synchronize()
    R, U = (int(v) for v in ref["totals"])
    got = {k: v.cpu().numpy() for k, v in lay.items() if k != "ws"}
    np.testing.assert_array_equal(got["totals"], ref["totals"], err_msg="totals")
    np.testing.assert_array_equal(got["expert_counts"][:d.L], ref["expert_counts"], err_msg="expert_counts")
    np.testing.assert_array_equal(got["expert_offsets"][:d.L + 1], ref["expert_offsets"], err_msg="expert_offsets")
    np.testing.assert_array_equal(got["src_slot_offsets"][:d.S + 1], ref["src_slot_offsets"],
                                  err_msg="src_slot_offsets")
    for key, n in (("row_slot", R), ("row_assign", R), ("slot_tok", U)):
        np.testing.assert_array_equal(got[key][:n], ref[key], err_msg=key)
        assert (got[key][n:] == POISON).all(), f"{key} written past its count"
    if d.T:
        np.testing.assert_array_equal(got["assign_row"][:d.T * d.k], ref["assign_row"], err_msg="assign_row")
        np.testing.assert_array_equal(got["tok_slot"][:d.T], ref["tok_slot"], err_msg="tok_slot")
    return lay


def bf16_half_ulp(r: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |r| (8 significant bits): the rounding any bf16
    output of the exact value r carries."""
    a = np.abs(np.asarray(r, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 8)


class Tol(NamedTuple):
    """A bf16 result against an fp32 reference: pass or fail and the figures."""
    ok: bool
    rel_l2: float
    max_excess: float     # max(|err| - half a bf16 ulp of the reference): the bound's subject
    rms: float            # rms of the reference
    max_abs: float        # the literal max |err|

    def __str__(self):
        r = self.rms if self.rms > 0 else 1.0
        return (f"rel_l2={self.rel_l2:.3e} max_abs={self.max_abs:.3e} ({self.max_abs / r:.4f} rms) "
                f"max_abs_beyond_half_ulp={self.max_excess:.3e} ({self.max_excess / r:.4f} rms) "
                f"rms={self.rms:.3e} ok={self.ok}")


def tolerance(got_bits: np.ndarray, ref_f32: np.ndarray) -> Tol:
    """A bf16 result against an fp32 reference.

    rel-L2 <= 1e-2, and every element within 2e-2 * rms(reference) beyond the
    half-ulp rounding of the bf16 output format itself: bf16 keeps 8
    significant bits, so rounding the exact value alone costs up to
    2^-8 * |y|, which exceeds 2e-2 * rms once |y| > 5.12 * rms; the max-abs
    bound is applied to the error on top of that rounding.  The literal
    max |err| is returned (and printed by the tests) beside it."""
    g = obf16.to_f32(got_bits).astype(np.float64)
    r = np.asarray(ref_f32, dtype=np.float64)
    diff = g - r
    nr = np.linalg.norm(r)
    rel = np.linalg.norm(diff) / nr if nr > 0 else float(np.linalg.norm(diff))
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    excess = np.abs(diff) - bf16_half_ulp(r)
    mx = float(excess.max()) if r.size else 0.0
    mabs = float(np.abs(diff).max()) if r.size else 0.0
    ok = rel <= REL_L2_TOL and mx <= MAX_ABS_TOL * rms + 1e-30
    return Tol(bool(ok), float(rel), mx, rms, mabs)
