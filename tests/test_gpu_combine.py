"""GPU parity: moe_combine vs the oracle within tolerance, bit-exact in the
exact special cases (identity experts with weights summing to 1, k=1 gathers),
and the tiny end-to-end chain layout -> quant -> GEMM1 -> combine."""
import numpy as np
import pytest
import torch

import combine_expert_histogram_amd as moe
import workloads
from gpu_helpers import (activations, dev, dims, host_u16, poisoned_layout, require_gpu, routing,
                         say, tolerance, weights)
from oracle import bf16 as obf16
from oracle import combine as ocombine
from oracle import gemm1 as ogemm1
from oracle import layout as olayout
from oracle import quant as oquant

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,sample", [("ep8_256x8_h7168", None), ("ep8_2048x8_h7168", None),
                                         ("ep8_2048x8_h4096", None)])
def test_combine_workloads(name, sample):
    """Full-expert layout (every assignment is a row), synthetic expert
    outputs [T*k, width], top-k routing weights."""
    require_gpu()
    w = workloads.get(name)
    d = dims(w, full=True)
    width = w.combine_width
    say(f"combine {name} T={d.T} width={width}")
    ids, wts = routing(name)
    Y = workloads.expert_outputs(w)
    ref = olayout.route_layout(ids, d.S, d.Ts, d.k, d.e0, d.L)
    lay = moe.route_layout(d, dev(ids.reshape(-1)), poisoned_layout(d))
    Yd = dev(Y.view(np.int16))
    out = moe.combine(d, width, Yd, lay["assign_row"], dev(wts.reshape(-1)))
    torch.cuda.synchronize()
    toks = np.arange(d.T) if sample is None else np.unique(
        np.concatenate([[0, d.T - 1], np.random.default_rng(2).choice(d.T, sample, replace=False)]))
    acc, _ = ocombine.combine(Y, ref["assign_row"], wts, d.T, d.k, tokens=toks)
    got = host_u16(out[torch.from_numpy(toks).cuda()])
    t = tolerance(got, acc)
    say(f"  tokens={toks.size} {t}")
    assert t.ok, str(t)


def test_combine_identity_experts_bit_exact():
    """Y[r] = x[token of r] over the full-expert layout; weights sum to 1 within
    2^-20, so fp32 gives x(1 +- ~2^-20) and bf16 rounding returns x exactly.
    The sum starts at +0, so an input -0 comes back as +0 (as in the oracle)."""
    require_gpu()
    name = "ep8_256x8_h7168"
    w = workloads.get(name)
    d = dims(w, full=True)
    ids, wts = routing(name)
    x = activations(name)
    lay = moe.route_layout(d, dev(ids.reshape(-1)), poisoned_layout(d))
    ref = olayout.route_layout(ids, d.S, d.Ts, d.k, d.e0, d.L)
    Y = x[ref["row_assign"] // d.k]
    out = moe.combine(d, w.H, dev(Y.view(np.int16)), lay["assign_row"], dev(wts.reshape(-1)))
    torch.cuda.synchronize()
    expect = np.where(x == 0x8000, np.uint16(0), x)
    np.testing.assert_array_equal(host_u16(out), expect)


def test_combine_k1_gather_and_missing_rows():
    require_gpu()
    rng = np.random.default_rng(3)
    T, R, width = 1000, 700, 1024
    d = moe.Dims(S=1, Ts=T, k=1, E=4, e0=0, L=4)
    Y = obf16.from_f32(rng.standard_normal((R, width)).astype(np.float32))
    ar = rng.integers(-1, R, T).astype(np.int32)
    ar[::97] = R + 5                          # rows past the end of y contribute nothing
    out = moe.combine(d, width, dev(Y.view(np.int16)), dev(ar), dev(np.ones(T, np.float32)))
    torch.cuda.synchronize()
    got = host_u16(out)
    ok = (ar >= 0) & (ar < R)
    np.testing.assert_array_equal(got[ok], Y[ar[ok]])
    assert (got[~ok] == 0).all()


@pytest.mark.parametrize("k", [3, 5, 9])
def test_combine_odd_k_vs_oracle(k):
    require_gpu()
    rng = np.random.default_rng(k)
    T, R, width = 513, 1500, 136
    d = moe.Dims(S=1, Ts=T, k=k, E=16, e0=0, L=16)
    Y = obf16.from_f32(rng.standard_normal((R, width)).astype(np.float32))
    ar = rng.integers(-1, R, T * k).astype(np.int32)
    wt = rng.uniform(0, 1, T * k).astype(np.float32)
    out = moe.combine(d, width, dev(Y.view(np.int16)), dev(ar), dev(wt))
    torch.cuda.synchronize()
    acc, _ = ocombine.combine(Y, ar, wt, T, k)
    t = tolerance(host_u16(out), acc)
    assert t.ok, str(t)


def test_tiny_chain_end_to_end():
    """layout -> quant -> GEMM1 -> combine of GEMM1's own output, against the
    oracle's chain (its own quant, fp32 GEMM1 rounded to bf16, combine)."""
    require_gpu()
    name = "tiny_t64_h256_e8"
    w = workloads.get(name)
    d = dims(w)
    ids, wts = routing(name)
    x = activations(name)
    wq, ws = weights(name)
    lay = moe.route_layout(d, dev(ids.reshape(-1)), poisoned_layout(d))
    q, qs = moe.quant_dispatch(d, dev(x.view(np.int16)), lay)
    y = moe.grouped_gemm1(d, w.N, q, qs, lay, dev(wq), dev(ws))
    out = moe.combine(d, w.N, y, lay["assign_row"], dev(wts.reshape(-1)))
    torch.cuda.synchronize()
    ref = olayout.route_layout(ids, d.S, d.Ts, d.k, d.e0, d.L)
    rq, rs = oquant.quant_dispatch(x, ref["slot_tok"])
    y32 = ogemm1.grouped_gemm1(rq, rs, ref["row_slot"], ref["expert_offsets"], wq, ws)
    acc, _ = ocombine.combine(obf16.from_f32(y32), ref["assign_row"], wts, d.T, d.k)
    t = tolerance(host_u16(out), acc)
    say(f"  chain {t}")
    assert t.ok, str(t)
