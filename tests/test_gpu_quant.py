"""GPU parity: moe_quant_dispatch vs the oracle, bit-exact fp8 payloads and
scales, on the workloads (full or sampled slots) and on crafted blocks that hit
every bf16 pattern, exact e4m3 rounding ties and near-ties."""
import numpy as np
import pytest
import torch

import combine_expert_histogram_amd as moe
import workloads
from gpu_helpers import activations, dev, dims, poisoned_layout, require_gpu, routing, say
from oracle import bf16 as obf16
from oracle import fp8 as ofp8
from oracle import layout as olayout
from oracle import quant as oquant

pytestmark = pytest.mark.gpu


def _run(d, ids, x_bits):
    lay = moe.route_layout(d, dev(ids.reshape(-1)), poisoned_layout(d))
    xt = dev(x_bits.view(np.int16))
    q = torch.full((d.T, d.H), 0xA5, dtype=torch.uint8, device="cuda")
    qs = torch.full((d.T, d.H // 128), -7.0, dtype=torch.float32, device="cuda")
    moe.quant_dispatch(d, xt, lay, q, qs)
    torch.cuda.synchronize()
    return lay, q, qs


def _compare(ref_lay, q, qs, x_bits, slots):
    rq, rs = oquant.quant_dispatch(x_bits, ref_lay["slot_tok"], slots=slots)
    sl = torch.from_numpy(np.asarray(slots, dtype=np.int64)).cuda()
    gq = q[sl].cpu().numpy()
    gs = qs[sl].cpu().numpy()
    bad = np.nonzero((gq != rq).any(axis=1))[0]
    assert bad.size == 0, f"payload mismatch in {bad.size} slots, first slot {slots[bad[0]]}"
    np.testing.assert_array_equal(gs.view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("name,sample", [
    ("tiny_t64_h256_e8", None), ("ep8_256x8_h7168", None), ("ep8_2048x8_h7168", None),
    ("ep8_2048x8_h4096", None), ("ep8_8192x8_h7168_zipf", 2048),
])
def test_quant_workloads(name, sample):
    require_gpu()
    w = workloads.get(name)
    d = dims(w)
    say(f"quant {name} T={d.T} H={d.H}")
    ids, _ = routing(name)
    x = activations(name)
    ref_lay = olayout.route_layout(ids, d.S, d.Ts, d.k, d.e0, d.L)
    U = int(ref_lay["totals"][1])
    lay, q, qs = _run(d, ids, x)
    if sample is None:
        slots = np.arange(U)
    else:
        rng = np.random.default_rng(17)
        slots = np.unique(np.concatenate([[0, U - 1], rng.choice(U, sample, replace=False)]))
    _compare(ref_lay, q, qs, x, slots)
    # rows past U are untouched
    assert (q[U:] == 0xA5).all() and (qs[U:] == -7.0).all()


def _quant_rows(x_f32_bits: np.ndarray):
    """Quantise every row of x (all tokens land: identity routing, k=1, L=E=1)."""
    T, H = x_f32_bits.shape
    d = moe.Dims(S=1, Ts=T, k=1, E=1, e0=0, L=1, H=H)
    ids = np.zeros((T, 1), np.int32)
    ref_lay = olayout.route_layout(ids, 1, T, 1, 0, 1)
    lay, q, qs = _run(d, ids, x_f32_bits)
    _compare(ref_lay, q, qs, x_f32_bits, np.arange(T))


def test_quant_every_bf16_pattern():
    """All 65280 finite bf16 values, shuffled into 128-element blocks several
    times, so each value is quantised under many different block scales."""
    require_gpu()
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    fin = bits[np.isfinite(vals)].astype(np.uint16)
    rng = np.random.default_rng(5)
    reps = [rng.permutation(fin) for _ in range(4)]
    allb = np.concatenate(reps)
    n = (allb.size // 1024) * 1024
    x = allb[:n].reshape(-1, 1024)
    say(f"quant every bf16 pattern rows={x.shape[0]}")
    _quant_rows(x)


def test_quant_exact_ties_and_near_ties():
    """Blocks whose amax is 448 (scale exactly 1) holding every e4m3 midpoint
    exactly, and blocks with an awkward scale holding values within a few ulps
    of midpoints after division."""
    require_gpu()
    mids = (ofp8.decode(np.arange(0x7E, dtype=np.uint8)).astype(np.float64)
            + ofp8.decode(np.arange(1, 0x7F, dtype=np.uint8)).astype(np.float64)) / 2
    rows = []
    # scale 1: x = midpoint exactly (every midpoint has <= 5 significant bits, so it is a bf16)
    m = np.concatenate([mids, -mids])
    for i in range(0, m.size, 127):
        blk = np.zeros(128, np.float64)
        part = m[i:i + 127]
        blk[:part.size] = part
        blk[127] = 448.0
        rows.append(blk)
    # awkward scales: amax a -> s = a/448; x = bf16 values nearest to midpoint * s
    rng = np.random.default_rng(9)
    for a in (3.0, 1.7, 0.09, 5.5e-3, 123.4, 2.0 ** -20 * 3):
        s = np.float32(np.float32(a) / np.float32(448.0))
        tgt = rng.choice(mids, 127) * float(s) * rng.choice([-1, 1], 127)
        blk = np.concatenate([tgt, [a]])
        rows.append(blk)
    x = np.stack(rows)                                    # [n, 128]
    pad = (-x.shape[0]) % 8
    if pad:
        x = np.concatenate([x, np.ones((pad, 128))])
    # eight blocks per row (H = 1024): several blocks per wavefront pass
    xb = obf16.from_f32(x.astype(np.float32)).reshape(-1, 1024)
    assert (obf16.to_f32(xb).reshape(-1, 128)[: len(rows) - 6, :127].astype(np.float64)
            == np.stack(rows[: len(rows) - 6])[:, :127]).all()     # midpoints are exact bf16
    _quant_rows(xb)


def test_quant_zero_and_sparse_blocks():
    require_gpu()
    rng = np.random.default_rng(4)
    x = np.zeros((64, 2048), np.float32)
    x[1::3] = rng.standard_normal((x[1::3].shape[0], 2048))
    x[2, 5] = -1e-30                  # lone tiny value
    x[4, 700] = -0.0
    x[5, 128:256] = -0.0              # block of negative zeros
    _quant_rows(obf16.from_f32(x))


def test_quant_ragged_hidden():
    """H = 128 * 9: the last 1024-element pass holds one block."""
    require_gpu()
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((300, 1152)) * np.exp2(rng.uniform(-8, 8, (300, 1)))).astype(np.float32)
    _quant_rows(obf16.from_f32(x))


def test_quant_out_of_range_tokens_leave_rows_unwritten():
    """Slot tokens outside [0, T) (the layout never produces them) are read as
    row 0 and their slot rows left unwritten; every other row is unchanged
    (H = 1152: the last pass holds one block, so lanes past it are live)."""
    require_gpu()
    rng = np.random.default_rng(8)
    T, H = 300, 1152
    x = obf16.from_f32((rng.standard_normal((T, H)) * np.exp2(rng.uniform(-8, 8, (T, 1)))).astype(np.float32))
    d = moe.Dims(S=1, Ts=T, k=1, E=1, e0=0, L=1, H=H)
    ids = np.zeros((T, 1), np.int32)
    ref_lay = olayout.route_layout(ids, 1, T, 1, 0, 1)
    lay = moe.route_layout(d, dev(ids.reshape(-1)), poisoned_layout(d))
    bad = [0, 5, 131, T - 1]
    lay["slot_tok"][bad[0]] = -1
    lay["slot_tok"][bad[1]] = T
    lay["slot_tok"][bad[2]] = T + 1000
    lay["slot_tok"][bad[3]] = -(1 << 30)
    q = torch.full((T, H), 0xA5, dtype=torch.uint8, device="cuda")
    qs = torch.full((T, H // 128), -7.0, dtype=torch.float32, device="cuda")
    moe.quant_dispatch(d, dev(x.view(np.int16)), lay, q, qs)
    torch.cuda.synchronize()
    good = np.setdiff1d(np.arange(T), bad)
    _compare(ref_lay, q, qs, x, good)
    for u in bad:
        assert (q[u] == 0xA5).all() and (qs[u] == -7.0).all(), f"slot {u} written"
