"""Seeded synthetic workloads for the MoE expert-dispatch hot path.

This module draws the random inputs that both the HIP path and the CPU oracle
consume.  It holds none of the hot path's arithmetic: no layout, no activation
quantisation, no GEMM and no combine.  The one piece of numeric preparation it
does is the weight-side input recipe (fp32 N(0, 0.02) -> bf16 -> fp8 e4m3 with
one fp32 scale per 128x128 block); that is done with torch's built-in CPU casts
so that neither the oracle's encoder nor the kernels' encoder is involved.

Shapes follow the MoE layers that "poc(cco): MegaMoE stage1 dispatch over
SDMA" measures (EP8 on MI355X, 256..8192 tokens per rank, uniform routing,
"Where we stand"), with E=256 experts and GEMM1 width 4096 as in TilePipe's
dispatch->GEMM command line.  The pages give no model dimensions, dataset or
benchmark suite; the hidden size 7168 (and 4096) and top-8 routing are the
stand-ins.

Every large array is drawn in fixed chunks, each from its own spawned seed, so
the bytes do not depend on the number of worker threads.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import hashlib
import os

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "routing", "activations", "weights",
    "expert_outputs", "weights2", "stage2_inputs", "weights_mx", "weights2_mx", "sha256",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One layer shape.  Notation: S sources x Ts tokens, top-k of E experts,
    local experts [e0, e0+L), hidden H, GEMM1 width N."""
    name: str
    S: int
    Ts: int
    H: int
    E: int
    e0: int
    L: int
    k: int
    N: int
    seed: int
    zipf_s: float | None = None     # per-expert logit bias (rank+1)^-s, rank = expert id
    combine_from_gemm1: bool = False  # combine reads GEMM1's own output (tiny case)

    @property
    def T(self) -> int:
        return self.S * self.Ts

    @property
    def combine_width(self) -> int:
        # The tiny case combines GEMM1's output (width N); the EP8 shares combine
        # stage2-width rows (width H) of synthetic expert outputs.
        return self.N if self.combine_from_gemm1 else self.H


WORKLOADS = {
    w.name: w for w in [
        # 1 source x 64 tokens, H=256, 8 experts all local, top-2, N=256.
        Workload("tiny_t64_h256_e8", S=1, Ts=64, H=256, E=8, e0=0, L=8, k=2, N=256,
                 seed=0, combine_from_gemm1=True),
        # One rank's share of EP8: 8 sources x 256 tokens, 32 of 256 experts local.
        Workload("ep8_256x8_h7168", S=8, Ts=256, H=7168, E=256, e0=0, L=32, k=8, N=4096, seed=1),
        # Same layer at 2048 tokens per source (16384 source tokens).
        Workload("ep8_2048x8_h7168", S=8, Ts=2048, H=7168, E=256, e0=0, L=32, k=8, N=4096, seed=2),
        # Load-imbalanced: 8192 tokens per source, Zipf(1.2) per-expert logit bias.
        Workload("ep8_8192x8_h7168_zipf", S=8, Ts=8192, H=7168, E=256, e0=0, L=32, k=8, N=4096,
                 seed=3, zipf_s=1.2),
        # Stage1 + combine at 16384 tokens with H=4096.
        Workload("ep8_2048x8_h4096", S=8, Ts=2048, H=4096, E=256, e0=0, L=32, k=8, N=4096, seed=4),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


# ----------------------------------------------------------------------------
# seeding
# appending a stream keeps the earlier streams' draws (SeedSequence children by index)
_STREAMS = ("routing", "activations", "weights", "expert_outputs", "weights2", "stage2_inputs")
_CHUNK_ROWS = 1024


def _stream(w_seed: int, which: str) -> np.random.SeedSequence:
    return np.random.SeedSequence(w_seed).spawn(len(_STREAMS))[_STREAMS.index(which)]


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunked_normal(ss: np.random.SeedSequence, rows: int, cols: int, sigma: float) -> np.ndarray:
    """fp32 N(0, sigma) [rows, cols], drawn in 1024-row chunks with one spawned
    seed per chunk (independent of the thread count)."""
    out = np.empty((rows, cols), dtype=np.float32)
    nchunks = (rows + _CHUNK_ROWS - 1) // _CHUNK_ROWS
    seeds = ss.spawn(nchunks) if nchunks else []

    def one(c):
        r0 = c * _CHUNK_ROWS
        r1 = min(rows, r0 + _CHUNK_ROWS)
        g = np.random.default_rng(seeds[c])
        g.standard_normal(size=(r1 - r0, cols), dtype=np.float32, out=out[r0:r1])
        if sigma != 1.0:
            out[r0:r1] *= np.float32(sigma)

    if nchunks <= 1:
        for c in range(nchunks):
            one(c)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(nchunks)))
    return out


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even) via torch's CPU cast; returns uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


# ----------------------------------------------------------------------------
# draws
def routing(w: Workload):
    """Router draw: fp32 N(0,1) logits [T,E] (plus the Zipf bias when set); the
    top-k ids by descending logit (ties to the lower id); routing weights are
    the softmax restricted to the selected k (float64, stored fp32)."""
    T, E, k = w.T, w.E, w.k
    logits = _chunked_normal(_stream(w.seed, "routing"), T, E, 1.0)
    if w.zipf_s is not None:
        bias = (np.arange(1, E + 1, dtype=np.float64) ** (-w.zipf_s)).astype(np.float32)
        logits += bias[None, :]
    if T == 0:
        return np.zeros((0, k), np.int32), np.zeros((0, k), np.float32)
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)
    sel = np.take_along_axis(logits, ids, axis=1).astype(np.float64)
    sel = np.exp(sel - sel.max(axis=1, keepdims=True))
    wts = (sel / sel.sum(axis=1, keepdims=True)).astype(np.float32)
    return np.ascontiguousarray(ids), np.ascontiguousarray(wts)


def activations(w: Workload) -> np.ndarray:
    """bf16 N(0,1) activations [T, H] as uint16 bit patterns."""
    return _to_bf16_bits(_chunked_normal(_stream(w.seed, "activations"), w.T, w.H, 1.0))


def weights(w: Workload, experts: range | None = None):
    """GEMM1 weights for the local experts (see ``_block_fp8_weights``).

    Logical weight of local expert le is [H, N] (K x N); it is stored
    K-contiguous as [N, H] bytes.

    Returns (w_e4m3 uint8 [L', N, H], w_scale float32 [L', N/128, H/128]).
    """
    return _block_fp8_weights(_stream(w.seed, "weights"), w.L, w.N, w.H, experts)


def weights2(w: Workload, experts: range | None = None):
    """GEMM2 (down projection) weights for the local experts: logical [I, H]
    (K = I = N/2 rows of GEMM1's output width, H output columns), stored
    K-contiguous as [H, I] bytes, same recipe as ``weights``.

    Returns (w2_e4m3 uint8 [L', H, I], w2_scale float32 [L', H/128, I/128]).
    """
    assert w.N % 256 == 0, "GEMM1 width must be 2*I with I a multiple of 128"
    return _block_fp8_weights(_stream(w.seed, "weights2"), w.L, w.H, w.N // 2, experts)


def _block_fp8_weights(ss: np.random.SeedSequence, L: int, N: int, K: int, experts):
    """[L', N, K] e4m3 bytes + [L', N/128, K/128] fp32 scales, expert le drawn from
    its own spawned seed.  Recipe: fp32 N(0, 0.02) -> bf16 (RNE) -> one fp32
    scale per 128(N) x 128(K) block = block |max| / 448 -> e4m3 bytes of
    value / scale (torch's float8_e4m3fn cast; every quotient is <= 448 in
    magnitude, so the cast never overflows).  An all-zero block gets scale 0
    and zero bytes."""
    import torch
    experts = range(L) if experts is None else experts
    seeds = ss.spawn(L)
    q = np.empty((len(experts), N, K), dtype=np.uint8)
    sc = np.empty((len(experts), N // 128, K // 128), dtype=np.float32)

    def one(i_le):
        i, le = i_le
        g = np.random.default_rng(seeds[le])
        wf = g.standard_normal(size=(N, K), dtype=np.float32)
        wf *= np.float32(0.02)
        t = torch.from_numpy(wf).to(torch.bfloat16).to(torch.float32)
        blk = t.view(N // 128, 128, K // 128, 128)
        amax = blk.abs().amax(dim=(1, 3))                       # [N/128, K/128]
        s = amax / torch.tensor(448.0, dtype=torch.float32)
        safe = torch.where(s > 0, s, torch.ones_like(s))
        v = blk / safe[:, None, :, None]
        v = torch.where((s > 0)[:, None, :, None], v, torch.zeros_like(v))
        q[i] = v.to(torch.float8_e4m3fn).view(torch.uint8).reshape(N, K).numpy()
        sc[i] = s.numpy()

    items = list(enumerate(experts))
    if len(items) <= 1:
        for it in items:
            one(it)
    else:
        with _cf.ThreadPoolExecutor(min(_threads(), 8)) as ex:
            list(ex.map(one, items))
    return q, sc


def stage2_inputs(w: Workload, rows: int | None = None) -> np.ndarray:
    """Synthetic GEMM1 outputs for testing stage2 apart from GEMM1: bf16
    N(0, 1.7) [rows, N] (default rows = T*k; 1.7 ~ the spread of GEMM1's
    outputs, sqrt(H) * 0.02 at H = 7168) as uint16 bits."""
    rows = w.T * w.k if rows is None else rows
    return _to_bf16_bits(_chunked_normal(_stream(w.seed, "stage2_inputs"), rows, w.N, 1.7))


def expert_outputs(w: Workload, rows: int | None = None, width: int | None = None) -> np.ndarray:
    """Synthetic expert outputs for the combine: bf16 N(0,1) [rows, width]
    (default rows = T*k, width = the combine width) as uint16 bits."""
    rows = w.T * w.k if rows is None else rows
    width = w.combine_width if width is None else width
    return _to_bf16_bits(_chunked_normal(_stream(w.seed, "expert_outputs"), rows, width, 1.0))


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()


def weights_mx(w: Workload, experts: range | None = None):
    """GEMM1 weights in the MX-style format: the same fp32 N(0, 0.02) -> bf16
    draws as ``weights``, quantised per column n and group of 32 consecutive K
    elements with a power-of-two scale (see ``_mx_weights``).

    Returns (w_e4m3 uint8 [L', N, H], w_scale uint32 [L', H/128, N]).
    """
    return _mx_weights(_stream(w.seed, "weights"), w.L, w.N, w.H, experts)


def weights2_mx(w: Workload, experts: range | None = None):
    """GEMM2 weights in the MX-style format: the same draws as ``weights2``.

    Returns (w2_e4m3 uint8 [L', H, I], w2_scale uint32 [L', I/128, H]).
    """
    assert w.N % 256 == 0, "GEMM1 width must be 2*I with I a multiple of 128"
    return _mx_weights(_stream(w.seed, "weights2"), w.L, w.H, w.N // 2, experts)


def _mx_weights(ss: np.random.SeedSequence, L: int, N: int, K: int, experts):
    """[L', N, K] e4m3 bytes + [L', K/128, N] packed e8m0 codes.  Expert le is
    drawn from its own spawned seed as in ``_block_fp8_weights``: fp32
    N(0, 0.02) -> bf16; per column n and group of 32 consecutive K elements,
    E = ceil(log2(group |max| / 448)) (the fp32 quotient's binary exponent; an
    all-zero group gets E = -127), payload = e4m3(value * 2^-E) (torch's
    float8_e4m3fn cast; exact scaling, every magnitude <= 448).  The codes
    E + 127 are packed four per uint32 (group 4kb+g in byte g) and stored
    K-block-major."""
    import torch
    experts = range(L) if experts is None else experts
    seeds = ss.spawn(L)
    q = np.empty((len(experts), N, K), dtype=np.uint8)
    sc = np.empty((len(experts), K // 128, N), dtype=np.uint32)

    def one(i_le):
        i, le = i_le
        g = np.random.default_rng(seeds[le])
        wf = g.standard_normal(size=(N, K), dtype=np.float32)
        wf *= np.float32(0.02)
        t = torch.from_numpy(wf).to(torch.bfloat16).to(torch.float32).view(N, K // 32, 32)
        amax = t.abs().amax(dim=2)
        m, e = torch.frexp(amax / torch.tensor(448.0, dtype=torch.float32))
        E = torch.where(m == 0.5, e - 1, e).to(torch.int64)
        E = torch.where(amax == 0, torch.full_like(E, -127), E).clamp(-127, 127)
        v = torch.ldexp(t.to(torch.float64), (-E)[:, :, None].to(torch.float64)).to(torch.float32)
        q[i] = v.to(torch.float8_e4m3fn).view(torch.uint8).reshape(N, K).numpy()
        c = (E + 127).to(torch.int64).view(N, K // 128, 4)
        packed = c[..., 0] | (c[..., 1] << 8) | (c[..., 2] << 16) | (c[..., 3] << 24)
        sc[i] = packed.t().numpy().astype(np.uint32)

    items = list(enumerate(experts))
    if len(items) <= 1:
        for it in items:
            one(it)
    else:
        with _cf.ThreadPoolExecutor(min(_threads(), 8)) as ex:
            list(ex.map(one, items))
    return q, sc
