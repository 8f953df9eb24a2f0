"""ctypes binding of libmoe_hotpath.so (the C ABI in include/moe_hotpath.h).

Argument marshalling only: torch tensors in, device pointers and sizes out to
the C functions of the same names, enqueued on torch's current HIP stream.
Every step of the path runs in the library's HIP kernels; there is no CPU
fallback, and loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_hotpath.so")

MOE_OK = 0
_STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_WORKSPACE",
           -3: "MOE_ERR_UNSUPPORTED", -4: "MOE_ERR_HIP"}

# every symbol include/moe_hotpath.h declares
EXPORTS = ("moe_status_string", "moe_capacity", "moe_route_layout_workspace", "moe_route_layout",
           "moe_route_layout_noalloc",
           "moe_quant_dispatch", "moe_grouped_gemm1_workspace", "moe_grouped_gemm1",
           "moe_quant_dispatch_mx", "moe_grouped_gemm1_mx", "moe_silu_mul_quant",
           "moe_grouped_gemm2_workspace", "moe_grouped_gemm2", "moe_silu_mul_quant_mx",
           "moe_grouped_gemm2_mx", "moe_combine")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)}")


class moe_dims(ctypes.Structure):
    _fields_ = [("num_sources", ctypes.c_int32), ("tokens_per_source", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("expert_begin", ctypes.c_int32), ("num_local_experts", ctypes.c_int32),
                ("hidden", ctypes.c_int32)]


@dataclass(frozen=True)
class Dims:
    S: int
    Ts: int
    k: int
    E: int
    e0: int
    L: int
    H: int = 128

    @property
    def T(self) -> int:
        return self.S * self.Ts

    def c(self) -> moe_dims:
        return moe_dims(self.S, self.Ts, self.k, self.E, self.e0, self.L, self.H)


_lib = None


def lib() -> ctypes.CDLL:
    """Loads the HIP library (built in-tree by combine_expert_histogram_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m combine_expert_histogram_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        D = ctypes.POINTER(moe_dims)
        sig = {
            "moe_status_string": (ctypes.c_char_p, [I32]),
            "moe_capacity": (I32, [D, ctypes.POINTER(I64), ctypes.POINTER(I64)]),
            "moe_route_layout_workspace": (I32, [D, ctypes.POINTER(SZ)]),
            "moe_route_layout": (I32, [D] + [P] * 10 + [P, SZ, P]),
            "moe_route_layout_noalloc": (I32, [D] + [P] * 10 + [P]),
            "moe_quant_dispatch": (I32, [D, P, P, P, P, P, P]),
            "moe_grouped_gemm1_workspace": (I32, [D, I32, ctypes.POINTER(SZ)]),
            "moe_grouped_gemm1": (I32, [D, I32] + [P] * 8 + [P, SZ, P]),
            "moe_quant_dispatch_mx": (I32, [D, P, P, P, P, P, P]),
            "moe_grouped_gemm1_mx": (I32, [D, I32] + [P] * 7 + [P, SZ, P]),
            "moe_silu_mul_quant": (I32, [D, I32, P, P, P, P, P]),
            "moe_grouped_gemm2_workspace": (I32, [D, I32, ctypes.POINTER(SZ)]),
            "moe_grouped_gemm2": (I32, [D, I32] + [P] * 8 + [P, SZ, P]),
            "moe_silu_mul_quant_mx": (I32, [D, I32, P, P, P, P, P]),
            "moe_grouped_gemm2_mx": (I32, [D, I32] + [P] * 8 + [P, SZ, P]),
            "moe_combine": (I32, [D, I32, P, I64, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None, name: str, nbytes_min: int = 0, elt: int | None = None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if elt is not None and t.element_size() != elt:
        raise ValueError(f"{name} must have {elt}-byte elements, got {t.dtype}")
    if t.numel() * t.element_size() < nbytes_min:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {nbytes_min}")
    return t.data_ptr()


def _i32(t, name, n):
    if t is not None and t.dtype != torch.int32:
        raise ValueError(f"{name} must be int32")
    return _ptr(t, name, 4 * n)


# ---------------------------------------------------------------- C ABI, same names
def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_capacity(d: Dims) -> tuple[int, int]:
    r, s = ctypes.c_int64(), ctypes.c_int64()
    _check("moe_capacity", lib().moe_capacity(ctypes.byref(d.c()), ctypes.byref(r), ctypes.byref(s)))
    return r.value, s.value


def moe_route_layout_workspace(d: Dims) -> int:
    b = ctypes.c_size_t()
    _check("moe_route_layout_workspace", lib().moe_route_layout_workspace(ctypes.byref(d.c()), ctypes.byref(b)))
    return b.value


def moe_grouped_gemm1_workspace(d: Dims, n: int) -> int:
    b = ctypes.c_size_t()
    _check("moe_grouped_gemm1_workspace",
           lib().moe_grouped_gemm1_workspace(ctypes.byref(d.c()), n, ctypes.byref(b)))
    return b.value


def moe_route_layout(d: Dims, topk_ids, expert_counts, expert_offsets, row_slot, row_assign,
                     assign_row, tok_slot, slot_tok, src_slot_offsets, totals, ws) -> None:
    T, k, L, S = d.T, d.k, d.L, d.S
    rows_cap, slots_cap = T * k, T
    ws_need = moe_route_layout_workspace(d)
    st = lib().moe_route_layout(
        ctypes.byref(d.c()), _i32(topk_ids, "topk_ids", T * k), _i32(expert_counts, "expert_counts", L),
        _i32(expert_offsets, "expert_offsets", L + 1), _i32(row_slot, "row_slot", rows_cap),
        _i32(row_assign, "row_assign", rows_cap), _i32(assign_row, "assign_row", T * k),
        _i32(tok_slot, "tok_slot", T), _i32(slot_tok, "slot_tok", slots_cap),
        _i32(src_slot_offsets, "src_slot_offsets", S + 1), _i32(totals, "totals", 2),
        _ptr(ws, "ws", ws_need), 0 if ws is None else ws.numel() * ws.element_size(), _stream())
    _check("moe_route_layout", st)


def moe_route_layout_noalloc(d: Dims, topk_ids, expert_counts, expert_offsets, row_slot, row_assign,
                             assign_row, tok_slot, slot_tok, src_slot_offsets, totals) -> None:
    T, k, L, S = d.T, d.k, d.L, d.S
    rows_cap, slots_cap = T * k, T
    st = lib().moe_route_layout_noalloc(
        ctypes.byref(d.c()), _i32(topk_ids, "topk_ids", T * k), _i32(expert_counts, "expert_counts", L),
        _i32(expert_offsets, "expert_offsets", L + 1), _i32(row_slot, "row_slot", rows_cap),
        _i32(row_assign, "row_assign", rows_cap), _i32(assign_row, "assign_row", T * k),
        _i32(tok_slot, "tok_slot", T), _i32(slot_tok, "slot_tok", slots_cap),
        _i32(src_slot_offsets, "src_slot_offsets", S + 1), _i32(totals, "totals", 2), _stream())
    _check("moe_route_layout_noalloc", st)


def moe_quant_dispatch(d: Dims, x_bf16, slot_tok, totals, q_e4m3, q_scale) -> None:
    T, H = d.T, d.H
    st = lib().moe_quant_dispatch(
        ctypes.byref(d.c()), _ptr(x_bf16, "x_bf16", 2 * T * H, 2), _i32(slot_tok, "slot_tok", T),
        _i32(totals, "totals", 2), _ptr(q_e4m3, "q_e4m3", T * H, 1),
        _ptr(q_scale, "q_scale", 4 * T * (H // 128), 4), _stream())
    _check("moe_quant_dispatch", st)


def moe_grouped_gemm1(d: Dims, n: int, q_e4m3, q_scale, row_slot, expert_offsets, totals,
                      w_e4m3, w_scale, y_bf16, ws=None) -> None:
    T, H, L = d.T, d.H, d.L
    rows_cap = T * d.k
    st = lib().moe_grouped_gemm1(
        ctypes.byref(d.c()), n, _ptr(q_e4m3, "q_e4m3", T * H, 1),
        _ptr(q_scale, "q_scale", 4 * T * (H // 128), 4), _i32(row_slot, "row_slot", rows_cap),
        _i32(expert_offsets, "expert_offsets", L + 1), _i32(totals, "totals", 2),
        _ptr(w_e4m3, "w_e4m3", L * n * H, 1), _ptr(w_scale, "w_scale", 4 * L * (n // 128) * (H // 128), 4),
        _ptr(y_bf16, "y_bf16", 2 * rows_cap * n, 2), _ptr(ws, "ws", moe_grouped_gemm1_workspace(d, n)),
        0 if ws is None else ws.numel() * ws.element_size(), _stream())
    _check("moe_grouped_gemm1", st)


def _u32(t, name, n):
    if t is not None and t.dtype not in (torch.int32, torch.uint32):
        raise ValueError(f"{name} must be a 32-bit integer tensor (packed e8m0 codes)")
    return _ptr(t, name, 4 * n)


def moe_quant_dispatch_mx(d: Dims, x_bf16, slot_tok, totals, q_e4m3, q_scale) -> None:
    T, H = d.T, d.H
    st = lib().moe_quant_dispatch_mx(
        ctypes.byref(d.c()), _ptr(x_bf16, "x_bf16", 2 * T * H, 2), _i32(slot_tok, "slot_tok", T),
        _i32(totals, "totals", 2), _ptr(q_e4m3, "q_e4m3", T * H, 1),
        _u32(q_scale, "q_scale", T * (H // 128)), _stream())
    _check("moe_quant_dispatch_mx", st)


def moe_grouped_gemm1_mx(d: Dims, n: int, q_e4m3, q_scale, row_slot, expert_offsets,
                         w_e4m3, w_scale, y_bf16, ws=None) -> None:
    T, H, L = d.T, d.H, d.L
    rows_cap = T * d.k
    st = lib().moe_grouped_gemm1_mx(
        ctypes.byref(d.c()), n, _ptr(q_e4m3, "q_e4m3", T * H, 1), _u32(q_scale, "q_scale", T * (H // 128)),
        _i32(row_slot, "row_slot", rows_cap), _i32(expert_offsets, "expert_offsets", L + 1),
        _ptr(w_e4m3, "w_e4m3", L * n * H, 1), _u32(w_scale, "w_scale", L * (H // 128) * n),
        _ptr(y_bf16, "y_bf16", 2 * rows_cap * n, 2), _ptr(ws, "ws", moe_grouped_gemm1_workspace(d, n)),
        0 if ws is None else ws.numel() * ws.element_size(), _stream())
    _check("moe_grouped_gemm1_mx", st)


def moe_silu_mul_quant(d: Dims, inter: int, y1_bf16, totals, h_e4m3, h_scale) -> None:
    rows_cap = d.T * d.k
    st = lib().moe_silu_mul_quant(
        ctypes.byref(d.c()), inter, _ptr(y1_bf16, "y1_bf16", 2 * rows_cap * 2 * inter, 2),
        _i32(totals, "totals", 2), _ptr(h_e4m3, "h_e4m3", rows_cap * inter, 1),
        _ptr(h_scale, "h_scale", 4 * rows_cap * (inter // 128), 4), _stream())
    _check("moe_silu_mul_quant", st)


def moe_grouped_gemm2_workspace(d: Dims, inter: int) -> int:
    b = ctypes.c_size_t()
    _check("moe_grouped_gemm2_workspace",
           lib().moe_grouped_gemm2_workspace(ctypes.byref(d.c()), inter, ctypes.byref(b)))
    return b.value


def moe_grouped_gemm2(d: Dims, inter: int, h_e4m3, h_scale, expert_offsets, row_assign, topk_w,
                      w2_e4m3, w2_scale, y2_bf16, ws=None) -> None:
    T, H, L = d.T, d.H, d.L
    rows_cap = T * d.k
    if topk_w is not None and topk_w.dtype != torch.float32:
        raise ValueError("topk_w must be float32")
    st = lib().moe_grouped_gemm2(
        ctypes.byref(d.c()), inter, _ptr(h_e4m3, "h_e4m3", rows_cap * inter, 1),
        _ptr(h_scale, "h_scale", 4 * rows_cap * (inter // 128), 4),
        _i32(expert_offsets, "expert_offsets", L + 1), _i32(row_assign, "row_assign", rows_cap),
        _ptr(topk_w, "topk_w", 4 * T * d.k, 4), _ptr(w2_e4m3, "w2_e4m3", L * H * inter, 1),
        _ptr(w2_scale, "w2_scale", 4 * L * (H // 128) * (inter // 128), 4),
        _ptr(y2_bf16, "y2_bf16", 2 * rows_cap * H, 2), _ptr(ws, "ws", moe_grouped_gemm2_workspace(d, inter)),
        0 if ws is None else ws.numel() * ws.element_size(), _stream())
    _check("moe_grouped_gemm2", st)


def moe_silu_mul_quant_mx(d: Dims, inter: int, y1_bf16, totals, h_e4m3, h_scale) -> None:
    rows_cap = d.T * d.k
    st = lib().moe_silu_mul_quant_mx(
        ctypes.byref(d.c()), inter, _ptr(y1_bf16, "y1_bf16", 2 * rows_cap * 2 * inter, 2),
        _i32(totals, "totals", 2), _ptr(h_e4m3, "h_e4m3", rows_cap * inter, 1),
        _u32(h_scale, "h_scale", rows_cap * (inter // 128)), _stream())
    _check("moe_silu_mul_quant_mx", st)


def moe_grouped_gemm2_mx(d: Dims, inter: int, h_e4m3, h_scale, expert_offsets, row_assign, topk_w,
                         w2_e4m3, w2_scale, y2_bf16, ws=None) -> None:
    T, H, L = d.T, d.H, d.L
    rows_cap = T * d.k
    if topk_w is not None and topk_w.dtype != torch.float32:
        raise ValueError("topk_w must be float32")
    st = lib().moe_grouped_gemm2_mx(
        ctypes.byref(d.c()), inter, _ptr(h_e4m3, "h_e4m3", rows_cap * inter, 1),
        _u32(h_scale, "h_scale", rows_cap * (inter // 128)),
        _i32(expert_offsets, "expert_offsets", L + 1), _i32(row_assign, "row_assign", rows_cap),
        _ptr(topk_w, "topk_w", 4 * T * d.k, 4), _ptr(w2_e4m3, "w2_e4m3", L * H * inter, 1),
        _u32(w2_scale, "w2_scale", L * (inter // 128) * H),
        _ptr(y2_bf16, "y2_bf16", 2 * rows_cap * H, 2), _ptr(ws, "ws", moe_grouped_gemm2_workspace(d, inter)),
        0 if ws is None else ws.numel() * ws.element_size(), _stream())
    _check("moe_grouped_gemm2_mx", st)


def moe_combine(d: Dims, width: int, y_bf16, assign_row, topk_w, out_bf16) -> None:
    T, k = d.T, d.k
    y_rows = 0 if y_bf16 is None else y_bf16.numel() // max(width, 1)
    if topk_w is not None and topk_w.dtype != torch.float32:
        raise ValueError("topk_w must be float32")
    st = lib().moe_combine(
        ctypes.byref(d.c()), width, _ptr(y_bf16, "y_bf16", 0, 2), y_rows,
        _i32(assign_row, "assign_row", T * k), _ptr(topk_w, "topk_w", 4 * T * k, 4),
        _ptr(out_bf16, "out_bf16", 2 * T * width, 2), _stream())
    _check("moe_combine", st)


# ---------------------------------------------------------------- conveniences
LAYOUT_KEYS = ("expert_counts", "expert_offsets", "row_slot", "row_assign", "assign_row",
               "tok_slot", "slot_tok", "src_slot_offsets", "totals")


def alloc_layout(d: Dims, device="cuda") -> dict:
    rows_cap, slots_cap = d.T * d.k, d.T
    sizes = dict(expert_counts=d.L, expert_offsets=d.L + 1, row_slot=rows_cap, row_assign=rows_cap,
                 assign_row=d.T * d.k, tok_slot=d.T, slot_tok=slots_cap, src_slot_offsets=d.S + 1,
                 totals=2)
    out = {k: torch.empty(max(v, 1), dtype=torch.int32, device=device) for k, v in sizes.items()}
    out["ws"] = torch.empty(max(moe_route_layout_workspace(d) // 4, 1), dtype=torch.int32, device=device)
    return out


def route_layout(d: Dims, topk_ids, out: dict | None = None) -> dict:
    out = alloc_layout(d, topk_ids.device) if out is None else out
    moe_route_layout(d, topk_ids, *(out[k] for k in LAYOUT_KEYS), out["ws"])
    return out


def quant_dispatch(d: Dims, x_bf16, lay: dict, q=None, q_scale=None):
    dev = x_bf16.device
    q = torch.empty((max(d.T, 1), d.H), dtype=torch.uint8, device=dev) if q is None else q
    q_scale = (torch.empty((max(d.T, 1), d.H // 128), dtype=torch.float32, device=dev)
               if q_scale is None else q_scale)
    moe_quant_dispatch(d, x_bf16, lay["slot_tok"], lay["totals"], q, q_scale)
    return q, q_scale


def alloc_gemm1_workspace(d: Dims, n: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(moe_grouped_gemm1_workspace(d, n) // 4, 1), dtype=torch.float32, device=device)


def grouped_gemm1(d: Dims, n: int, q, q_scale, lay: dict, w_e4m3, w_scale, y=None, ws=None):
    y = torch.empty((max(d.T * d.k, 1), n), dtype=torch.bfloat16, device=q.device) if y is None else y
    ws = alloc_gemm1_workspace(d, n, q.device) if ws is None else ws
    moe_grouped_gemm1(d, n, q, q_scale, lay["row_slot"], lay["expert_offsets"], lay["totals"],
                      w_e4m3, w_scale, y, ws)
    return y


def quant_dispatch_mx(d: Dims, x_bf16, lay: dict, q=None, q_scale=None):
    dev = x_bf16.device
    q = torch.empty((max(d.T, 1), d.H), dtype=torch.uint8, device=dev) if q is None else q
    q_scale = (torch.empty((max(d.T, 1), d.H // 128), dtype=torch.int32, device=dev)
               if q_scale is None else q_scale)
    moe_quant_dispatch_mx(d, x_bf16, lay["slot_tok"], lay["totals"], q, q_scale)
    return q, q_scale


def grouped_gemm1_mx(d: Dims, n: int, q, q_scale, lay: dict, w_e4m3, w_scale, y=None, ws=None):
    y = torch.empty((max(d.T * d.k, 1), n), dtype=torch.bfloat16, device=q.device) if y is None else y
    ws = alloc_gemm1_workspace(d, n, q.device) if ws is None else ws
    moe_grouped_gemm1_mx(d, n, q, q_scale, lay["row_slot"], lay["expert_offsets"], w_e4m3, w_scale, y, ws)
    return y


def silu_mul_quant(d: Dims, inter: int, y1, lay: dict, h=None, h_scale=None):
    rows = max(d.T * d.k, 1)
    h = torch.empty((rows, inter), dtype=torch.uint8, device=y1.device) if h is None else h
    h_scale = (torch.empty((rows, inter // 128), dtype=torch.float32, device=y1.device)
               if h_scale is None else h_scale)
    moe_silu_mul_quant(d, inter, y1, lay["totals"], h, h_scale)
    return h, h_scale


def alloc_gemm2_workspace(d: Dims, inter: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(moe_grouped_gemm2_workspace(d, inter) // 4, 1), dtype=torch.float32, device=device)


def grouped_gemm2(d: Dims, inter: int, h, h_scale, lay: dict, topk_w, w2_e4m3, w2_scale, y2=None, ws=None):
    y2 = torch.empty((max(d.T * d.k, 1), d.H), dtype=torch.bfloat16, device=h.device) if y2 is None else y2
    ws = alloc_gemm2_workspace(d, inter, h.device) if ws is None else ws
    moe_grouped_gemm2(d, inter, h, h_scale, lay["expert_offsets"], lay["row_assign"], topk_w, w2_e4m3, w2_scale,
                      y2, ws)
    return y2


def silu_mul_quant_mx(d: Dims, inter: int, y1, lay: dict, h=None, h_scale=None):
    rows = max(d.T * d.k, 1)
    h = torch.empty((rows, inter), dtype=torch.uint8, device=y1.device) if h is None else h
    h_scale = (torch.empty((rows, inter // 128), dtype=torch.int32, device=y1.device)
               if h_scale is None else h_scale)
    moe_silu_mul_quant_mx(d, inter, y1, lay["totals"], h, h_scale)
    return h, h_scale


def grouped_gemm2_mx(d: Dims, inter: int, h, h_scale, lay: dict, topk_w, w2_e4m3, w2_scale, y2=None, ws=None):
    y2 = torch.empty((max(d.T * d.k, 1), d.H), dtype=torch.bfloat16, device=h.device) if y2 is None else y2
    ws = alloc_gemm2_workspace(d, inter, h.device) if ws is None else ws
    moe_grouped_gemm2_mx(d, inter, h, h_scale, lay["expert_offsets"], lay["row_assign"], topk_w, w2_e4m3,
                         w2_scale, y2, ws)
    return y2


def combine(d: Dims, width: int, y_bf16, assign_row, topk_w, out=None):
    out = torch.empty((max(d.T, 1), width), dtype=torch.bfloat16, device=y_bf16.device) if out is None else out
    moe_combine(d, width, y_bf16, assign_row, topk_w, out)
    return out
