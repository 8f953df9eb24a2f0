"""MoE expert-dispatch hot path on one MI355X (gfx950).

The four steps (layout, quant + dispatch, grouped GEMM1, combine), and the
MX-style variants of quant and GEMM1 (e8m0 scales per 32 K elements) and
stage2 (silu(gate) * up with its fp8 quant, the grouped GEMM2), are HIP
kernels behind the C ABI in include/moe_hotpath.h (libmoe_hotpath.so, built
in-tree by ``python -m combine_expert_histogram_amd.build``); ``binding`` is
the ctypes layer that passes torch device tensors and torch's current stream.
"""
from .binding import (  # noqa: F401
    Dims, MoeError, alloc_gemm1_workspace, alloc_layout, combine, grouped_gemm1, lib, moe_capacity, moe_combine,
    grouped_gemm1_mx, moe_grouped_gemm1, moe_grouped_gemm1_mx, moe_grouped_gemm1_workspace, moe_quant_dispatch,
    moe_quant_dispatch_mx, moe_route_layout, moe_route_layout_noalloc, moe_route_layout_workspace, moe_status_string, quant_dispatch,
    quant_dispatch_mx, route_layout, silu_mul_quant, grouped_gemm2, alloc_gemm2_workspace, moe_silu_mul_quant,
    moe_grouped_gemm2, moe_grouped_gemm2_workspace, silu_mul_quant_mx, grouped_gemm2_mx, moe_silu_mul_quant_mx,
    moe_grouped_gemm2_mx,
)
