"""The C ABI library loads, exports every symbol include/moe_hotpath.h declares,
and its host-only paths (capacities, workspace sizes, argument validation)
behave as documented.  No kernel is launched, so this runs without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_hotpath.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:moe_status|const char\*)\s+(moe_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    from combine_expert_histogram_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from combine_expert_histogram_amd import build
        build.build()
    return binding.lib()


def test_header_declares_the_four_steps():
    names = _declared()
    for n in ("moe_route_layout", "moe_quant_dispatch", "moe_grouped_gemm1", "moe_combine"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    from combine_expert_histogram_amd import binding
    names = _declared()
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    from combine_expert_histogram_amd import binding as b
    assert b.moe_status_string(0) == "ok"
    assert "argument" in b.moe_status_string(-1)
    assert "workspace" in b.moe_status_string(-2)


def test_capacity_and_workspace(L):
    from combine_expert_histogram_amd import binding as b
    d = b.Dims(S=8, Ts=2048, k=8, E=256, e0=0, L=32, H=7168)
    assert b.moe_capacity(d) == (16384 * 8, 16384)
    ws = b.moe_route_layout_workspace(d)
    assert ws > 0 and ws % 256 == 0
    # the row-scale table (H/128 K blocks x (rows_cap + one 256-row tile, 64-aligned) floats,
    # 256 B aligned), then 16 B tile descriptors: one count + (rows_cap/128 + L) x (n/256)
    table = (56 * ((16384 * 8 + 256 + 63) // 64 * 64) * 4 + 255) // 256 * 256
    assert b.moe_grouped_gemm1_workspace(d, 4096) == table + (1 + (16384 * 8 // 128 + 32) * 16 + 1024) * 16
    # the full-expert layout used by the combine
    assert b.moe_route_layout_workspace(b.Dims(S=8, Ts=2048, k=8, E=256, e0=0, L=256)) > 0


@pytest.mark.parametrize("bad", [
    dict(S=0), dict(Ts=-1), dict(k=0), dict(k=300), dict(e0=-1), dict(L=0), dict(e0=250, L=8),
])
def test_invalid_dims_rejected(L, bad):
    from combine_expert_histogram_amd import binding as b
    args = dict(S=8, Ts=16, k=8, E=256, e0=0, L=32, H=256)
    args.update(bad)
    with pytest.raises(b.MoeError) as ei:
        b.moe_capacity(b.Dims(**args))
    assert ei.value.status == -1


def test_hidden_must_be_a_multiple_of_128(L):
    from combine_expert_histogram_amd import binding as b
    for H in (0, 64, 200):
        with pytest.raises(b.MoeError):
            b.moe_grouped_gemm1_workspace(b.Dims(S=1, Ts=4, k=2, E=8, e0=0, L=8, H=H), 128)
    with pytest.raises(b.MoeError):
        b.moe_grouped_gemm1_workspace(b.Dims(S=1, Ts=4, k=2, E=8, e0=0, L=8, H=256), 100)


def test_null_pointers_and_short_workspace_rejected_before_any_launch(L):
    from combine_expert_histogram_amd import binding as b
    d = b.Dims(S=1, Ts=64, k=2, E=8, e0=0, L=8, H=256).c()
    P = ctypes.c_void_p
    fake = P(4096)   # never dereferenced: validation fails first
    # null outputs
    assert L.moe_route_layout(ctypes.byref(d), fake, *([None] * 9), fake, 1 << 20, None) == -1
    # workspace too small
    args = [fake] * 10
    assert L.moe_route_layout(ctypes.byref(d), *args, fake, 4, None) == -2
    assert L.moe_quant_dispatch(ctypes.byref(d), None, fake, fake, fake, fake, None) == -1
    assert L.moe_grouped_gemm1(ctypes.byref(d), 256, *([None] * 8), None, 0, None) == -1
    assert L.moe_combine(ctypes.byref(d), 12, fake, 10, fake, fake, fake, None) == -1   # width % 8
    assert L.moe_combine(ctypes.byref(d), 256, fake, 10, None, fake, fake, None) == -1
    # too many local experts for the layout kernels
    big = b.Dims(S=1, Ts=4, k=2, E=4096, e0=0, L=2048).c()
    sz = ctypes.c_size_t()
    assert L.moe_route_layout_workspace(ctypes.byref(big), ctypes.byref(sz)) == -3


def test_empty_input_calls_are_noops(L):
    """T = 0: quant, GEMM1 and combine return MOE_OK without launching."""
    from combine_expert_histogram_amd import binding as b
    d = b.Dims(S=2, Ts=0, k=2, E=8, e0=0, L=8, H=256).c()
    assert L.moe_quant_dispatch(ctypes.byref(d), None, None, None, None, None, None) == 0
    assert L.moe_grouped_gemm1(ctypes.byref(d), 256, *([None] * 8), None, 0, None) == 0
    assert L.moe_combine(ctypes.byref(d), 256, None, 0, None, None, None, None) == 0


def test_stage2_and_mx_workspaces(L):
    from combine_expert_histogram_amd import binding as b
    d = b.Dims(S=8, Ts=2048, k=8, E=256, e0=0, L=32, H=7168)
    # GEMM2: K = inter, n = H; the same table + descriptor layout as GEMM1's
    inter = 2048
    table = ((inter // 128) * ((16384 * 8 + 256 + 63) // 64 * 64) * 4 + 255) // 256 * 256
    desc_end = table + (1 + (16384 * 8 // 128 + 32) * (7168 // 256) + 1024) * 16
    # then one float per row, from a 256 B boundary
    assert b.moe_grouped_gemm2_workspace(d, inter) == (desc_end + 255) // 256 * 256 + 16384 * 8 * 4
    for bad in (0, 64, 200):
        with pytest.raises(b.MoeError):
            b.moe_grouped_gemm2_workspace(d, bad)


def test_stage2_and_mx_validation_before_any_launch(L):
    from combine_expert_histogram_amd import binding as b
    d = b.Dims(S=1, Ts=64, k=2, E=8, e0=0, L=8, H=256).c()
    fake = ctypes.c_void_p(4096)   # never dereferenced: validation fails first
    assert L.moe_quant_dispatch_mx(ctypes.byref(d), None, fake, fake, fake, fake, None) == -1
    assert L.moe_grouped_gemm1_mx(ctypes.byref(d), 256, *([None] * 7), None, 0, None) == -1
    assert L.moe_grouped_gemm1_mx(ctypes.byref(d), 200, *([fake] * 7), fake, 1 << 30, None) == -1   # n % 128
    assert L.moe_silu_mul_quant(ctypes.byref(d), 100, fake, fake, fake, fake, None) == -1          # inter % 128
    assert L.moe_silu_mul_quant(ctypes.byref(d), 128, None, fake, fake, fake, None) == -1
    # GEMM2 needs the row weights (row_assign and topk_w)
    args = [fake, fake, fake, None, fake, fake, fake, fake]
    assert L.moe_grouped_gemm2(ctypes.byref(d), 128, *args, fake, 1 << 30, None) == -1
    # a short workspace
    assert L.moe_grouped_gemm2(ctypes.byref(d), 128, *([fake] * 8), fake, 16, None) == -2
    assert L.moe_grouped_gemm2_mx(ctypes.byref(d), 128, *args, fake, 1 << 30, None) == -1
    assert L.moe_grouped_gemm2_mx(ctypes.byref(d), 128, *([fake] * 8), fake, 16, None) == -2
    assert L.moe_silu_mul_quant_mx(ctypes.byref(d), 100, fake, fake, fake, fake, None) == -1


def test_stage2_and_mx_empty_input_calls_are_noops(L):
    from combine_expert_histogram_amd import binding as b
    d = b.Dims(S=2, Ts=0, k=2, E=8, e0=0, L=8, H=256).c()
    assert L.moe_quant_dispatch_mx(ctypes.byref(d), None, None, None, None, None, None) == 0
    assert L.moe_grouped_gemm1_mx(ctypes.byref(d), 256, *([None] * 7), None, 0, None) == 0
    assert L.moe_silu_mul_quant(ctypes.byref(d), 128, None, None, None, None, None) == 0
    assert L.moe_grouped_gemm2(ctypes.byref(d), 128, *([None] * 8), None, 0, None) == 0
    assert L.moe_silu_mul_quant_mx(ctypes.byref(d), 128, None, None, None, None, None) == 0
    assert L.moe_grouped_gemm2_mx(ctypes.byref(d), 128, *([None] * 8), None, 0, None) == 0


def test_noalloc_layout_size_limit(L):
    """The allocation-free layout holds its workspace in a 256 KiB static array:
    every configuration with T*L <= 2^22 fits it, and a larger one is refused
    with MOE_ERR_WORKSPACE before anything touches the GPU."""
    from combine_expert_histogram_amd import binding as b
    cap = 256 * 1024
    for S, Ts, Lx in ((1, 1 << 21, 1), (1, (1 << 21) - 64, 1), (2, 1 << 20, 2), (8, 2048, 256),
                      (8, 8192, 32), (4, 1024, 1024), (1, 4096, 1000), (8, 2048, 32)):
        d = b.Dims(S=S, Ts=Ts, k=min(8, Lx), E=max(Lx, 8), e0=0, L=Lx)
        assert S * Ts * Lx <= 1 << 22
        assert b.moe_route_layout_workspace(d) <= cap, (S, Ts, Lx)
    big = b.Dims(S=8, Ts=1 << 17, k=8, E=1024, e0=0, L=1024)
    assert b.moe_route_layout_workspace(big) > cap
    P = ctypes.c_void_p
    fake = P(4096)   # never dereferenced: the size check comes first
    assert L.moe_route_layout_noalloc(ctypes.byref(big.c()), *([fake] * 10), None) == -2
    # null outputs are refused like moe_route_layout's
    small = b.Dims(S=1, Ts=64, k=2, E=8, e0=0, L=8)
    assert L.moe_route_layout_noalloc(ctypes.byref(small.c()), fake, *([None] * 9), None) == -1
