"""The benchmark's measurement kernels (libmoe_ceiling.so, not part of the hot
path's C ABI): the library exports them, and on the GPU each computes what its
rate assumes it moves — the read stream folds every word of its buffer, the
read/write streams write every output word from its two, four or eight source
words — so a ceiling the benchmark reports is a measured pass over all of its
bytes."""
import ctypes
import os

import numpy as np
import pytest

from combine_expert_histogram_amd import build as cbuild

SYMBOLS = ("moe_ceiling_read_stream", "moe_ceiling_rw_stream", "moe_ceiling_mfma_fp8",
           "moe_ceiling_mfma_fp8_scaled")


def _lib():
    if not os.path.exists(cbuild.CEILING_LIB):
        pytest.skip("libmoe_ceiling.so not built")
    lib = ctypes.CDLL(cbuild.CEILING_LIB)
    lib.moe_ceiling_read_stream.restype = ctypes.c_int
    lib.moe_ceiling_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_void_p]
    lib.moe_ceiling_rw_stream.restype = ctypes.c_int
    lib.moe_ceiling_rw_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_void_p]
    return lib


def test_ceiling_library_exports_its_kernels():
    lib = _lib()
    for name in SYMBOLS:
        assert hasattr(lib, name), name


def test_ceiling_calls_reject_bad_arguments_without_launching():
    lib = _lib()
    # null buffers, sizes that are not whole 16 B words, empty grids: -1 before any launch
    assert lib.moe_ceiling_rw_stream(None, None, 1024, 2, None) == -1
    assert lib.moe_ceiling_rw_stream(ctypes.c_void_p(16), ctypes.c_void_p(16), 1000, 2, None) == -1
    assert lib.moe_ceiling_rw_stream(ctypes.c_void_p(16), ctypes.c_void_p(16), 1024, 3, None) == -1
    assert lib.moe_ceiling_read_stream(None, 1024, 4, 0, ctypes.c_void_p(16), None) == -1
    assert lib.moe_ceiling_read_stream(ctypes.c_void_p(16), 1000, 4, 0, ctypes.c_void_p(16), None) == -1


@pytest.mark.gpu
@pytest.mark.parametrize("ratio", [2, 4, 8])
@pytest.mark.parametrize("out_words", [1 << 16, 123457, 37])
def test_rw_stream_writes_the_xor_of_each_source_group(out_words, ratio):
    import torch
    from gpu_helpers import require_gpu, say
    require_gpu()
    say(f"rw stream {out_words} words, ratio {ratio}")
    lib = _lib()
    rng = np.random.default_rng(5)
    src = rng.integers(0, 2**32, size=(ratio, out_words, 4), dtype=np.uint32)
    src_d = torch.from_numpy(src.view(np.int32)).cuda()
    dst_d = torch.full((out_words, 4), -7, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    assert lib.moe_ceiling_rw_stream(ctypes.c_void_p(src_d.data_ptr()), ctypes.c_void_p(dst_d.data_ptr()),
                                     out_words * 16, ratio, ctypes.c_void_p(st.cuda_stream)) == 0
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(src, axis=0)
    assert np.array_equal(dst_d.cpu().numpy().view(np.uint32), want)


@pytest.mark.gpu
@pytest.mark.parametrize("temporal", [0, 1])
def test_read_stream_folds_every_word(temporal):
    import torch
    from gpu_helpers import require_gpu, say
    require_gpu()
    say(f"read stream temporal={temporal}")
    lib = _lib()
    words = (1 << 20) + 5 * 4                       # a ragged tail past the last full pass
    rng = np.random.default_rng(6)
    buf = rng.integers(0, 2**32, size=words, dtype=np.uint32)
    buf_d = torch.from_numpy(buf.view(np.int32)).cuda()
    grid = 96
    out_d = torch.zeros(grid * 256, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    assert lib.moe_ceiling_read_stream(ctypes.c_void_p(buf_d.data_ptr()), words * 4, grid, temporal,
                                       ctypes.c_void_p(out_d.data_ptr()), ctypes.c_void_p(st.cuda_stream)) == 0
    torch.cuda.synchronize()
    # every thread folds the words it loaded by xor; together they cover the buffer once
    got = np.bitwise_xor.reduce(out_d.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(buf)
