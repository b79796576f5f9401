"""The allocation-free split-K entry point (q4_0_gemv_splitk_noalloc) against
the entry point it is a variant of (q4_0_gemv_splitk with a caller
workspace), through the C ABI: bit-identical outputs, on two calls in a row,
the second with a smaller input (the library's array keeps the first call's
contents, which the second must not depend on)."""
import ctypes

import numpy as np
import pytest

from bit_block_quantized_dequant_amd import synth
from gpu_helpers import T, assert_bits, empty, host

pytestmark = pytest.mark.gpu


def _splitk(dev, w, x, M, N, K):
    import torch
    import bit_block_quantized_dequant_amd as q4
    L = q4.lib()
    b = ctypes.c_int64(0)
    assert L.q4_splitk_workspace(0, M, N, K, ctypes.byref(b)) == 0
    ws = torch.full((max(b.value, 256),), 0x5A, dtype=torch.uint8, device=dev)
    y = empty((M, N), dev)
    st = L.q4_0_gemv_splitk(ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                            ctypes.c_void_p(x.data_ptr()), M, N, K,
                            ctypes.c_void_p(ws.data_ptr()), b.value, None)
    assert st == 0, q4.q4_strerror(st)
    return host(y)


def _noalloc(dev, w, x, M, N, K):
    import bit_block_quantized_dequant_amd as q4
    y = empty((M, N), dev)
    st = q4.lib().q4_0_gemv_splitk_noalloc(ctypes.c_void_p(y.data_ptr()),
                                           ctypes.c_void_p(w.data_ptr()),
                                           ctypes.c_void_p(x.data_ptr()), M, N, K, None)
    assert st == 0, q4.q4_strerror(st)
    return host(y)


def test_noalloc_equals_workspace_call_twice(dev):
    import bit_block_quantized_dequant_amd as q4
    assert q4.lib().q4_noalloc_scratch_bytes() == 8 << 20
    rng = synth.make_rng(7000)
    # first call: 16 tokens, 4096 rows (about 2 MiB of the array); second:
    # a smaller one, 5 tokens of 777 rows with K = 1408
    for M, N, K in ((16, 4096, 4096), (5, 777, 1408)):
        w = synth.q4_0_matrix(rng, N, K)
        x = synth.activations(rng, M, K)
        wd, xd = T(w, dev), T(x, dev)
        a = _noalloc(dev, wd, xd, M, N, K)
        b = _splitk(dev, wd, xd, M, N, K)
        assert not np.any(np.isnan(a))
        assert_bits(a, b, "noalloc vs workspace M=%d N=%d K=%d" % (M, N, K))


def test_noalloc_refuses_beyond_its_array(dev):
    import bit_block_quantized_dequant_amd as q4
    L = q4.lib()
    # at the longest K each part's staging must fit in LDS, so the K split
    # takes about 200 parts: partials of about 56 MiB for 4096 rows
    M, N, K = 16, 4096, 1 << 20
    b = ctypes.c_int64(0)
    assert L.q4_splitk_workspace(0, M, N, K, ctypes.byref(b)) == 0
    assert b.value > L.q4_noalloc_scratch_bytes()
    # refused on the host before anything is launched
    A = ctypes.c_void_p(0x7F0000000000)
    assert L.q4_0_gemv_splitk_noalloc(A, A, A, M, N, K, None) == 2
    # a shape that fits still runs (the split-K path, with the array)
    assert L.q4_splitk_workspace(0, 8, 4096, 4096, ctypes.byref(b)) == 0
    assert 0 < b.value <= L.q4_noalloc_scratch_bytes()
