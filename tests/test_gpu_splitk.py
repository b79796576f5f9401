"""GPU parity of the split-K batched GEMV (q4_0_gemv_splitk, q4k_gemv_splitk)
against the CPU oracle through the C ABI, within 1e-4 * sum_k |w x|: the
batched Q4_0 workload's shape, long K, K tails, ragged N, 16 tokens; tokens
whose K parts differ wildly in magnitude or are all zero (each part has its
own power-of-two scale, merged at a common one); a token's row does not
depend on the batch (the split depends on N, K and the device only); one
workspace serves call after call and holds nothing between calls; and the
workspace checks."""
import ctypes

import numpy as np
import pytest

from bit_block_quantized_dequant_amd import synth
from gpu_helpers import NT, T, assert_bits, assert_bound, empty, host

pytestmark = pytest.mark.gpu

Q4_0, Q4K = 0, 1


def ws_bytes(fmt, M, N, K):
    import bit_block_quantized_dequant_amd as q4
    b = ctypes.c_int64(-1)
    st = q4.lib().q4_splitk_workspace(fmt, M, N, K, ctypes.byref(b))
    assert st == 0, q4.q4_strerror(st)
    return b.value


def workspace(dev, nbytes):
    import torch
    # any content: filled with garbage on purpose
    return torch.full((max(nbytes, 256),), 0x7F, dtype=torch.uint8, device=dev)


def run(dev, fmt, y, w, x, M, N, K, ws):
    import bit_block_quantized_dequant_amd as q4
    L = q4.lib()
    f = L.q4_0_gemv_splitk if fmt == Q4_0 else L.q4k_gemv_splitk
    st = f(ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(w.data_ptr()),
           ctypes.c_void_p(x.data_ptr()), M, N, K, ctypes.c_void_p(ws.data_ptr()),
           ws.numel(), None)
    assert st == 0, q4.q4_strerror(st)


def case(dev, orc, fmt, M, N, K, seed, x=None, ws=None):
    rng = synth.make_rng(seed)
    w = synth.q4_0_matrix(rng, N, K) if fmt == Q4_0 else synth.q4k_matrix(rng, N, K)
    if x is None:
        x = synth.activations(rng, M, K)
    if ws is None:
        ws = workspace(dev, ws_bytes(fmt, M, N, K))
    y = empty((M, N), dev)
    run(dev, fmt, y, T(w, dev), T(x, dev), M, N, K, ws)
    ref, ab = (orc.q4_0_gemv if fmt == Q4_0 else orc.q4k_gemv)(w, x, N, K, NT)
    got = host(y)
    assert_bound(got, ref, ab, "splitk fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K))
    return got, w, x, ws


@pytest.mark.parametrize("fmt,M,N,K", [
    (Q4_0, 3, 4096, 4096), (Q4_0, 4, 4096, 4096), (Q4_0, 8, 4096, 4096),
    (Q4_0, 16, 4096, 4096), (Q4K, 4, 4096, 14336), (Q4K, 16, 2048, 4096),
    (Q4_0, 5, 777, 1408), (Q4K, 6, 513, 2080), (Q4K, 8, 33, 32768), (Q4_0, 12, 16, 4096),
    # rows of more than 256 steps with many tile groups: parts of 6-7 steps,
    # staged in two passes from global memory
    (Q4_0, 3, 1024, 131072), (Q4K, 12, 512, 98304),
])
def test_splitk_parity(dev, orc, fmt, M, N, K):
    assert ws_bytes(fmt, M, N, K) > 0
    case(dev, orc, fmt, M, N, K, 6000 + M + N + K)


def test_splitk_part_magnitudes(dev, orc):
    """Tokens whose K parts differ by up to 2^200 in magnitude, a token zero
    in most parts, an all-zero token."""
    rng = synth.make_rng(6100)
    M, N, K = 6, 1024, 4096
    x = synth.activations(rng, M, K)
    x[0, :2048] *= np.float32(2.0 ** 100)
    x[0, 2048:] *= np.float32(2.0 ** -100)
    x[1, :3840] = 0.0
    x[2] = 0.0
    x[3] *= np.float32(2.0 ** -120)
    x[4, ::2] *= np.float32(2.0 ** 60)
    got, *_ = case(dev, orc, Q4_0, M, N, K, 6101, x=x)
    assert np.all(got[2] == 0.0)


@pytest.mark.parametrize("fmt", [Q4_0, Q4K])
def test_splitk_rows_independent_of_batch(dev, fmt):
    rng = synth.make_rng(6200 + fmt)
    N, K = 2048, 4096
    w = synth.q4_0_matrix(rng, N, K) if fmt == Q4_0 else synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, 16, K)
    wd = T(w, dev)
    ws = workspace(dev, ws_bytes(fmt, 16, N, K))
    yb = empty((16, N), dev)
    run(dev, fmt, yb, wd, T(x, dev), 16, N, K, ws)
    yb = host(yb)
    for sub in ([5, 0, 9], [15, 1, 2, 3, 4, 6, 7, 8], list(range(10))):
        ys = empty((len(sub), N), dev)
        run(dev, fmt, ys, wd, T(x[sub], dev), len(sub), N, K, ws)
        ys = host(ys)
        for j, m in enumerate(sub):
            assert_bits(ys[j], yb[m], "split-K fmt %d token %d in a batch of %d" % (fmt, m, len(sub)))


def test_splitk_workspace_reuse(dev, orc):
    """One workspace, call after call and shape after shape; repeated calls
    are bit-identical."""
    big = max(ws_bytes(Q4_0, 16, 4096, 4096), ws_bytes(Q4K, 8, 3000, 8192))
    ws = workspace(dev, big)
    a1, w, x, _ = case(dev, orc, Q4_0, 8, 4096, 4096, 6300, ws=ws)
    case(dev, orc, Q4K, 8, 3000, 8192, 6301, ws=ws)
    case(dev, orc, Q4_0, 16, 4096, 4096, 6302, ws=ws)
    y = empty((8, 4096), dev)
    for _ in range(3):
        run(dev, Q4_0, y, T(w, dev), T(x, dev), 8, 4096, 4096, ws)
        assert_bits(host(y), a1, "repeated split-K call")


def test_splitk_workspace_checks(dev):
    import torch
    import bit_block_quantized_dequant_amd as q4
    L = q4.lib()
    M, N, K = 8, 4096, 4096
    need = ws_bytes(Q4_0, M, N, K)
    w = torch.zeros(N * K // 32 * 18, dtype=torch.uint8, device=dev)
    x = torch.zeros(M * K, device=dev)
    y = torch.zeros(M * N, device=dev)
    ws = torch.zeros(need + 512, dtype=torch.uint8, device=dev)
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)
    assert L.q4_0_gemv_splitk(P(y), P(w), P(x), M, N, K, P(ws), need - 256, None) == 2
    assert L.q4_0_gemv_splitk(P(y), P(w), P(x), M, N, K, None, need, None) == 1
    assert L.q4_0_gemv_splitk(P(y), P(w), P(x), M, N, K, P(ws, 16), need, None) == 4
    # M <= 2 needs no workspace (the VALU kernel runs)
    assert ws_bytes(Q4_0, 2, N, K) == 0
    assert L.q4_0_gemv_splitk(P(y), P(w), P(x), 2, N, K, None, 0, None) == 0
    torch.cuda.synchronize()
    assert np.all(host(y)[:2 * N] == 0.0)
    b = ctypes.c_int64(0)
    assert L.q4_splitk_workspace(7, M, N, K, ctypes.byref(b)) == 5
