"""GPU parity for batches of 9 to 16 token rows (two 8-token A tiles on the
matrix cores) and for calls whose activations do not fit in LDS at once
(staged in K slices), against the CPU oracle through the C ABI, within
1e-4 * sum_k |w x|; plus the design's bit-identity: a token's row does not
depend on the batch it is computed in, whether the batch is staged whole or
in slices (each wave keeps its K range and its step order)."""
import numpy as np
import pytest

from bit_block_quantized_dequant_amd import synth
from gpu_helpers import NT, T, assert_bits, assert_bound, assert_silu, empty, host

pytestmark = pytest.mark.gpu


def _gemv(dev, orc, fmt, M, N, K, seed, sigma=1.0):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(seed)
    w = synth.q4_0_matrix(rng, N, K) if fmt == "q4_0" else synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, M, K, sigma)
    y = empty((M, N), dev)
    (q4.q4_0_gemv if fmt == "q4_0" else q4.q4k_gemv)(y, T(w, dev), T(x, dev), M, N, K)
    ref, ab = (orc.q4_0_gemv if fmt == "q4_0" else orc.q4k_gemv)(w, x, N, K, NT)
    assert_bound(host(y), ref, ab, "%s M=%d N=%d K=%d" % (fmt, M, N, K))


@pytest.mark.parametrize("fmt", ["q4_0", "q4k"])
@pytest.mark.parametrize("M", [9, 10, 11, 12, 13, 14, 15, 16])
def test_batches_9_to_16(dev, orc, fmt, M):
    """Whole-row staging (K = 2048) for every M of the second tile."""
    _gemv(dev, orc, fmt, M, 333, 2048, 3000 + M)


@pytest.mark.parametrize("fmt,M,N,K", [
    ("q4_0", 16, 4096, 4096),   # 8 waves per tile: wave positions staged in 2 groups
    ("q4k", 16, 1000, 4096),
    ("q4k", 4, 4096, 14336),    # the dense down-projection at batch 4
    ("q4_0", 4, 1500, 14336),
    ("q4k", 8, 700, 8192),
    ("q4_0", 3, 513, 16384),
    ("q4k", 2, 257, 16448),     # M = 2 beyond the VALU kernel's staging
    ("q4_0", 2, 300, 16448),
    ("q4k", 12, 301, 3616),     # K tail, 12 tokens
    ("q4k", 16, 77, 32768),
])
def test_sliced_staging(dev, orc, fmt, M, N, K):
    _gemv(dev, orc, fmt, M, N, K, 3100 + M + K)


@pytest.mark.parametrize("M,K", [(16, 4096), (12, 2048), (5, 14336)])
def test_wide_rmsnorm_and_pair_calls(dev, orc, M, K):
    """RMSNorm, gate+up and their SiLU-gated and fused forms at wide or
    sliced shapes."""
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(3200 + M + K)
    N = 203
    wg, wu = synth.q4k_matrix(rng, N, K), synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, M, K, 2.0)
    gam = synth.gamma(rng, K)
    Wg, Wu, X, G = T(wg, dev), T(wu, dev), T(x, dev), T(gam, dev)
    y = empty((M, N), dev)
    q4.fused_rmsnorm_q4k_gemv(y, Wg, X, G, 1e-5, M, N, K)
    ref, ab, _ = orc.fused_rmsnorm_q4k_gemv(wg, x, gam, 1e-5, N, K, NT)
    assert_bound(host(y), ref, ab, "rmsnorm M=%d K=%d" % (M, K))
    g, u = empty((M, N), dev), empty((M, N), dev)
    q4.fused_gate_up_q4k_gemv(g, u, Wg, Wu, X, M, N, K)
    rg, ru, ag, au = orc.gate_up_q4k_gemv(wg, wu, x, N, K, NT)
    assert_bound(host(g), rg, ag, "gate M=%d K=%d" % (M, K))
    assert_bound(host(u), ru, au, "up M=%d K=%d" % (M, K))
    h = empty((M, N), dev)
    q4.fused_gate_up_silu_q4k_gemv(h, Wg, Wu, X, M, N, K)
    assert_silu(orc, host(h), rg, ru, ag, au, "silu M=%d K=%d" % (M, K))
    xh = orc.rmsnorm(x, gam, 1e-5)
    ng, nu, nag, nau = orc.gate_up_q4k_gemv(wg, wu, xh, N, K, NT)
    h2 = empty((M, N), dev)
    q4.fused_rmsnorm_gate_up_silu_q4k_gemv(h2, Wg, Wu, X, G, 1e-5, M, N, K)
    assert_silu(orc, host(h2), ng, nu, nag, nau, "norm silu M=%d K=%d" % (M, K))


@pytest.mark.parametrize("fmt,N,K", [("q4_0", 777, 4096), ("q4k", 777, 4096),
                                     ("q4k", 300, 14336)])
def test_rows_independent_of_batch_and_slicing(dev, fmt, N, K):
    """A token's row is bit-identical in batches of 3..16, staged whole
    (small M) or in K slices (large M): every wave keeps its K range and
    its step order."""
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(3300 + K)
    w = synth.q4_0_matrix(rng, N, K) if fmt == "q4_0" else synth.q4k_matrix(rng, N, K)
    f = q4.q4_0_gemv if fmt == "q4_0" else q4.q4k_gemv
    x = synth.activations(rng, 16, K)
    x[3] *= np.float32(2.0 ** 40)
    x[11] *= np.float32(2.0 ** -50)
    wd = T(w, dev)
    yb = empty((16, N), dev)
    f(yb, wd, T(x, dev), 16, N, K)
    yb = host(yb)
    for sub in ([11, 3, 0], [15, 14, 13, 12, 11, 10, 9, 8, 7], [3, 11, 5, 6],
                list(range(12))):
        ys = empty((len(sub), N), dev)
        f(ys, wd, T(x[sub], dev), len(sub), N, K)
        ys = host(ys)
        for j, m in enumerate(sub):
            assert_bits(ys[j], yb[m], "%s K=%d token %d at row %d of %d vs row %d of 16"
                        % (fmt, K, m, j, len(sub), m))


@pytest.mark.parametrize("M,K", [(16, 4096), (4, 14336), (12, 2048)])
def test_wide_pure_read_checksums(dev, orc, M, K):
    import torch
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(3400 + M + K)
    N = 301
    for fmt, kid in (("q4_0", q4.Q4_READ_Q4_0_GEMV), ("q4k", q4.Q4_READ_Q4K_GEMV)):
        w = synth.q4_0_matrix(rng, N, K) if fmt == "q4_0" else synth.q4k_matrix(rng, N, K)
        rb = synth.q4_0_row_bytes(K) if fmt == "q4_0" else synth.q4k_row_bytes(K)
        c = empty((N,), dev, torch.int32)
        q4.q4_pure_read(c, kid, T(w, dev), None, None, M, 0, 0, N, K)
        assert np.array_equal(host(c).view(np.uint32), orc.row_checksum(w, N, rb)), (fmt, M, K)
