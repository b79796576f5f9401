"""GPU parity for K tails: Q4_K rows that end inside their last super-block
(K % 32 == 0, K % 256 != 0; the rest of that super-block is padding that
no result depends on) and Q4_0 rows of an even block count that is not a
multiple of 8 (K % 64 == 0, K % 256 != 0), against the CPU oracle through
the C ABI, to the same bars as the whole-super-block calls: dequantization
bit-exact, GEMV within 1e-4 * sum_k |w x|.  Both kernels are covered:
M = 1, 2 run the VALU kernel (whose last unit is half used when
K % 64 == 32), M >= 3 the matrix-core kernel (whose last 256-column step
is partial).  The padding is drawn random like the rest of the row, and a
second copy with every padding bit flipped must give bit-identical outputs.
"""
import numpy as np
import pytest

from bit_block_quantized_dequant_amd import synth
from gpu_helpers import NT, T, assert_bits, assert_bound, assert_silu, empty, host
from oracle_pins import _q4k_padding_mask

pytestmark = pytest.mark.gpu

Q4K_TAILS = [32, 96, 288, 1408, 2080, 3616]
Q4_0_TAILS = [64, 192, 1408]


def _fits(M, K):
    return M * ((K + 63) // 64) * 64 <= 32768


@pytest.mark.parametrize("K", Q4K_TAILS + [14336])
def test_dequant_q4k_tail(dev, orc, K):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(900 + K)
    N = 37
    w = synth.q4k_matrix(rng, N, K)
    out = empty((N, K), dev)
    q4.dequant_q4k(out, T(w, dev), N, K)
    assert_bits(host(out), orc.dequant_q4k(w, N, K), "dequant_q4k K=%d" % K)


@pytest.mark.parametrize("K", Q4_0_TAILS + [14336])
def test_dequant_q4_0_tail(dev, orc, K):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(950 + K)
    N = 37
    w = synth.q4_0_matrix(rng, N, K)
    out = empty((N, K), dev)
    q4.dequant_q4_0(out, T(w, dev), N, K)
    assert_bits(host(out), orc.dequant_q4_0(w, N, K), "dequant_q4_0 K=%d" % K)


@pytest.mark.parametrize("K", Q4K_TAILS)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 8])
def test_q4k_gemv_tail(dev, orc, M, K):
    import bit_block_quantized_dequant_amd as q4
    if not _fits(M, K):
        pytest.skip("M * K over the staging limit")
    rng = synth.make_rng(1000 + 10 * K + M)
    N = 301
    w = synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, M, K)
    y = empty((M, N), dev)
    q4.q4k_gemv(y, T(w, dev), T(x, dev), M, N, K)
    ref, ab = orc.q4k_gemv(w, x, N, K, NT)
    got = host(y)
    assert_bound(got, ref, ab, "q4k_gemv M=%d K=%d" % (M, K))
    # the padding decides nothing: every padding bit flipped, same outputs
    if K % 256:
        w2 = w ^ _q4k_padding_mask(K)[None, :]
        y2 = empty((M, N), dev)
        q4.q4k_gemv(y2, T(w2, dev), T(x, dev), M, N, K)
        assert np.array_equal(host(y2), got), "padding changed the result, M=%d K=%d" % (M, K)


@pytest.mark.parametrize("K", Q4_0_TAILS)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 8])
def test_q4_0_gemv_tail(dev, orc, M, K):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(1100 + 10 * K + M)
    N = 299
    w = synth.q4_0_matrix(rng, N, K)
    x = synth.activations(rng, M, K)
    y = empty((M, N), dev)
    q4.q4_0_gemv(y, T(w, dev), T(x, dev), M, N, K)
    ref, ab = orc.q4_0_gemv(w, x, N, K, NT)
    assert_bound(host(y), ref, ab, "q4_0_gemv M=%d K=%d" % (M, K))


@pytest.mark.parametrize("fmt,M", [("q4_0", 1), ("q4_0", 2), ("q4k", 1), ("q4k", 2)])
def test_gemv_k14336(dev, orc, fmt, M):
    """The down-projection shape of the 4096 x 14336 dense model: K = 14336
    (224 units per row, many steps per lane)."""
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(1200 + M)
    N, K = 4096, 14336
    w = synth.q4_0_matrix(rng, N, K) if fmt == "q4_0" else synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, M, K)
    y = empty((M, N), dev)
    if fmt == "q4_0":
        q4.q4_0_gemv(y, T(w, dev), T(x, dev), M, N, K)
        ref, ab = orc.q4_0_gemv(w, x, N, K, NT)
    else:
        q4.q4k_gemv(y, T(w, dev), T(x, dev), M, N, K)
        ref, ab = orc.q4k_gemv(w, x, N, K, NT)
    assert_bound(host(y), ref, ab, "%s K=14336 M=%d" % (fmt, M))


@pytest.mark.parametrize("K", [96, 1408, 2080])
@pytest.mark.parametrize("M", [1, 2, 4])
def test_fused_rmsnorm_tail(dev, orc, M, K):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(1300 + K + M)
    N = 257
    w = synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, M, K, 2.0)
    g = synth.gamma(rng, K)
    y = empty((M, N), dev)
    q4.fused_rmsnorm_q4k_gemv(y, T(w, dev), T(x, dev), T(g, dev), 1e-5, M, N, K)
    ref, ab, _ = orc.fused_rmsnorm_q4k_gemv(w, x, g, 1e-5, N, K, NT)
    assert_bound(host(y), ref, ab, "fused_rmsnorm M=%d K=%d" % (M, K))


@pytest.mark.parametrize("K", [288, 1408, 2080])
@pytest.mark.parametrize("M", [1, 2, 4])
def test_gate_up_tail(dev, orc, M, K):
    """gate+up, its SiLU-gated single output, and both behind RMSNorm."""
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(1400 + K + M)
    N = 203
    wg, wu = synth.q4k_matrix(rng, N, K), synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, M, K)
    gam = synth.gamma(rng, K)
    Wg, Wu, X = T(wg, dev), T(wu, dev), T(x, dev)
    g, u = empty((M, N), dev), empty((M, N), dev)
    q4.fused_gate_up_q4k_gemv(g, u, Wg, Wu, X, M, N, K)
    rg, ru, ag, au = orc.gate_up_q4k_gemv(wg, wu, x, N, K, NT)
    assert_bound(host(g), rg, ag, "gate M=%d K=%d" % (M, K))
    assert_bound(host(u), ru, au, "up M=%d K=%d" % (M, K))
    h = empty((M, N), dev)
    q4.fused_gate_up_silu_q4k_gemv(h, Wg, Wu, X, M, N, K)
    assert_silu(orc, host(h), rg, ru, ag, au, "gate_up_silu M=%d K=%d" % (M, K))
    xh = orc.rmsnorm(x, gam, 1e-5)
    ng, nu, nag, nau = orc.gate_up_q4k_gemv(wg, wu, xh, N, K, NT)
    g2, u2 = empty((M, N), dev), empty((M, N), dev)
    q4.fused_rmsnorm_gate_up_q4k_gemv(g2, u2, Wg, Wu, X, T(gam, dev), 1e-5, M, N, K)
    assert_bound(host(g2), ng, nag, "norm gate M=%d K=%d" % (M, K))
    assert_bound(host(u2), nu, nau, "norm up M=%d K=%d" % (M, K))
    h2 = empty((M, N), dev)
    q4.fused_rmsnorm_gate_up_silu_q4k_gemv(h2, Wg, Wu, X, T(gam, dev), 1e-5, M, N, K)
    assert_silu(orc, host(h2), ng, nu, nag, nau, "norm gate_up_silu M=%d K=%d" % (M, K))


@pytest.mark.parametrize("M", [1, 4])
def test_moe_and_router_k1408(dev, orc, M):
    """The expert gate/up call and the router at K = 1408 (44 Q4_0 blocks)."""
    import torch
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(1500 + M)
    E, N, K, top_k = 16, 160, 1408, 4
    wg, wu = synth.q4_0_matrix(rng, E * N, K), synth.q4_0_matrix(rng, E * N, K)
    x = synth.activations(rng, M, K)
    ids = synth.expert_ids(rng, M, top_k, E)
    g, u = empty((M, top_k, N), dev), empty((M, top_k, N), dev)
    q4.moe_q4_gemv(g, u, T(wg, dev), T(wu, dev), T(x, dev), T(ids, dev), M, top_k, E, N, K)
    rg, ru, ag, au = orc.moe_q4_0_gemv(wg, wu, x, ids, E, N, K, NT)
    assert_bound(host(g), rg, ag, "moe gate K=1408 M=%d" % M)
    assert_bound(host(u), ru, au, "moe up K=1408 M=%d" % M)
    wr = synth.q4_0_matrix(rng, 64, K)
    ri = empty((M, 6), dev, torch.int32)
    rw = empty((M, 6), dev)
    q4.moe_router_q4_0(ri, rw, T(wr, dev), T(x, dev), M, 64, K, 6, 1)
    want_ids, _, lg, ab = orc.moe_router_q4_0(wr, x, 64, K, 6, True)
    got_ids = host(ri)
    # selections equal where the logits are further apart than the bound
    for m in range(M):
        order = np.argsort(-lg[m], kind="stable")
        gap = np.abs(np.diff(lg[m][order[:7]]))
        tol = 2e-4 * ab[m][order[:7]].max()
        if np.all(gap > tol):
            assert np.array_equal(got_ids[m], want_ids[m]), m


def _q4k_read_checksum(w, K):
    """Word sums of what a Q4_K call reads per row: every super-block header,
    and every 32-byte nibble chunk that holds an element < K."""
    N = w.shape[0]
    S = (K + 255) // 256
    words = np.ascontiguousarray(w).reshape(N, S, 144).view("<u4").astype(np.uint64)
    tot = words[:, :, :4].sum(axis=(1, 2))
    for s in range(S):
        for g in range(4):
            if 256 * s + 64 * g < K:
                tot += words[:, s, 4 + 8 * g:12 + 8 * g].sum(axis=1)
    return (tot % (1 << 32)).astype(np.uint32)


@pytest.mark.parametrize("M", [1, 2, 3, 8])
def test_pure_read_tail_checksums(dev, orc, M):
    """The pure-read mirror of a tail call reads what the call reads: the
    headers and the nibble chunks holding elements < K (a padding chunk of
    the last super-block is never read), for both kernels."""
    import torch
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(1600 + M)
    for K in (96, 288, 2080):
        if not _fits(M, K):
            continue
        N = 131
        w0 = synth.q4k_matrix(rng, N, K)
        c = empty((N,), dev, torch.int32)
        q4.q4_pure_read(c, q4.Q4_READ_Q4K_GEMV, T(w0, dev), None, None, M, 0, 0, N, K)
        assert np.array_equal(host(c).view(np.uint32), _q4k_read_checksum(w0, K)), (M, K)
    for K in (192, 1408):
        N = 133
        w0 = synth.q4_0_matrix(rng, N, K)
        c = empty((N,), dev, torch.int32)
        q4.q4_pure_read(c, q4.Q4_READ_Q4_0_GEMV, T(w0, dev), None, None, M, 0, 0, N, K)
        want = orc.row_checksum(w0, N, synth.q4_0_row_bytes(K))
        assert np.array_equal(host(c).view(np.uint32), want), (M, K)


@pytest.mark.parametrize("K", [64, 192])
def test_router_short_rows(dev, orc, K):
    """Router rows of one and three block pairs (lane groups of 4)."""
    import torch
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(1700 + K)
    M, E, top_k = 3, 40, 5
    wr = synth.q4_0_matrix(rng, E, K)
    x = synth.activations(rng, M, K)
    ri = empty((M, top_k), dev, torch.int32)
    rw = empty((M, top_k), dev)
    q4.moe_router_q4_0(ri, rw, T(wr, dev), T(x, dev), M, E, K, top_k, 1)
    want_ids, want_w, lg, ab = orc.moe_router_q4_0(wr, x, E, K, top_k, True)
    got_ids, got_w = host(ri), host(rw)
    for m in range(M):
        order = np.argsort(-lg[m], kind="stable")
        gap = np.abs(np.diff(lg[m][order[:top_k + 1]]))
        if np.all(gap > 2e-4 * ab[m].max()):
            assert np.array_equal(got_ids[m], want_ids[m]), m
            assert np.allclose(got_w[m], want_w[m], rtol=1e-3, atol=1e-6), m
