"""GPU parity for the activation staging's batched tails: rows longer than
the chunks each thread holds in registers are staged in batches of loads
(the single-token call with rows over 64 units, the two-token VALU call,
the expert call at K > 2048, the expert down-projection's pair rows, and the
batched kernel's K-sliced staging).  The K values leave a last batch that
is partly past the end of the rows, and some end in a half-used 64-weight
unit (K % 64 == 32; Q4_0 rows, whose K is a multiple of 64, take the K
below).  Against the CPU oracle through the C ABI, within 1e-4 * sum_k |w x|.
"""
import numpy as np
import pytest

from bit_block_quantized_dequant_amd import synth
from gpu_helpers import NT, T, assert_bound, empty, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K", [4128, 8224, 14368, 32768])
def test_single_token_long_rows(dev, orc, K):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(7000 + K)
    N = 97
    K0 = K // 64 * 64
    wk, w0 = synth.q4k_matrix(rng, N, K), synth.q4_0_matrix(rng, N, K0)
    x = synth.activations(rng, 1, K)
    g = synth.gamma(rng, K)
    y = empty((1, N), dev)
    q4.q4k_gemv(y, T(wk, dev), T(x, dev), 1, N, K)
    ref, ab = orc.q4k_gemv(wk, x, N, K, NT)
    assert_bound(host(y), ref, ab, "q4k_gemv M=1 K=%d" % K)
    x0 = np.ascontiguousarray(x[:, :K0])
    q4.q4_0_gemv(y, T(w0, dev), T(x0, dev), 1, N, K0)
    ref, ab = orc.q4_0_gemv(w0, x0, N, K0, NT)
    assert_bound(host(y), ref, ab, "q4_0_gemv M=1 K=%d" % K0)
    q4.fused_rmsnorm_q4k_gemv(y, T(wk, dev), T(x, dev), T(g, dev), 1e-5, 1, N, K)
    ref, ab, _ = orc.fused_rmsnorm_q4k_gemv(wk, x, g, 1e-5, N, K, NT)
    assert_bound(host(y), ref, ab, "fused_rmsnorm M=1 K=%d" % K)


@pytest.mark.parametrize("K", [4160, 8224, 16384])
def test_two_tokens_long_rows(dev, orc, K):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(7100 + K)
    N = 131
    K0 = K // 64 * 64
    w0 = synth.q4_0_matrix(rng, N, K0)
    x = synth.activations(rng, 2, K)
    g = synth.gamma(rng, K)
    wk = synth.q4k_matrix(rng, N, K)
    y = empty((2, N), dev)
    x0 = np.ascontiguousarray(x[:, :K0])
    q4.q4_0_gemv(y, T(w0, dev), T(x0, dev), 2, N, K0)
    ref, ab = orc.q4_0_gemv(w0, x0, N, K0, NT)
    assert_bound(host(y), ref, ab, "q4_0_gemv M=2 K=%d" % K0)
    q4.fused_rmsnorm_q4k_gemv(y, T(wk, dev), T(x, dev), T(g, dev), 1e-5, 2, N, K)
    ref, ab, _ = orc.fused_rmsnorm_q4k_gemv(wk, x, g, 1e-5, N, K, NT)
    assert_bound(host(y), ref, ab, "fused_rmsnorm M=2 K=%d" % K)


@pytest.mark.parametrize("M,K", [(4, 4096), (3, 2112), (8, 4096), (1, 8256)])
def test_expert_calls_long_rows(dev, orc, M, K):
    """The gate/up expert call (tail staging beyond 2048 columns per token)
    and the down-projection (pair rows staged in batches) on the same ids."""
    import bit_block_quantized_dequant_amd as q4
    E, top_k, N = 12, 3, 45
    rng = synth.make_rng(7200 + M + K)
    wg, wu = synth.q4_0_matrix(rng, E * N, K), synth.q4_0_matrix(rng, E * N, K)
    wd = synth.q4_0_matrix(rng, E * N, K)
    x = synth.activations(rng, M, K)
    h = synth.activations(rng, M * top_k, K).reshape(M, top_k, K)
    ids = synth.expert_ids(rng, M, top_k, E)
    ids[0, 0] = ids[M - 1, top_k - 1]  # one expert shared by two tokens
    if M == 1:
        ids[0, 1] = ids[0, 0]          # (or listed twice by one token)
    g, u = empty((M, top_k, N), dev), empty((M, top_k, N), dev)
    q4.moe_q4_gemv(g, u, T(wg, dev), T(wu, dev), T(x, dev), T(ids, dev), M, top_k, E, N, K)
    rg, ru, ag, au = orc.moe_q4_0_gemv(wg, wu, x, ids, E, N, K, NT)
    assert_bound(host(g), rg, ag, "moe gate M=%d K=%d" % (M, K))
    assert_bound(host(u), ru, au, "moe up M=%d K=%d" % (M, K))
    yd = empty((M, top_k, N), dev)
    q4.moe_q4_gemv_down(yd, T(wd, dev), T(h, dev), T(ids, dev), M, top_k, E, N, K)
    rd, ad = orc.moe_q4_0_down(wd, h, ids, E, N, K, NT)
    assert_bound(host(yd), rd, ad, "moe down M=%d K=%d" % (M, K))


@pytest.mark.parametrize("M,K", [(16, 4096), (12, 8224), (5, 14368)])
def test_sliced_batches(dev, orc, M, K):
    """Batches whose staged rows do not fit in LDS at once (K-sliced
    staging), both formats and the RMSNorm call."""
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(7300 + M + K)
    N = 150
    K0 = K // 64 * 64
    wk, w0 = synth.q4k_matrix(rng, N, K), synth.q4_0_matrix(rng, N, K0)
    x = synth.activations(rng, M, K)
    g = synth.gamma(rng, K)
    y = empty((M, N), dev)
    q4.q4k_gemv(y, T(wk, dev), T(x, dev), M, N, K)
    ref, ab = orc.q4k_gemv(wk, x, N, K, NT)
    assert_bound(host(y), ref, ab, "q4k_gemv M=%d K=%d" % (M, K))
    x0 = np.ascontiguousarray(x[:, :K0])
    q4.q4_0_gemv(y, T(w0, dev), T(x0, dev), M, N, K0)
    ref, ab = orc.q4_0_gemv(w0, x0, N, K0, NT)
    assert_bound(host(y), ref, ab, "q4_0_gemv M=%d K=%d" % (M, K0))
    q4.fused_rmsnorm_q4k_gemv(y, T(wk, dev), T(x, dev), T(g, dev), 1e-5, M, N, K)
    ref, ab, _ = orc.fused_rmsnorm_q4k_gemv(wk, x, g, 1e-5, N, K, NT)
    assert_bound(host(y), ref, ab, "fused_rmsnorm M=%d K=%d" % (M, K))
