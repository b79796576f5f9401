"""GPU parity of the expert down-projection (moe_q4_gemv_down) against the
CPU oracle through the C ABI: every (token, slot) pair's own input row times
the Q4_0 down matrix of its expert, within 1e-4 * sum_k |w h| per output.
Cases: the decode shape that follows the expert gate/up call (4 tokens,
top-6 of 64 experts, 2048 rows of K = 1408), every batch M = 1..8, experts
shared by several tokens, a token that lists one expert several times (more
pairs for one expert than staged rows at once), invalid ids (NaN rows), and
the pure-read mirror's checksums."""
import numpy as np
import pytest

from bit_block_quantized_dequant_amd import synth
from gpu_helpers import NT, T, assert_bound, empty, host

pytestmark = pytest.mark.gpu


def _down(dev, orc, wd, h, ids, E, N, K, what):
    import bit_block_quantized_dequant_amd as q4
    M, top_k = ids.shape
    y = empty((M, top_k, N), dev)
    q4.moe_q4_gemv_down(y, T(wd, dev), T(h, dev), T(ids, dev), M, top_k, E, N, K)
    ref, ab = orc.moe_q4_0_down(wd, h, ids, E, N, K, NT)
    got = host(y)
    bad = (ids < 0) | (ids >= E)
    assert np.all(np.isnan(got[bad])), "%s: invalid pairs must be NaN" % what
    ok = ~bad
    assert_bound(got[ok], ref[ok], ab[ok], what)
    return got


def test_down_decode_shape(dev, orc):
    """4 tokens, top-6 of 64 experts, N = 2048 rows, K = 1408 (the width of
    the gated activation of the expert gate/up workload)."""
    rng = synth.make_rng(2001)
    M, top_k, E, N, K = 4, 6, 64, 2048, 1408
    wd = synth.q4_0_matrix(rng, E * N, K)
    h = synth.pair_activations(rng, M, top_k, K)
    ids = synth.expert_ids(rng, M, top_k, E)
    _down(dev, orc, wd, h, ids, E, N, K, "down M=4 top6 E=64")


@pytest.mark.parametrize("M", [1, 2, 3, 5, 6, 7, 8])
def test_down_batches(dev, orc, M):
    rng = synth.make_rng(2010 + M)
    top_k, E, N, K = 6, 64, 301, 1408
    wd = synth.q4_0_matrix(rng, E * N, K)
    h = synth.pair_activations(rng, M, top_k, K)
    ids = synth.expert_ids(rng, M, top_k, E)
    _down(dev, orc, wd, h, ids, E, N, K, "down M=%d" % M)


def test_down_shared_repeated_and_invalid_ids(dev, orc):
    rng = synth.make_rng(2020)
    E, N, K = 9, 130, 192
    wd = synth.q4_0_matrix(rng, E * N, K)
    # token 0 lists expert 5 three times (three pairs of one expert, one
    # token: staged one row at a time when M = 1); experts shared across
    # tokens; ids outside [0, E)
    for ids in (np.array([[5, 5, 2, 5]], np.int32),
                np.array([[1, 4, 8], [4, 1, 0], [8, 4, 7], [2, 9, -1]], np.int32),
                np.array([[3, 3], [3, 3], [3, 3]], np.int32),
                np.array([[-5, 100]], np.int32)):
        M, top_k = ids.shape
        h = synth.pair_activations(rng, M, top_k, K)
        _down(dev, orc, wd, h, ids, E, N, K, "down ids %s" % ids.tolist())


@pytest.mark.parametrize("K", [64, 2048, 4096])
def test_down_widths(dev, orc, K):
    """Rows of 1, 32 and 64 units (lane groups of 4, 32 and 64 lanes)."""
    rng = synth.make_rng(2030 + K)
    M, top_k, E, N = 2, 4, 16, 257
    wd = synth.q4_0_matrix(rng, E * N, K)
    h = synth.pair_activations(rng, M, top_k, K)
    ids = synth.expert_ids(rng, M, top_k, E)
    _down(dev, orc, wd, h, ids, E, N, K, "down K=%d" % K)


def test_down_token_magnitudes(dev, orc):
    """Every pair row is scaled by its own power of two: rows of very
    different magnitudes in one call stay within the bound."""
    rng = synth.make_rng(2040)
    M, top_k, E, N, K = 3, 4, 12, 200, 1408
    wd = synth.q4_0_matrix(rng, E * N, K)
    h = synth.pair_activations(rng, M, top_k, K)
    scales = 2.0 ** np.array([-120, -40, 0, 40, 90, -130, 20, 60, -60, 100, 5, -10])
    h = (h * scales.reshape(M, top_k, 1)).astype(np.float32)
    ids = np.array([[1, 2, 3, 4], [1, 5, 6, 2], [7, 3, 1, 11]], np.int32)
    _down(dev, orc, wd, h, ids, E, N, K, "down magnitudes")


def test_down_pure_read_checksums(dev, orc):
    import torch
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(2050)
    M, top_k, E, N, K = 4, 6, 64, 333, 1408
    wd = synth.q4_0_matrix(rng, E * N, K)
    ids = synth.expert_ids(rng, M, top_k, E)
    ids[1, 2] = ids[3, 0]
    ids[2, 5] = E + 1
    c = empty((M, top_k, N), dev, torch.int32)
    q4.q4_pure_read(c, q4.Q4_READ_MOE_DOWN, T(wd, dev), None, T(ids, dev), M, top_k, E, N, K)
    got = host(c).view(np.uint32)
    rb = synth.q4_0_row_bytes(K)
    for m in range(M):
        for s in range(top_k):
            e = ids[m, s]
            if 0 <= e < E:
                want = orc.row_checksum(wd[e * N:(e + 1) * N], N, rb)
            else:
                want = np.full(N, 0xFFFFFFFF, np.uint32)
            assert np.array_equal(got[m, s], want), (m, s)
