"""GPU parity at the edges of the input range that include/q4gemv.h states,
for every kernel path: the VALU kernel (dense calls with M = 1, 2, and the
expert call), the matrix-core kernel (dense calls with M >= 3), the RMSNorm
calls, and the router's softmax on logits without a finite maximum.

Every token row is scaled by a power of two inside the library, so the
stated bound |y - y_ref| <= 1e-4 * sum_k |w x| + 2^-149 must hold from
subnormal tokens (2^-140) up to 2^100, and for the RMSNorm calls for any
finite x (up to 2^120 here, where the mean square overflows fp32 and the
normalized row is 0 by definition).  Two conditions of the header are
exercised at their limits with tokens dominated by one element: the
factored dequant-dot (the two exact parts a, b of each weight w = a - b
summed separately) is guaranteed while sum (|a| + |b|) |x| <= 8 sum |w x|,
and the matrix-core kernel carries an element below 2^-38 * max|x| of its
token with an absolute error up to 2^-39 * max|x|.
"""
import numpy as np
import pytest

from bit_block_quantized_dequant_amd import synth
from gpu_helpers import NT, T, assert_bound, assert_silu, empty, host, split_sum

pytestmark = pytest.mark.gpu

# token magnitudes 2^s (rows of N(0,1) * 2^s): subnormal, smallest normal,
# tiny, small, unit, large, the stated upper end
SCALES = [-140, -126, -100, -60, 0, 60, 100]
N, K = 64, 1024


def tokens(rng, scales, K):
    x = synth.activations(rng, len(scales), K).astype(np.float64)
    return (x * (2.0 ** np.array(scales, dtype=np.float64))[:, None]).astype(np.float32)


def batches(M):
    """Token-scale batches for a call of M rows covering every scale."""
    if M == 1:
        return [[s] for s in SCALES]
    if M == 2:
        return [[-140, 100], [-60, 60], [0, -126], [-100, -100]]
    return [[SCALES[(i + j) % len(SCALES)] for i in range(M)] for j in range(2)]


@pytest.mark.parametrize("fmt", ["q4_0", "q4k"])
@pytest.mark.parametrize("M", [1, 2, 3, 8])
def test_dense_token_magnitudes(dev, orc, fmt, M):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(900 + M)
    w = synth.q4_0_matrix(rng, N, K) if fmt == "q4_0" else synth.q4k_matrix(rng, N, K)
    call = q4.q4_0_gemv if fmt == "q4_0" else q4.q4k_gemv
    ref_fn = orc.q4_0_gemv if fmt == "q4_0" else orc.q4k_gemv
    wd = T(w, dev)
    for sc in batches(M):
        x = tokens(rng, sc, K)
        y = empty((M, N), dev)
        call(y, wd, T(x, dev), M, N, K)
        ref, ab = ref_fn(w, x, N, K, NT)
        assert_bound(host(y), ref, ab, "%s M=%d scales %s" % (fmt, M, sc))


@pytest.mark.parametrize("M", [1, 2, 4])
def test_gate_up_token_magnitudes(dev, orc, M):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(910 + M)
    wg, wu = synth.q4k_matrix(rng, N, K), synth.q4k_matrix(rng, N, K)
    for sc in batches(M):
        x = tokens(rng, sc, K)
        g, u = empty((M, N), dev), empty((M, N), dev)
        q4.fused_gate_up_q4k_gemv(g, u, T(wg, dev), T(wu, dev), T(x, dev), M, N, K)
        rg, ru, ag, au = orc.gate_up_q4k_gemv(wg, wu, x, N, K, NT)
        assert_bound(host(g), rg, ag, "gate M=%d scales %s" % (M, sc))
        assert_bound(host(u), ru, au, "up M=%d scales %s" % (M, sc))


# the RMSNorm calls take any finite x: up to 2^120 the mean square can
# overflow fp32 (then r = 0 and the normalized row is 0, on both sides)
NORM_SCALES = [-140, -100, -60, 0, 60, 100, 120]


@pytest.mark.parametrize("M", [1, 2, 3, 8])
def test_rmsnorm_token_magnitudes(dev, orc, M):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(920 + M)
    w = synth.q4k_matrix(rng, N, K)
    gam = synth.gamma(rng, K)
    scs = [[s] for s in NORM_SCALES] if M == 1 else \
        [[NORM_SCALES[(i + j) % len(NORM_SCALES)] for i in range(M)] for j in range(2)]
    for sc in scs:
        x = tokens(rng, sc, K)
        y = empty((M, N), dev)
        q4.fused_rmsnorm_q4k_gemv(y, T(w, dev), T(x, dev), T(gam, dev), 1e-5, M, N, K)
        ref, ab, _ = orc.fused_rmsnorm_q4k_gemv(w, x, gam, 1e-5, N, K, NT)
        assert_bound(host(y), ref, ab, "rmsnorm M=%d scales %s" % (M, sc))


@pytest.mark.parametrize("M", [1, 2, 4])
def test_rmsnorm_gate_up_silu_token_magnitudes(dev, orc, M):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(930 + M)
    wg, wu = synth.q4k_matrix(rng, N, K), synth.q4k_matrix(rng, N, K)
    gam = synth.gamma(rng, K)
    for j in range(2):
        sc = [NORM_SCALES[(i + 3 * j) % len(NORM_SCALES)] for i in range(M)]
        x = tokens(rng, sc, K)
        xh = orc.rmsnorm(x, gam, 1e-5)
        rg, ru, ag, au = orc.gate_up_q4k_gemv(wg, wu, xh, N, K, NT)
        g, u = empty((M, N), dev), empty((M, N), dev)
        q4.fused_rmsnorm_gate_up_q4k_gemv(g, u, T(wg, dev), T(wu, dev), T(x, dev), T(gam, dev),
                                          1e-5, M, N, K)
        assert_bound(host(g), rg, ag, "rmsnorm gate M=%d scales %s" % (M, sc))
        assert_bound(host(u), ru, au, "rmsnorm up M=%d scales %s" % (M, sc))
        h = empty((M, N), dev)
        q4.fused_rmsnorm_gate_up_silu_q4k_gemv(h, T(wg, dev), T(wu, dev), T(x, dev),
                                               T(gam, dev), 1e-5, M, N, K)
        assert_silu(orc, host(h), rg, ru, ag, au, "rmsnorm silu M=%d scales %s" % (M, sc))


def test_moe_token_magnitudes(dev, orc):
    import torch

    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(940)
    E, top_k, NE = 8, 3, 40
    wg, wu = synth.q4_0_matrix(rng, E * NE, K), synth.q4_0_matrix(rng, E * NE, K)
    ids = synth.expert_ids(rng, 4, top_k, E)
    for sc in ([-140, -60, 60, 100], [-126, 0, -100, 100]):
        x = tokens(rng, sc, K)
        g, u = empty((4, top_k, NE), dev), empty((4, top_k, NE), dev)
        q4.moe_q4_gemv(g, u, T(wg, dev), T(wu, dev), T(x, dev), T(ids, dev), 4, top_k, E, NE, K)
        rg, ru, ag, au = orc.moe_q4_0_gemv(wg, wu, x, ids, E, NE, K, NT)
        assert_bound(host(g), rg, ag, "moe gate scales %s" % sc)
        assert_bound(host(u), ru, au, "moe up scales %s" % sc)
    del torch


@pytest.mark.parametrize("fmt", ["q4_0", "q4k"])
@pytest.mark.parametrize("M", [1, 2, 3, 8])
def test_lopsided_tokens_at_the_stated_limits(dev, orc, fmt, M):
    """Tokens dominated by one element (1.0 at column 5), all others
    2^-40 * N(0,1) -- below the matrix-core path's 2^-38 * max|x|, so those
    are carried with its absolute floor.  The weight at column 5 is chosen
    so that its two parts nearly cancel, putting sum (|a|+|b|)|x| at 6-7
    times sum |w x|, just inside the stated limit of 8: Q4_0 q = 11
    (a = 11 d, b = 8 d, w = 3 d); Q4_K sc = 10, q = 15, m = 55 with
    dmin = 2 d (a = 150 d, b = 110 d, w = 40 d).  M = 1, 2 run the VALU
    kernel, M = 3, 8 the matrix cores."""
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(950 + M + (10 if fmt == "q4k" else 0))
    if fmt == "q4_0":
        w = synth.q4_0_matrix(rng, N, K)
        w[:, 2 + 5] = (w[:, 2 + 5] & 0xF0) | 11  # element 5: low nibble of byte 5
    else:
        w = synth.q4k_matrix(rng, N, K)
        sb = w.reshape(N, K // 256, 144)
        d = np.float16(0.02)
        sb[:, 0, 0:2] = np.frombuffer(d.tobytes(), np.uint8)
        sb[:, 0, 2:4] = np.frombuffer(np.float16(2 * d).tobytes(), np.uint8)
        # sub-block 0: sc = S[0] & 63 = 10, m = S[4] & 63 = 55 (top bits 0)
        sb[:, 0, 4] = 10
        sb[:, 0, 8] = 55
        # element 5: chunk 0, byte 5, low nibble
        sb[:, 0, 16 + 5] = (sb[:, 0, 16 + 5] & 0xF0) | 15
    x = (synth.activations(rng, M, K).astype(np.float64) * 2.0 ** -40).astype(np.float32)
    x[:, 5] = 1.0
    ref_fn = orc.q4_0_gemv if fmt == "q4_0" else orc.q4k_gemv
    ref, ab = ref_fn(w, x, N, K, NT)
    r = split_sum(orc, fmt, w, x, N, K) / ab
    assert np.all(r <= 8.0) and np.all(r >= 6.0), (r.min(), r.max())
    y = empty((M, N), dev)
    (q4.q4_0_gemv if fmt == "q4_0" else q4.q4k_gemv)(y, T(w, dev), T(x, dev), M, N, K)
    assert_bound(host(y), ref, ab, "lopsided %s M=%d" % (fmt, M))
