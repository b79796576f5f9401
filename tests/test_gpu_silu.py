"""GPU parity of the SiLU-gated calls, fused_gate_up_silu_q4k_gemv,
fused_rmsnorm_gate_up_silu_q4k_gemv and moe_q4_gemv_silu, through the C ABI.

Two bars per output element h = silu(g) * u:
  * against the oracle: g and u are each within 1e-4 * sum_k |w x| of the
    oracle's g and u (the GEMV bar), and silu has a slope of at most 1.1 in
    absolute value, so
        |h_gpu - h_ref| <= 1.1 dg (|u| + du) + |silu(g)| du
                           + 2^-20 (|silu(g)| + 1.1 dg) (|u| + du)
                           + 2^-140 (|g| + 1) (|u| + du) + 2^-149
    with dg = 1e-4 sum|w_g x|, du = 1e-4 sum|w_u x|; the last terms are the
    fp32 epilogue: a few ulp of the product, and where exp(-|g|) is an fp32
    subnormal (g < -87) an absolute error below (|g| + 1) 2^-148 of silu;
  * the epilogue alone: the SiLU call accumulates g and u exactly as the
    plain gate+up (or expert) call does, so h_gpu must equal the oracle's
    silu(g_gpu) * u_gpu of the plain call's outputs to within
    2^-20 |silu(g_gpu) u_gpu| + 2^-140 (|g_gpu| + 1) |u_gpu| + 2^-149.
The two named gate/up workloads run at full size; small shapes cover ragged
row counts (the 8 + 8-row tiles of the matrix-core path), K = 256 .. 8192
and M = 1 .. 8; an invalid expert id yields NaN rows of h.
"""
import numpy as np
import pytest

from bit_block_quantized_dequant_amd import synth

from gpu_helpers import NT, T, assert_epilogue, assert_silu, empty, host

pytestmark = pytest.mark.gpu

def run_gate_up(dev, orc, wg, wu, x, M, N, K, what):
    import bit_block_quantized_dequant_amd as q4
    tg, tu, tx = T(wg, dev), T(wu, dev), T(x, dev)
    h = empty((M, N), dev)
    q4.fused_gate_up_silu_q4k_gemv(h, tg, tu, tx, M, N, K)
    g, u = empty((M, N), dev), empty((M, N), dev)
    q4.fused_gate_up_q4k_gemv(g, u, tg, tu, tx, M, N, K)
    h, g, u = host(h), host(g), host(u)
    rg, ru, ag, au = orc.gate_up_q4k_gemv(wg, wu, x, N, K, NT)
    assert_silu(orc, h, rg, ru, ag, au, what)
    assert_epilogue(orc, h, g, u, what + " (epilogue)")


@pytest.mark.parametrize("M", [1, 4])
def test_workload4_gate_up_silu(dev, orc, M):
    d = synth.workload_inputs(4, M=M)
    run_gate_up(dev, orc, d["w_gate"], d["w_up"], d["x"], M, d["N"], d["K"],
                "workload 4 silu M=%d" % M)


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (1, 37, 3584), (2, 300, 1024), (3, 77, 512),
                                   (4, 8, 256), (5, 129, 2048), (6, 9, 4096), (7, 1000, 1024),
                                   (8, 40, 4096), (2, 3, 8192), (8, 17, 2048)])
def test_gate_up_silu_shapes(dev, orc, M, N, K):
    rng = synth.make_rng(6000 + M + N + K)
    wg, wu = synth.q4k_matrix(rng, N, K), synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, M, K, sigma=3.0)
    run_gate_up(dev, orc, wg, wu, x, M, N, K, "silu M=%d N=%d K=%d" % (M, N, K))


def run_norm_gate_up(dev, orc, wg, wu, x, gam, M, N, K, what):
    import bit_block_quantized_dequant_amd as q4
    tg, tu, tx, tga = T(wg, dev), T(wu, dev), T(x, dev), T(gam, dev)
    h = empty((M, N), dev)
    q4.fused_rmsnorm_gate_up_silu_q4k_gemv(h, tg, tu, tx, tga, 1e-5, M, N, K)
    g, u = empty((M, N), dev), empty((M, N), dev)
    q4.fused_rmsnorm_gate_up_q4k_gemv(g, u, tg, tu, tx, tga, 1e-5, M, N, K)
    h, g, u = host(h), host(g), host(u)
    xhat = orc.rmsnorm(x, gam, 1e-5)
    rg, ru, ag, au = orc.gate_up_q4k_gemv(wg, wu, xhat, N, K, NT)
    assert_silu(orc, h, rg, ru, ag, au, what)
    assert_epilogue(orc, h, g, u, what + " (epilogue)")


@pytest.mark.parametrize("M,N,K", [(1, 14336, 4096), (4, 14336, 4096), (1, 37, 3584),
                                   (2, 300, 1024), (3, 77, 512), (8, 17, 2048), (6, 9, 4096)])
def test_rmsnorm_gate_up_silu(dev, orc, M, N, K):
    """RMSNorm feeding the SiLU-gated pair, against the oracle's normalized
    rows, gate and up; and the epilogue against the GPU's own RMSNorm +
    gate/up call."""
    rng = synth.make_rng(6500 + M + N + K)
    wg, wu = synth.q4k_matrix(rng, N, K), synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, M, K, sigma=2.0)
    gam = synth.gamma(rng, K)
    run_norm_gate_up(dev, orc, wg, wu, x, gam, M, N, K, "norm silu M=%d N=%d K=%d" % (M, N, K))


def run_moe(dev, orc, wg, wu, x, ids, E, N, K, what):
    import bit_block_quantized_dequant_amd as q4
    M, top_k = ids.shape
    tg, tu, tx, ti = T(wg, dev), T(wu, dev), T(x, dev), T(ids, dev)
    h = empty((M, top_k, N), dev)
    q4.moe_q4_gemv_silu(h, tg, tu, tx, ti, M, top_k, E, N, K)
    g, u = empty((M, top_k, N), dev), empty((M, top_k, N), dev)
    q4.moe_q4_gemv(g, u, tg, tu, tx, ti, M, top_k, E, N, K)
    h, g, u = host(h), host(g), host(u)
    rg, ru, ag, au = orc.moe_q4_0_gemv(wg, wu, x, ids, E, N, K, NT)
    assert_silu(orc, h, rg, ru, ag, au, what)
    assert_epilogue(orc, h, g, u, what + " (epilogue)")


def test_workload5_moe_silu(dev, orc):
    d = synth.workload_inputs(5)
    run_moe(dev, orc, d["w_gate"], d["w_up"], d["x"], d["ids"], d["E"], d["N"], d["K"],
            "workload 5 silu")


def test_workload5_moe_silu_all_distinct_and_invalid(dev, orc):
    d = synth.workload_inputs(5)
    M, top_k = d["M"], d["top_k"]
    ids = np.arange(M * top_k, dtype=np.int32).reshape(M, top_k) * 2 + 1
    run_moe(dev, orc, d["w_gate"], d["w_up"], d["x"], ids, d["E"], d["N"], d["K"],
            "workload 5 silu, all distinct")
    ids[1, 2] = -1
    ids[3, 0] = d["E"]
    run_moe(dev, orc, d["w_gate"], d["w_up"], d["x"], ids, d["E"], d["N"], d["K"],
            "workload 5 silu, two invalid ids")


@pytest.mark.parametrize("M,top_k,E,N,K", [(1, 1, 1, 5, 256), (2, 3, 4, 70, 512),
                                           (8, 8, 16, 33, 1024), (3, 2, 7, 200, 4096),
                                           (5, 4, 9, 64, 2048)])
def test_moe_silu_shapes(dev, orc, M, top_k, E, N, K):
    rng = synth.make_rng(7000 + N + K + M + E)
    wg, wu = synth.q4_0_matrix(rng, E * N, K), synth.q4_0_matrix(rng, E * N, K)
    x = synth.activations(rng, M, K, sigma=3.0)
    ids = synth.expert_ids(rng, M, top_k, E)
    run_moe(dev, orc, wg, wu, x, ids, E, N, K,
            "moe silu M=%d top_k=%d E=%d N=%d K=%d" % (M, top_k, E, N, K))
