"""GPU parity of split-array Q4_0 (f16 scales, 16-byte nibble blocks)
against the CPU oracle through the C ABI: the repack is bit-exact against
the oracle's byte split, and the GEMV is within 1e-4 * sum_k |w x| for odd
and even block counts and every batch M = 1..8.  At M = 1, 2 both layouts
run the same VALU arithmetic in the same order, so the split form's result
equals q4_0_gemv's bit for bit; at M >= 3 both run the matrix-core kernel
with the same K split and step order, so they agree bit for bit too."""
import numpy as np
import pytest

from bit_block_quantized_dequant_amd import synth
from gpu_helpers import NT, T, assert_bits, assert_bound, empty, host

pytestmark = pytest.mark.gpu


def _soa(dev, w, N, K):
    import torch
    import bit_block_quantized_dequant_amd as q4
    nb = N * (K // 32)
    sc = torch.empty(2 * nb, dtype=torch.uint8, device=dev)
    qs = torch.empty(16 * nb, dtype=torch.uint8, device=dev)
    q4.q4_0_repack_soa(sc, qs, T(w, dev), N, K)
    return sc, qs


@pytest.mark.parametrize("K", [32, 96, 2080, 4096])
def test_repack_bitexact(dev, orc, K):
    rng = synth.make_rng(5000 + K)
    N = 123
    w = synth.q4_0_matrix(rng, N, K)
    sc, qs = _soa(dev, w, N, K)
    want_sc, want_qs = orc.q4_0_to_soa(w, N, K)
    assert np.array_equal(host(sc), want_sc.reshape(-1)), K
    assert np.array_equal(host(qs), want_qs.reshape(-1)), K


@pytest.mark.parametrize("K", [32, 96, 1408, 2080, 4096, 14336])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 13, 16])
def test_soa_gemv(dev, orc, M, K):
    """M >= 3 on the matrix cores (K-sliced where needed; a partial last
    step at K = 32, 96, 1408, 2080)."""
    import bit_block_quantized_dequant_amd as q4
    if M == 1 and K > 32768:
        pytest.skip("over the staging limit")
    rng = synth.make_rng(5100 + 10 * K + M)
    N = 301
    w = synth.q4_0_matrix(rng, N, K)
    x = synth.activations(rng, M, K)
    sc, qs = _soa(dev, w, N, K)
    y = empty((M, N), dev)
    q4.q4_0_gemv_soa(y, sc, qs, T(x, dev), M, N, K)
    hsc, hqs = orc.q4_0_to_soa(w, N, K)
    ref, ab = orc.q4_0_soa_gemv(hsc, hqs, x, N, K, NT)
    got = host(y)
    assert_bound(got, ref, ab, "q4_0_gemv_soa M=%d K=%d" % (M, K))
    if M <= 2 and K % 64 == 0 and M * K <= 32768:
        y2 = empty((M, N), dev)
        q4.q4_0_gemv(y2, T(w, dev), T(x, dev), M, N, K)
        assert_bits(got, host(y2), "split arrays vs 18-byte blocks M=%d K=%d" % (M, K))
    if M >= 3 and K % 64 == 0:
        y3 = empty((M, N), dev)
        q4.q4_0_gemv(y3, T(w, dev), T(x, dev), M, N, K)
        assert_bits(got, host(y3), "split arrays vs 18-byte blocks M=%d K=%d" % (M, K))


def test_soa_workload2_shape(dev, orc):
    """The batched Q4_0 workload's matrix (4096 x 4096) in split arrays."""
    import bit_block_quantized_dequant_amd as q4
    for M in (1, 8):
        d = synth.workload_inputs(2, M=M)
        N, K = d["N"], d["K"]
        sc, qs = _soa(dev, d["w"], N, K)
        y = empty((M, N), dev)
        q4.q4_0_gemv_soa(y, sc, qs, T(d["x"], dev), M, N, K)
        ref, ab = orc.q4_0_gemv(d["w"], d["x"], N, K, NT)
        assert_bound(host(y), ref, ab, "q4_0_gemv_soa workload 2 M=%d" % M)
