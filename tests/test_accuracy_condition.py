"""The accuracy condition that include/q4gemv.h states for the factored
dequant-dot holds on the workloads' input distributions (CPU only).

The kernels sum the two exact parts of every weight w = a - b separately
(Q4_0: a = d q, b = 8 d; Q4_K: a = d sc q, b = dmin m), so their rounding
error scales with sum_k (|a_k| + |b_k|) |x_k|; the 1e-4 * sum |w x| bound
is guaranteed while that sum is at most 8 * sum |w x|.  On seeded rows of
workload 2 (Q4_0) and workload 4 (Q4_K) the ratio is about 3.9 and 1.3.
"""
import numpy as np
import pytest

from bit_block_quantized_dequant_amd import synth
from gpu_helpers import split_sum


@pytest.mark.parametrize("fmt", ["q4_0", "q4k"])
def test_workloads_inside_the_cancellation_limit(orc, fmt):
    rng = synth.config_rng(2 if fmt == "q4_0" else 4)
    w = synth.q4_0_matrix(rng, 64, 4096) if fmt == "q4_0" else synth.q4k_matrix(rng, 64, 4096)
    x = synth.activations(rng, 4, 4096)
    _, ab = (orc.q4_0_gemv if fmt == "q4_0" else orc.q4k_gemv)(w, x, 64, 4096)
    r = split_sum(orc, fmt, w, x, 64, 4096) / ab
    assert np.all(r <= 8.0) and np.max(r) < (5.0 if fmt == "q4_0" else 2.0), np.max(r)
