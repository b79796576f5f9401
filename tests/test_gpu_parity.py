"""GPU parity: every libq4gemv call against the CPU oracle, through the C ABI
(the Python binding only marshals pointers).

Bars:
  * dequantization: bit-exact (NaN == NaN, +0 == -0);
  * GEMV outputs: |y_gpu - y_ref| <= 1e-4 * sum_k |w[n,k] * x[m,k]| per output
    element, y_ref and the sum from the oracle in float64;
  * pure-read checksums: bit-exact against the oracle's row word sums;
  * invariants the design promises bit-exactly: a token row of a batched
    call does not depend on the other rows or its position, gate/up equal
    two single-matrix calls, the single-token expert call equals
    per-slot single calls and a batched one depends neither on slot order
    nor on the other tokens' routing, y(2x) = 2 y(x), one-hot x gives the
    dequantized column.
All five named workloads run at full size; smaller shapes cover ragged row
counts, every lane-group width (K = 256 .. 32768) and every batch M = 1..8.
"""
import os

import numpy as np
import pytest

from bit_block_quantized_dequant_amd import synth
from gpu_helpers import NT, T, assert_bits, assert_bound, empty, host

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# dequantization (bit-exact)
# ---------------------------------------------------------------------------
def special_q4k_rows():
    """Hand-made Q4_K super-blocks: subnormal, zero, negative, huge, inf and NaN
    scales, extreme 6-bit fields, all nibble values."""
    rng = synth.make_rng(5)
    blocks = []
    for d, dmin in [(2.0 ** -24, 2.0 ** -24), (0.0, 0.0), (-0.5, 0.25), (65504.0, 65504.0),
                    (np.inf, 1.0), (1.0, np.inf), (np.nan, 0.5), (-0.0, -0.0), (6.1e-5, 3e-8),
                    (1.0, 1.0)]:
        hdr = np.concatenate([np.frombuffer(np.float16(d).tobytes(), np.uint8),
                              np.frombuffer(np.float16(dmin).tobytes(), np.uint8)])
        for scales in (rng.integers(0, 256, 12), np.full(12, 0xFF), np.zeros(12)):
            qs = rng.integers(0, 256, 128)
            blocks.append(np.concatenate([hdr, scales, qs]).astype(np.uint8))
    w = np.stack(blocks)
    return w.reshape(-1, 144 * 2)  # two super-blocks per row: K = 512


def special_q4_0_rows():
    rng = synth.make_rng(6)
    blocks = []
    for d in (2.0 ** -24, 0.0, -0.5, 65504.0, np.inf, np.nan, -0.0, 6.1e-5, 1.0, 3e-3):
        for _ in range(8):
            blocks.append(np.concatenate([np.frombuffer(np.float16(d).tobytes(), np.uint8),
                                          rng.integers(0, 256, 16)]).astype(np.uint8))
    w = np.stack(blocks)
    return w.reshape(-1, 18 * 8)  # 8 blocks per row: K = 256


def test_dequant_q4k_bitexact(dev, orc):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.config_rng(3)
    cases = [("workload-3 rows", synth.q4k_matrix(rng, 300, 3584), 3584),
             ("special values", special_q4k_rows(), 512),
             ("K=256 one row", synth.q4k_matrix(rng, 1, 256), 256)]
    for name, w, K in cases:
        N = w.shape[0]
        out = empty((N, K), dev)
        q4.dequant_q4k(out, T(w, dev), N, K)
        assert_bits(host(out), orc.dequant_q4k(w, N, K), "dequant_q4k " + name)


def test_dequant_q4_0_bitexact(dev, orc):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.config_rng(2)
    cases = [("workload-2 rows", synth.q4_0_matrix(rng, 257, 4096), 4096),
             ("special values", special_q4_0_rows(), 256)]
    for name, w, K in cases:
        N = w.shape[0]
        out = empty((N, K), dev)
        q4.dequant_q4_0(out, T(w, dev), N, K)
        assert_bits(host(out), orc.dequant_q4_0(w, N, K), "dequant_q4_0 " + name)


# ---------------------------------------------------------------------------
# the five named workloads at full size
# ---------------------------------------------------------------------------
def test_workload1_q4_0_gemv(dev, orc):
    import bit_block_quantized_dequant_amd as q4
    d = synth.workload_inputs(1)
    M, N, K = d["M"], d["N"], d["K"]
    y = empty((M, N), dev)
    q4.q4_0_gemv(y, T(d["w"], dev), T(d["x"], dev), M, N, K)
    ref, ab = orc.q4_0_gemv(d["w"], d["x"], N, K, NT)
    assert_bound(host(y), ref, ab, "workload 1")


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_workload2_q4_0_gemv_batched(dev, orc, M):
    import bit_block_quantized_dequant_amd as q4
    d = synth.workload_inputs(2, M=M)
    N, K = d["N"], d["K"]
    y = empty((M, N), dev)
    q4.q4_0_gemv(y, T(d["w"], dev), T(d["x"], dev), M, N, K)
    ref, ab = orc.q4_0_gemv(d["w"], d["x"], N, K, NT)
    assert_bound(host(y), ref, ab, "workload 2 M=%d" % M)


def test_workload3_fused_rmsnorm(dev, orc):
    import bit_block_quantized_dequant_amd as q4
    d = synth.workload_inputs(3)
    M, N, K = d["M"], d["N"], d["K"]
    y = empty((M, N), dev)
    q4.fused_rmsnorm_q4k_gemv(y, T(d["w"], dev), T(d["x"], dev), T(d["gamma"], dev), d["eps"],
                              M, N, K)
    ref, ab, _ = orc.fused_rmsnorm_q4k_gemv(d["w"], d["x"], d["gamma"], d["eps"], N, K, NT)
    assert_bound(host(y), ref, ab, "workload 3")


@pytest.mark.parametrize("M", [1, 4])
def test_workload4_gate_up(dev, orc, M):
    import bit_block_quantized_dequant_amd as q4
    d = synth.workload_inputs(4, M=M)
    N, K = d["N"], d["K"]
    g, u = empty((M, N), dev), empty((M, N), dev)
    q4.fused_gate_up_q4k_gemv(g, u, T(d["w_gate"], dev), T(d["w_up"], dev), T(d["x"], dev),
                              M, N, K)
    rg, ru, ag, au = orc.gate_up_q4k_gemv(d["w_gate"], d["w_up"], d["x"], N, K, NT)
    assert_bound(host(g), rg, ag, "workload 4 gate M=%d" % M)
    assert_bound(host(u), ru, au, "workload 4 up M=%d" % M)


def _moe_case(dev, orc, d, ids, what):
    import bit_block_quantized_dequant_amd as q4
    M, N, K, E = d["M"], d["N"], d["K"], d["E"]
    top_k = ids.shape[1]
    g, u = empty((M, top_k, N), dev), empty((M, top_k, N), dev)
    wg, wu = T(d["w_gate"], dev), T(d["w_up"], dev)
    q4.moe_q4_gemv(g, u, wg, wu, T(d["x"], dev), T(ids, dev), M, top_k, E, N, K)
    rg, ru, ag, au = orc.moe_q4_0_gemv(d["w_gate"], d["w_up"], d["x"], ids, E, N, K, NT)
    return host(g), host(u), rg, ru, ag, au


def test_workload5_moe(dev, orc):
    d = synth.workload_inputs(5)
    g, u, rg, ru, ag, au = _moe_case(dev, orc, d, d["ids"], "workload 5")
    assert_bound(g, rg, ag, "workload 5 gate")
    assert_bound(u, ru, au, "workload 5 up")


def test_workload5_moe_all_distinct_and_repeats(dev, orc):
    d = synth.workload_inputs(5)
    M, top_k = d["M"], d["top_k"]
    distinct = np.arange(M * top_k, dtype=np.int32).reshape(M, top_k) * 2 + 1
    g, u, rg, ru, ag, au = _moe_case(dev, orc, d, distinct, "all distinct")
    assert_bound(g, rg, ag, "all-distinct gate")
    assert_bound(u, ru, au, "all-distinct up")
    # every token picks the same six experts (in different slot orders)
    same = np.array([np.roll(np.array([3, 9, 27, 40, 51, 63]), k) for k in range(M)], np.int32)
    g, u, rg, ru, ag, au = _moe_case(dev, orc, d, same, "shared experts")
    assert_bound(g, rg, ag, "shared gate")
    assert_bound(u, ru, au, "shared up")
    # a token lists one expert in two slots: both slots are written
    dup = same.copy()
    dup[:, 1] = dup[:, 0]
    dup[2, 4] = dup[2, 5]
    g, u, rg, ru, ag, au = _moe_case(dev, orc, d, dup, "repeated within a token")
    assert_bound(g, rg, ag, "repeated gate")
    assert_bound(u, ru, au, "repeated up")


def test_moe_invalid_ids_give_nan(dev, orc):
    d = synth.workload_inputs(5)
    ids = d["ids"].copy()
    ids[1, 2] = 64
    ids[3, 0] = -7
    g, u, rg, ru, ag, au = _moe_case(dev, orc, d, ids, "invalid ids")
    for (m, s) in [(1, 2), (3, 0)]:
        assert np.all(np.isnan(g[m, s])) and np.all(np.isnan(u[m, s]))
    ok = ~np.isnan(rg)
    assert np.all(np.abs(g[ok] - rg[ok]) <= 1e-4 * ag[ok])
    assert np.all(np.abs(u[ok] - ru[ok]) <= 1e-4 * au[ok])


def test_moe_dedupe_extremes(dev, orc):
    """The in-kernel dedupe at its ends, for the gate/up, SiLU-gated and
    down-projection expert calls: all 64 pairs on one expert (one unique
    expert, every slot written), and every pair invalid (no expert to read,
    every row NaN)."""
    import bit_block_quantized_dequant_amd as q4
    M, top_k, E, N, K = 8, 8, 9, 40, 512  # (top_k <= E)
    rng = synth.make_rng(5077)
    wg, wu = synth.q4_0_matrix(rng, E * N, K), synth.q4_0_matrix(rng, E * N, K)
    wd = synth.q4_0_matrix(rng, E * N, K)
    x = synth.activations(rng, M, K)
    h = synth.activations(rng, M * top_k, K).reshape(M, top_k, K)
    for ids, what in ((np.full((M, top_k), 3, np.int32), "one expert for all 64 pairs"),
                      (np.full((M, top_k), E, np.int32), "every id invalid")):
        g, u = empty((M, top_k, N), dev), empty((M, top_k, N), dev)
        hs, yd = empty((M, top_k, N), dev), empty((M, top_k, N), dev)
        q4.moe_q4_gemv(g, u, T(wg, dev), T(wu, dev), T(x, dev), T(ids, dev), M, top_k, E, N, K)
        q4.moe_q4_gemv_silu(hs, T(wg, dev), T(wu, dev), T(x, dev), T(ids, dev), M, top_k, E, N,
                            K)
        q4.moe_q4_gemv_down(yd, T(wd, dev), T(h, dev), T(ids, dev), M, top_k, E, N, K)
        g, u, hs, yd = host(g), host(u), host(hs), host(yd)
        if ids[0, 0] >= E:
            for a, nm in ((g, "gate"), (u, "up"), (hs, "silu"), (yd, "down")):
                assert np.all(np.isnan(a)), "%s: %s rows must be NaN" % (what, nm)
            continue
        rg, ru, ag, au = orc.moe_q4_0_gemv(wg, wu, x, ids, E, N, K, NT)
        assert_bound(g, rg, ag, what + " gate")
        assert_bound(u, ru, au, what + " up")
        rd, ad = orc.moe_q4_0_down(wd, h, ids, E, N, K, NT)
        assert_bound(yd, rd, ad, what + " down")
        ref = orc.silu_mul(rg, ru)
        dg, du = 1e-4 * ag, 1e-4 * au
        sg = np.abs(orc.silu_mul(rg, np.ones_like(rg)))
        uu = np.abs(ru) + du
        bound = 1.1 * dg * uu + sg * du + 2.0 ** -20 * (sg + 1.1 * dg) * uu + 1e-30
        assert np.all(np.abs(hs - ref) <= bound), what + " silu"


# ---------------------------------------------------------------------------
# shape sweep: ragged N, every lane-group width, every M
# ---------------------------------------------------------------------------
SHAPES = [(1, 1, 256), (3, 5, 256), (8, 37, 512), (2, 129, 1024), (5, 1000, 2048),
          (7, 333, 3584), (1, 4097, 4096), (4, 250, 8192), (1, 77, 32768), (8, 61, 4096),
          (6, 3, 5120)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_q4k_gemv_shapes(dev, orc, M, N, K):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(1000 + N + K + M)
    w = synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, M, K)
    y = empty((M, N), dev)
    q4.q4k_gemv(y, T(w, dev), T(x, dev), M, N, K)
    ref, ab = orc.q4k_gemv(w, x, N, K, NT)
    assert_bound(host(y), ref, ab, "q4k_gemv M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_q4_0_gemv_shapes(dev, orc, M, N, K):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(2000 + N + K + M)
    w = synth.q4_0_matrix(rng, N, K)
    x = synth.activations(rng, M, K)
    y = empty((M, N), dev)
    q4.q4_0_gemv(y, T(w, dev), T(x, dev), M, N, K)
    ref, ab = orc.q4_0_gemv(w, x, N, K, NT)
    assert_bound(host(y), ref, ab, "q4_0_gemv M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(1, 7, 256), (3, 100, 1024), (8, 45, 4096), (2, 33, 3584)])
def test_fused_rmsnorm_shapes(dev, orc, M, N, K):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(3000 + N + K + M)
    w = synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, M, K, 2.0)
    g = synth.gamma(rng, K)
    y = empty((M, N), dev)
    q4.fused_rmsnorm_q4k_gemv(y, T(w, dev), T(x, dev), T(g, dev), 1e-5, M, N, K)
    ref, ab, _ = orc.fused_rmsnorm_q4k_gemv(w, x, g, 1e-5, N, K, NT)
    assert_bound(host(y), ref, ab, "fused_rmsnorm M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (3, 41, 512), (8, 130, 4096), (2, 9, 8192)])
def test_gate_up_shapes(dev, orc, M, N, K):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(4000 + N + K + M)
    wg, wu = synth.q4k_matrix(rng, N, K), synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, M, K)
    g, u = empty((M, N), dev), empty((M, N), dev)
    q4.fused_gate_up_q4k_gemv(g, u, T(wg, dev), T(wu, dev), T(x, dev), M, N, K)
    rg, ru, ag, au = orc.gate_up_q4k_gemv(wg, wu, x, N, K, NT)
    assert_bound(host(g), rg, ag, "gate M=%d N=%d K=%d" % (M, N, K))
    assert_bound(host(u), ru, au, "up M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M,top_k,E,N,K", [(1, 1, 1, 5, 256), (2, 3, 4, 70, 512),
                                           (8, 8, 16, 33, 1024), (3, 2, 7, 200, 4096)])
def test_moe_shapes(dev, orc, M, top_k, E, N, K):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(5000 + N + K + M + E)
    wg, wu = synth.q4_0_matrix(rng, E * N, K), synth.q4_0_matrix(rng, E * N, K)
    x = synth.activations(rng, M, K)
    ids = synth.expert_ids(rng, M, top_k, E)
    g, u = empty((M, top_k, N), dev), empty((M, top_k, N), dev)
    q4.moe_q4_gemv(g, u, T(wg, dev), T(wu, dev), T(x, dev), T(ids, dev), M, top_k, E, N, K)
    rg, ru, ag, au = orc.moe_q4_0_gemv(wg, wu, x, ids, E, N, K, NT)
    assert_bound(host(g), rg, ag, "moe gate")
    assert_bound(host(u), ru, au, "moe up")


# ---------------------------------------------------------------------------
# pure-read ceiling: checksums prove every byte was read
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M", [1, 2, 3, 8])
def test_pure_read_checksums(dev, orc, M):
    """The pure-read pass of each call (VALU addressing at M <= 2, matrix-core
    addressing at M >= 3) touches every weight word exactly once."""
    import torch
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(77)
    N, K = 301, 3584
    w0 = synth.q4k_matrix(rng, N, K)
    w1 = synth.q4k_matrix(rng, N, K)
    rb = synth.q4k_row_bytes(K)
    c = empty((2 * N,), dev, torch.int32)
    q4.q4_pure_read(c, q4.Q4_READ_GATE_UP, T(w0, dev), T(w1, dev), None, M, 0, 0, N, K)
    got = host(c).view(np.uint32)
    want = np.concatenate([orc.row_checksum(w0, N, rb), orc.row_checksum(w1, N, rb)])
    assert np.array_equal(got, want)
    c = empty((N,), dev, torch.int32)
    q4.q4_pure_read(c, q4.Q4_READ_Q4K_GEMV, T(w0, dev), None, None, M, 0, 0, N, K)
    assert np.array_equal(host(c).view(np.uint32), orc.row_checksum(w0, N, rb))
    N, K = 1000, 2048
    w0 = synth.q4_0_matrix(rng, N, K)
    rb = synth.q4_0_row_bytes(K)
    c = empty((N,), dev, torch.int32)
    q4.q4_pure_read(c, q4.Q4_READ_Q4_0_GEMV, T(w0, dev), None, None, M, 0, 0, N, K)
    assert np.array_equal(host(c).view(np.uint32), orc.row_checksum(w0, N, rb))


@pytest.mark.parametrize("N,K", [(1, 256), (37, 512), (301, 3584), (1000, 4096), (3, 32768),
                                 (28672, 4096)])
def test_stream_read_checksums(dev, orc, N, K):
    """The reference stream reads every byte of N * K * 9/16 bytes once: one
    word sum per 4 KiB block (the last one partial), up to the headline's
    66 MB (many blocks per wave)."""
    import torch
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(78 + N)
    w = synth.q4k_matrix(rng, N, K)
    nbytes = w.size
    nblk = (nbytes + 4095) // 4096
    c = empty((nblk,), dev, torch.int32)
    q4.q4_pure_read(c, q4.Q4_READ_STREAM, T(w, dev), None, None, 1, 0, 0, N, K)
    padded = np.zeros(nblk * 4096, np.uint8)
    padded[:nbytes] = w.reshape(-1)
    assert np.array_equal(host(c).view(np.uint32), orc.row_checksum(padded, nblk, 4096))


def test_pure_read_moe_checksums(dev, orc):
    import torch
    import bit_block_quantized_dequant_amd as q4
    d = synth.workload_inputs(5)
    M, N, K, E, top_k = d["M"], d["N"], d["K"], d["E"], d["top_k"]
    ids = d["ids"].copy()
    ids[0, 1] = ids[2, 3]  # a shared expert
    ids[3, 5] = E + 3      # an invalid id
    c = empty((2, M, top_k, N), dev, torch.int32)
    q4.q4_pure_read(c, q4.Q4_READ_MOE, T(d["w_gate"], dev), T(d["w_up"], dev), T(ids, dev),
                    M, top_k, E, N, K)
    got = host(c).view(np.uint32)
    rb = synth.q4_0_row_bytes(K)
    for mt, w in enumerate((d["w_gate"], d["w_up"])):
        for m in range(M):
            for s in range(top_k):
                e = ids[m, s]
                if 0 <= e < E:
                    want = orc.row_checksum(w[e * N:(e + 1) * N], N, rb)
                else:
                    want = np.full(N, 0xFFFFFFFF, np.uint32)
                assert np.array_equal(got[mt, m, s], want), (mt, m, s)


# ---------------------------------------------------------------------------
# bit-exact invariants of the design
# ---------------------------------------------------------------------------
def test_batch_rows_independent_of_batch(dev):
    """Batches of M >= 3 (matrix-core kernel) compute every token row on its
    own: the rows of an M=8 batch equal, bit for bit, the same tokens run in
    smaller batches at other positions.  (M = 1, 2 run the VALU kernel, whose
    rounding differs; they are held to the oracle bound like every call.)"""
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(31)
    N, K, M = 777, 4096, 8
    for fmt in ("q4_0", "q4k"):
        w = synth.q4_0_matrix(rng, N, K) if fmt == "q4_0" else synth.q4k_matrix(rng, N, K)
        f = q4.q4_0_gemv if fmt == "q4_0" else q4.q4k_gemv
        x = synth.activations(rng, M, K)
        wd, xd = T(w, dev), T(x, dev)
        yb = empty((M, N), dev)
        f(yb, wd, xd, M, N, K)
        yb = host(yb)
        for sub in ([7, 0, 2], [3, 5, 1, 6], [6, 2, 4, 0, 1], [1, 2, 3, 4, 5, 6, 7]):
            ys = empty((len(sub), N), dev)
            f(ys, wd, T(x[sub], dev), len(sub), N, K)
            ys = host(ys)
            for j, m in enumerate(sub):
                assert_bits(ys[j], yb[m], "%s token %d at row %d of %d vs row %d of 8"
                            % (fmt, m, j, len(sub), m))


@pytest.mark.parametrize("fmt", ["q4_0", "q4k"])
def test_batched_token_magnitudes(dev, orc, fmt):
    """Each token of a batch is scaled by its own power of two before its f16
    split: tokens 1e-30 and 1e30 apart, and an all-zero token, in one batch."""
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(34)
    N, K, M = 200, 2048, 6
    w = synth.q4_0_matrix(rng, N, K) if fmt == "q4_0" else synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, M, K)
    x[0] *= np.float32(1e-30)
    x[1] *= np.float32(1e30)
    x[2] = 0.0
    x[3, ::7] = 0.0
    x[4] *= np.float32(2.0 ** -60)
    y = empty((M, N), dev)
    f = q4.q4_0_gemv if fmt == "q4_0" else q4.q4k_gemv
    f(y, T(w, dev), T(x, dev), M, N, K)
    ref, ab = (orc.q4_0_gemv if fmt == "q4_0" else orc.q4k_gemv)(w, x, N, K, NT)
    y = host(y)
    assert_bound(y, ref, ab, fmt + " mixed token magnitudes")
    assert np.all(y[2] == 0.0)


@pytest.mark.parametrize("M,N,K", [(1, 14336, 4096), (4, 14336, 4096), (1, 37, 3584),
                                   (2, 300, 1024), (3, 77, 512), (8, 40, 4096), (5, 1, 256)])
def test_rmsnorm_gate_up(dev, orc, M, N, K):
    """RMSNorm feeding the gate+up pair: against the oracle's normalized rows
    and its plain GEMVs, within 1e-4 * sum |w xhat| (xhat as the oracle
    computes it)."""
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(4400 + M + N + K)
    wg, wu = synth.q4k_matrix(rng, N, K), synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, M, K, sigma=2.0)
    gam = synth.gamma(rng, K)
    g, u = empty((M, N), dev), empty((M, N), dev)
    q4.fused_rmsnorm_gate_up_q4k_gemv(g, u, T(wg, dev), T(wu, dev), T(x, dev), T(gam, dev),
                                      1e-5, M, N, K)
    xhat = orc.rmsnorm(x, gam, 1e-5)
    rg, ru, ag, au = orc.gate_up_q4k_gemv(wg, wu, xhat, N, K, NT)
    assert_bound(host(g), rg, ag, "norm gate M=%d N=%d K=%d" % (M, N, K))
    assert_bound(host(u), ru, au, "norm up M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 2, 4])
def test_rmsnorm_gate_up_equals_two_norm_calls(dev, M):
    """Each output equals fused_rmsnorm_q4k_gemv on that matrix, bit for bit
    (same staging, same accumulation; N = 513 gives both calls the same K
    split on the matrix cores)."""
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(33)
    N, K = 513, 4096
    wg, wu = synth.q4k_matrix(rng, N, K), synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, M, K, sigma=2.0)
    gam = synth.gamma(rng, K)
    wgd, wud, xd, gd = T(wg, dev), T(wu, dev), T(x, dev), T(gam, dev)
    g, u, g1, u1 = (empty((M, N), dev) for _ in range(4))
    q4.fused_rmsnorm_gate_up_q4k_gemv(g, u, wgd, wud, xd, gd, 1e-5, M, N, K)
    q4.fused_rmsnorm_q4k_gemv(g1, wgd, xd, gd, 1e-5, M, N, K)
    q4.fused_rmsnorm_q4k_gemv(u1, wud, xd, gd, 1e-5, M, N, K)
    assert_bits(host(g), host(g1), "norm gate vs fused_rmsnorm_q4k_gemv M=%d" % M)
    assert_bits(host(u), host(u1), "norm up vs fused_rmsnorm_q4k_gemv M=%d" % M)


def test_gate_up_equals_two_single_calls(dev):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(32)
    N, K, M = 513, 4096, 4
    wg, wu = synth.q4k_matrix(rng, N, K), synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, M, K)
    wgd, wud, xd = T(wg, dev), T(wu, dev), T(x, dev)
    g, u, g1, u1 = (empty((M, N), dev) for _ in range(4))
    q4.fused_gate_up_q4k_gemv(g, u, wgd, wud, xd, M, N, K)
    q4.q4k_gemv(g1, wgd, xd, M, N, K)
    q4.q4k_gemv(u1, wud, xd, M, N, K)
    assert_bits(host(g), host(g1), "gate vs q4k_gemv")
    assert_bits(host(u), host(u1), "up vs q4k_gemv")
    # equal matrices give equal outputs
    q4.fused_gate_up_q4k_gemv(g, u, wgd, wgd, xd, M, N, K)
    assert_bits(host(g), host(u), "gate == up for Wg == Wu")


@pytest.mark.parametrize("N", [300, 4096])
@pytest.mark.parametrize("M", [1, 2])
def test_long_rows_pair_equals_two_single_calls(dev, M, N):
    """Rows over 64 units at one or two tokens (one row per lane in the
    single-matrix call; 32-lane groups where their workgroups fill the CUs
    evenly, as at N = 4096 on 256 CUs, else 64): the gate+up pair and its
    RMSNorm form still equal two single-matrix calls bit for bit."""
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(34 + M + N)
    K = 8224
    wg, wu = synth.q4k_matrix(rng, N, K), synth.q4k_matrix(rng, N, K)
    x = synth.activations(rng, M, K, sigma=2.0)
    gam = synth.gamma(rng, K)
    wgd, wud, xd, gd = T(wg, dev), T(wu, dev), T(x, dev), T(gam, dev)
    g, u, g1, u1 = (empty((M, N), dev) for _ in range(4))
    q4.fused_gate_up_q4k_gemv(g, u, wgd, wud, xd, M, N, K)
    q4.q4k_gemv(g1, wgd, xd, M, N, K)
    q4.q4k_gemv(u1, wud, xd, M, N, K)
    assert_bits(host(g), host(g1), "gate vs q4k_gemv M=%d K=%d" % (M, K))
    assert_bits(host(u), host(u1), "up vs q4k_gemv M=%d K=%d" % (M, K))
    q4.fused_rmsnorm_gate_up_q4k_gemv(g, u, wgd, wud, xd, gd, 1e-5, M, N, K)
    q4.fused_rmsnorm_q4k_gemv(g1, wgd, xd, gd, 1e-5, M, N, K)
    q4.fused_rmsnorm_q4k_gemv(u1, wud, xd, gd, 1e-5, M, N, K)
    assert_bits(host(g), host(g1), "norm gate M=%d K=%d" % (M, K))
    assert_bits(host(u), host(u1), "norm up M=%d K=%d" % (M, K))


def test_moe_single_token_equals_single_calls(dev):
    """At M = 1 the expert call runs on the VALU kernel: each (slot) output
    equals the single-matrix q4_0_gemv on that expert, bit for bit, for rows
    of at most 64 units (K <= 4096; longer dense rows take narrower lane
    groups than the expert call)."""
    import bit_block_quantized_dequant_amd as q4
    d = synth.workload_inputs(5)
    N, K, E, top_k = d["N"], d["K"], d["E"], d["top_k"]
    ids = d["ids"][:1].copy()
    wg, wu, xd = T(d["w_gate"], dev), T(d["w_up"], dev), T(d["x"][:1], dev)
    g, u = empty((1, top_k, N), dev), empty((1, top_k, N), dev)
    q4.moe_q4_gemv(g, u, wg, wu, xd, T(ids, dev), 1, top_k, E, N, K)
    g, u = host(g), host(u)
    for s in range(top_k):
        e = int(ids[0, s])
        for mat, out in ((wg, g), (wu, u)):
            y1 = empty((1, N), dev)
            q4.q4_0_gemv(y1, mat[e * N:(e + 1) * N], xd, 1, N, K)
            assert_bits(host(y1)[0], out[0, s], "moe slot %d vs q4_0_gemv" % s)


def test_moe_rows_independent_of_routing(dev):
    """Batched expert call (matrix cores): permuting a token's slots permutes
    its outputs, and other tokens' choices do not change them, bit for bit."""
    import bit_block_quantized_dequant_amd as q4
    d = synth.workload_inputs(5)
    M, N, K, E, top_k = d["M"], d["N"], d["K"], d["E"], d["top_k"]
    wg, wu, xd = T(d["w_gate"], dev), T(d["w_up"], dev), T(d["x"], dev)

    def run(ids):
        g, u = empty((M, top_k, N), dev), empty((M, top_k, N), dev)
        q4.moe_q4_gemv(g, u, wg, wu, xd, T(ids, dev), M, top_k, E, N, K)
        return host(g), host(u)

    ids = d["ids"].copy()
    ids[1, 0] = ids[0, 4]  # one expert shared by two tokens
    g0, u0 = run(ids)
    perm = np.array([3, 0, 5, 1, 4, 2])
    ids_p = ids.copy()
    ids_p[2] = ids[2][perm]
    g1, u1 = run(ids_p)
    for s in range(top_k):
        assert_bits(g1[2, s], g0[2, perm[s]], "gate, permuted slot %d" % s)
        assert_bits(u1[2, s], u0[2, perm[s]], "up, permuted slot %d" % s)
    rng = synth.make_rng(36)
    ids_o = ids.copy()
    for m in range(1, M):  # other tokens: new draws (token 0 keeps its experts)
        ids_o[m] = rng.choice(E, size=top_k, replace=False)
    g2, u2 = run(ids_o)
    assert_bits(g2[0], g0[0], "token 0 gate with other routing")
    assert_bits(u2[0], u0[0], "token 0 up with other routing")


def test_scaling_onehot_zero(dev, orc):
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(33)
    N, K = 300, 2048
    for fmt in ("q4_0", "q4k"):
        w = synth.q4_0_matrix(rng, N, K) if fmt == "q4_0" else synth.q4k_matrix(rng, N, K)
        f = q4.q4_0_gemv if fmt == "q4_0" else q4.q4k_gemv
        deq = orc.dequant_q4_0(w, N, K) if fmt == "q4_0" else orc.dequant_q4k(w, N, K)
        wd = T(w, dev)
        x = synth.activations(rng, 2, K)
        y1, y2 = empty((2, N), dev), empty((2, N), dev)
        f(y1, wd, T(x, dev), 2, N, K)
        f(y2, wd, T(2 * x, dev), 2, N, K)
        assert_bits(host(y2), 2 * host(y1), fmt + " y(2x) = 2 y(x)")
        cols = [0, 1, 31, 32, 63, 255, 1000, 2047]
        eye = np.zeros((len(cols), K), np.float32)
        eye[np.arange(len(cols)), cols] = 1.0
        ye = empty((len(cols), N), dev)
        f(ye, wd, T(eye, dev), len(cols), N, K)
        assert_bits(host(ye), deq[:, cols].T, fmt + " one-hot x gives the weights")
        z = empty((1, N), dev)
        f(z, wd, T(np.zeros((1, K), np.float32), dev), 1, N, K)
        assert np.all(host(z) == 0.0)


def test_graph_replay_matches_eager(dev):
    """The calls can be captured in a HIP graph (no allocation, no memset in
    the library): every replay, with other eager work and synchronizations
    between replays, equals the eager call bit for bit."""
    import torch
    import bit_block_quantized_dequant_amd as q4
    rng = synth.make_rng(35)
    N, K = 1000, 4096
    wg, wu = synth.q4k_matrix(rng, N, K), synth.q4k_matrix(rng, N, K)
    w0 = synth.q4_0_matrix(rng, N, K)
    gam = synth.gamma(rng, K)
    x = synth.activations(rng, 8, K)
    wgd, wud, w0d, gd, xd = T(wg, dev), T(wu, dev), T(w0, dev), T(gam, dev), T(x, dev)
    outs = {k: empty((8, N), dev) for k in ("g1", "u1", "n1", "k4", "q8", "h1", "h5")}
    # the router (64 Q4_0 expert rows) and the SiLU expert call on its ids,
    # whose ids stay on the device between the two captured launches
    E, NE, top_k = 64, 40, 4
    wr = T(synth.q4_0_matrix(rng, E, K), dev)
    mg, mu = T(synth.q4_0_matrix(rng, E * NE, K), dev), T(synth.q4_0_matrix(rng, E * NE, K), dev)
    outs["ids"] = empty((4, top_k), dev, dtype=torch.int32)
    outs["wts"] = empty((4, top_k), dev)
    outs["hm"] = empty((4, top_k, NE), dev)
    # split-K (two kernels and a caller workspace), its allocation-free form,
    # split-array Q4_0, and the expert down-projection on the router's ids
    wsb = max(q4.splitk_workspace_bytes(q4.Q4_FORMAT_Q4_0, 8, N, K),
              q4.splitk_workspace_bytes(q4.Q4_FORMAT_Q4K, 4, N, K))
    assert wsb > 0
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    for k, m in (("sk8", 8), ("skk4", 4), ("na6", 6), ("soa3", 3)):
        outs[k] = empty((m, N), dev)
    nb = N * (K // 32)
    sc = torch.empty(2 * nb, dtype=torch.uint8, device=dev)
    qs = torch.empty(16 * nb, dtype=torch.uint8, device=dev)
    q4.q4_0_repack_soa(sc, qs, w0d, N, K)
    KD, ND = 128, 64
    wdn = T(synth.q4_0_matrix(rng, E * ND, KD), dev)
    hd = T(synth.activations(rng, 4 * top_k, KD), dev)
    outs["dn"] = empty((4, top_k, ND), dev)

    def calls(stream):
        q4.fused_gate_up_q4k_gemv(outs["g1"], outs["u1"], wgd, wud, xd, 1, N, K, stream=stream)
        q4.fused_rmsnorm_q4k_gemv(outs["n1"], wgd, xd, gd, 1e-5, 3, N, K, stream=stream)
        q4.q4k_gemv(outs["k4"], wud, xd, 4, N, K, stream=stream)
        q4.q4_0_gemv(outs["q8"], w0d, xd, 8, N, K, stream=stream)
        q4.fused_gate_up_silu_q4k_gemv(outs["h1"], wgd, wud, xd, 1, N, K, stream=stream)
        q4.fused_gate_up_silu_q4k_gemv(outs["h5"], wgd, wud, xd, 5, N, K, stream=stream)
        q4.moe_router_q4_0(outs["ids"], outs["wts"], wr, xd, 4, E, K, top_k, 1, stream=stream)
        q4.moe_q4_gemv_silu(outs["hm"], mg, mu, xd, outs["ids"], 4, top_k, E, NE, K,
                            stream=stream)
        q4.q4_0_gemv_splitk(outs["sk8"], w0d, xd, 8, N, K, ws, stream=stream)
        q4.q4k_gemv_splitk(outs["skk4"], wgd, xd, 4, N, K, ws, stream=stream)
        q4.q4_0_gemv_splitk_noalloc(outs["na6"], w0d, xd, 6, N, K, stream=stream)
        q4.q4_0_gemv_soa(outs["soa3"], sc, qs, xd, 3, N, K, stream=stream)
        q4.moe_q4_gemv_down(outs["dn"], wdn, hd, outs["ids"], 4, top_k, E, ND, KD,
                            stream=stream)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        calls(s)
    torch.cuda.synchronize()
    want = {k: host(v).copy() for k, v in outs.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        g.capture_begin()
        calls(s)
        g.capture_end()
    for rep in range(3):
        for v in outs.values():
            v.fill_(float("nan") if v.dtype == torch.float32 else -7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert_bits(host(v), want[k], "graph replay %d, %s" % (rep, k))


def test_moe_matrix_core_path_in_child_process():
    """The matrix-core expert path (opt-in, Q4GEMV_MOE_MFMA=1; the switch is
    read once per process) against the oracle, in one child process; some
    tokens list one expert in two slots, and both slots must be written."""
    import subprocess
    import sys
    code = (
        "import numpy as np, torch, sys\n"
        "sys.path.insert(0, %r)\n"
        "import bit_block_quantized_dequant_amd as q4\n"
        "from bit_block_quantized_dequant_amd import synth\n"
        "from oracle import oracle\n"
        "o = oracle.default(); dev = torch.device('cuda:0')\n"
        "T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)\n"
        "for (M, top_k, E, N, K, seed) in [(4, 6, 64, 1408, 2048, 0), (2, 3, 4, 70, 512, 1),\n"
        "                                   (8, 8, 16, 33, 1024, 2), (3, 2, 7, 200, 4096, 3)]:\n"
        "    rng = synth.make_rng(5100 + seed)\n"
        "    wg, wu = synth.q4_0_matrix(rng, E * N, K), synth.q4_0_matrix(rng, E * N, K)\n"
        "    x = synth.activations(rng, M, K)\n"
        "    ids = synth.expert_ids(rng, M, top_k, E)\n"
        "    if seed == 1: ids[1, 0] = -3\n"
        "    if seed in (0, 2): ids[1, 0] = ids[1, 2]  # one expert in two slots of a token\n"
        "    g = torch.full((M, top_k, N), float('nan'), device=dev)\n"
        "    u = torch.full((M, top_k, N), float('nan'), device=dev)\n"
        "    q4.moe_q4_gemv(g, u, T(wg), T(wu), T(x), T(ids), M, top_k, E, N, K)\n"
        "    torch.cuda.synchronize()\n"
        "    rg, ru, ag, au = o.moe_q4_0_gemv(wg, wu, x, ids, E, N, K)\n"
        "    for got, ref, ab in ((g, rg, ag), (u, ru, au)):\n"
        "        got = got.cpu().numpy().astype(np.float64)\n"
        "        assert np.array_equal(np.isnan(got), np.isnan(ref))\n"
        "        ok = ~np.isnan(ref)\n"
        "        assert np.all(np.abs(got[ok] - ref[ok]) <= 1e-4 * ab[ok]), (M, top_k, E, N, K)\n"
        "print('ok')\n" % os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    env = dict(os.environ, Q4GEMV_MOE_MFMA="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


def test_forced_lane_groups_in_child_process():
    """Single-token calls with the lanes per row group forced to 8 and 16
    (Q4GEMV_LG, read once per process; this also turns off the
    register-resident activations) against the oracle, one child process
    per width."""
    import subprocess
    import sys
    code = (
        "import numpy as np, torch, sys\n"
        "sys.path.insert(0, %r)\n"
        "import bit_block_quantized_dequant_amd as q4\n"
        "from bit_block_quantized_dequant_amd import synth\n"
        "from oracle import oracle\n"
        "o = oracle.default(); dev = torch.device('cuda:0')\n"
        "T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)\n"
        "def close(y, ref, ab, what):\n"
        "    y = y.cpu().numpy().astype(np.float64).reshape(ref.shape)\n"
        "    assert np.all(np.abs(y - ref) <= 1e-4 * ab), what\n"
        "for (N, K, seed) in [(37, 3584, 0), (300, 1024, 1), (1000, 4096, 2), (5, 256, 3)]:\n"
        "    rng = synth.make_rng(5200 + seed)\n"
        "    wk, wk2, w0 = synth.q4k_matrix(rng, N, K), synth.q4k_matrix(rng, N, K), synth.q4_0_matrix(rng, N, K)\n"
        "    x = synth.activations(rng, 1, K); gam = synth.gamma(rng, K)\n"
        "    y = torch.empty(1, N, device=dev); u = torch.empty(1, N, device=dev)\n"
        "    q4.q4k_gemv(y, T(wk), T(x), 1, N, K); torch.cuda.synchronize()\n"
        "    ry, ab = o.q4k_gemv(wk, x, N, K); close(y, ry, ab, ('q4k', N, K))\n"
        "    q4.q4_0_gemv(y, T(w0), T(x), 1, N, K); torch.cuda.synchronize()\n"
        "    ry, ab = o.q4_0_gemv(w0, x, N, K); close(y, ry, ab, ('q4_0', N, K))\n"
        "    q4.fused_rmsnorm_q4k_gemv(y, T(wk), T(x), T(gam), 1e-5, 1, N, K); torch.cuda.synchronize()\n"
        "    ry, ab, _ = o.fused_rmsnorm_q4k_gemv(wk, x, gam, 1e-5, N, K); close(y, ry, ab, ('norm', N, K))\n"
        "    q4.fused_gate_up_q4k_gemv(y, u, T(wk), T(wk2), T(x), 1, N, K); torch.cuda.synchronize()\n"
        "    rg, ru, ag, au = o.gate_up_q4k_gemv(wk, wk2, x, N, K)\n"
        "    close(y, rg, ag, ('gate', N, K)); close(u, ru, au, ('up', N, K))\n"
        "print('ok')\n" % os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    for lg in ("8", "16"):
        env = dict(os.environ, Q4GEMV_LG=lg)
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                           timeout=300)
        assert r.returncode == 0 and r.stdout.strip().endswith("ok"), lg + r.stdout + r.stderr


def test_valu_kernel_for_batches_in_child_process():
    """Batches of M >= 3 on the VALU kernel (Q4GEMV_MFMA=0, read once per
    process; the library sends such batches to the matrix cores by default)
    against the oracle: every dense call, the SiLU-gated one included."""
    import subprocess
    import sys
    code = (
        "import numpy as np, torch, sys\n"
        "sys.path.insert(0, %r)\n"
        "import bit_block_quantized_dequant_amd as q4\n"
        "from bit_block_quantized_dequant_amd import synth\n"
        "from oracle import oracle\n"
        "o = oracle.default(); dev = torch.device('cuda:0')\n"
        "T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)\n"
        "def close(y, ref, ab, what):\n"
        "    y = y.cpu().numpy().astype(np.float64).reshape(ref.shape)\n"
        "    assert np.all(np.abs(y - ref) <= 1e-4 * ab), what\n"
        "for (M, N, K, seed) in [(3, 37, 1024, 0), (5, 130, 2048, 1), (8, 64, 4096, 2), (4, 9, 256, 3)]:\n"
        "    rng = synth.make_rng(5300 + seed)\n"
        "    wk, wk2, w0 = synth.q4k_matrix(rng, N, K), synth.q4k_matrix(rng, N, K), synth.q4_0_matrix(rng, N, K)\n"
        "    x = synth.activations(rng, M, K); gam = synth.gamma(rng, K)\n"
        "    y = torch.empty(M, N, device=dev); u = torch.empty(M, N, device=dev)\n"
        "    q4.q4k_gemv(y, T(wk), T(x), M, N, K); torch.cuda.synchronize()\n"
        "    ry, ab = o.q4k_gemv(wk, x, N, K); close(y, ry, ab, ('q4k', M, N, K))\n"
        "    q4.q4_0_gemv(y, T(w0), T(x), M, N, K); torch.cuda.synchronize()\n"
        "    ry, ab = o.q4_0_gemv(w0, x, N, K); close(y, ry, ab, ('q4_0', M, N, K))\n"
        "    q4.fused_rmsnorm_q4k_gemv(y, T(wk), T(x), T(gam), 1e-5, M, N, K); torch.cuda.synchronize()\n"
        "    ry, ab, _ = o.fused_rmsnorm_q4k_gemv(wk, x, gam, 1e-5, N, K); close(y, ry, ab, ('norm', M, N, K))\n"
        "    q4.fused_gate_up_q4k_gemv(y, u, T(wk), T(wk2), T(x), M, N, K); torch.cuda.synchronize()\n"
        "    rg, ru, ag, au = o.gate_up_q4k_gemv(wk, wk2, x, N, K)\n"
        "    close(y, rg, ag, ('gate', M, N, K)); close(u, ru, au, ('up', M, N, K))\n"
        "    h = torch.empty(M, N, device=dev)\n"
        "    q4.fused_gate_up_silu_q4k_gemv(h, T(wk), T(wk2), T(x), M, N, K); torch.cuda.synchronize()\n"
        "    hh = h.cpu().numpy().astype(np.float64); ref = o.silu_mul(y.cpu().numpy().astype(np.float64),\n"
        "                                                         u.cpu().numpy().astype(np.float64))\n"
        "    assert np.all(np.abs(hh - ref) <= 2.0 ** -20 * np.abs(ref) + 1e-30), ('silu', M, N, K)\n"
        "print('ok')\n" % os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    env = dict(os.environ, Q4GEMV_MFMA="0")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
