"""CPU proof that the GEMV kernel's weight loads stay in bounds: the host
model in addr_model.py replays the launch plan, the strided task split, the
cursors and the address clamping of every lane for each call shape the GPU
tests use, plus adversarial ones (waves without tasks, padded expert row
groups, one-row matrices)."""
import pytest

import addr_model as A

DENSE = [(1, 1, 256), (3, 5, 256), (8, 37, 512), (2, 129, 1024), (5, 1000, 2048),
         (7, 333, 3584), (1, 4097, 4096), (4, 250, 8192), (1, 77, 32768), (8, 61, 4096),
         (6, 3, 5120), (1, 256, 512), (1, 4096, 4096), (1, 18944, 3584), (2, 2, 256)]


@pytest.mark.parametrize("fmt", ["q4k", "q4_0"])
@pytest.mark.parametrize("M,N,K", DENSE)
def test_single_matrix_loads_in_bounds(fmt, M, N, K):
    assert A.check(fmt, M, N, K, RR=2, nmat=1, cus=8) > 0


@pytest.mark.parametrize("fmt", ["q4k", "q4_0"])
@pytest.mark.parametrize("N,K", [(1, 256), (37, 512), (256, 512), (1000, 2048), (77, 4096)])
def test_single_token_one_row_per_lane_loads_in_bounds(fmt, N, K):
    # single-matrix calls too small for one task per CU at two rows per lane
    # run one row per lane (run_m)
    assert A.check(fmt, 1, N, K, RR=1, nmat=1, cus=8) > 0
    assert A.check(fmt, 1, N, K, RR=1, nmat=1, cus=256) > 0


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (3, 41, 512), (8, 130, 4096), (2, 9, 8192),
                                   (1, 14336, 4096)])
def test_two_matrix_loads_in_bounds(M, N, K):
    assert A.check("q4k", M, N, K, RR=1, nmat=2, cus=8) > 0


@pytest.mark.parametrize("fmt,N,K,nmat", [("q4_0", 4096, 4096, 1), ("q4_0", 256, 512, 1),
                                          ("q4k", 18944, 3584, 1), ("q4k", 3, 4096, 2)])
def test_single_token_plans_at_full_chip(fmt, N, K, nmat):
    # 256 CUs: up to three workgroups per CU, the grid cut to two steps per
    # wave (down to one workgroup per CU)
    RR = 2 if nmat == 1 else 1
    pl = A.plan(1, K, N, RR, False, 1, cus=256)
    assert pl["nwaves"] <= 3 * 4 * 256 and pl["nwaves"] * 4 >= min(pl["ntasks"], 4 * 256)
    assert A.check(fmt, 1, N, K, RR=RR, nmat=nmat, cus=256) > 0


@pytest.mark.parametrize("lg", [4, 8, 16, 32])
@pytest.mark.parametrize("fmt,N,K,nmat", [("q4k", 18944, 3584, 1), ("q4k", 14336, 4096, 2),
                                          ("q4_0", 37, 3584, 1), ("q4k", 5, 1024, 2)])
def test_lane_group_overrides_load_in_bounds(lg, fmt, N, K, nmat):
    # Q4GEMV_LG forces the lanes per row group; the kernel's clamping must
    # keep every lane in bounds for any power-of-two width
    RR = 2 if nmat == 1 else 1
    assert A.check(fmt, 1, N, K, RR=RR, nmat=nmat, cus=256, lg=lg) > 0


@pytest.mark.parametrize("experts,E,N,K,npairs", [([0], 1, 5, 256, 1), ([3, 1], 4, 70, 512, 6),
                                                  ([15, 0, 7], 16, 33, 1024, 64),
                                                  ([6, 2, 5], 7, 200, 4096, 6),
                                                  ([63, 0, 31, 5], 64, 1408, 2048, 24),
                                                  ([], 4, 16, 256, 8)])
@pytest.mark.parametrize("bpc", [3, 4])
def test_expert_loads_in_bounds(experts, E, N, K, npairs, bpc):
    A.check("q4_0", 4, N, K, RR=1, nmat=2, moe_experts=experts, E=E, npairs_max=npairs, cus=8,
            bpc=bpc)


def test_model_catches_the_unclamped_base():
    # Without the clamp of the uniform base row, a wave with no tasks
    # (t0 >= ntasks, strided split) starts past N and its 32-bit lane offset
    # wraps: the model must flag that form of the code.
    import os
    src = open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "addr_model.py")).read()
    unclamped = src.replace("R0c = max(0, min(R0, N - 1))", "R0c = R0")
    assert unclamped != src
    ns = {}
    exec(compile(unclamped, "addr_model_unclamped", "exec"), ns)
    with pytest.raises(AssertionError):
        ns["check"]("q4k", 1, 1, 256, 2, 1, cus=8)


# ---------------------------------------------------------------------------
# matrix-core kernel of the batched calls (M >= 2)
# ---------------------------------------------------------------------------
BATCHED = [(M, N, K) for (M, N, K) in DENSE if M >= 2] + [
    (8, 4096, 4096), (4, 14336, 4096), (2, 16, 16384), (8, 17, 256), (2, 1, 256)]


@pytest.mark.parametrize("fmt", ["q4k", "q4_0"])
@pytest.mark.parametrize("M,N,K", BATCHED)
def test_batched_loads_in_bounds(fmt, M, N, K):
    # few CUs so that workgroups run several rounds and waves prefetch across
    # them; many CUs so that the K split and idle tile groups come into play
    assert A.mfma_check(fmt, M, N, K, nmat=1, cus=4) > 0
    if N * K <= 4096 * 4096:
        assert A.mfma_check(fmt, M, N, K, nmat=1, cus=256) > 0


@pytest.mark.parametrize("M,N,K", [(3, 41, 512), (8, 130, 4096), (2, 9, 8192), (4, 14336, 4096)])
def test_batched_two_matrix_loads_in_bounds(M, N, K):
    assert A.mfma_check("q4k", M, N, K, nmat=2, cus=4) > 0
    assert A.mfma_check("q4k", M, N, K, nmat=2, cus=256) > 0


@pytest.mark.parametrize("fmt", ["q4k", "q4_0"])
@pytest.mark.parametrize("M,K", [(2, 256), (3, 512), (8, 4096), (2, 16384), (4, 8192),
                                 (7, 3584), (5, 2048)])
def test_batched_lds_regions(fmt, M, K):
    assert A.mfma_lds_check(fmt, M, K)


def test_batched_lds_fits_every_shape():
    for fmt in ("q4k", "q4_0"):
        for M in range(2, 9):
            for K in range(256, 32768 // M + 1, 256):
                assert A.mlayout(fmt, M, K)["bytes"] <= A.LDS_CAP, (fmt, M, K)


def test_batched_ks_choices():
    # one tile, long rows: all 8 waves split K; short rows cap the split
    assert A.mfma_ks(1, 32, 256) == 8
    assert A.mfma_ks(1, 1, 256) == 1
    assert A.mfma_ks(1, 3, 256) == 2
    # plenty of tiles: no split (1792 tiles give 7/8 of the 2048 wanted waves)
    assert A.mfma_ks(4096, 16, 256) == 1
    assert A.mfma_ks(1792, 16, 256) == 1
    assert A.mfma_ks(1536, 16, 256) == 1
    assert A.mfma_ks(1535, 16, 256) == 2
    # the small Q4_0 call: 256 tiles, split eight ways
    assert A.mfma_ks(256, 16, 256) == 8


@pytest.mark.parametrize("experts,E,N,K,M,top_k", [([0], 1, 5, 256, 2, 1),
                                                   ([3, 1], 4, 70, 512, 2, 3),
                                                   ([15, 0, 7], 16, 33, 1024, 8, 8),
                                                   ([6, 2, 5], 7, 200, 4096, 3, 2),
                                                   ([63, 0, 31, 5], 64, 1408, 2048, 4, 6),
                                                   ([], 4, 16, 256, 4, 2)])
def test_batched_expert_loads_in_bounds(experts, E, N, K, M, top_k):
    umax = min(M * top_k, E)
    for cus in (4, 256):
        A.mfma_check("q4_0", M, N, K, 2, cus=cus, experts=experts, umax=umax, E=E)


@pytest.mark.parametrize("M,N,K", [(3, 1, 256), (4, 8, 256), (5, 9, 512), (8, 17, 2048),
                                   (6, 40, 4096), (7, 1000, 1024), (4, 14336, 4096),
                                   (2, 3, 8192)])
def test_batched_silu_pair_loads_in_bounds(M, N, K):
    # SiLU-gated gate+up on the matrix cores: 8 gate rows + the same 8 up rows
    # per tile, each lane reading its own matrix
    assert A.mfma_check("q4k", M, N, K, 2, cus=8, pair=True) > 0
    assert A.mfma_check("q4k", M, N, K, 2, cus=256, pair=True) > 0


@pytest.mark.parametrize("E,K", [(1, 256), (3, 256), (8, 512), (64, 2048), (65, 1024), (7, 64), (9, 128),
                                 (100, 4096), (1024, 512), (7, 32768)])
def test_router_loads_in_bounds(E, K):
    assert A.router_check(E, K) > 0


# ---------------------------------------------------------------------------
# K tails: Q4_K rows ending inside their last super-block (K % 32 == 0),
# Q4_0 rows of an even block count (K % 64 == 0)
# ---------------------------------------------------------------------------
Q4K_TAIL_K = [32, 96, 288, 1408, 2080, 3616]
Q4_0_TAIL_K = [64, 192, 1408]


@pytest.mark.parametrize("K", Q4K_TAIL_K + [14336])
@pytest.mark.parametrize("M", [1, 2])
def test_tail_loads_in_bounds_q4k(M, K):
    assert A.check("q4k", M, 301, K, RR=2, nmat=1, cus=8) > 0
    assert A.check("q4k", M, 301, K, RR=1, nmat=1, cus=8) > 0  # one row per lane at M <= 2
    assert A.check("q4k", M, 203, K, RR=1, nmat=2, cus=8) > 0


@pytest.mark.parametrize("K", Q4_0_TAIL_K + [14336])
@pytest.mark.parametrize("M", [1, 2])
def test_tail_loads_in_bounds_q4_0(M, K):
    assert A.check("q4_0", M, 299, K, RR=2, nmat=1, cus=8) > 0
    assert A.check("q4_0", M, 299, K, RR=1, nmat=1, cus=8) > 0


@pytest.mark.parametrize("K", Q4K_TAIL_K)
@pytest.mark.parametrize("M", [3, 8])
def test_tail_batched_loads_in_bounds_q4k(M, K):
    if M * ((K + 63) // 64) * 64 > 32768:
        pytest.skip("over the staging limit")
    assert A.mfma_check("q4k", M, 301, K, 1, cus=8) > 0
    assert A.mfma_check("q4k", M, 203, K, 2, cus=8, pair=True) > 0
    assert A.mfma_lds_check("q4k", M, K)


@pytest.mark.parametrize("K", Q4_0_TAIL_K)
@pytest.mark.parametrize("M", [3, 8])
def test_tail_batched_loads_in_bounds_q4_0(M, K):
    assert A.mfma_check("q4_0", M, 299, K, 1, cus=8) > 0
    assert A.mfma_lds_check("q4_0", M, K)


def test_tail_expert_and_router_loads_in_bounds():
    assert A.check("q4_0", 4, 160, 1408, RR=1, nmat=2, moe_experts=[3, 0, 15, 7], E=16,
                   npairs_max=16, cus=8) > 0
    assert A.router_check(64, 1408) > 0


def test_odd_q4_0_block_count_would_misalign():
    """Why Q4_0 rows need K % 64 == 0: with an odd block count, every other
    row starts 2 bytes off a word boundary."""
    with pytest.raises(AssertionError, match="alignment"):
        A.check("q4_0", 1, 4, 96, RR=2, nmat=1, cus=8)


@pytest.mark.parametrize("experts,E,N,K,npairs", [([0], 1, 5, 64, 1), ([3, 1], 4, 70, 1408, 6),
                                                  ([63, 0, 17], 64, 333, 2048, 24),
                                                  ([5], 8, 1, 1408, 8),
                                                  (list(range(20)), 20, 200, 192, 20)])
@pytest.mark.parametrize("wgc", [1, 2, 4])
@pytest.mark.parametrize("RR", [1, 2])
def test_down_loads_in_bounds(experts, E, N, K, npairs, wgc, RR):
    assert A.down_check(N, K, experts, E, npairs, cus=8, wgc=wgc, RR=RR) > 0


def test_down_lane_groups():
    # rows of 22 units (K = 1408): 8 lanes x 3 units (2 idle of 24), not 32
    assert A.choose_lg_waste(22) == 8
    assert A.choose_lg_waste(32) == 32 and A.choose_lg_waste(64) == 64
    assert A.choose_lg_waste(56) == 64 and A.choose_lg_waste(1) == 4


@pytest.mark.parametrize("fmt", ["q4k", "q4_0"])
@pytest.mark.parametrize("M,N,K", [(16, 4096, 4096), (16, 14336, 4096), (4, 4096, 14336),
                                   (8, 4096, 14336), (9, 777, 2048), (16, 40, 32768),
                                   (3, 4096, 65536), (2, 4096, 16448), (12, 300, 3616),
                                   (16, 1, 256), (5, 513, 1 << 20)])
def test_slice_plans(fmt, M, N, K):
    if fmt == "q4_0" and K % 64:
        pytest.skip("Q4_0 rows take K % 64 == 0")
    A.slice_check(fmt, M, N, K)


def test_slicing_keeps_small_batches_whole():
    # the workloads' batches stage whole (no change to their kernels)
    for fmt, M, N, K in (("q4_0", 8, 4096, 4096), ("q4k", 8, 14336, 4096),
                         ("q4k", 4, 18944, 3584), ("q4_0", 3, 4096, 4096)):
        assert A.slice_plan(fmt, M, N, K)[0], (fmt, M, N, K)
    assert not A.slice_plan("q4_0", 16, 4096, 4096)[0]


@pytest.mark.parametrize("K", [32, 96, 1408, 2080, 4096])
@pytest.mark.parametrize("M", [1, 2, 5, 8])
def test_soa_loads_in_bounds(M, K):
    """Split-array Q4_0: nibble blocks 16-byte aligned, scales 2-byte aligned,
    an odd block count's last unit clamped to the row's last block."""
    if M * ((K + 63) // 64) * 64 > 32768:
        pytest.skip("over the staging limit")
    assert A.check("q4_0s", M, 301, K, RR=2, nmat=1, cus=8) > 0


@pytest.mark.parametrize("K", [32, 96, 1408, 2080, 4096])
@pytest.mark.parametrize("M", [3, 8])
def test_soa_batched_loads_in_bounds(M, K):
    assert A.mfma_check("q4_0s", M, 301, K, 1, cus=8) > 0


@pytest.mark.parametrize("fmt,M,N,K", [("q4_0", 8, 4096, 4096), ("q4_0", 16, 4096, 4096),
                                       ("q4k", 4, 4096, 14336), ("q4_0", 5, 777, 1408),
                                       ("q4k", 6, 513, 2080), ("q4k", 8, 33, 32768),
                                       ("q4_0", 12, 16, 4096), ("q4_0", 3, 4096, 4096),
                                       ("q4k", 16, 4096, 14336), ("q4_0", 7, 256, 1 << 20)])
def test_splitk_plans(fmt, M, N, K):
    pl = A.splitk_check(fmt, M, N, K)
    assert pl["kp"] >= 1


def test_long_row_lane_groups_fill_the_chip_evenly():
    # dense rows over 64 units at M <= 2 take 32-lane groups only where their
    # 512-thread workgroups fill the CUs evenly (plan() in q4_host.h)
    assert A.plan(1, 14336, 4096, 1, False, 1, cus=256)["lg"] == 32   # 256 groups
    assert A.plan(2, 28672, 8192, 1, False, 1, cus=256)["lg"] == 32   # 512 groups
    assert A.plan(1, 13824, 5120, 1, False, 1, cus=256)["lg"] == 64   # 320 groups
    assert A.plan(1, 14336, 1024, 1, False, 1, cus=256)["lg"] == 64   # 64 groups
    assert A.plan(1, 4096, 5120, 2, False, 1, cus=256)["lg"] == 64    # rows of 64 units
    assert A.check("q4k", 1, 640, 13824, RR=1, nmat=1, cus=32) > 0   # 40 groups on 32 CUs
    assert A.check("q4k", 2, 512, 13824, RR=1, nmat=2, cus=32) > 0   # 32 groups on 32 CUs
