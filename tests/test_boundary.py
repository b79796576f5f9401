"""The C-ABI boundary on the CPU: libq4gemv.so loads, exports every call that
include/q4gemv.h declares, and refuses invalid arguments with the documented
status before any HIP call (so none of these tests needs a GPU; no call here
has a fully valid argument list, so nothing is ever launched)."""
import ctypes
import os
import re

import pytest

import bit_block_quantized_dequant_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4gemv.h")

OK, NULL, SHAPE, BATCH, ALIGN, ARG, HIP = range(7)
# fake, never dereferenced addresses: aligned and misaligned
A = 0x7F0000000000
MIS = A + 2


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ["q4_0_gemv", "q4k_gemv", "fused_rmsnorm_q4k_gemv", "fused_gate_up_q4k_gemv",
              "fused_rmsnorm_gate_up_q4k_gemv", "fused_gate_up_silu_q4k_gemv",
              "fused_rmsnorm_gate_up_silu_q4k_gemv", "moe_q4_gemv",
              "moe_q4_gemv_silu", "moe_q4_gemv_down", "moe_router_q4_0",
              "dequant_q4k", "dequant_q4_0", "q4_pure_read", "q4_strerror",
              "q4_version"]:
        assert n in names, n


def test_library_exports_every_declared_symbol(q4lib):
    for n in declared_functions():
        assert hasattr(q4lib, n), "libq4gemv.so does not export %s" % n


def test_exports_are_c_symbols(q4lib):
    # no C++ mangling on the ABI
    out = os.popen("nm -D --defined-only %s" % q4.LIB_PATH).read()
    for n in declared_functions():
        assert re.search(r"\bT %s$" % n, out, flags=re.M), n


def test_version_and_strerror(q4lib):
    assert q4.q4_version() == 1
    for s in range(7):
        assert q4.q4_strerror(s) and q4.q4_strerror(s) != "unknown status"
    assert q4.q4_strerror(99) == "unknown status"


def L():
    return q4.lib()


@pytest.mark.parametrize("args,want", [
    ((None, A, A, 1, 16, 256, None), NULL),
    ((A, None, A, 1, 16, 256, None), NULL),
    ((A, A, None, 1, 16, 256, None), NULL),
    ((A, A, A, 0, 16, 256, None), BATCH),
    ((A, A, A, 17, 16, 256, None), BATCH),
    ((A, A, A, -1, 16, 256, None), BATCH),
    ((A, A, A, 1, 0, 256, None), SHAPE),
    ((A, A, A, 1, 2 ** 31, 256, None), SHAPE),
    ((A, A, A, 1, 16, 0, None), SHAPE),
    ((A, A, A, 1, 16, 272, None), SHAPE),  # not a multiple of 32
    ((A, A, A, 1, 16, -256, None), SHAPE),
    ((A, A, A, 1, 16, 32832, None), SHAPE),  # one token over the VALU staging limit
    ((A, A, A, 2, 16, (1 << 20) + 256, None), SHAPE),  # over Q4_MAX_K
    ((A, MIS, A, 1, 16, 256, None), ALIGN),
    ((A, A + 4, A, 1, 16, 256, None), ALIGN),
    ((A, A, A + 8, 1, 16, 256, None), ALIGN),
    ((A + 1, A, A, 1, 16, 256, None), ALIGN),
])
@pytest.mark.parametrize("fn", ["q4_0_gemv", "q4k_gemv"])
def test_dense_validation(q4lib, fn, args, want):
    assert getattr(L(), fn)(*args) == want


def test_k_granularity(q4lib):
    """Q4_K rows may end at any multiple of 32 (inside their last
    super-block); Q4_0 rows need an even block count (K % 64 == 0).  A
    shape that passes is shown by the next check refusing a misaligned
    pointer instead."""
    for K in (32, 96, 288, 1408, 2080):
        assert L().q4k_gemv(A, MIS, A, 1, 16, K, None) == ALIGN, K
        assert L().dequant_q4k(A, MIS, 16, K, None) == ALIGN, K
    for K in (32, 96, 288, 2080):
        assert L().q4_0_gemv(A, MIS, A, 1, 16, K, None) == SHAPE, K
        assert L().dequant_q4_0(A, MIS, 16, K, None) == SHAPE, K
    for K in (64, 1408, 14336):
        assert L().q4_0_gemv(A, MIS, A, 1, 16, K, None) == ALIGN, K
    # a single token is staged whole: ceil(K/64) * 64 <= 32768; batches
    # stage K in slices when needed (no M * K limit)
    assert L().q4k_gemv(A, MIS, A, 1, 16, 32800, None) == SHAPE
    assert L().q4k_gemv(A, MIS, A, 1, 16, 32768, None) == ALIGN
    for M in (2, 3, 16):
        assert L().q4k_gemv(A, MIS, A, M, 16, 65536, None) == ALIGN, M
    assert L().q4_0_gemv(A, MIS, A, 16, 16, 14336, None) == ALIGN


def test_rmsnorm_validation(q4lib):
    f = L().fused_rmsnorm_q4k_gemv
    assert f(A, A, A, None, 1e-5, 1, 16, 256, None) == NULL
    assert f(A, A, A, A + 4, 1e-5, 1, 16, 256, None) == ALIGN
    assert f(A, A, A, A, -1.0, 1, 16, 256, None) == ARG
    assert f(A, A, A, A, float("nan"), 1, 16, 256, None) == ARG
    assert f(A, A, A, A, float("inf"), 1, 16, 256, None) == ARG
    assert f(A, A, A, A, 1e-5, 17, 16, 256, None) == BATCH


def test_gate_up_validation(q4lib):
    f = L().fused_gate_up_q4k_gemv
    assert f(A, None, A, A, A, 1, 16, 256, None) == NULL
    assert f(A, A, A, None, A, 1, 16, 256, None) == NULL
    assert f(A, A, A, A + 4, A, 1, 16, 256, None) == ALIGN
    assert f(A, A + 2, A, A, A, 1, 16, 256, None) == ALIGN
    assert f(A, A, A, A, A, 1, 16, 100, None) == SHAPE


def test_rmsnorm_gate_up_validation(q4lib):
    f = L().fused_rmsnorm_gate_up_q4k_gemv
    assert f(A, A, A, A, A, None, 1e-5, 1, 16, 256, None) == NULL
    assert f(A, None, A, A, A, A, 1e-5, 1, 16, 256, None) == NULL
    assert f(A, A, A, A, A, A + 4, 1e-5, 1, 16, 256, None) == ALIGN
    assert f(A, A + 2, A, A, A, A, 1e-5, 1, 16, 256, None) == ALIGN
    assert f(A, A, A, A, A, A, -1.0, 1, 16, 256, None) == ARG
    assert f(A, A, A, A, A, A, float("nan"), 1, 16, 256, None) == ARG
    assert f(A, A, A, A, A, A, 1e-5, 17, 16, 256, None) == BATCH
    assert f(A, A, A, A, A, A, 1e-5, 1, 16, 100, None) == SHAPE


def test_rmsnorm_gate_up_silu_validation(q4lib):
    f = L().fused_rmsnorm_gate_up_silu_q4k_gemv
    assert f(None, A, A, A, A, 1e-5, 1, 16, 256, None) == NULL
    assert f(A, A, A, A, None, 1e-5, 1, 16, 256, None) == NULL
    assert f(A + 2, A, A, A, A, 1e-5, 1, 16, 256, None) == ALIGN
    assert f(A, A, A, A, A + 4, 1e-5, 1, 16, 256, None) == ALIGN
    assert f(A, A, A, A, A, -1.0, 1, 16, 256, None) == ARG
    assert f(A, A, A, A, A, 1e-5, 17, 16, 256, None) == BATCH
    assert f(A, A, A, A, A, 1e-5, 1, 16, 100, None) == SHAPE


def test_gate_up_silu_validation(q4lib):
    f = L().fused_gate_up_silu_q4k_gemv
    assert f(None, A, A, A, 1, 16, 256, None) == NULL
    assert f(A, A, None, A, 1, 16, 256, None) == NULL
    assert f(A, A, A, None, 1, 16, 256, None) == NULL
    assert f(A + 2, A, A, A, 1, 16, 256, None) == ALIGN
    assert f(A, A + 4, A, A, 1, 16, 256, None) == ALIGN
    assert f(A, A, A, A + 8, 1, 16, 256, None) == ALIGN
    assert f(A, A, A, A, 1, 16, 100, None) == SHAPE
    assert f(A, A, A, A, 17, 16, 256, None) == BATCH
    assert f(A, A, A, A, 0, 16, 256, None) == BATCH


@pytest.mark.parametrize("M,top_k,E,N,K,want", [
    (4, 0, 64, 1408, 2048, SHAPE),
    (4, 65, 64, 1408, 2048, SHAPE),
    (4, 6, 0, 1408, 2048, SHAPE),
    (4, 6, 2 ** 20, 1408, 2048, SHAPE),
    (8, 9, 64, 16, 256, SHAPE),         # 72 (token, slot) pairs > 64
    (4, 6, 64, 2 ** 26, 256, SHAPE),    # E * N >= 2^31
    (9, 6, 64, 1408, 2048, BATCH),
    (4, 6, 64, 1408, 2000, SHAPE),
])
def test_moe_validation(q4lib, M, top_k, E, N, K, want):
    assert L().moe_q4_gemv(A, A, A, A, A, A, M, top_k, E, N, K, None) == want
    assert L().moe_q4_gemv_silu(A, A, A, A, A, M, top_k, E, N, K, None) == want
    assert L().moe_q4_gemv_down(A, A, A, A, M, top_k, E, N, K, None) == want


def test_moe_null_and_align(q4lib):
    f = L().moe_q4_gemv
    assert f(A, A, A, A, A, None, 4, 6, 64, 1408, 2048, None) == NULL
    assert f(A, A, A, A, A, A + 2, 4, 6, 64, 1408, 2048, None) == ALIGN
    g = L().moe_q4_gemv_silu
    assert g(None, A, A, A, A, 4, 6, 64, 1408, 2048, None) == NULL
    assert g(A, A, A, A, None, 4, 6, 64, 1408, 2048, None) == NULL
    assert g(A + 2, A, A, A, A, 4, 6, 64, 1408, 2048, None) == ALIGN
    assert g(A, A, A, A, A + 2, 4, 6, 64, 1408, 2048, None) == ALIGN
    d = L().moe_q4_gemv_down
    for i in range(4):
        args = [A] * 4
        args[i] = None
        assert d(*args, 4, 6, 64, 2048, 1408, None) == NULL, i
        args[i] = A + 2 if i != 1 else A + 4
        assert d(*args, 4, 6, 64, 2048, 1408, None) == ALIGN, i
    assert d(A, A, A + 8, A, 4, 6, 64, 2048, 1408, None) == ALIGN  # h: 16 bytes
    assert d(A, A, A, A, 4, 6, 64, 2048, 1376, None) == SHAPE      # K % 64 != 0


@pytest.mark.parametrize("args,want", [
    ((None, A, A, A, 4, 64, 2048, 6, 1, None), NULL),
    ((A, None, A, A, 4, 64, 2048, 6, 1, None), NULL),
    ((A, A, None, A, 4, 64, 2048, 6, 1, None), NULL),
    ((A, A, A, None, 4, 64, 2048, 6, 1, None), NULL),
    ((A, A, A, A, 0, 64, 2048, 6, 1, None), BATCH),
    ((A, A, A, A, 9, 64, 2048, 6, 1, None), BATCH),
    ((A, A, A, A, 4, 0, 2048, 1, 1, None), SHAPE),
    ((A, A, A, A, 4, 1025, 2048, 6, 1, None), SHAPE),
    ((A, A, A, A, 4, 64, 2000, 6, 1, None), SHAPE),
    ((A, A, A, A, 4, 64, 65536, 6, 1, None), SHAPE),
    ((A, A, A, A, 4, 64, 2048, 0, 1, None), SHAPE),
    ((A, A, A, A, 4, 64, 2048, 65, 1, None), SHAPE),
    ((A, A, A, A, 4, 100, 2048, 65, 1, None), SHAPE),
    ((A, A, A, A, 4, 4, 2048, 5, 1, None), SHAPE),
    ((A, A, A, A, 4, 64, 2048, 6, 2, None), ARG),
    ((A, A, A, A, 4, 64, 2048, 6, -1, None), ARG),
    ((A + 2, A, A, A, 4, 64, 2048, 6, 1, None), ALIGN),
    ((A, A + 2, A, A, 4, 64, 2048, 6, 1, None), ALIGN),
    ((A, A, A + 4, A, 4, 64, 2048, 6, 1, None), ALIGN),
    ((A, A, A, A + 8, 4, 64, 2048, 6, 1, None), ALIGN),
])
def test_router_validation(q4lib, args, want):
    assert L().moe_router_q4_0(*args) == want


def test_dequant_validation(q4lib):
    for f in (L().dequant_q4k, L().dequant_q4_0):
        assert f(None, A, 4, 256, None) == NULL
        assert f(A, None, 4, 256, None) == NULL
        assert f(A, A, 0, 256, None) == SHAPE
        assert f(A, A, 4, 100, None) == SHAPE
        assert f(A + 4, A, 4, 256, None) == ALIGN
        assert f(A, A + 4, 4, 256, None) == ALIGN


def test_pure_read_validation(q4lib):
    f = L().q4_pure_read
    assert f(A, 9, A, A, None, 1, 0, 0, 16, 256, None) == ARG
    assert f(A, -1, A, A, None, 1, 0, 0, 16, 256, None) == ARG
    assert f(None, 0, A, None, None, 1, 0, 0, 16, 256, None) == NULL
    assert f(A, 2, A, None, None, 1, 0, 0, 16, 256, None) == NULL  # gate/up needs w1
    assert f(A, 3, A, A, None, 4, 6, 64, 16, 256, None) == NULL    # moe needs ids
    assert f(A, 1, A, None, None, 1, 0, 0, 16, 300, None) == SHAPE
    assert f(A, 3, A, A, A, 4, 0, 64, 16, 256, None) == SHAPE
    assert f(A + 1, 0, A, None, None, 1, 0, 0, 16, 256, None) == ALIGN
    # reference stream (kernel_id 4)
    assert f(A, 6, A, None, None, 1, 0, 0, 16, 256, None) == ARG
    assert f(A, 5, A, None, None, 4, 6, 64, 16, 1408, None) == NULL  # down needs ids
    assert f(A, 5, A, None, A, 4, 6, 64, 16, 1376, None) == SHAPE
    assert f(A, 4, A, None, None, 1, 0, 0, 16, 300, None) == SHAPE
    assert f(A, 4, A, None, None, 1, 0, 0, 0, 256, None) == SHAPE
    assert f(A, 4, A + 4, None, None, 1, 0, 0, 16, 256, None) == ALIGN
    assert f(None, 4, A, None, None, 1, 0, 0, 16, 256, None) == NULL


def test_binding_refuses_host_tensors():
    import torch
    y = torch.zeros(16)
    w = torch.zeros(16 * 144, dtype=torch.uint8)
    x = torch.zeros(256)
    with pytest.raises(ValueError, match="GPU tensor"):
        q4.q4k_gemv(y, w, x, 1, 16, 256)
    with pytest.raises(ValueError, match="GPU tensor"):
        q4.dequant_q4k(torch.zeros(16, 256), w, 16, 256)


def test_binding_refuses_wrong_dtypes():
    """int64 ids (what torch.topk returns), half or double activations and
    outputs, and non-byte weights are refused before any pointer is used."""
    import torch
    w = torch.zeros(16 * 144, dtype=torch.uint8)
    x = torch.zeros(256)
    y = torch.zeros(16)
    with pytest.raises(ValueError, match="x must be a float32"):
        q4.q4k_gemv(y, w, x.half(), 1, 16, 256)
    with pytest.raises(ValueError, match="y must be a float32"):
        q4.q4k_gemv(y.double(), w, x, 1, 16, 256)
    with pytest.raises(ValueError, match="w must be a uint8"):
        q4.q4k_gemv(y, w.float(), x, 1, 16, 256)
    gate = torch.zeros(1, 2, 16)
    ids64 = torch.zeros(1, 2, dtype=torch.int64)
    wq = torch.zeros(4 * 16 * 144, dtype=torch.uint8)
    with pytest.raises(ValueError, match="ids must be a int32"):
        q4.moe_q4_gemv(gate, gate.clone(), wq, wq, torch.zeros(1, 256), ids64, 1, 2, 4, 16, 256)
    with pytest.raises(ValueError, match="ids must be a int32"):
        q4.moe_router_q4_0(ids64, torch.zeros(1, 2), wq, torch.zeros(1, 256), 1, 4, 256, 2, 1)
    with pytest.raises(ValueError, match="gamma must be a float32"):
        q4.fused_rmsnorm_q4k_gemv(y, w, x, x.half(), 1e-5, 1, 16, 256)
    with pytest.raises(ValueError, match="checksum must be a checksum"):
        q4.q4_pure_read(torch.zeros(16), q4.Q4_READ_Q4K_GEMV, w, None, None, 1, 0, 0, 16, 256)


def test_binding_raises_q4error(q4lib):
    # a NULL output through the binding surfaces as Q4Error(Q4_ERR_NULL)
    with pytest.raises(q4.Q4Error) as ei:
        q4._ok(L().q4k_gemv(None, A, A, 1, 16, 256, None), "q4k_gemv")
    assert ei.value.status == NULL


def test_soa_validation(q4lib):
    g = L().q4_0_gemv_soa
    assert g(None, A, A, A, 1, 16, 96, None) == NULL
    assert g(A, None, A, A, 1, 16, 96, None) == NULL
    assert g(A, A, A, A, 17, 16, 96, None) == BATCH
    assert g(A, A, A, A, 1, 16, 48, None) == SHAPE       # K % 32
    assert g(A, A, A, A, 1, 16, 32800, None) == SHAPE    # staging limit
    assert g(A, A + 1, A, A, 1, 16, 96, None) == ALIGN   # scales: 2 bytes
    assert g(A, A, A + 8, A, 1, 16, 96, None) == ALIGN   # quants: 16 bytes
    assert g(A + 2, A + 2, A, A + 4, 1, 16, 2080, None) == ALIGN  # odd block count passes
    r = L().q4_0_repack_soa
    assert r(None, A, A, 16, 96, None) == NULL
    assert r(A, A, A, 16, 48, None) == SHAPE
    assert r(A, A + 8, A, 16, 96, None) == ALIGN
    assert r(A, A, A + 1, 16, 96, None) == ALIGN


def test_splitk_validation(q4lib):
    b = ctypes.c_int64(0)
    assert L().q4_splitk_workspace(7, 8, 16, 256, ctypes.byref(b)) == ARG
    assert L().q4_splitk_workspace(0, 17, 16, 256, ctypes.byref(b)) == BATCH
    assert L().q4_splitk_workspace(0, 8, 16, 96, ctypes.byref(b)) == SHAPE
    assert L().q4_splitk_workspace(0, 8, 16, 256, None) == NULL
    f = L().q4_0_gemv_splitk
    assert f(None, A, A, 8, 16, 256, A, 1 << 20, None) == NULL
    assert f(A, A, A, 17, 16, 256, A, 1 << 20, None) == BATCH
    assert f(A, MIS, A, 8, 16, 256, A, 1 << 20, None) == ALIGN
    assert L().q4k_gemv_splitk(A, A, A, 8, 16, 48, A, 1 << 20, None) == SHAPE


def test_splitk_noalloc_validation(q4lib):
    """The allocation-free split-K call refuses bad arguments on the host,
    before it takes its workspace's address."""
    f = L().q4_0_gemv_splitk_noalloc
    assert f(None, A, A, 8, 16, 256, None) == NULL
    assert f(A, None, A, 8, 16, 256, None) == NULL
    assert f(A, A, A, 0, 16, 256, None) == BATCH
    assert f(A, A, A, 17, 16, 256, None) == BATCH
    assert f(A, A, A, 8, 16, 96, None) == SHAPE          # Q4_0: K % 64
    assert f(A, A, A, 8, 0, 256, None) == SHAPE
    assert f(A, MIS, A, 8, 16, 256, None) == ALIGN
    assert f(A, A, A + 4, 8, 16, 256, None) == ALIGN     # x: 16 bytes
    assert L().q4_noalloc_scratch_bytes() == 8 << 20


def test_binding_noalloc_refuses_host_tensors():
    import torch
    y = torch.zeros(8 * 16)
    w = torch.zeros(16 * 144, dtype=torch.uint8)
    x = torch.zeros(8 * 256)
    with pytest.raises(ValueError, match="GPU tensor"):
        q4.q4_0_gemv_splitk_noalloc(y, w, x, 8, 16, 256)
