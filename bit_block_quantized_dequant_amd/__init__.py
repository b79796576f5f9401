"""Python binding of libq4gemv: decode-time GEMV over 4-bit block-quantized
weights on AMD MI355X (gfx950).

Argument marshalling only.  Every function has the name and argument order of
the C call in include/q4gemv.h; tensors are torch device tensors (their
data_ptr() is passed), sizes are ints, and `stream` defaults to torch's
current stream on the tensors' device.  All arithmetic runs in the HIP
kernels of libq4gemv.so; there is no other implementation to fall back to,
and a missing library raises ImportError on first use.

The binding adds guards the C ABI cannot make by itself: every tensor must
have the call's element type (float32 activations, gamma and outputs, int32
expert ids, byte weights), live on a GPU, be contiguous and be at least as
large as the call will touch, so that a wrong argument raises here instead of
reaching a kernel.  A nonzero
status from the library raises Q4Error.
"""
import ctypes
import os

__all__ = [
    "Q4Error", "lib", "q4_version", "q4_strerror", "q4_0_gemv", "q4k_gemv",
    "fused_rmsnorm_q4k_gemv", "fused_gate_up_q4k_gemv", "fused_rmsnorm_gate_up_q4k_gemv",
    "fused_gate_up_silu_q4k_gemv", "fused_rmsnorm_gate_up_silu_q4k_gemv",
    "moe_q4_gemv", "moe_q4_gemv_silu", "moe_q4_gemv_down", "moe_router_q4_0", "dequant_q4k",
    "q4_0_gemv_soa", "q4_0_repack_soa", "q4_0_gemv_splitk", "q4k_gemv_splitk",
    "splitk_workspace_bytes", "q4_0_gemv_splitk_noalloc", "noalloc_scratch_bytes",
    "Q4_FORMAT_Q4_0", "Q4_FORMAT_Q4K",
    "dequant_q4_0", "q4_pure_read", "Q4_READ_Q4_0_GEMV", "Q4_READ_Q4K_GEMV",
    "Q4_READ_GATE_UP", "Q4_READ_MOE", "Q4_READ_STREAM", "Q4_READ_MOE_DOWN", "LIB_PATH", "q4_0_row_bytes",
    "q4k_row_bytes",
]

# Q4GEMV_LIB may name another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("Q4GEMV_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libq4gemv.so")

Q4_READ_Q4_0_GEMV = 0
Q4_READ_Q4K_GEMV = 1
Q4_READ_GATE_UP = 2
Q4_READ_MOE = 3
Q4_READ_STREAM = 4
Q4_READ_MOE_DOWN = 5
Q4_FORMAT_Q4_0 = 0
Q4_FORMAT_Q4K = 1

STATUS = {0: "Q4_OK", 1: "Q4_ERR_NULL", 2: "Q4_ERR_SHAPE", 3: "Q4_ERR_BATCH", 4: "Q4_ERR_ALIGN",
          5: "Q4_ERR_ARG", 6: "Q4_ERR_HIP"}

_LIB = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64


class Q4Error(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (call, STATUS.get(status, status),
                                                 q4_strerror(status)))


def lib() -> ctypes.CDLL:
    """The loaded libq4gemv.so (raises ImportError if it was never built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libq4gemv.so is not built at %s; build it with "
                              "`python -m bit_block_quantized_dequant_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        L.q4_strerror.argtypes = [ctypes.c_int]
        L.q4_strerror.restype = ctypes.c_char_p
        L.q4_version.argtypes = []
        L.q4_version.restype = ctypes.c_int
        sigs = {
            "q4_0_gemv": [_vp, _vp, _vp, _i64, _i64, _i64, _vp],
            "q4k_gemv": [_vp, _vp, _vp, _i64, _i64, _i64, _vp],
            "fused_rmsnorm_q4k_gemv": [_vp, _vp, _vp, _vp, ctypes.c_float, _i64, _i64, _i64,
                                       _vp],
            "fused_gate_up_q4k_gemv": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp],
            "fused_rmsnorm_gate_up_q4k_gemv": [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float,
                                               _i64, _i64, _i64, _vp],
            "fused_gate_up_silu_q4k_gemv": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp],
            "fused_rmsnorm_gate_up_silu_q4k_gemv": [_vp, _vp, _vp, _vp, _vp, ctypes.c_float,
                                                    _i64, _i64, _i64, _vp],
            "moe_q4_gemv_silu": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp],
            "moe_q4_gemv_down": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp],
            "moe_router_q4_0": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int, _vp],
            "moe_q4_gemv": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp],
            "dequant_q4k": [_vp, _vp, _i64, _i64, _vp],
            "q4_0_gemv_soa": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp],
            "q4_0_repack_soa": [_vp, _vp, _vp, _i64, _i64, _vp],
            "q4_splitk_workspace": [ctypes.c_int, _i64, _i64, _i64, _vp],
            "q4_0_gemv_splitk": [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp],
            "q4k_gemv_splitk": [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp],
            "q4_0_gemv_splitk_noalloc": [_vp, _vp, _vp, _i64, _i64, _i64, _vp],
            "dequant_q4_0": [_vp, _vp, _i64, _i64, _vp],
            "q4_pure_read": [_vp, ctypes.c_int, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                             _vp],
        }
        for name, args in sigs.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.q4_noalloc_scratch_bytes.argtypes = []
        L.q4_noalloc_scratch_bytes.restype = ctypes.c_longlong
        _LIB = L
    return _LIB


def q4_version() -> int:
    return int(lib().q4_version())


def q4_strerror(status: int) -> str:
    return lib().q4_strerror(int(status)).decode()


def q4_0_row_bytes(K: int) -> int:
    return K // 32 * 18


def q4k_row_bytes(K: int) -> int:
    return (K + 255) // 256 * 144


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
F32, I32, U8, CKS = "float32", "int32", "uint8", "checksum"


def _dtype_ok(t, kind):
    import torch
    if kind == F32:
        return t.dtype == torch.float32
    if kind == I32:
        return t.dtype == torch.int32
    if kind == U8:  # packed weight bytes
        return t.dtype in (torch.uint8, torch.int8)
    if kind == CKS:  # 32-bit checksum words
        return t.dtype in (torch.int32, getattr(torch, "uint32", torch.int32))
    raise AssertionError(kind)


def _ptr(t, name, min_bytes=None, device=None, kind=None):
    """Device pointer of tensor `t` (None passes NULL), after the guards:
    dtype (`kind`: float32 activations/outputs, int32 ids, byte weights,
    32-bit checksums), GPU residence, contiguity, a common device and size."""
    if t is None:
        return None, device
    if isinstance(t, int):  # a raw device address, passed through unchecked
        return t, device
    if kind is not None and not _dtype_ok(t, kind):
        raise ValueError("%s must be a %s tensor, got %s" % (name, kind, t.dtype))
    if not getattr(t, "is_cuda", False):
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, other arguments on %s" % (name, t.device, device))
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError("%s holds %d bytes, the call needs %d" %
                         (name, t.numel() * t.element_size(), min_bytes))
    return t.data_ptr(), t.device


def _ptrs(*specs):
    """Pointers of (tensor, name, min_bytes, kind) specs: every dtype is
    checked before any other guard, then each tensor as _ptr checks it, all
    on one device.  Returns (pointers, device)."""
    for t, name, _, kind in specs:
        if t is not None and not isinstance(t, int) and not _dtype_ok(t, kind):
            raise ValueError("%s must be a %s tensor, got %s" % (name, kind, t.dtype))
    ptrs, dev = [], None
    for t, name, min_bytes, kind in specs:
        p, dev = _ptr(t, name, min_bytes, dev, kind)
        ptrs.append(p)
    return ptrs, dev


def _stream(stream, device):
    if stream is None:
        import torch
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ok(status, call):
    if status != 0:
        raise Q4Error(status, call)


def _sz(v, per):
    # bytes a call touches for a size that may be invalid (the library refuses those)
    return max(0, int(v)) * per


# --------------------------------------------------------------------------
# calls (names and argument order of include/q4gemv.h)
# --------------------------------------------------------------------------
def q4_0_gemv(y, w, x, M, N, K, stream=None):
    """y[M,N] = x[M,K] . W^T, W Q4_0 [N rows]."""
    (py, pw, px), dev = _ptrs((y, "y", _sz(M * N, 4), F32),
                              (w, "w", _sz(N, q4_0_row_bytes(K)), U8),
                              (x, "x", _sz(M * K, 4), F32))
    _ok(lib().q4_0_gemv(py, pw, px, M, N, K, _stream(stream, dev)), "q4_0_gemv")


def q4k_gemv(y, w, x, M, N, K, stream=None):
    """y[M,N] = x[M,K] . W^T, W Q4_K [N rows]."""
    (py, pw, px), dev = _ptrs((y, "y", _sz(M * N, 4), F32),
                              (w, "w", _sz(N, q4k_row_bytes(K)), U8),
                              (x, "x", _sz(M * K, 4), F32))
    _ok(lib().q4k_gemv(py, pw, px, M, N, K, _stream(stream, dev)), "q4k_gemv")


def fused_rmsnorm_q4k_gemv(y, w, x, gamma, eps, M, N, K, stream=None):
    """y = RMSNorm(x; gamma, eps) . W^T, W Q4_K."""
    (py, pw, px, pg), dev = _ptrs((y, "y", _sz(M * N, 4), F32),
                                  (w, "w", _sz(N, q4k_row_bytes(K)), U8),
                                  (x, "x", _sz(M * K, 4), F32),
                                  (gamma, "gamma", _sz(K, 4), F32))
    _ok(lib().fused_rmsnorm_q4k_gemv(py, pw, px, pg, float(eps), M, N, K, _stream(stream, dev)),
        "fused_rmsnorm_q4k_gemv")


def fused_gate_up_q4k_gemv(gate, up, w_gate, w_up, x, M, N, K, stream=None):
    """gate = x . Wg^T, up = x . Wu^T (Q4_K), one staging of x."""
    (pg, pu, pwg, pwu, px), dev = _ptrs((gate, "gate", _sz(M * N, 4), F32),
                                        (up, "up", _sz(M * N, 4), F32),
                                        (w_gate, "w_gate", _sz(N, q4k_row_bytes(K)), U8),
                                        (w_up, "w_up", _sz(N, q4k_row_bytes(K)), U8),
                                        (x, "x", _sz(M * K, 4), F32))
    _ok(lib().fused_gate_up_q4k_gemv(pg, pu, pwg, pwu, px, M, N, K, _stream(stream, dev)),
        "fused_gate_up_q4k_gemv")


def moe_q4_gemv(gate, up, w_gate, w_up, x, ids, M, top_k, E, N, K, stream=None):
    """gate/up[M, top_k, N] of the selected Q4_0 experts (expert-stacked rows)."""
    (pg, pu, pwg, pwu, px, pi), dev = _ptrs((gate, "gate", _sz(M * top_k * N, 4), F32),
                                            (up, "up", _sz(M * top_k * N, 4), F32),
                                            (w_gate, "w_gate", _sz(E * N, q4_0_row_bytes(K)), U8),
                                            (w_up, "w_up", _sz(E * N, q4_0_row_bytes(K)), U8),
                                            (x, "x", _sz(M * K, 4), F32),
                                            (ids, "ids", _sz(M * top_k, 4), I32))
    _ok(lib().moe_q4_gemv(pg, pu, pwg, pwu, px, pi, M, top_k, E, N, K, _stream(stream, dev)),
        "moe_q4_gemv")


def fused_rmsnorm_gate_up_q4k_gemv(gate, up, w_gate, w_up, x, gamma, eps, M, N, K,
                                   stream=None):
    """gate/up = RMSNorm(x; gamma, eps) . Wg^T / Wu^T (Q4_K), one staging."""
    (pg, pu, pwg, pwu, px, pga), dev = _ptrs((gate, "gate", _sz(M * N, 4), F32),
                                             (up, "up", _sz(M * N, 4), F32),
                                             (w_gate, "w_gate", _sz(N, q4k_row_bytes(K)), U8),
                                             (w_up, "w_up", _sz(N, q4k_row_bytes(K)), U8),
                                             (x, "x", _sz(M * K, 4), F32),
                                             (gamma, "gamma", _sz(K, 4), F32))
    _ok(lib().fused_rmsnorm_gate_up_q4k_gemv(pg, pu, pwg, pwu, px, pga, float(eps), M, N, K,
                                             _stream(stream, dev)),
        "fused_rmsnorm_gate_up_q4k_gemv")


def fused_gate_up_silu_q4k_gemv(h, w_gate, w_up, x, M, N, K, stream=None):
    """h = silu(x . Wg^T) * (x . Wu^T) (Q4_K), one staging of x, one output."""
    (ph, pwg, pwu, px), dev = _ptrs((h, "h", _sz(M * N, 4), F32),
                                    (w_gate, "w_gate", _sz(N, q4k_row_bytes(K)), U8),
                                    (w_up, "w_up", _sz(N, q4k_row_bytes(K)), U8),
                                    (x, "x", _sz(M * K, 4), F32))
    _ok(lib().fused_gate_up_silu_q4k_gemv(ph, pwg, pwu, px, M, N, K, _stream(stream, dev)),
        "fused_gate_up_silu_q4k_gemv")


def fused_rmsnorm_gate_up_silu_q4k_gemv(h, w_gate, w_up, x, gamma, eps, M, N, K,
                                        stream=None):
    """h = silu(xhat . Wg^T) * (xhat . Wu^T), xhat = RMSNorm(x; gamma, eps); one launch."""
    (ph, pwg, pwu, px, pga), dev = _ptrs((h, "h", _sz(M * N, 4), F32),
                                         (w_gate, "w_gate", _sz(N, q4k_row_bytes(K)), U8),
                                         (w_up, "w_up", _sz(N, q4k_row_bytes(K)), U8),
                                         (x, "x", _sz(M * K, 4), F32),
                                         (gamma, "gamma", _sz(K, 4), F32))
    _ok(lib().fused_rmsnorm_gate_up_silu_q4k_gemv(ph, pwg, pwu, px, pga, float(eps), M, N, K,
                                                  _stream(stream, dev)),
        "fused_rmsnorm_gate_up_silu_q4k_gemv")


def moe_q4_gemv_silu(h, w_gate, w_up, x, ids, M, top_k, E, N, K, stream=None):
    """h[M, top_k, N] = silu(gate) * up of the selected Q4_0 experts."""
    (ph, pwg, pwu, px, pi), dev = _ptrs((h, "h", _sz(M * top_k * N, 4), F32),
                                        (w_gate, "w_gate", _sz(E * N, q4_0_row_bytes(K)), U8),
                                        (w_up, "w_up", _sz(E * N, q4_0_row_bytes(K)), U8),
                                        (x, "x", _sz(M * K, 4), F32),
                                        (ids, "ids", _sz(M * top_k, 4), I32))
    _ok(lib().moe_q4_gemv_silu(ph, pwg, pwu, px, pi, M, top_k, E, N, K, _stream(stream, dev)),
        "moe_q4_gemv_silu")


def moe_q4_gemv_down(y, w_down, h, ids, M, top_k, E, N, K, stream=None):
    """y[M, top_k, N] = each (token, slot) pair's own row h[m, s] times the
    down matrix of its selected Q4_0 expert."""
    (py, pw, ph, pi), dev = _ptrs((y, "y", _sz(M * top_k * N, 4), F32),
                                  (w_down, "w_down", _sz(E * N, q4_0_row_bytes(K)), U8),
                                  (h, "h", _sz(M * top_k * K, 4), F32),
                                  (ids, "ids", _sz(M * top_k, 4), I32))
    _ok(lib().moe_q4_gemv_down(py, pw, ph, pi, M, top_k, E, N, K, _stream(stream, dev)),
        "moe_q4_gemv_down")


def moe_router_q4_0(ids, weights, w_router, x, M, E, K, top_k, normalize, stream=None):
    """ids/weights[M, top_k]: each token's top_k experts by Q4_0 gate logit and
    their softmax weights (normalized over the selection, or the full softmax's)."""
    (pi, pw, pr, px), dev = _ptrs((ids, "ids", _sz(M * top_k, 4), I32),
                                  (weights, "weights", _sz(M * top_k, 4), F32),
                                  (w_router, "w_router", _sz(E, q4_0_row_bytes(K)), U8),
                                  (x, "x", _sz(M * K, 4), F32))
    _ok(lib().moe_router_q4_0(pi, pw, pr, px, M, E, K, top_k, int(normalize),
                              _stream(stream, dev)), "moe_router_q4_0")


def q4_0_repack_soa(scales, quants, w, N, K, stream=None):
    """Split N rows of 18-byte Q4_0 blocks into f16 scales [N, K/32] and
    16-byte nibble blocks [N, K/32, 16] (byte copies)."""
    nb = N * (K // 32)
    (ps, pq, pw), dev = _ptrs((scales, "scales", 2 * nb, U8), (quants, "quants", 16 * nb, U8),
                              (w, "w", 18 * nb, U8))
    _ok(lib().q4_0_repack_soa(ps, pq, pw, N, K, _stream(stream, dev)), "q4_0_repack_soa")


def q4_0_gemv_soa(y, scales, quants, x, M, N, K, stream=None):
    """y[M, N] = X . W^T over split-array Q4_0 (scales, quants)."""
    nb = N * (K // 32)
    (py, ps, pq, px), dev = _ptrs((y, "y", _sz(M * N, 4), F32), (scales, "scales", 2 * nb, U8),
                                  (quants, "quants", 16 * nb, U8), (x, "x", _sz(M * K, 4), F32))
    _ok(lib().q4_0_gemv_soa(py, ps, pq, px, M, N, K, _stream(stream, dev)), "q4_0_gemv_soa")


def splitk_workspace_bytes(fmt, M, N, K) -> int:
    """Workspace bytes the split-K calls need for this shape on the current
    device (0: the call does not split)."""
    b = ctypes.c_int64(0)
    _ok(lib().q4_splitk_workspace(int(fmt), M, N, K, ctypes.byref(b)), "q4_splitk_workspace")
    return int(b.value)


def _splitk(name, fmt, y, w, x, M, N, K, workspace, stream):
    rb = q4_0_row_bytes(K) if fmt == Q4_FORMAT_Q4_0 else q4k_row_bytes(K)
    need = splitk_workspace_bytes(fmt, M, N, K)
    specs = [(y, "y", _sz(M * N, 4), F32), (w, "w", _sz(N, rb), U8), (x, "x", _sz(M * K, 4), F32)]
    if need:
        specs.append((workspace, "workspace", need, U8))
    ptrs, dev = _ptrs(*specs)
    pws = ptrs[3] if need else None
    _ok(getattr(lib(), name)(ptrs[0], ptrs[1], ptrs[2], M, N, K, pws, need,
                             _stream(stream, dev)), name)


def q4_0_gemv_splitk(y, w, x, M, N, K, workspace, stream=None):
    """q4_0_gemv with K split over workgroups (workspace: device bytes of at
    least splitk_workspace_bytes(Q4_FORMAT_Q4_0, M, N, K), any content; the
    call writes it before reading it and leaves nothing in it that a later
    call needs)."""
    _splitk("q4_0_gemv_splitk", Q4_FORMAT_Q4_0, y, w, x, M, N, K, workspace, stream)


def noalloc_scratch_bytes() -> int:
    """Size of the library's own split-K workspace (per GPU)."""
    return int(lib().q4_noalloc_scratch_bytes())


def q4_0_gemv_splitk_noalloc(y, w, x, M, N, K, stream=None):
    """q4_0_gemv_splitk with the library's own workspace: allocates nothing
    (for graph capture and serving loops).  Calls that overlap on one GPU race
    on that workspace and must not be made."""
    rb = q4_0_row_bytes(K)
    (py, pw, px), dev = _ptrs((y, "y", _sz(M * N, 4), F32), (w, "w", _sz(N, rb), U8),
                              (x, "x", _sz(M * K, 4), F32))
    _ok(lib().q4_0_gemv_splitk_noalloc(py, pw, px, M, N, K, _stream(stream, dev)),
        "q4_0_gemv_splitk_noalloc")


def q4k_gemv_splitk(y, w, x, M, N, K, workspace, stream=None):
    """q4k_gemv with K split over workgroups (workspace as q4_0_gemv_splitk's)."""
    _splitk("q4k_gemv_splitk", Q4_FORMAT_Q4K, y, w, x, M, N, K, workspace, stream)


def dequant_q4k(out, w, N, K, stream=None):
    """out[N,K] fp32 = the Q4_K weights, bit-exact."""
    (po, pw), dev = _ptrs((out, "out", _sz(N * K, 4), F32),
                          (w, "w", _sz(N, q4k_row_bytes(K)), U8))
    _ok(lib().dequant_q4k(po, pw, N, K, _stream(stream, dev)), "dequant_q4k")


def dequant_q4_0(out, w, N, K, stream=None):
    """out[N,K] fp32 = the Q4_0 weights, bit-exact."""
    (po, pw), dev = _ptrs((out, "out", _sz(N * K, 4), F32),
                          (w, "w", _sz(N, q4_0_row_bytes(K)), U8))
    _ok(lib().dequant_q4_0(po, pw, N, K, _stream(stream, dev)), "dequant_q4_0")


def q4_pure_read(checksum, kernel_id, w0, w1, ids, M, top_k, E, N, K, stream=None):
    """Read the weight bytes of the named call with its addressing; write row checksums."""
    if kernel_id == Q4_READ_MOE:
        rows, nmat, rb = E * N, 2, q4_0_row_bytes(K)
        ncks = 2 * M * top_k * N
    elif kernel_id == Q4_READ_MOE_DOWN:
        rows, nmat, rb = E * N, 1, q4_0_row_bytes(K)
        ncks = M * top_k * N
    elif kernel_id == Q4_READ_STREAM:
        rows, nmat, rb = N, 1, q4k_row_bytes(K)
        ncks = (max(0, N) * rb + 4095) // 4096  # one checksum per 4 KiB block
    else:
        nmat = 2 if kernel_id == Q4_READ_GATE_UP else 1
        rb = q4_0_row_bytes(K) if kernel_id == Q4_READ_Q4_0_GEMV else q4k_row_bytes(K)
        rows, ncks = N, nmat * N
    ids_bytes = _sz(M * top_k, 4) if kernel_id in (Q4_READ_MOE, Q4_READ_MOE_DOWN) else None
    (pc, p0, p1, pi), dev = _ptrs((checksum, "checksum", _sz(ncks, 4), CKS),
                                  (w0, "w0", _sz(rows, rb), U8),
                                  (w1, "w1", _sz(rows, rb) if nmat == 2 else None, U8),
                                  (ids, "ids", ids_bytes, I32))
    _ok(lib().q4_pure_read(pc, int(kernel_id), p0, p1, pi, M, top_k, E, N, K,
                           _stream(stream, dev)), "q4_pure_read")
