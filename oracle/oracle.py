"""ctypes wrapper around the plain-C oracle (``q4_oracle.c``).

Test infrastructure only: used by the tests, the smoke check and the
benchmark's CPU baseline, never by the library or its binding.  Every array
crosses as a contiguous numpy array; results come back as float64 (GEMV
values and the matching sum of |w*x|) or float32 (dequantized weights and
normalized activations), exactly as the C code computes them.

``Oracle(path)`` binds one compiled copy of the oracle (the tests also bind
deliberately broken copies to show that the pins catch them); the module
level functions use the default build in this directory.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_u8p = ctypes.POINTER(ctypes.c_uint8)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_i64 = ctypes.c_int64
_int = ctypes.c_int


def _p(a, t):
    return a.ctypes.data_as(t)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s array, got %s" % (np.dtype(dtype), a.dtype))
    return a


class Oracle:
    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f32.restype = ctypes.c_float
        L.oracle_q4k_scale_min.argtypes = [_u8p, _int, ctypes.POINTER(_int), ctypes.POINTER(_int)]
        L.oracle_q4k_scale_min.restype = None
        for name in ("oracle_dequant_q4_0", "oracle_dequant_q4k"):
            f = getattr(L, name)
            f.argtypes = [_u8p, _i64, _i64, _f32p]
            f.restype = None
        for name in ("oracle_q4_0_gemv", "oracle_q4k_gemv"):
            f = getattr(L, name)
            f.argtypes = [_u8p, _f32p, _i64, _i64, _i64, _f64p, _f64p, _int]
            f.restype = None
        L.oracle_rmsnorm.argtypes = [_f32p, _f32p, ctypes.c_float, _i64, _i64, _f32p]
        L.oracle_rmsnorm.restype = None
        L.oracle_fused_rmsnorm_q4k_gemv.argtypes = [_u8p, _f32p, _f32p, ctypes.c_float, _i64,
                                                    _i64, _i64, _f64p, _f64p, _f32p, _int]
        L.oracle_fused_rmsnorm_q4k_gemv.restype = None
        L.oracle_gate_up_q4k_gemv.argtypes = [_u8p, _u8p, _f32p, _i64, _i64, _i64, _f64p, _f64p,
                                              _f64p, _f64p, _int]
        L.oracle_gate_up_q4k_gemv.restype = None
        L.oracle_moe_q4_0_gemv.argtypes = [_u8p, _u8p, _f32p, _i32p, _i64, _i64, _i64, _i64,
                                           _i64, _f64p, _f64p, _f64p, _f64p, _int]
        L.oracle_moe_q4_0_gemv.restype = None
        L.oracle_moe_q4_0_down.argtypes = [_u8p, _f32p, _i32p, _i64, _i64, _i64, _i64, _i64,
                                           _f64p, _f64p, _int]
        L.oracle_moe_q4_0_down.restype = None
        L.oracle_dequant_q4_0_soa.argtypes = [_u8p, _u8p, _i64, _i64, _f32p]
        L.oracle_dequant_q4_0_soa.restype = None
        L.oracle_q4_0_to_soa.argtypes = [_u8p, _i64, _i64, _u8p, _u8p]
        L.oracle_q4_0_to_soa.restype = None
        L.oracle_q4_0_soa_gemv.argtypes = [_u8p, _u8p, _f32p, _i64, _i64, _i64, _f64p, _f64p,
                                           _int]
        L.oracle_q4_0_soa_gemv.restype = None
        L.oracle_silu_mul.argtypes = [_f64p, _f64p, _i64, _f64p]
        L.oracle_silu_mul.restype = None
        L.oracle_topk_softmax.argtypes = [_f64p, _i64, _i64, _i64, _int, _i32p, _f64p]
        L.oracle_topk_softmax.restype = None
        L.oracle_moe_router_q4_0.argtypes = [_u8p, _f32p, _i64, _i64, _i64, _i64, _int, _i32p,
                                             _f64p, _f64p, _f64p]
        L.oracle_moe_router_q4_0.restype = None
        L.oracle_row_checksum.argtypes = [_u8p, _i64, _i64, _u32p]
        L.oracle_row_checksum.restype = None
        self.L = L
        self.path = path

    def f16_to_f32(self, bits: int) -> float:
        return float(self.L.oracle_f16_to_f32(int(bits) & 0xFFFF))

    def q4k_scale_min(self, scale_bytes, j: int):
        S = _c(np.asarray(scale_bytes, dtype=np.uint8), np.uint8)
        assert S.size == 12
        sc, m = _int(), _int()
        self.L.oracle_q4k_scale_min(_p(S, _u8p), int(j), ctypes.byref(sc), ctypes.byref(m))
        return sc.value, m.value

    def dequant_q4_0(self, w, N: int, K: int) -> np.ndarray:
        w = _c(w, np.uint8)
        assert w.size == N * (K // 32) * 18
        out = np.empty((N, K), dtype=np.float32)
        self.L.oracle_dequant_q4_0(_p(w, _u8p), N, K, _p(out, _f32p))
        return out

    def dequant_q4k(self, w, N: int, K: int) -> np.ndarray:
        w = _c(w, np.uint8)
        assert w.size == N * ((K + 255) // 256) * 144
        out = np.empty((N, K), dtype=np.float32)
        self.L.oracle_dequant_q4k(_p(w, _u8p), N, K, _p(out, _f32p))
        return out

    def dequant_q4_0_soa(self, scales, quants, N: int, K: int) -> np.ndarray:
        sc = _c(scales, np.uint8)
        qs = _c(quants, np.uint8)
        nb = N * (K // 32)
        assert sc.size == 2 * nb and qs.size == 16 * nb
        out = np.empty((N, K), dtype=np.float32)
        self.L.oracle_dequant_q4_0_soa(_p(sc, _u8p), _p(qs, _u8p), N, K, _p(out, _f32p))
        return out

    def q4_0_to_soa(self, w, N: int, K: int):
        """(scales uint8 [N, K/32*2], quants uint8 [N, K/32*16]) of Q4_0 rows."""
        w = _c(w, np.uint8)
        nb = K // 32
        assert w.size == N * nb * 18
        sc = np.empty((N, nb * 2), dtype=np.uint8)
        qs = np.empty((N, nb * 16), dtype=np.uint8)
        self.L.oracle_q4_0_to_soa(_p(w, _u8p), N, K, _p(sc, _u8p), _p(qs, _u8p))
        return sc, qs

    def q4_0_soa_gemv(self, scales, quants, x, N: int, K: int, nthreads: int = 1):
        """Returns (y, absdot), each float64 [M, N]."""
        sc = _c(scales, np.uint8)
        qs = _c(quants, np.uint8)
        x = _c(np.atleast_2d(x), np.float32)
        M = x.shape[0]
        assert x.shape[1] == K
        y = np.empty((M, N), dtype=np.float64)
        a = np.empty((M, N), dtype=np.float64)
        self.L.oracle_q4_0_soa_gemv(_p(sc, _u8p), _p(qs, _u8p), _p(x, _f32p), M, N, K,
                                    _p(y, _f64p), _p(a, _f64p), int(nthreads))
        return y, a

    def _gemv(self, fname, w, x, N, K, nthreads):
        w = _c(w, np.uint8)
        x = _c(np.atleast_2d(x), np.float32)
        M = x.shape[0]
        assert x.shape[1] == K
        y = np.empty((M, N), dtype=np.float64)
        a = np.empty((M, N), dtype=np.float64)
        getattr(self.L, fname)(_p(w, _u8p), _p(x, _f32p), M, N, K, _p(y, _f64p),
                               _p(a, _f64p), int(nthreads))
        return y, a

    def q4_0_gemv(self, w, x, N: int, K: int, nthreads: int = 1):
        """Returns (y, absdot), each float64 [M, N]."""
        return self._gemv("oracle_q4_0_gemv", w, x, N, K, nthreads)

    def q4k_gemv(self, w, x, N: int, K: int, nthreads: int = 1):
        """Returns (y, absdot), each float64 [M, N]."""
        return self._gemv("oracle_q4k_gemv", w, x, N, K, nthreads)

    def rmsnorm(self, x, gamma, eps: float) -> np.ndarray:
        x = _c(np.atleast_2d(x), np.float32)
        g = _c(gamma, np.float32)
        M, K = x.shape
        assert g.size == K
        out = np.empty((M, K), dtype=np.float32)
        self.L.oracle_rmsnorm(_p(x, _f32p), _p(g, _f32p), float(eps), M, K, _p(out, _f32p))
        return out

    def fused_rmsnorm_q4k_gemv(self, w, x, gamma, eps: float, N: int, K: int,
                               nthreads: int = 1):
        """Returns (y, absdot, xhat): float64 [M,N] twice and the float32 normalized input."""
        w = _c(w, np.uint8)
        x = _c(np.atleast_2d(x), np.float32)
        g = _c(gamma, np.float32)
        M = x.shape[0]
        y = np.empty((M, N), dtype=np.float64)
        a = np.empty((M, N), dtype=np.float64)
        xh = np.empty((M, K), dtype=np.float32)
        self.L.oracle_fused_rmsnorm_q4k_gemv(_p(w, _u8p), _p(x, _f32p), _p(g, _f32p),
                                             float(eps), M, N, K, _p(y, _f64p), _p(a, _f64p),
                                             _p(xh, _f32p), int(nthreads))
        return y, a, xh

    def gate_up_q4k_gemv(self, wg, wu, x, N: int, K: int, nthreads: int = 1):
        """Returns (gate, up, absgate, absup), each float64 [M, N]."""
        wg = _c(wg, np.uint8)
        wu = _c(wu, np.uint8)
        x = _c(np.atleast_2d(x), np.float32)
        M = x.shape[0]
        outs = [np.empty((M, N), dtype=np.float64) for _ in range(4)]
        self.L.oracle_gate_up_q4k_gemv(_p(wg, _u8p), _p(wu, _u8p), _p(x, _f32p), M, N, K,
                                       *[_p(o, _f64p) for o in outs], int(nthreads))
        return tuple(outs)

    def moe_q4_0_gemv(self, wg, wu, x, ids, E: int, N: int, K: int, nthreads: int = 1):
        """Returns (gate, up, absgate, absup), each float64 [M, top_k, N]."""
        wg = _c(wg, np.uint8)
        wu = _c(wu, np.uint8)
        x = _c(np.atleast_2d(x), np.float32)
        ids = _c(np.atleast_2d(ids), np.int32)
        M, top_k = ids.shape
        assert x.shape == (M, K)
        outs = [np.empty((M, top_k, N), dtype=np.float64) for _ in range(4)]
        self.L.oracle_moe_q4_0_gemv(_p(wg, _u8p), _p(wu, _u8p), _p(x, _f32p), _p(ids, _i32p),
                                    M, top_k, E, N, K, *[_p(o, _f64p) for o in outs],
                                    int(nthreads))
        return tuple(outs)

    def moe_q4_0_down(self, wd, h, ids, E: int, N: int, K: int, nthreads: int = 1):
        """Down-projection of every (token, slot) pair's own input row h[m, s]
        by its expert's matrix.  Returns (y, absy), each float64 [M, top_k, N]."""
        wd = _c(wd, np.uint8)
        ids = _c(np.atleast_2d(ids), np.int32)
        M, top_k = ids.shape
        h = _c(np.asarray(h, dtype=np.float32).reshape(M, top_k, K), np.float32)
        y = np.empty((M, top_k, N), dtype=np.float64)
        a = np.empty((M, top_k, N), dtype=np.float64)
        self.L.oracle_moe_q4_0_down(_p(wd, _u8p), _p(h, _f32p), _p(ids, _i32p), M, top_k, E, N,
                                    K, _p(y, _f64p), _p(a, _f64p), int(nthreads))
        return y, a

    def silu_mul(self, g, u) -> np.ndarray:
        """h = silu(g) * u elementwise, float64, same shape as g."""
        g = _c(np.asarray(g, dtype=np.float64), np.float64)
        u = _c(np.asarray(u, dtype=np.float64), np.float64)
        assert g.shape == u.shape
        h = np.empty_like(g)
        self.L.oracle_silu_mul(_p(g, _f64p), _p(u, _f64p), g.size, _p(h, _f64p))
        return h

    def topk_softmax(self, logits, top_k: int, normalize: bool):
        """Returns (ids int32 [M, top_k], weights float64 [M, top_k])."""
        lg = _c(np.atleast_2d(np.asarray(logits, dtype=np.float64)), np.float64)
        M, E = lg.shape
        ids = np.empty((M, top_k), dtype=np.int32)
        wts = np.empty((M, top_k), dtype=np.float64)
        self.L.oracle_topk_softmax(_p(lg, _f64p), M, E, top_k, int(bool(normalize)),
                                   _p(ids, _i32p), _p(wts, _f64p))
        return ids, wts

    def moe_router_q4_0(self, w, x, E: int, K: int, top_k: int, normalize: bool):
        """Returns (ids, weights, logits, abslogits): int32 [M, top_k], float64
        [M, top_k], float64 [M, E] twice."""
        w = _c(w, np.uint8)
        x = _c(np.atleast_2d(x), np.float32)
        M = x.shape[0]
        assert x.shape[1] == K and w.size == E * (K // 32) * 18
        ids = np.empty((M, top_k), dtype=np.int32)
        wts = np.empty((M, top_k), dtype=np.float64)
        lg = np.empty((M, E), dtype=np.float64)
        ab = np.empty((M, E), dtype=np.float64)
        self.L.oracle_moe_router_q4_0(_p(w, _u8p), _p(x, _f32p), M, E, K, top_k,
                                      int(bool(normalize)), _p(ids, _i32p), _p(wts, _f64p),
                                      _p(lg, _f64p), _p(ab, _f64p))
        return ids, wts, lg, ab

    def row_checksum(self, w, nrows: int, row_bytes: int) -> np.ndarray:
        w = _c(w, np.uint8)
        assert w.size >= nrows * row_bytes and row_bytes % 4 == 0
        out = np.empty(nrows, dtype=np.uint32)
        self.L.oracle_row_checksum(_p(w, _u8p), nrows, row_bytes, _p(out, _u32p))
        return out


_DEFAULT = None


def default() -> Oracle:
    """The oracle built in this directory, compiled first if never built."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _DEFAULT = Oracle(_build.LIB)
    return _DEFAULT


def __getattr__(name):
    # module-level access (oracle.q4k_gemv(...)) forwards to the default build
    if name.startswith("_"):
        raise AttributeError(name)
    return getattr(default(), name)
