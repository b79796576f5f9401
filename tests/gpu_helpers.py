"""Helpers shared by the parity tests: host/device copies, NaN-filled
outputs (an output a kernel forgets to write fails), and the two comparison
bars (bit-exact, and |y - y_ref| <= 1e-4 * sum_k |w x| per element)."""
import os

import numpy as np

NT = min(16, os.cpu_count() or 1)


def T(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def empty(shape, dev, dtype=None):
    import torch
    # filled with NaN so that an output the kernel forgets to write fails
    t = torch.empty(shape, dtype=dtype or torch.float32, device=dev)
    if t.dtype == torch.float32:
        t.fill_(float("nan"))
    else:
        t.fill_(0x5A5A5A5A)
    return t


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


# the fp32 output's own quantum in the subnormal range: no fp32 result can be
# closer than half of it to an exact value that falls there
OUT_Q = 2.0 ** -149


def assert_bound(y, ref, absdot, what):
    y = np.asarray(y, dtype=np.float64).reshape(ref.shape)
    assert not np.any(np.isnan(y)), "%s: NaN in output" % what
    err = np.abs(y - ref)
    bound = 1e-4 * absdot + OUT_Q
    bad = err > bound
    if np.any(bad):
        i = np.unravel_index(np.argmax(err / np.maximum(bound, 1e-300)), err.shape)
        raise AssertionError("%s: %d outputs out of bound; worst at %s: gpu %r ref %r bound %r"
                             % (what, int(bad.sum()), i, y[i], ref[i], bound[i]))


def assert_bits(got, want, what):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), "%s: NaN positions differ" % what
    g = got[~gn]
    w = want[~wn]
    same = (g.view(np.uint32) == w.view(np.uint32)) | ((g == 0) & (w == 0))
    if not np.all(same):
        i = int(np.argmin(same))
        raise AssertionError("%s: %d values differ, first %r vs %r" % (what, int((~same).sum()),
                                                                        g[i], w[i]))


# SiLU-gated outputs: the bars are derived in test_gpu_silu.py's docstring.
EPI = 2.0 ** -20    # relative: the fp32 epilogue
UNDER = 2.0 ** -140  # absolute, per unit of (|g| + 1) |u|: fp32 subnormal exp(-|g|)


def silu_bound(orc, g, u, ag, au):
    dg, du = 1e-4 * ag, 1e-4 * au
    s = np.abs(orc.silu_mul(g, np.ones_like(g)))
    uu = np.abs(u) + du
    return (1.1 * dg * uu + s * du + EPI * (s + 1.1 * dg) * uu
            + UNDER * (np.abs(g) + 1.0) * uu + 2.0 ** -149)


def assert_silu(orc, h, g, u, ag, au, what):
    h = np.asarray(h, np.float64).reshape(g.shape)
    ref = orc.silu_mul(g, u)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(h), nan), "%s: NaN positions differ" % what
    ok = ~nan
    err = np.abs(h[ok] - ref[ok])
    bound = silu_bound(orc, g[ok], u[ok], ag[ok], au[ok])
    bad = err > bound
    if np.any(bad):
        i = int(np.argmax(err / np.maximum(bound, 1e-300)))
        raise AssertionError("%s: %d outputs out of bound; worst gpu %r ref %r bound %r"
                             % (what, int(bad.sum()), h[ok][i], ref[ok][i], bound[i]))


def assert_epilogue(orc, h, g_gpu, u_gpu, what):
    g = np.asarray(g_gpu, np.float64)
    u = np.asarray(u_gpu, np.float64).reshape(g.shape)
    h = np.asarray(h, np.float64).reshape(g.shape)
    ref = orc.silu_mul(g, u)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(h), nan), "%s: NaN positions differ" % what
    err = np.abs(h[~nan] - ref[~nan])
    bound = (EPI * np.abs(ref[~nan]) + UNDER * (np.abs(g[~nan]) + 1.0) * np.abs(u[~nan])
             + 2.0 ** -149)
    assert np.all(err <= bound), "%s: epilogue off by %g (relative)" % (
        what, float(np.max(err / np.maximum(np.abs(ref[~nan]), 1e-300))))


def split_sum(orc, fmt, w, x, N, K):
    """sum_k (|a_k| + |b_k|) |x_k| per output, with w = a - b the two exact
    parts the kernels sum separately (Q4_0: a = d q, b = 8 d; Q4_K:
    a = d sc q, b = dmin m), from the oracle's dequantization of the same
    rows with every nibble forced to 0 (which leaves -b)."""
    deq = (orc.dequant_q4_0 if fmt == "q4_0" else orc.dequant_q4k)(w, N, K).astype(np.float64)
    w0 = w.copy()
    if fmt == "q4_0":
        blk = w0.reshape(N, K // 32, 18)
        blk[:, :, 2:] = 0
    else:
        sb = w0.reshape(N, (K + 255) // 256, 144)
        sb[:, :, 16:] = 0
    b = -(orc.dequant_q4_0 if fmt == "q4_0" else orc.dequant_q4k)(w0, N, K).astype(np.float64)
    a = deq + b
    return np.abs(x.astype(np.float64)) @ (np.abs(a) + np.abs(b)).T
