"""GPU parity of the expert router, moe_router_q4_0, through the C ABI.

The selection is an integer decision taken on fp32 logits, each within
b_e = 1e-4 * sum_k |w_e x| of the exact one, so where two experts' logits
are closer than b_e + b_e' either order is correct.  The tests check what is
unique and that the rest is valid, against the oracle's fp64 logits l:
  * the ids of a token are distinct and in [0, E);
  * consecutive picks are in order within the bound:
        l[S_s] + b[S_s] + b[S_s+1] >= l[S_s+1];
  * no expert left out is clearly larger than one picked:
        min_s (l[S_s] + b[S_s]) >= max_{e not in S} (l[e] - b[e]);
  * where the oracle's margins exceed the bound, the ids equal the oracle's;
  * rows of the router matrix that are byte-identical give bit-equal logits,
    and the lower expert index must come first (the tie rule);
  * weights against the oracle's softmax of its own logits at the GPU's ids:
    each log-weight moves by at most b_s + B (B the largest b over the
    softmax's denominator set), so
        |p_gpu - p_ref| <= p_ref (expm1(b_s + B) + 2^-16),
    the last term the fp32 evaluation (exp, the sum, the division);
  * chained on the device, the ids drive moe_q4_gemv_silu unchanged.
"""
import numpy as np
import pytest

from bit_block_quantized_dequant_amd import synth

from gpu_helpers import NT, T, assert_silu, empty, host

pytestmark = pytest.mark.gpu


def router_inputs(seed, M, E, K, dup=False):
    rng = synth.make_rng(seed)
    w = synth.q4_0_matrix(rng, E, K)
    if dup:
        # experts 2 and 5 (and 7 and 1) carry the same bytes: exact ties
        w[5] = w[2]
        w[1] = w[7]
    x = synth.activations(rng, M, K)
    return w, x


def run_router(dev, w, x, E, K, top_k, normalize):
    import torch

    import bit_block_quantized_dequant_amd as q4
    M = x.shape[0]
    ids = empty((M, top_k), dev, dtype=torch.int32)
    wts = empty((M, top_k), dev)
    q4.moe_router_q4_0(ids, wts, T(w, dev), T(x, dev), M, E, K, top_k, normalize)
    return host(ids), host(wts)


def check_router(orc, ids, wts, w, x, E, K, top_k, normalize, what):
    rid, rw, lg, ab = orc.moe_router_q4_0(w, x, E, K, top_k, normalize)
    M = x.shape[0]
    b = 1e-4 * ab
    exact = 0
    for m in range(M):
        S = ids[m].astype(np.int64)
        assert len(set(S.tolist())) == top_k and S.min() >= 0 and S.max() < E, (what, m, S)
        l, bb = lg[m], b[m]
        for s in range(top_k - 1):
            assert l[S[s]] + bb[S[s]] + bb[S[s + 1]] >= l[S[s + 1]], (what, m, s)
        rest = np.setdiff1d(np.arange(E), S)
        if rest.size:
            assert np.min(l[S] + bb[S]) >= np.max(l[rest] - bb[rest]), (what, m)
        # the oracle's order is forced where its consecutive gaps (through
        # the first excluded expert) exceed the bound
        order = np.argsort(-l, kind="stable")
        n = min(top_k + 1, E)
        gaps = l[order[:n - 1]] - l[order[1:n]]
        if np.all(gaps > bb[order[:n - 1]] + bb[order[1:n]]):
            assert np.array_equal(S, rid[m]), (what, m, S, rid[m])
            exact += 1
        # weights
        den_set = S if normalize else np.arange(E)
        L = np.max(l[den_set])
        pref = np.exp(l[S] - L) / np.sum(np.exp(l[den_set] - L))
        B = np.max(bb[den_set])
        with np.errstate(over="ignore", invalid="ignore"):
            bound = pref * (np.expm1(bb[S] + B) + 2.0 ** -16)
        # logits known only to more than ~700 (huge tokens) leave the weights
        # undetermined by the bar: inf * 0 there means no bound
        bound = np.where(np.isnan(bound), np.inf, bound)
        got = wts[m].astype(np.float64)
        assert np.all((got >= 0.0) & (got <= 1.0)), (what, m, got)
        assert np.all(np.abs(got - pref) <= bound), (what, m, got, pref, bound)
        if normalize:
            assert abs(got.sum() - 1.0) <= top_k * 2.0 ** -21, (what, m)
    return exact


@pytest.mark.parametrize("normalize", [1, 0])
def test_workload5_router(dev, orc, normalize):
    # the expert call's shape: 4 tokens, 64 experts, K = 2048, top-6
    d = synth.workload_inputs(5)
    M, E, K, top_k = d["M"], d["E"], d["K"], d["top_k"]
    w, _ = router_inputs(8100, 1, E, K)
    ids, wts = run_router(dev, w, d["x"], E, K, top_k, normalize)
    exact = check_router(orc, ids, wts, w, d["x"], E, K, top_k, normalize, "workload 5 router")
    assert exact >= 1  # the exact-match branch is exercised, not vacuous


@pytest.mark.parametrize("M,E,K,top_k,normalize", [(1, 1, 256, 1, 1), (1, 3, 256, 3, 0),
                                                   (2, 8, 512, 2, 1), (8, 1024, 512, 64, 1),
                                                   (3, 100, 4096, 8, 0), (2, 7, 32768, 7, 1),
                                                   (5, 65, 1024, 13, 1), (4, 256, 2048, 8, 0)])
def test_router_shapes(dev, orc, M, E, K, top_k, normalize):
    w, x = router_inputs(8200 + M + E + K, M, E, K)
    ids, wts = run_router(dev, w, x, E, K, top_k, normalize)
    check_router(orc, ids, wts, w, x, E, K, top_k, normalize,
                 "router M=%d E=%d K=%d top_k=%d" % (M, E, K, top_k))


def test_router_ties_take_the_lower_index(dev, orc):
    M, E, K = 6, 16, 1024
    w, x = router_inputs(8300, M, E, K, dup=True)
    ids, wts = run_router(dev, w, x, E, K, E, 1)
    check_router(orc, ids, wts, w, x, E, K, E, 1, "router ties")
    for m in range(M):
        pos = {int(e): s for s, e in enumerate(ids[m])}
        assert pos[2] < pos[5], (m, ids[m])
        assert pos[1] < pos[7], (m, ids[m])
        assert abs(pos[2] - pos[5]) == 1 and abs(pos[1] - pos[7]) == 1, (m, ids[m])
        assert wts[m][pos[2]] == wts[m][pos[5]] and wts[m][pos[1]] == wts[m][pos[7]]


def test_router_then_silu_expert_call_on_device(dev, orc):
    """The router's ids feed moe_q4_gemv_silu without leaving the GPU."""
    import torch

    import bit_block_quantized_dequant_amd as q4
    M, E, K, N, top_k = 3, 16, 1024, 96, 4
    rng = synth.make_rng(8400)
    wr = synth.q4_0_matrix(rng, E, K)
    wg, wu = synth.q4_0_matrix(rng, E * N, K), synth.q4_0_matrix(rng, E * N, K)
    x = synth.activations(rng, M, K)
    tx = T(x, dev)
    ids = empty((M, top_k), dev, dtype=torch.int32)
    wts = empty((M, top_k), dev)
    q4.moe_router_q4_0(ids, wts, T(wr, dev), tx, M, E, K, top_k, 1)
    h = empty((M, top_k, N), dev)
    q4.moe_q4_gemv_silu(h, T(wg, dev), T(wu, dev), tx, ids, M, top_k, E, N, K)
    ids_h, wts_h, h = host(ids), host(wts), host(h)
    check_router(orc, ids_h, wts_h, wr, x, E, K, top_k, 1, "chained router")
    rg, ru, ag, au = orc.moe_q4_0_gemv(wg, wu, x, ids_h, E, N, K, NT)
    assert_silu(orc, h, rg, ru, ag, au, "chained silu expert call")


def q4_0_rows_const(E, K, d, nib):
    """E rows of Q4_0 blocks with scale d and every nibble equal to nib."""
    blk = np.empty((E * (K // 32), 18), np.uint8)
    blk[:, 0:2] = np.frombuffer(np.float16(d).tobytes(), np.uint8)
    blk[:, 2:] = nib | (nib << 4)
    return blk.reshape(E, (K // 32) * 18)


def test_router_degenerate_logits(dev, orc):
    """Logits without a finite maximum.  d = +inf with all nibbles 0 makes
    every weight -inf (a -inf logit against x > 0), nibbles 15 make +inf; NaN
    tokens make NaN logits.  Ids must equal the oracle's (ties to the lower
    index, NaN as -inf) and the weights its closed forms: uniform over
    experts tied at -inf, shared by experts tied at +inf, 0 for NaN, 0
    everywhere for an all-NaN row."""
    E, K, top_k = 8, 256, 3
    rng = synth.make_rng(8200)
    x = np.abs(synth.activations(rng, 2, K)) + 0.5
    cases = []
    w = q4_0_rows_const(E, K, np.inf, 0)  # every expert -inf
    cases.append(("all -inf", w, x))
    w = synth.q4_0_matrix(rng, E, K)
    w[[2, 6]] = q4_0_rows_const(2, K, np.inf, 15)  # two experts +inf
    w[[0, 4]] = q4_0_rows_const(2, K, np.inf, 0)   # two experts -inf
    cases.append(("+inf ties", w, x))
    cases.append(("NaN tokens", synth.q4_0_matrix(rng, E, K),
                  np.full((2, K), np.nan, np.float32)))
    for name, w, xx in cases:
        for normalize in (1, 0):
            ids, wts = run_router(dev, w, xx, E, K, top_k, normalize)
            rid, rw, lg, _ = orc.moe_router_q4_0(w, xx, E, K, top_k, normalize)
            assert np.array_equal(ids, rid), (name, normalize, ids, rid)
            assert np.all(np.abs(wts - rw) <= 2.0 ** -22 * np.abs(rw)), (name, normalize, wts, rw)
    # the closed forms the oracle gives for these rows
    _, rw, _, _ = orc.moe_router_q4_0(cases[0][1], x, E, K, top_k, 1)
    assert np.allclose(rw, 1.0 / 3.0, rtol=1e-15)
    _, rw, _, _ = orc.moe_router_q4_0(cases[1][1], x, E, K, top_k, 1)
    assert np.array_equal(rw[:, :2], np.full((2, 2), 0.5)) and np.all(rw[:, 2] == 0.0)
    _, rw, _, _ = orc.moe_router_q4_0(cases[2][1], cases[2][2], E, K, top_k, 0)
    assert np.all(rw == 0.0)


@pytest.mark.parametrize("scale", [-140, -60, 60, 100])
def test_router_token_magnitudes(dev, orc, scale):
    """The router's logits take the same per-token scaling as the GEMV
    kernels: top-k validity and weights against the oracle hold from
    subnormal tokens to 2^100."""
    E, K, top_k, M = 64, 2048, 6, 3
    w, x = router_inputs(8300 + scale, M, E, K)
    x = (x.astype(np.float64) * 2.0 ** scale).astype(np.float32)
    for normalize in (1, 0):
        ids, wts = run_router(dev, w, x, E, K, top_k, normalize)
        check_router(orc, ids, wts, w, x, E, K, top_k, normalize, "scale 2^%d" % scale)
