"""Seeded synthetic inputs for the 4-bit block-quantized GEMV workloads.

This module holds random draws and byte layout only -- none of the
dequantization or GEMV arithmetic.  Both the CPU oracle (in the tests and
the benchmark's CPU baseline) and the GPU library are fed from here.

Block layouts (little-endian):
  Q4_0 block, 18 bytes per 32 weights: f16 d, then 16 nibble bytes.
  Q4_K super-block, 144 bytes per 256 weights: f16 d, f16 dmin, 12 packed
  scale/min bytes, 128 nibble bytes.

Distributions of the workloads:
  * d (Q4_0) uniform in [0.01, 0.1], d and dmin (Q4_K) uniform in
    [0.005, 0.05]; each drawn in float64 and rounded to f16 (round to
    nearest even, numpy's conversion).
  * Nibbles uniform in 0..15: every nibble byte is a uniform random byte.
  * Q4_K 6-bit scales and mins uniform in 0..63: the 12 packed bytes are
    uniform random bytes.  Each of the 16 six-bit fields is a function of
    its own disjoint set of 6 of those 96 bits, so uniform bytes give
    independent uniform 6-bit values, with no packing step needed.
  * x ~ N(0, sigma) fp32; gamma ~ N(1, 0.1) fp32; expert ids per token drawn
    uniformly without replacement.
Draw order inside each helper is fixed: scales first, then scale/min bytes,
then nibble bytes; callers draw weights, then x, then gamma, then ids.
"""
import numpy as np

SEED_BASE = 20261202


def make_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def config_rng(config_index: int) -> np.random.Generator:
    """Generator of the named workload number (1-based), seed 20261202 + index."""
    return make_rng(SEED_BASE + int(config_index))


def f16_uniform_bits(rng, n: int, lo: float, hi: float) -> np.ndarray:
    return rng.uniform(lo, hi, size=n).astype(np.float16).view(np.uint16)


def _put_f16(dst: np.ndarray, col: int, bits: np.ndarray) -> None:
    dst[:, col] = (bits & 0xFF).astype(np.uint8)
    dst[:, col + 1] = (bits >> 8).astype(np.uint8)


def q4_0_matrix(rng, rows: int, K: int, dlo: float = 0.01, dhi: float = 0.1) -> np.ndarray:
    """Random Q4_0 weights, uint8 [rows, K/32*18]."""
    assert K % 32 == 0
    nb = rows * (K // 32)
    d = f16_uniform_bits(rng, nb, dlo, dhi)
    qs = rng.integers(0, 256, size=(nb, 16), dtype=np.uint8)
    blk = np.empty((nb, 18), dtype=np.uint8)
    _put_f16(blk, 0, d)
    blk[:, 2:] = qs
    return blk.reshape(rows, (K // 32) * 18)


def q4k_matrix(rng, rows: int, K: int, lo: float = 0.005, hi: float = 0.05) -> np.ndarray:
    """Random Q4_K weights, uint8 [rows, ceil(K/256)*144].  For K not a
    multiple of 256 the last super-block of every row is only partly used;
    its unused part is drawn like the rest (random bytes)."""
    assert K % 32 == 0
    nb = rows * ((K + 255) // 256)
    d = f16_uniform_bits(rng, nb, lo, hi)
    dmin = f16_uniform_bits(rng, nb, lo, hi)
    scales = rng.integers(0, 256, size=(nb, 12), dtype=np.uint8)
    qs = rng.integers(0, 256, size=(nb, 128), dtype=np.uint8)
    blk = np.empty((nb, 144), dtype=np.uint8)
    _put_f16(blk, 0, d)
    _put_f16(blk, 2, dmin)
    blk[:, 4:16] = scales
    blk[:, 16:] = qs
    return blk.reshape(rows, ((K + 255) // 256) * 144)


def activations(rng, M: int, K: int, sigma: float = 1.0) -> np.ndarray:
    return (rng.standard_normal((M, K)) * sigma).astype(np.float32)


def gamma(rng, K: int) -> np.ndarray:
    return (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32)


def expert_ids(rng, M: int, top_k: int, E: int) -> np.ndarray:
    return np.stack([rng.choice(E, size=top_k, replace=False) for _ in range(M)]).astype(np.int32)


def expert_ids_distinct(rng, M: int, top_k: int, E: int) -> np.ndarray:
    """All M * top_k ids distinct (every pair reads its own expert)."""
    return rng.choice(E, size=M * top_k, replace=False).reshape(M, top_k).astype(np.int32)


def q4_0_row_bytes(K: int) -> int:
    return (K // 32) * 18


def q4k_row_bytes(K: int) -> int:
    return ((K + 255) // 256) * 144


def q4_0_soa_split(w: np.ndarray):
    """The split-array form of 18-byte Q4_0 rows: (f16 scale bytes
    [rows, K/32*2], nibble bytes [rows, K/32*16]) -- a byte split, no
    arithmetic."""
    rows = w.shape[0]
    blk = np.ascontiguousarray(w).reshape(rows, -1, 18)
    return (np.ascontiguousarray(blk[:, :, 0:2]).reshape(rows, -1),
            np.ascontiguousarray(blk[:, :, 2:18]).reshape(rows, -1))


def pair_activations(rng, M: int, top_k: int, K: int, sigma: float = 1.0) -> np.ndarray:
    """Inputs of the expert down-projection, fp32 [M, top_k, K]: one row per
    (token, slot) pair."""
    return (rng.standard_normal((M, top_k, K)) * sigma).astype(np.float32)


# The five named workloads (sizes and distributions of the decode path).
WORKLOADS = {
    1: dict(name="q4_0_gemv M=1 K=512 N=256", op="q4_0_gemv", M=(1,), K=512, N=256),
    2: dict(name="q4_0_gemv K=4096 N=4096 M=1,2,4,8", op="q4_0_gemv", M=(1, 2, 4, 8),
            K=4096, N=4096),
    3: dict(name="fused_rmsnorm_q4k_gemv M=1 K=3584 N=18944", op="fused_rmsnorm_q4k_gemv",
            M=(1,), K=3584, N=18944, x_sigma=2.0, eps=1e-5),
    4: dict(name="fused_gate_up_q4k_gemv K=4096 N=14336x2 M=1,4", op="fused_gate_up_q4k_gemv",
            M=(1, 4), K=4096, N=14336),
    5: dict(name="moe_q4_gemv M=4 E=64 top_k=6 N=1408 K=2048", op="moe_q4_gemv", M=(4,),
            K=2048, N=1408, E=64, top_k=6),
}


# The step after the expert gate/up call: the down-projection of the SiLU-
# gated rows, one Q4_0 matrix of 2048 rows x 1408 columns per expert, same
# experts and ids as the gate/up workload (draws from their own seed).
DOWN = dict(name="moe_q4_gemv_down M=4 E=64 top_k=6 N=2048 K=1408", E=64, top_k=6, N=2048,
            K=1408)

# The dense down-projection after the gate+up pair of the 14336 x 4096
# workload: Q4_K, 4096 rows x 14336 columns.
DENSE_DOWN = dict(N=4096, K=14336)


def down_inputs(M: int = 4, distinct: bool = False) -> dict:
    """Inputs of the expert down-projection at batch M: the gate/up
    workload's ids, then (seed 20261202 + 6) the expert-stacked down
    matrices and one N(0, 1) input row per (token, slot) pair."""
    d5 = workload_inputs(5, M=M, distinct=distinct)
    rng = config_rng(6)
    E, N, K, top_k = DOWN["E"], DOWN["N"], DOWN["K"], DOWN["top_k"]
    return dict(M=M, E=E, N=N, K=K, top_k=top_k, ids=d5["ids"],
                w_down=q4_0_matrix(rng, E * N, K), h=pair_activations(rng, M, top_k, K))


def workload_inputs(index: int, M: int = None, rows: int = None, distinct: bool = False) -> dict:
    """Inputs of workload `index` (1..5) at batch M; `rows` < N draws only the
    first rows of every matrix (the same bytes the full draw would not give, so
    use it only where a reduced problem is wanted).  For workload 5,
    distinct=True replaces the ids by a draw of M * top_k distinct experts."""
    wl = WORKLOADS[index]
    M = wl["M"][0] if M is None else M
    N = wl["N"] if rows is None else rows
    K = wl["K"]
    rng = config_rng(index)
    out = dict(M=M, N=N, K=K, op=wl["op"])
    if index in (1, 2):
        out["w"] = q4_0_matrix(rng, N, K)
        out["x"] = activations(rng, M, K)
    elif index == 3:
        out["w"] = q4k_matrix(rng, N, K)
        out["x"] = activations(rng, M, K, wl["x_sigma"])
        out["gamma"] = gamma(rng, K)
        out["eps"] = wl["eps"]
    elif index == 4:
        out["w_gate"] = q4k_matrix(rng, N, K)
        out["w_up"] = q4k_matrix(rng, N, K)
        out["x"] = activations(rng, M, K)
    elif index == 5:
        E = wl["E"]
        out["E"] = E
        out["top_k"] = wl["top_k"]
        out["w_gate"] = q4_0_matrix(rng, E * N, K)
        out["w_up"] = q4_0_matrix(rng, E * N, K)
        out["x"] = activations(rng, M, K)
        out["ids"] = expert_ids(rng, M, wl["top_k"], E)
        if distinct:  # drawn after the primary ids, so the weights are the same
            out["ids"] = expert_ids_distinct(rng, M, wl["top_k"], E)
    return out
