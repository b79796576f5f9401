/*
 * q4gemv.h -- C ABI of libq4gemv: decode-time GEMV over 4-bit
 * block-quantized weights on AMD Instinct MI355X (gfx950).
 *
 * Weight formats (little-endian, rows contiguous, row n of a matrix starts at
 * byte n * row_bytes):
 *
 *   Q4_0, 18 bytes per block of 32 weights, row_bytes = K/32 * 18:
 *     +0  f16 d
 *     +2  16 bytes of nibbles: the low nibble of byte j is element j, the
 *         high nibble is element j+16; weight = d * (q - 8).
 *     (inferencelayer 0.2.13, src/bin/kernel_lab.rs, GEMV_F16S WGSL:
 *      q4_lo / q4_hi and the per-block scale.)
 *
 *   Q4_K, 144 bytes per super-block of 256 weights,
 *   row_bytes = ceil(K/256) * 144:
 *     +0  f16 d, +2 f16 dmin, +4 twelve bytes S packing eight 6-bit scales
 *     and eight 6-bit mins, +16 128 bytes of nibbles.  Sub-block j (32
 *     weights) has scale sc_j and min m_j: for j < 4, sc_j = S[j] & 63 and
 *     m_j = S[j+4] & 63; for j >= 4, sc_j = (S[j+4] & 15) | (S[j-4] >> 6) << 4
 *     and m_j = (S[j+4] >> 4) | (S[j] >> 6) << 4.  Element t of the
 *     super-block is in byte 32*(t/64) + t%32 of the nibbles, low nibble when
 *     t%64 < 32, high nibble otherwise; weight = d*sc_j*q - dmin*m_j with
 *     j = t/32.  When K is not a multiple of 256 (it must be one of 32),
 *     a row's last super-block holds only its first K % 256 weights; the
 *     rest of it (nibbles and the 6-bit fields of the unused sub-blocks) is
 *     padding that no result depends on.
 *     (trueno-gpu 0.4.11, src/kernels/quantize/fused.rs,
 *      FusedRmsNormQ4KGemvKernel::build_ptx, PHASE 3; that page sizes a row
 *      by ceiling division, (K + 255) / 256 super-blocks.)
 *
 * Activations x / X are fp32 [M, K] row-major; outputs are fp32 [M, N]
 * row-major (for the expert call, [M, top_k, N]).  GEMV means
 * y[m, n] = sum_k w[n, k] * x[m, k], evaluated in fp32 with fp32
 * accumulation.
 *
 * Accuracy of every GEMV output (per token row m and output row n):
 *     |y - y_exact| <= 1e-4 * sum_k |w[n,k] * x[m,k]| + 2^-149
 * (the last term is the fp32 output's own quantum in the subnormal range),
 * for every finite x whose outputs are representable (sum_k |w x| < 2^126),
 * provided two conditions hold; neither depends on the token's magnitude,
 * because every token row is scaled by a power of two before use:
 *   (1) the dequant-dot sums the two exact parts of each weight w = a - b
 *       separately (Q4_0: a = d*q, b = 8*d; Q4_K: a = d*sc*q, b = dmin*m),
 *       so its rounding error scales with sum_k (|a_k| + |b_k|) |x_k|; the
 *       bound is guaranteed while that sum is at most 8 * sum_k |w_k x_k|
 *       (random weights of the formats' usual distributions give about 3.9
 *       for Q4_0 and 1.3 for Q4_K; a token concentrated on weights whose
 *       two parts cancel can exceed it);
 *   (2) batched dense calls with M >= 3, and any batch the VALU kernel
 *       cannot stage whole (the matrix-core path), carry each
 *       x as two f16 parts of x * 2^e, which represents elements down to
 *       2^-38 * max_k |x[m,k]| to 22 bits and smaller ones with an absolute
 *       error up to 2^-39 * max_k |x[m,k]|; the bound holds while
 *       sum_k |w x| >= 2^-24 * max_k |x[m,k]| * sum_k |w[n,k]|.  The other
 *       paths carry every element at fp32 precision.
 * The RMSNorm calls accept any finite x and gamma: the normalized row is
 * the fp32 value of the definition (its sum of squares accumulated in
 * fp64, so it cannot overflow; a mean square beyond the fp32 range gives
 * r = 0 and a zero row), and the bound applies with x replaced by it.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers (memory of the current HIP device) unless
 *     stated otherwise.  The caller owns every buffer; the library never
 *     allocates, frees or keeps a pointer, and keeps no per-call state.
 *   - Inputs are read-only; outputs are fully overwritten (never
 *     accumulated into) and must not alias any input.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *     null stream).  Results are valid once work queued later on the same
 *     stream can observe them.
 *   - Arguments are validated on the host before any HIP call; on a
 *     validation error nothing is launched and a status > 0 is returned.
 *     Q4_ERR_HIP means the launch itself failed; kernel faults surface, as
 *     usual for HIP, on a later synchronization.
 *   - Limits: 1 <= M <= Q4_MAX_M for the dense calls, 1 <= M <= 8 for the
 *     expert calls and the router (Q4_ERR_BATCH); 0 < K <= Q4_MAX_K with
 *     K % 32 == 0 for Q4_K and K % 64 == 0 for Q4_0 (an even block count
 *     keeps every Q4_0 row 4-byte aligned); a single token (M = 1) and the
 *     expert calls: M * ceil(K/64) * 64 <= Q4_MAX_MK (their activations are
 *     staged whole in LDS); dense batches of M >= 2 have no M * K limit
 *     (the matrix-core kernel stages K in slices when the rows do not fit
 *     at once, with the same results bit for bit); 1 <= N < 2^31
 *     (Q4_ERR_SHAPE).  Weight and x
 *     pointers 16-byte aligned, all other pointers 4-byte aligned
 *     (Q4_ERR_ALIGN).  Values out of range are refused, never clamped.
 *   - The library is re-entrant; calls on different streams may overlap.
 *
 * Environment variables (read once per process; for measurements and
 * comparisons only, results stay within the same bounds):
 *   Q4GEMV_MFMA=0          batches of M >= 3 on the VALU kernel instead of
 *                          the matrix cores
 *   Q4GEMV_MOE_MFMA=1      the expert call (M >= 2) on the matrix cores
 *   Q4GEMV_XR=0            single-token activations read from LDS instead of
 *                          registers
 *   Q4GEMV_LG=n            lanes per row group of the VALU kernel (power of
 *                          two, 4..64)
 *   Q4GEMV_WG_PER_CU=n     at most n resident workgroups per CU
 *   Q4GEMV_BLOCKS_PER_CU=n workgroups per CU in the VALU kernel's grid
 *   Q4GEMV_MFMA_KS=n       waves splitting a matrix-core tile's K range
 *                          (1, 2, 4 or 8)
 *   Q4GEMV_SPLITK_KP=n     K parts of the split-K calls (their workspace
 *                          size follows)
 *   Q4GEMV_DOWN_RR=n       rows per lane of the expert down-projection (1 or 2)
 *   Q4GEMV_DOWN_WG_PER_CU=n  resident workgroups per CU of the expert
 *                          down-projection
 */
#ifndef Q4GEMV_H
#define Q4GEMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    Q4_OK = 0,
    Q4_ERR_NULL = 1,   /* a required pointer is NULL */
    Q4_ERR_SHAPE = 2,  /* N, K, E, top_k or M*K outside the documented limits */
    Q4_ERR_BATCH = 3,  /* M outside [1, 16] (dense calls) or [1, 8] (experts, router) */
    Q4_ERR_ALIGN = 4,  /* a pointer is not aligned as documented */
    Q4_ERR_ARG = 5,    /* another argument is invalid (eps, kernel id) */
    Q4_ERR_HIP = 6     /* the HIP runtime refused the launch */
};

/* Largest M * K (K rounded up to a multiple of 64) of a call whose
 * activations are staged whole in the 160 KB LDS of a compute unit: single
 * tokens and the expert calls. */
#define Q4_MAX_MK 32768

/* Largest batch M of the dense calls, and largest K of any call. */
#define Q4_MAX_M 16
#define Q4_MAX_K (1 << 20)

/* Human-readable text of a status code (static storage, never NULL). */
const char* q4_strerror(int status);

/* ABI version of this header (incremented on any signature change). */
int q4_version(void);

/*
 * y[M, N] = X[M, K] . W^T with W in Q4_0 (N rows).  The weights are read
 * once for all M rows of X.
 * (inferencelayer 0.2.13, src/bin/kernel_lab.rs: GEMV_F16S, several
 *  activation columns per weight read.)
 */
int q4_0_gemv(float* y, const void* w, const float* x,
              int64_t M, int64_t N, int64_t K, void* stream);

/*
 * y[M, N] = X[M, K] . W^T with W in Q4_K (N rows), weights read once for all M.
 * (trueno-gpu 0.4.11, fused.rs, FusedRmsNormQ4KGemvKernel PHASE 3.)
 */
int q4k_gemv(float* y, const void* w, const float* x,
             int64_t M, int64_t N, int64_t K, void* stream);

/*
 * RMSNorm of every row of X, then Q4_K GEMV of the normalized rows:
 *   r_m = 1 / sqrt(sum_k x[m,k]^2 / K + eps),  xhat[m,k] = (x[m,k] * r_m) * gamma[k],
 *   y[m, n] = sum_k w[n,k] * xhat[m,k].
 * The normalization is fp32 and never leaves the chip.  gamma: fp32 [K].
 * eps must be finite and >= 0 (Q4_ERR_ARG).
 * (trueno-gpu 0.4.11, fused.rs, FusedRmsNormQ4KGemvKernel, PHASE 1 to 3.)
 */
int fused_rmsnorm_q4k_gemv(float* y, const void* w, const float* x, const float* gamma,
                           float eps, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * gate[M, N] = X . Wg^T and up[M, N] = X . Wu^T, both Q4_K with N rows, from
 * one staging of X.  gate and up must not overlap.
 * (trueno-gpu 0.4.11, fused.rs, FusedGateUpQ4KGemvKernel.)
 */
int fused_gate_up_q4k_gemv(float* gate, float* up, const void* w_gate, const void* w_up,
                           const float* x, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * RMSNorm feeding the gate+up pair in one launch: with xhat the normalized
 * rows of fused_rmsnorm_q4k_gemv (fp32, on chip, never written out),
 *   gate[M, N] = Xhat . Wg^T and up[M, N] = Xhat . Wu^T,
 * both Q4_K with N rows, from one staging of the normalized rows (same
 * layouts, limits and eps rule as the two calls it combines).  gate and up
 * must not overlap.  (trueno-gpu 0.4.11, fused.rs: FusedRmsNormQ4KGemvKernel,
 * the normalization kept on chip, and FusedGateUpQ4KGemvKernel, the pair
 * that shares one input load.)
 */
int fused_rmsnorm_gate_up_q4k_gemv(float* gate, float* up, const void* w_gate,
                                   const void* w_up, const float* x, const float* gamma,
                                   float eps, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * SiLU-gated gate+up: the one output
 *   h[m, n] = silu(gate[m, n]) * up[m, n],  silu(g) = g / (1 + exp(-g)),
 * with gate and up the two products of fused_gate_up_q4k_gemv (same layouts,
 * same limits), computed from one staging of X and never written out.  h is
 * fp32 [M, N] and must not overlap the inputs.  The epilogue is fp32 (a few
 * ulp); gate and up are accumulated exactly as fused_gate_up_q4k_gemv
 * accumulates them.  The pages' expert kernel emits one output per (token,
 * slot, row) from the gate and up matrices; this call is that single output
 * for the dense pair (inferencelayer 0.2.13, kernel_lab.rs, moe_lab: one
 * [columns, top_k, rows] output; trueno-gpu 0.4.11, fused.rs,
 * FusedGateUpQ4KGemvKernel: the pair that shares one input load).
 */
int fused_gate_up_silu_q4k_gemv(float* h, const void* w_gate, const void* w_up,
                                const float* x, int64_t M, int64_t N, int64_t K,
                                void* stream);

/*
 * The two above together: RMSNorm feeding the gate+up pair, with the one
 * output h[m, n] = silu(gate[m, n]) * up[m, n] of fused_rmsnorm_gate_up_q4k_gemv's
 * gate and up (same layouts, limits and eps rule; gate and up are never
 * written out).
 */
int fused_rmsnorm_gate_up_silu_q4k_gemv(float* h, const void* w_gate, const void* w_up,
                                        const float* x, const float* gamma, float eps,
                                        int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Expert-selected gate/up GEMV over Q4_0 experts.  w_gate and w_up each hold
 * E expert matrices of N rows, stacked: expert e's row r is global row
 * e*N + r.  ids: int32 [M, top_k], the experts chosen for each token.  For
 * token m and slot s with e = ids[m, s]:
 *   gate[m, s, r] = sum_k Wg[e*N + r, k] * x[m, k]   (likewise up),
 * gate and up being fp32 [M, top_k, N].  Only the selected experts' rows
 * are read, each selected expert once per call however many tokens chose it.
 * Precondition 0 <= ids < E (the ids live on the device, so they cannot be
 * checked without a synchronization): an id outside it reads nothing and
 * yields NaN in that (token, slot)'s rows.  Limits: 1 <= E < 2^20,
 * 1 <= top_k <= E, M * top_k <= 64, E * N < 2^31 (Q4_ERR_SHAPE).
 * (inferencelayer 0.2.13, src/bin/kernel_lab.rs: moe_lab and MOE_PURE_READ.)
 */
int moe_q4_gemv(float* gate, float* up, const void* w_gate, const void* w_up,
                const float* x, const int32_t* ids, int64_t M, int64_t top_k, int64_t E,
                int64_t N, int64_t K, void* stream);

/*
 * SiLU-gated expert call: the one output
 *   h[m, s, r] = silu(gate[m, s, r]) * up[m, s, r]
 * with gate and up as moe_q4_gemv computes them (same layouts, limits, id
 * precondition and expert dedupe; an invalid id yields NaN rows of h).  h is
 * fp32 [M, top_k, N].  (inferencelayer 0.2.13, kernel_lab.rs, moe_lab: the
 * expert kernel writes one [columns, top_k, rows] output from w1 and w3.)
 */
int moe_q4_gemv_silu(float* h, const void* w_gate, const void* w_up, const float* x,
                     const int32_t* ids, int64_t M, int64_t top_k, int64_t E, int64_t N,
                     int64_t K, void* stream);

/*
 * Expert down-projection over the selected experts, Q4_0: every (token,
 * slot) pair p = m * top_k + s has its own input row h[m, s] (the gated
 * activation of its expert) and is multiplied by the down matrix of the
 * same expert e = ids[m, s]:
 *   y[m, s, r] = sum_k Wd[e*N + r, k] * h[m, s, k],
 * w_down holding E expert matrices of N rows and K columns, stacked as for
 * moe_q4_gemv (expert e's row r is global row e*N + r).  h: fp32
 * [M, top_k, K]; y: fp32 [M, top_k, N].  Only the selected experts' rows
 * are read, each once per call however many pairs chose it; per expert,
 * only the input rows of the pairs that chose it are staged on chip.  Same
 * id precondition (an invalid id yields NaN rows of y), limits and
 * alignment (w_down and h 16 bytes) as moe_q4_gemv.
 * (inferencelayer 0.2.13, kernel_lab.rs, moe_lab: expert-stacked rows and
 * the per-(column, slot) expert selection, here for the projection that
 * follows the gate and up matrices.)
 */
int moe_q4_gemv_down(float* y, const void* w_down, const float* h, const int32_t* ids,
                     int64_t M, int64_t top_k, int64_t E, int64_t N, int64_t K,
                     void* stream);

/*
 * Expert router: the gate logits of each token row against E expert rows,
 * then its top_k experts and their softmax weights, in one launch
 * (atlas, spark_model/layers/ops/gemm_quant.rs, moe_gate_topk_fused: gate
 * GEMV over the experts, top-K indices and softmax weights, normalize flag;
 * here over Q4_0 router weights and for M <= 8 token rows).
 *   logits l[m, e] = sum_k Wr[e, k] * x[m, k], Wr: E rows of Q4_0 (K/32
 *                    blocks of 18 bytes each), x: fp32 [M, K]
 *   ids[m, s]      int32 [M, top_k]: the s-th largest logit's expert, s = 0
 *                  first; equal logits go to the lower expert index and a
 *                  NaN logit ranks as -inf
 *   weights[m, s]  fp32 [M, top_k]: exp(l - lmax) / D, with D summed over
 *                  the selected experts (normalize = 1: the weights sum to
 *                  1) or over all E experts (normalize = 0: the entries of
 *                  the full softmax); lmax is the largest non-NaN logit, a
 *                  logit equal to lmax weighs exactly 1 (experts tied at an
 *                  infinite maximum share the weight, as equal logits do),
 *                  a NaN logit weighs 0, and a zero D gives zero weights
 * The ids are in the layout moe_q4_gemv and moe_q4_gemv_silu take.  The
 * logits are fp32 sums within 1e-4 * sum_k |w x| of the exact ones; where
 * two experts' logits are closer than that, either order is correct.
 * Limits: M in [1, 8] (Q4_ERR_BATCH); K % 64 == 0 and K <= 32768;
 * 1 <= E <= 1024; 1 <= top_k <= min(E, 64) (Q4_ERR_SHAPE); normalize 0 or
 * 1 (Q4_ERR_ARG).  Alignment: Wr and x 16 bytes, ids and weights 4.
 */
int moe_router_q4_0(int32_t* ids, float* weights, const void* w_router, const float* x,
                    int64_t M, int64_t E, int64_t K, int64_t top_k, int normalize,
                    void* stream);

/*
 * Split-K batched GEMV with a caller workspace: y[M, N] = X[M, K] . W^T,
 * as q4_0_gemv / q4k_gemv, for batches whose activations cost more to stage
 * in every workgroup than the weights they meet there (few output rows, long
 * K).  A workgroup serves 8 tiles of 16 rows and one of kp parts of K: it
 * stages only that part of X, scaled per token by a power of two of its
 * own, and writes its partial sums to the workspace; a second kernel on the
 * same stream adds the kp partials in a fixed order, each brought to a
 * common scale, and writes y.  kp depends on N, K and the device only, so a
 * token's row does not depend on the batch.  Same bound as the two calls.
 *   q4_splitk_workspace: *bytes = the workspace these calls need for this
 *     shape on the current device (0 if the call would not split: M <= 2,
 *     which runs the VALU kernel, or a plan of one part, which runs the
 *     ordinary call).  format: Q4_FORMAT_Q4_0 or Q4_FORMAT_Q4K (Q4_ERR_ARG).
 *   workspace: device memory of at least that many bytes, 256-byte aligned,
 *     any content (it holds nothing between calls); calls that share a
 *     workspace must not overlap.  A smaller workspace: Q4_ERR_SHAPE; NULL
 *     where one is needed: Q4_ERR_NULL.  Other limits and alignment as
 *     q4_0_gemv / q4k_gemv.
 * It pays where staging dominates, i.e. for few output rows (on MI355X,
 * 4096 x 4096 at 4 / 8 / 16 tokens: 9.3 / 10.0 / 12.0 against 9.9 / 11.5 /
 * 28.0 us; the 4096 x 14336 down-projection at 4 tokens: 15.3 against
 * 25.9 us); with many output rows the ordinary call already shares its
 * staging among 128 rows per workgroup.  (The pages' kernels stage x once
 * per workgroup; splitting K over workgroups is this library's answer to
 * the staging cost of batches on a 256-CU part.)
 */
enum { Q4_FORMAT_Q4_0 = 0, Q4_FORMAT_Q4K = 1 };
int q4_splitk_workspace(int format, int64_t M, int64_t N, int64_t K, int64_t* bytes);
int q4_0_gemv_splitk(float* y, const void* w, const float* x, int64_t M, int64_t N, int64_t K,
                     void* workspace, int64_t workspace_bytes, void* stream);
int q4k_gemv_splitk(float* y, const void* w, const float* x, int64_t M, int64_t N, int64_t K,
                    void* workspace, int64_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid it):
 * q4_0_gemv_splitk_noalloc is q4_0_gemv_splitk with the library's own
 * workspace, a device array of q4_noalloc_scratch_bytes() bytes (8 MiB) per
 * GPU, held until the process ends; it allocates nothing.  A shape whose
 * workspace (q4_splitk_workspace) exceeds it: Q4_ERR_SHAPE, before any
 * launch (16 tokens of 4096 rows at K = 4096 need 2 MiB; very long K needs
 * more parts and can exceed it).  Every call on one GPU uses that GPU's one array: calls that
 * overlap on one GPU (different streams, or host threads) race and must not
 * be made.  Results equal q4_0_gemv_splitk's bit for bit.
 */
long long q4_noalloc_scratch_bytes(void);
int q4_0_gemv_splitk_noalloc(float* y, const void* w, const float* x, int64_t M, int64_t N,
                             int64_t K, void* stream);

/*
 * Q4_0 in split arrays (inferencelayer 0.2.13, kernel_lab.rs, GEMV_F16S:
 * `scales: array<f16>`, `quants: array<vec4<u32>>`): row n's block b has
 * its f16 scale at scales[n * K/32 + b] and its 16 nibble bytes at
 * quants + (n * K/32 + b) * 16, the nibbles meaning what they mean in an
 * 18-byte Q4_0 block.  Every nibble block is 16-byte aligned, so K may be
 * any multiple of 32 (an odd block count too).
 *
 * q4_0_repack_soa: the split form of N rows of 18-byte Q4_0 blocks (a byte
 * copy; scales: N * K/32 * 2 bytes, 2-byte aligned; quants: N * K/32 * 16
 * bytes, 16-byte aligned; w 2-byte aligned).
 * q4_0_gemv_soa: y[M, N] = X[M, K] . W^T over the split form, the weights
 * read once for all M; the results are those of q4_0_gemv on the 18-byte
 * form within the same bound (bit for bit at M <= 2, where both run the
 * VALU kernel).  Limits as q4_0_gemv's, with K % 32 == 0; alignment:
 * quants and x 16 bytes, scales 2, y 4.
 */
int q4_0_repack_soa(void* scales, void* quants, const void* w, int64_t N, int64_t K,
                    void* stream);
int q4_0_gemv_soa(float* y, const void* scales, const void* quants, const float* x,
                  int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Dequantize N rows of Q4_K to fp32 out[N, K], bit-exact: every weight is
 * the correctly rounded fp32 value of d*sc*q - dmin*m.
 * (trueno-gpu 0.4.11, fused.rs, FusedRmsNormQ4KGemvKernel PHASE 3.)
 */
int dequant_q4k(float* out, const void* w, int64_t N, int64_t K, void* stream);

/*
 * Dequantize N rows of Q4_0 to fp32 out[N, K], bit-exact (d*(q-8) is exact).
 * (inferencelayer 0.2.13, kernel_lab.rs, GEMV_F16S: q4_lo / q4_hi.)
 */
int dequant_q4_0(float* out, const void* w, int64_t N, int64_t K, void* stream);

/*
 * Pure-read bandwidth ceiling: reads exactly the weight bytes that the named
 * GEMV call reads, with the same addressing, work split and launch shape,
 * but does no unpack, no arithmetic on x and never reads x.  To prove every
 * byte was read it writes, for every weight row it visited, the sum of that
 * row's little-endian 32-bit words modulo 2^32.
 * (inferencelayer 0.2.13, kernel_lab.rs: MOE_PURE_READ and the pure_read
 *  variant of the dense lab, whose ratio to the real kernel separates an
 *  access-pattern limit from an arithmetic limit.)
 *
 *   kernel_id           reads                               checksum layout (uint32)
 *   Q4_READ_Q4_0_GEMV   w0: Q4_0 [N, K]                     [N]
 *   Q4_READ_Q4K_GEMV    w0: Q4_K [N, K]                     [N]
 *   Q4_READ_GATE_UP     w0, w1: Q4_K [N, K] each            [2, N]  (w0 rows, then w1)
 *   Q4_READ_MOE         w0, w1: Q4_0 experts as moe_q4_gemv [2, M, top_k, N]
 *   Q4_READ_STREAM      w0: N * K * 9/16 bytes              [ceil(bytes / 4096)]
 *   Q4_READ_MOE_DOWN    w0: Q4_0 experts as moe_q4_gemv_down [M, top_k, N]
 *
 * For a Q4_K row whose K is not a multiple of 256, the checksum covers what
 * the call reads: the super-block headers and the 32-byte nibble chunks
 * that hold an element < K (a chunk of padding only is not read).
 * Q4_READ_STREAM (K % 256 == 0) is the reference stream of the same byte count as a GEMV
 * of N rows and K columns (both formats use 9/16 byte per weight), read the
 * fastest way measured on this part: contiguous 1 KiB wave instructions
 * with the non-temporal hint, 4 KiB blocks per wave step with the next
 * block in flight, blocks strided over two 256-thread workgroups per CU.
 * Its checksums are per 4 KiB block of the range (the last one partial),
 * not per row.  M is ignored.
 *
 * M selects the launch shape of the mirrored call (and, for Q4_READ_MOE,
 * the number of tokens); ids, top_k and E are used by Q4_READ_MOE only
 * (pass NULL / 0 otherwise).  For an expert id outside [0, E) the checksum
 * rows are 0xFFFFFFFF.  Unknown kernel_id: Q4_ERR_ARG.
 */
enum {
    Q4_READ_Q4_0_GEMV = 0,
    Q4_READ_Q4K_GEMV = 1,
    Q4_READ_GATE_UP = 2,
    Q4_READ_MOE = 3,
    Q4_READ_STREAM = 4,
    Q4_READ_MOE_DOWN = 5
};
int q4_pure_read(uint32_t* checksum, int kernel_id, const void* w0, const void* w1,
                 const int32_t* ids, int64_t M, int64_t top_k, int64_t E, int64_t N, int64_t K,
                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4GEMV_H */
