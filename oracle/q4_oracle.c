/*
 * q4_oracle.c -- plain, slow, obviously-correct CPU oracle for 4-bit
 * block-quantized dequantization and GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no source, header, table or helper with the
 * HIP library; it is written from the format definitions on the pages below.
 *
 * Sources (the pages):
 *  [TG]  trueno-gpu 0.4.11, src/kernels/quantize/fused.rs
 *        - FusedRmsNormQ4KGemvKernel::build_ptx, PHASE 1 and PHASE 2
 *          (sum of squares, rsqrt(mean + eps), x * rms_inv * gamma)
 *        - FusedRmsNormQ4KGemvKernel::build_ptx, PHASE 3 (Q4_K super-block:
 *          f16 d at +0, f16 dmin at +2, 12 scale bytes at +4, qs at +16;
 *          6-bit scale/min extraction for sub-blocks 0-3 and 4-7; 64-value
 *          qs chunks with low nibbles first; value = d*scale*q - dmin*min)
 *        - FusedGateUpQ4KGemvKernel doc comment (two outputs, one input)
 *  [AT]  atlas, spark_model/layers/ops/gemm_quant.rs
 *        - moe_gate_topk_fused (router: gate GEMV over the experts, top-K
 *          indices and softmax weights, normalize flag)
 *  [IL]  inferencelayer 0.2.13, src/bin/kernel_lab.rs
 *        - GEMV_F16S WGSL (q4_lo / q4_hi: low nibble of byte j is element j,
 *          high nibble is element j+16, both minus 8, times the f16 scale)
 *        - MOE_PURE_READ WGSL and moe_lab (expert-stacked rows
 *          row = eid*rows + r, selection per (column, slot); one output
 *          per (column, slot, row) from the gate and up matrices)
 *
 * Arithmetic: every dequantized weight is formed exactly in double and
 * rounded to float once (the one correct fp32 value); every GEMV sum is a
 * double accumulation of exact double products of fp32 operands; RMSNorm is
 * in fp32 apart from the sum of squares, which is accumulated in double.
 * Build with -ffp-contract=off (no fused multiply-add anywhere).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define Q4_0_BLOCK_ELEMS 32
#define Q4_0_BLOCK_BYTES 18
#define Q4K_SB_ELEMS 256
#define Q4K_SB_BYTES 144

/* ------------------------------------------------------------------------
 * IEEE-754 binary16 -> value, from the bit layout: 1 sign bit, 5 exponent
 * bits (bias 15), 10 fraction bits.  [TG] loads d and dmin as f16 and
 * converts to f32; [IL] reads f16 scales.  Returned as double; the value is
 * always exactly representable as a float.
 * ---------------------------------------------------------------------- */
static double f16_value(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 31;
    int frac = h & 1023;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);               /* zero and subnormals */
    else if (expo == 31)
        v = frac ? (double)NAN : (double)INFINITY;   /* inf and NaN */
    else
        v = ldexp((double)(1024 + frac), expo - 25); /* normals */
    return sign ? -v : v;
}

float oracle_f16_to_f32(uint16_t h) { return (float)f16_value(h); }

static uint16_t le16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ------------------------------------------------------------------------
 * Q4_K 6-bit scale and min of sub-block j (0..7) from the 12 packed bytes S.
 * [TG] PHASE 3: sub-blocks 0-3 take the low 6 bits of S[j] and S[j+4];
 * sub-blocks 4-7 take a low nibble from S[j+4] and two high bits from the
 * top of S[j-4] (scale) or S[j] (min).
 * ---------------------------------------------------------------------- */
void oracle_q4k_scale_min(const uint8_t* S, int j, int* sc, int* m)
{
    if (j < 4) {
        *sc = S[j] & 63;
        *m = S[j + 4] & 63;
    } else {
        *sc = (S[j + 4] & 0x0F) | ((S[j - 4] >> 6) << 4);
        *m = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);
    }
}

/* One Q4_0 block (18 bytes) -> 32 floats.  [IL] GEMV_F16S: element j takes
 * the low nibble of qs byte j, element j+16 its high nibble; w = d*(q-8). */
static void dequant_q4_0_block(const uint8_t* blk, float* out)
{
    double d = f16_value(le16(blk));
    const uint8_t* qs = blk + 2;
    for (int j = 0; j < 16; ++j) {
        int lo = qs[j] & 0x0F;
        int hi = qs[j] >> 4;
        out[j] = (float)(d * (double)(lo - 8));
        out[j + 16] = (float)(d * (double)(hi - 8));
    }
}

/* One Q4_K super-block (144 bytes) -> 256 floats.  [TG] PHASE 3: element t
 * lives in qs chunk c = t/64 at byte 32c + t%32, low nibble when t%64 < 32
 * and high nibble otherwise; it belongs to sub-block t/32.  The value
 * d*sc*q - dmin*m is exact in double (at most 50 significant bits between
 * the two products) and is rounded to float once. */
static void dequant_q4k_superblock(const uint8_t* sb, float* out)
{
    double d = f16_value(le16(sb));
    double dmin = f16_value(le16(sb + 2));
    const uint8_t* S = sb + 4;
    const uint8_t* qs = sb + 16;
    for (int t = 0; t < Q4K_SB_ELEMS; ++t) {
        int c = t / 64;
        int i = t % 32;
        int h = (t % 64) / 32;
        int q = (qs[32 * c + i] >> (4 * h)) & 0x0F;
        int sc, m;
        oracle_q4k_scale_min(S, t / 32, &sc, &m);
        out[t] = (float)(d * (double)sc * (double)q - dmin * (double)m);
    }
}

/* Dequantize N rows of K weights (row-major, rows contiguous). */
void oracle_dequant_q4_0(const uint8_t* w, int64_t N, int64_t K, float* out)
{
    int64_t nb = K / Q4_0_BLOCK_ELEMS;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nb; ++b)
            dequant_q4_0_block(w + (n * nb + b) * Q4_0_BLOCK_BYTES,
                               out + n * K + b * Q4_0_BLOCK_ELEMS);
}

/* ------------------------------------------------------------------------
 * Q4_0 in split arrays ([IL] GEMV_F16S: `scales: array<f16>` and `quants:
 * array<vec4<u32>>`, one f16 scale and one 16-byte vector per block of 32
 * weights).  Row n holds nb = K/32 blocks: scale of block b at
 * scales[n*nb + b], its 16 nibble bytes at quants[(n*nb + b)*16 ..]; the
 * nibbles mean what they mean in an 18-byte block (q4_lo / q4_hi: the low
 * nibble of byte j is element j, the high nibble element j+16, minus 8).
 * ---------------------------------------------------------------------- */
void oracle_dequant_q4_0_soa(const uint8_t* scales, const uint8_t* quants, int64_t N,
                             int64_t K, float* out)
{
    int64_t nb = K / Q4_0_BLOCK_ELEMS;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nb; ++b) {
            double d = f16_value(le16(scales + 2 * (n * nb + b)));
            const uint8_t* q = quants + 16 * (n * nb + b);
            float* o = out + n * K + b * Q4_0_BLOCK_ELEMS;
            for (int j = 0; j < 32; ++j) {
                int v = j < 16 ? (q[j] & 0x0F) : (q[j - 16] >> 4);
                o[j] = (float)(d * (double)(v - 8));
            }
        }
}

/* The split-array form of N rows of 18-byte Q4_0 blocks: a byte copy. */
void oracle_q4_0_to_soa(const uint8_t* w, int64_t N, int64_t K, uint8_t* scales,
                        uint8_t* quants)
{
    int64_t nblk = N * (K / Q4_0_BLOCK_ELEMS);
    for (int64_t i = 0; i < nblk; ++i) {
        memcpy(scales + 2 * i, w + Q4_0_BLOCK_BYTES * i, 2);
        memcpy(quants + 16 * i, w + Q4_0_BLOCK_BYTES * i + 2, 16);
    }
}

/* Q4_K rows whose K is not a multiple of 256 ([TG] PHASE 3 sizes a row by
 * ceiling division, (K + 255) / 256 super-blocks, while the format defines
 * whole super-blocks only).  The reading taken here: a row is
 * ceil(K/256) super-blocks of 144 bytes, its elements are the first K of
 * their 256 * ceil(K/256) values, and the rest of the last super-block is
 * padding that no result depends on. */
static int64_t q4k_row_superblocks(int64_t K)
{
    return (K + Q4K_SB_ELEMS - 1) / Q4K_SB_ELEMS;
}

void oracle_dequant_q4k(const uint8_t* w, int64_t N, int64_t K, float* out)
{
    int64_t nb = q4k_row_superblocks(K);
    float tmp[Q4K_SB_ELEMS];
    for (int64_t n = 0; n < N; ++n)
        for (int64_t s = 0; s < nb; ++s) {
            int64_t k0 = s * Q4K_SB_ELEMS;
            int64_t cnt = K - k0 < Q4K_SB_ELEMS ? K - k0 : Q4K_SB_ELEMS;
            dequant_q4k_superblock(w + (n * nb + s) * Q4K_SB_BYTES, tmp);
            memcpy(out + n * K + k0, tmp, sizeof(float) * (size_t)cnt);
        }
}

/* ------------------------------------------------------------------------
 * GEMV y[m,n] = sum_k w[n,k] * x[m,k] (the plain definition), with
 * absdot[m,n] = sum_k |w[n,k] * x[m,k]| beside it.  Both in double: each
 * product of two floats is exact in double.
 * ---------------------------------------------------------------------- */
typedef struct {
    int fmt; /* 0 = Q4_0, 1 = Q4_K, 2 = Q4_0 split arrays (w: scales, w2: quants) */
    const uint8_t* w;
    const uint8_t* w2;
    const float* x;
    int64_t M, N, K;
    double* y;
    double* absdot;
    int64_t row0, row1;
} gemv_job;

static void* gemv_worker(void* arg)
{
    gemv_job* j = (gemv_job*)arg;
    float* row = (float*)malloc(sizeof(float) * (size_t)j->K);
    int64_t row_bytes = j->fmt == 0 ? (j->K / Q4_0_BLOCK_ELEMS) * Q4_0_BLOCK_BYTES
                                    : q4k_row_superblocks(j->K) * Q4K_SB_BYTES;
    for (int64_t n = j->row0; n < j->row1; ++n) {
        if (j->fmt == 0)
            oracle_dequant_q4_0(j->w + n * row_bytes, 1, j->K, row);
        else if (j->fmt == 1)
            oracle_dequant_q4k(j->w + n * row_bytes, 1, j->K, row);
        else
            oracle_dequant_q4_0_soa(j->w + n * (j->K / Q4_0_BLOCK_ELEMS) * 2,
                                    j->w2 + n * (j->K / Q4_0_BLOCK_ELEMS) * 16, 1, j->K, row);
        for (int64_t m = 0; m < j->M; ++m) {
            const float* xm = j->x + m * j->K;
            double acc = 0.0, aacc = 0.0;
            for (int64_t k = 0; k < j->K; ++k) {
                double p = (double)row[k] * (double)xm[k];
                acc += p;
                aacc += fabs(p);
            }
            j->y[m * j->N + n] = acc;
            if (j->absdot) j->absdot[m * j->N + n] = aacc;
        }
    }
    free(row);
    return NULL;
}

static void gemv_run(int fmt, const uint8_t* w, const uint8_t* w2, const float* x, int64_t M,
                     int64_t N, int64_t K, double* y, double* absdot, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > N) nthreads = (int)N;
    if (nthreads <= 1) {
        gemv_job j = {fmt, w, w2, x, M, N, K, y, absdot, 0, N};
        gemv_worker(&j);
        return;
    }
    pthread_t tid[256];
    gemv_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        gemv_job j = {fmt, w, w2, x, M, N, K, y, absdot,
                      N * t / nthreads, N * (t + 1) / nthreads};
        jobs[t] = j;
        pthread_create(&tid[t], NULL, gemv_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(tid[t], NULL);
}

void oracle_q4_0_gemv(const uint8_t* w, const float* x, int64_t M, int64_t N, int64_t K,
                      double* y, double* absdot, int nthreads)
{
    gemv_run(0, w, NULL, x, M, N, K, y, absdot, nthreads);
}

void oracle_q4k_gemv(const uint8_t* w, const float* x, int64_t M, int64_t N, int64_t K,
                     double* y, double* absdot, int nthreads)
{
    gemv_run(1, w, NULL, x, M, N, K, y, absdot, nthreads);
}

void oracle_q4_0_soa_gemv(const uint8_t* scales, const uint8_t* quants, const float* x,
                          int64_t M, int64_t N, int64_t K, double* y, double* absdot,
                          int nthreads)
{
    gemv_run(2, scales, quants, x, M, N, K, y, absdot, nthreads);
}

/* ------------------------------------------------------------------------
 * RMSNorm per row, [TG] PHASE 1 and PHASE 2: ms = sum(x^2)/K,
 * r = 1/sqrt(ms + eps), xhat = (x * r) * gamma.  fp32 throughout, except
 * that the sum of squares is accumulated in double and rounded once.
 * ---------------------------------------------------------------------- */
void oracle_rmsnorm(const float* x, const float* gamma, float eps, int64_t M, int64_t K,
                    float* xhat)
{
    for (int64_t m = 0; m < M; ++m) {
        const float* xm = x + m * K;
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) ss += (double)xm[k] * (double)xm[k];
        float ms = (float)(ss / (double)K);
        float r = 1.0f / sqrtf(ms + eps);
        for (int64_t k = 0; k < K; ++k) xhat[m * K + k] = (xm[k] * r) * gamma[k];
    }
}

/* RMSNorm followed by Q4_K GEMV on the normalized rows ([TG] doc of
 * FusedRmsNormQ4KGemvKernel: normalize, then multiply). xhat_out may be NULL. */
void oracle_fused_rmsnorm_q4k_gemv(const uint8_t* w, const float* x, const float* gamma,
                                   float eps, int64_t M, int64_t N, int64_t K, double* y,
                                   double* absdot, float* xhat_out, int nthreads)
{
    float* xhat = (float*)malloc(sizeof(float) * (size_t)(M * K));
    oracle_rmsnorm(x, gamma, eps, M, K, xhat);
    oracle_q4k_gemv(w, xhat, M, N, K, y, absdot, nthreads);
    if (xhat_out) memcpy(xhat_out, xhat, sizeof(float) * (size_t)(M * K));
    free(xhat);
}

/* Gate and up projections of the same input ([TG] FusedGateUpQ4KGemvKernel
 * doc): two independent GEMVs. */
void oracle_gate_up_q4k_gemv(const uint8_t* wg, const uint8_t* wu, const float* x, int64_t M,
                             int64_t N, int64_t K, double* gate, double* up,
                             double* absgate, double* absup, int nthreads)
{
    oracle_q4k_gemv(wg, x, M, N, K, gate, absgate, nthreads);
    oracle_q4k_gemv(wu, x, M, N, K, up, absup, nthreads);
}

/* ------------------------------------------------------------------------
 * Expert-selected gate/up Q4_0 GEMV ([IL] moe_lab, MOE_PURE_READ): the
 * weights are expert-stacked, expert e's row r being global row e*N + r.
 * For token m and slot s the expert is e = ids[m*top_k + s] and
 * gate[m,s,r] = sum_k Wg[e][r][k] * x[m,k] (likewise up).  An id outside
 * [0, E) yields NaN rows (the library's documented behaviour).
 * ---------------------------------------------------------------------- */
void oracle_moe_q4_0_gemv(const uint8_t* wg, const uint8_t* wu, const float* x,
                          const int32_t* ids, int64_t M, int64_t top_k, int64_t E, int64_t N,
                          int64_t K, double* gate, double* up, double* absgate,
                          double* absup, int nthreads)
{
    int64_t mat_bytes = N * (K / Q4_0_BLOCK_ELEMS) * Q4_0_BLOCK_BYTES;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t s = 0; s < top_k; ++s) {
            int64_t p = m * top_k + s;
            int32_t e = ids[p];
            double* g = gate + p * N;
            double* u = up + p * N;
            double* ag = absgate ? absgate + p * N : NULL;
            double* au = absup ? absup + p * N : NULL;
            if (e < 0 || e >= E) {
                for (int64_t r = 0; r < N; ++r) {
                    g[r] = NAN;
                    u[r] = NAN;
                    if (ag) ag[r] = NAN;
                    if (au) au[r] = NAN;
                }
                continue;
            }
            oracle_q4_0_gemv(wg + e * mat_bytes, x + m * K, 1, N, K, g, ag, nthreads);
            oracle_q4_0_gemv(wu + e * mat_bytes, x + m * K, 1, N, K, u, au, nthreads);
        }
    }
}

/* ------------------------------------------------------------------------
 * SiLU-gated product of a gate and an up projection, elementwise:
 *   h = silu(g) * u,  silu(g) = g * sigmoid(g) = g / (1 + exp(-g)).
 * [IL] moe_lab: the expert kernel writes ONE [columns, top_k, rows] output
 * from the gate (w1) and up (w3) matrices; this is the reading of that
 * single output (the SwiGLU gate of the two projections).  Double
 * throughout; a NaN in g or u gives a NaN.
 * ---------------------------------------------------------------------- */
void oracle_silu_mul(const double* g, const double* u, int64_t n, double* h)
{
    for (int64_t i = 0; i < n; ++i) {
        double s = g[i] / (1.0 + exp(-g[i]));
        h[i] = s * u[i];
    }
}

/* ------------------------------------------------------------------------
 * Expert down-projection over the selected experts, Q4_0: every (token,
 * slot) pair p = m*top_k + s has its own input row h[p] (the gated
 * activation its expert produced) and is multiplied by the down matrix of
 * the same expert e = ids[p]:
 *   y[p, r] = sum_k Wd[e*N + r, k] * h[p, k].
 * [IL] moe_lab: expert-stacked rows and the per-(column, slot) selection,
 * here applied to the projection that follows the gate and up matrices.
 * An id outside [0, E) yields NaN rows, as for the gate/up call.
 * ---------------------------------------------------------------------- */
void oracle_moe_q4_0_down(const uint8_t* wd, const float* h, const int32_t* ids, int64_t M,
                          int64_t top_k, int64_t E, int64_t N, int64_t K, double* y,
                          double* absy, int nthreads)
{
    int64_t mat_bytes = N * (K / Q4_0_BLOCK_ELEMS) * Q4_0_BLOCK_BYTES;
    for (int64_t p = 0; p < M * top_k; ++p) {
        int32_t e = ids[p];
        double* yp = y + p * N;
        double* ap = absy ? absy + p * N : NULL;
        if (e < 0 || e >= E) {
            for (int64_t r = 0; r < N; ++r) {
                yp[r] = NAN;
                if (ap) ap[r] = NAN;
            }
            continue;
        }
        oracle_q4_0_gemv(wd + e * mat_bytes, h + p * K, 1, N, K, yp, ap, nthreads);
    }
}

/* ------------------------------------------------------------------------
 * Router top-k with softmax weights, per token row of logits [M, E]
 * ([AT] moe_gate_topk_fused: gate logits over the experts, then the top-K
 * indices and their softmax weights, with a normalize flag).
 *   ids[m, s]: the s-th largest logit's expert (s = 0 first), by repeated
 *              argmax; equal logits go to the lower expert index, and a NaN
 *              logit ranks as -inf.
 *   weights:   p_e = exp(l_e - lmax) / D with lmax the largest non-NaN
 *              logit and D the sum over the selected experts (normalize !=
 *              0) or over all E experts (normalize == 0: the full softmax's
 *              entries).  The page gives no rule for infinite or NaN logits;
 *              the reading here: a logit equal to lmax has term exactly 1
 *              (also for an infinite lmax), a NaN logit term 0, and a zero
 *              D gives zero weights.
 * Double throughout.
 * ---------------------------------------------------------------------- */
/* The unnormalized softmax term of logit v against the largest logit lmax:
 * exp(v - lmax), with v - lmax taken as 0 where v equals lmax (experts tied
 * at an infinite maximum share its weight, as equal logits do) and 0 for a
 * NaN logit. */
static double softmax_term(double v, double lmax)
{
    if (isnan(v)) return 0.0;
    if (v == lmax) return 1.0;
    return exp(v - lmax);
}

void oracle_topk_softmax(const double* logits, int64_t M, int64_t E, int64_t top_k,
                         int normalize, int32_t* ids, double* weights)
{
    char* taken = (char*)malloc((size_t)E);
    for (int64_t m = 0; m < M; ++m) {
        const double* l = logits + m * E;
        memset(taken, 0, (size_t)E);
        for (int64_t s = 0; s < top_k; ++s) {
            int64_t best = -1;
            double bv = 0.0;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                double v = isnan(l[e]) ? -INFINITY : l[e];
                if (best < 0 || v > bv) {
                    best = e;
                    bv = v;
                }
            }
            taken[best] = 1;
            ids[m * top_k + s] = (int32_t)best;
        }
        /* lmax: the largest non-NaN logit (NaN when every logit is NaN). */
        double lmax = NAN;
        for (int64_t e = 0; e < E; ++e)
            if (!isnan(l[e]) && (isnan(lmax) || l[e] > lmax)) lmax = l[e];
        double den = 0.0;
        if (normalize) {
            for (int64_t s = 0; s < top_k; ++s) den += softmax_term(l[ids[m * top_k + s]], lmax);
        } else {
            for (int64_t e = 0; e < E; ++e) den += softmax_term(l[e], lmax);
        }
        for (int64_t s = 0; s < top_k; ++s) {
            double t = softmax_term(l[ids[m * top_k + s]], lmax);
            weights[m * top_k + s] = den > 0.0 ? t / den : 0.0;
        }
    }
    free(taken);
}

/* The router: Q4_0 gate logits over E expert rows (the plain GEMV), then
 * oracle_topk_softmax.  logits / abslogits ([M, E], may be NULL) receive the
 * logits and their sums of |w x|. */
void oracle_moe_router_q4_0(const uint8_t* w, const float* x, int64_t M, int64_t E, int64_t K,
                            int64_t top_k, int normalize, int32_t* ids, double* weights,
                            double* logits, double* abslogits)
{
    double* l = (double*)malloc(sizeof(double) * (size_t)(M * E));
    double* a = (double*)malloc(sizeof(double) * (size_t)(M * E));
    oracle_q4_0_gemv(w, x, M, E, K, l, a, 1);
    oracle_topk_softmax(l, M, E, top_k, normalize, ids, weights);
    if (logits) memcpy(logits, l, sizeof(double) * (size_t)(M * E));
    if (abslogits) memcpy(abslogits, a, sizeof(double) * (size_t)(M * E));
    free(l);
    free(a);
}

/* Per-row checksum of packed weight rows: the sum of the row's little-endian
 * 32-bit words, modulo 2^32 (what a pure-read pass over the same bytes must
 * report).  row_bytes must be a multiple of 4. */
void oracle_row_checksum(const uint8_t* w, int64_t nrows, int64_t row_bytes, uint32_t* out)
{
    for (int64_t n = 0; n < nrows; ++n) {
        const uint8_t* r = w + n * row_bytes;
        uint32_t s = 0;
        for (int64_t b = 0; b + 4 <= row_bytes; b += 4)
            s += (uint32_t)r[b] | ((uint32_t)r[b + 1] << 8) | ((uint32_t)r[b + 2] << 16) |
                 ((uint32_t)r[b + 3] << 24);
        out[n] = s;
    }
}

int oracle_abi_version(void) { return 2; }
