// q4_router.h -- the expert router of libq4gemv: gate logits of one token
// row against E Q4_0 expert rows, then the top-k experts and their softmax
// weights, in one launch (atlas, spark_model/layers/ops/gemm_quant.rs,
// moe_gate_topk_fused: the gate GEMV over the experts, the top-K indices and
// their softmax weights with a normalize flag, one launch instead of two).
//
// One 512-thread workgroup per token row.  The row is staged in LDS as for
// the GEMV kernel (pre-scaled chunks and per-32 sums, q4_kernels.h).  The
// logits are split over the 8 waves: a lane group of lg lanes (the power of
// two covering the row's block pairs, at most 64) takes one expert row, a
// wave 64 / lg rows at a time and kRouterRows of those at once, so that the
// loads of all its rows are in flight together before any arithmetic (the
// call is latency-bound: 73 KB at the expert call's shape).  The top k
// then come from ranks, not from k rounds of an argmax (measured: each
// round of a wave-wide argmax cost ~0.9 us at E = 64): every thread counts,
// for its expert(s), how many experts are ahead (larger logit first, the
// lower expert index on equal logits, a NaN logit ranked as -inf), so the
// cost does not grow with k.  Weights, in fp32 by wave 0:
// p = exp(l - lmax) / D, D summed over the selected experts (normalize) or
// over all E (the full softmax's entries); lmax is the largest non-NaN
// logit, a NaN logit weighs 0, a logit equal to lmax weighs exactly 1.
//
// Loads stay in bounds: unit indices are clamped to the row's last block
// pair (lanes past the end compute on it and drop the result), expert rows
// are < E, and the staging clamps its activation reads to the row.
#pragma once

#include "q4_kernels.h"

namespace q4 {

constexpr int kRouterBlock = 512;
constexpr int kRouterRows = 4;  // rows per lane group whose loads go out together
constexpr int kRouterMaxE = 1024;
constexpr int kRouterMaxTopK = kWave;  // lane s of wave 0 writes pick s
constexpr int kRouterMaxK = 32768;
static_assert(kRouterBlock / kWave <= kMaxStageWaves, "staging scratch holds 8 waves");

// dynamic LDS: the staged row (chunks and run sums), E logits (padded to
// a multiple of 4), E 64-bit rank keys, the picks
inline size_t router_lds_bytes(int K, int E) {
    return (size_t)(K / kUnitElems) * kUnitChunks * 16 + (size_t)(K / 32) * 4 +
           (size_t)((E + 3) & ~3) * 4 + (size_t)E * 8 + (size_t)kRouterMaxTopK * 8;
}

static __global__ __launch_bounds__(kRouterBlock) void router_kernel(int32_t* __restrict__ ids,
                                                              float* __restrict__ weights,
                                                              const uint8_t* __restrict__ w,
                                                              const float* __restrict__ x, int E,
                                                              int K, int top_k, int normalize) {
    extern __shared__ float4 smem[];
    __shared__ StageRed red;  // staging scratch
    const int m = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    constexpr int kWaves = kRouterBlock / kWave;
    const int kq = xrow_chunks(K / kUnitElems);
    const int k64 = K >> 6;
    float4* xl = smem;
    float* xsum = (float*)(smem + kq);
    float* lg = xsum + (K >> 5);

    GemvParams p = {};
    p.x = x + (long long)m * K;
    p.K = K;
    p.upr = K / kUnitElems;
    XStage<> st;
    int xe[1];  // the row's scale exponent: the staged row is x * 2^xe
    stage_x_issue<kModeDense>(p, 1, st, kRouterBlock);
    stage_x_finish<kFmtQ4_0, 1, kModeDense, true>(p, st, xl, xsum, red, xe, kRouterBlock);
    __syncthreads();

    // ---- logits ----
    const int upr = K / kUnitElems;
    int lgw = 4;  // (group_total sums at least a quad)
    while (lgw < upr && lgw < kWave) lgw <<= 1;
    const int rpp = kWave / lgw;           // rows per wave pass
    const int gi = lane / lgw, li = lane - gi * lgw;
    const int upl = (upr + lgw - 1) / lgw;  // block pairs per lane per row
    const long long rb = (long long)(K / 32) * 18;
    const int step = kWaves * rpp * kRouterRows;
    for (int e0 = wave * rpp * kRouterRows; e0 < E; e0 += step) {
        float acc[kRouterRows][1];
#pragma unroll
        for (int q = 0; q < kRouterRows; ++q) acc[q][0] = 0.f;
        for (int i = 0; i < upl; ++i) {
            const int u = li + lgw * i;
            const bool act = u < upr;
            const int uc = act ? u : upr - 1;
            uint32_t r[kRouterRows][kUnitWords];
#pragma unroll
            for (int q = 0; q < kRouterRows; ++q) {
                // rows past E re-read row E - 1 and are never written
                const int e = min(e0 + q * rpp + gi, E - 1);
                load_unit<kFmtQ4_0>(w + (long long)e * rb + (long long)uc * kQ4_0PairBytes, 0,
                                    r[q]);
            }
            rows_dot<kFmtQ4_0, 1, kRouterRows>(r, uc, 0u, xl, kq, (const float2*)xsum, k64, acc,
                                               act);
        }
#pragma unroll
        for (int q = 0; q < kRouterRows; ++q) {
            const int e = e0 + q * rpp + gi;
            const float t = __builtin_ldexpf(group_total(acc[q][0], lgw), -xe[0]);
            if (li == lgw - 1 && e < E) lg[e] = t;
        }
    }
    __syncthreads();

    // ---- top k by rank: expert e's rank is the number of experts ahead of
    // it (larger logit, or an equal logit and a lower index); ranks 0 ..
    // top_k - 1 are the picks.  Each expert gets a 64-bit key, the logit's
    // order-preserving integer image (a NaN logit as -inf) above the
    // complement of its index, so "j ahead of e" is key_j > key_e and all
    // keys differ. ----
    // (after the logits padded to a multiple of 4: 16-byte aligned for the
    // two-key reads)
    unsigned long long* key = (unsigned long long*)(lg + ((E + 3) & ~3));
    int* sel_e = (int*)(key + E);                      // [top_k] expert of rank s
    float* sel_v = (float*)(sel_e + kRouterMaxTopK);   // [top_k] its logit
    for (int e = threadIdx.x; e < E; e += kRouterBlock) {
        const float v = lg[e];
        const uint32_t b = __builtin_bit_cast(uint32_t, v != v ? -__builtin_inff() : v);
        const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
        key[e] = ((unsigned long long)o << 32) | (uint32_t)~(uint32_t)e;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kRouterBlock) {
        const unsigned long long ke = key[e];
        int rank = 0;
        int j = 0;
        // the whole wave reads the same addresses (broadcast), two keys a read
        for (; j + 4 <= E; j += 4) {
            const ulonglong2 a = *(const ulonglong2*)(key + j);
            const ulonglong2 c = *(const ulonglong2*)(key + j + 2);
            rank += (a.x > ke) + (a.y > ke) + (c.x > ke) + (c.y > ke);
        }
        for (; j < E; ++j) rank += key[j] > ke;
        if (rank < top_k) {
            sel_e[rank] = e;
            sel_v[rank] = lg[e];
        }
    }
    __syncthreads();
    if (wave != 0) return;

    // ---- softmax weights (wave 0; lane s writes pick s) ----
    // lmax: the largest non-NaN logit (fmaxf drops NaN; NaN if all are NaN).
    // A logit's term is exp(l - lmax), taken as exp(0) = 1 where l equals
    // lmax (so experts tied at an infinite maximum share its weight, the
    // limit of equal logits), 0 for a NaN logit; with a zero denominator
    // (every term 0) the weights are 0.
    float lmax = __builtin_nanf("");
    for (int e = lane; e < E; e += kWave) lmax = fmaxf(lmax, lg[e]);
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, k, kWave));
    auto term = [&](float v) { return v != v ? 0.f : (v == lmax ? 1.f : expf(v - lmax)); };
    float ex = 0.f;
    if (normalize) {
        if (lane < top_k) ex = term(sel_v[lane]);
    } else {
        for (int e = lane; e < E; e += kWave) ex += term(lg[e]);
    }
    // wave total in lane 63, then to every lane
    ex = group_total(ex, kWave);
    ex = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), kWave - 1));
    if (lane < top_k) {
        ids[(long long)m * top_k + lane] = sel_e[lane];
        weights[(long long)m * top_k + lane] = ex > 0.f ? term(sel_v[lane]) / ex : 0.f;
    }
}

}  // namespace q4
