// q4_moe_down.h -- the expert down-projection of libq4gemv: every (token,
// slot) pair multiplies its own input row (the gated activation its expert
// produced) by the Q4_0 down matrix of the same expert
// (inferencelayer 0.2.13, kernel_lab.rs, moe_lab: expert-stacked rows and
// the per-(column, slot) expert selection, applied to the projection that
// follows the gate and up matrices).
//
// Unlike the gate/up call, whose tokens share one input row per token, here
// every pair has a row of its own, so staging all of them in every
// workgroup would cost M * top_k rows of LDS (147 KB at 4 tokens, top-6,
// K = 1408; too much at 8 tokens).  Instead:
//   * The selected experts are deduped in the kernel (as for gate/up); the
//     grid holds ks workgroups per possible unique expert, and workgroup b
//     serves expert b / ks and the (b % ks)-th share of its rows
//     (workgroups past the dedupe's count exit at once).
//   * The workgroup stages only the rows of the pairs that chose its
//     expert (at most M with distinct ids per token; more are staged M at
//     a time), each scaled by its own power of two, then streams its share
//     of the expert's rows: lanes in groups of lg over a row's 64-weight
//     units, RR rows per group, the next step's weights in flight while
//     the current one is computed (the first step's before the staging).
//   * Every weight byte is read once for all pairs of its expert.
// The activation staging is the GEMV kernel's (pre-scaled chunks and
// 32-element run sums in LDS, q4_kernels.h) with a row map; rows are
// scaled by 2^e, e chosen so the row's largest magnitude lies in
// [2^kXTarget, 2^(kXTarget+1)), and outputs by 2^-e.
#pragma once

#include "q4_kernels.h"

namespace q4 {

constexpr int kDownBlock = 256;
#ifndef Q4_DOWN_BATCH
#define Q4_DOWN_BATCH 2
#endif
constexpr int kDownBatch = Q4_DOWN_BATCH;  // staging chunks per thread per wait
constexpr int kDownWaves = kDownBlock / kWave;
static_assert(kDownWaves <= kMaxStageWaves, "staging scratch holds 8 waves");

// LDS bytes of one workgroup: M staged rows (the GEMV kernel's layout).
inline size_t down_lds_bytes(int M, int upr) {
    return (size_t)M * upr * kUnitChunks * 16 + (size_t)M * upr * 2 * 4;
}

// y[p, r] = sum_k Wd[ids[p] * N + r, k] * h[p, k] for every pair p of M
// tokens x top_k slots.  Workgroup b serves unique expert b / p.ks and the
// (b % p.ks)-th of p.ks equal shares of its p.nrg row groups (RR rows each);
// p.upr, p.lg, p.upl, p.rgw as for the GEMV kernel.  PURE: the same weight
// loads, and per-row word checksums in place of outputs.
template <int M, int RR, bool PURE>
__global__ __launch_bounds__(kDownBlock) void moe_down_kernel(const GemvParams p) {
    constexpr int FMT = kFmtQ4_0;
    constexpr int NR = RR;
    extern __shared__ float4 smem[];
    __shared__ MoeShared moe;
    __shared__ StageRed red;
    __shared__ int sh_pr[M];  // pair of staged row j
    __shared__ int sh_e[M];   // its scale exponent
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kq = xrow_chunks(p.upr);  // LDS float4 chunks per staged row
    const int k64 = p.upr;
    float4* xl = smem;
    float* xsum = (float*)(smem + M * kq);

    moe_dedupe<M>(p, moe, moe_load_id<M>(p));
    __syncthreads();
    const int nu = __builtin_amdgcn_readfirstlane(moe.nu);
    // rows of pairs with an invalid id: NaN (or an all-ones checksum)
    if (moe.invalid) {
        const long long total = (long long)M * p.top_k * p.N;
        for (long long i = (long long)blockIdx.x * kDownBlock + tid; i < total;
             i += (long long)gridDim.x * kDownBlock) {
            const int pr = (int)(i / p.N);
            if ((moe.invalid >> pr) & 1ull) {
                if constexpr (PURE)
                    p.cks[i] = 0xFFFFFFFFu;
                else
                    p.y0[i] = __builtin_nanf("");
            }
        }
    }
    // this workgroup's expert and share of its row groups (uniform exits,
    // before any further barrier)
    const int ux = blockIdx.x / p.ks;
    const int part = blockIdx.x - ux * p.ks;
    if (ux >= nu) return;
    const int g0 = part * p.nrg / p.ks, g1 = (part + 1) * p.nrg / p.ks;
    if (g0 >= g1) return;
    const int e = __builtin_amdgcn_readfirstlane(moe.uexp[ux]);
    const unsigned long long pairs = moe.upairs[ux];
    const long long ebase = (long long)e * p.N;  // the expert's first row

    const int gi = lane / p.lg;       // row group of this lane within a wave pass
    const int li = lane - gi * p.lg;  // lane within its row group
    const int u_last = p.upr - 1;
    const uint32_t rb = (uint32_t)p.row_bytes;
    const int per_pass = kDownWaves * p.rgw;  // row groups per workgroup pass
    const int npass = (g1 - g0 + per_pass - 1) / per_pass;
    const int nsteps = npass * p.upl;

    // the weights of step q (pass q / upl, unit step q % upl) of this lane:
    // the wave's first row group of the pass kept inside the share
    // (uniform), the lane's rows clamped to the expert
    auto load = [&](int q, uint32_t (&dst)[NR][kUnitWords]) {
        const int pass = q / p.upl, ui = q - pass * p.upl;
        const int u = li + ui * p.lg;
        const uint32_t uoff = (uint32_t)min(u, u_last) * kQ4_0PairBytes;
        const int gw = min(g0 + pass * per_pass + wave * p.rgw, g1 - 1);
        const int R0 = gw * RR;
        const long long sbase = (ebase + R0) * p.row_bytes;
        const int lrow_max = p.N - 1 - R0;  // >= 0
#pragma unroll
        for (int r = 0; r < RR; ++r) {
            const uint32_t lr = (uint32_t)min(gi * RR + r, lrow_max);
            load_unit_at<FMT>(p.w0 + sbase, lr * rb + uoff, 0u, dst[r]);
        }
    };

    // pair batches of at most M staged rows (one batch unless a token chose
    // this expert twice); a pure-read pass reads once
    unsigned long long rest = pairs;
    bool first = true;
    while (rest) {
        uint32_t bufA[NR][kUnitWords], bufB[NR][kUnitWords];
        load(0, bufA);  // issued ahead of the staging
        int nb = 0;
        if constexpr (PURE) {
            rest = 0;
        } else {
            // (a later batch: every wave is done writing the previous
            // batch's outputs, which read sh_pr and sh_e)
            if (!first) sync_lds();
            first = false;
            // ---- stage the batch's rows: largest |h| per row, then the
            // scaled chunks and run sums (all threads; a run's 8 lanes are
            // active together: nb * K/4 and the block size are multiples
            // of 8) ----
            nb = min(__popcll(rest), M);
            if (tid < M) {
                unsigned long long r2 = rest;
                for (int j = 0; j < tid && r2; ++j) r2 &= r2 - 1ull;
                sh_pr[tid] = r2 ? __builtin_ctzll(r2) : 0;
            }
            for (int j = 0; j < nb; ++j) rest &= rest - 1ull;
            sync_lds();
            const int kq4 = p.K >> 2;
            const int total = nb * kq4;
            const float4* h4 = (const float4*)p.x;
            float am[M];
#pragma unroll
            for (int j = 0; j < M; ++j) am[j] = 0.f;
            // kDownBatch chunks per wait (a wait also waits for the weight
            // loads issued before it), kept unscaled in their LDS slots for
            // the second pass; chunks past the end are clamped duplicates
            const int kqr = xrow_chunks(p.upr);
            auto slot = [&](int j, int c) { return j * kqr + xchunk(c >> 4, c & 15); };
            ChunkWalk w(tid, kDownBlock, kq4);
            for (int i0 = tid; i0 < total; i0 += kDownBatch * kDownBlock) {
                float4 t[kDownBatch];
                int tj[kDownBatch], tc[kDownBatch];
                bool ok[kDownBatch];
#pragma unroll
                for (int k = 0; k < kDownBatch; ++k) {
                    ok[k] = i0 + k * kDownBlock < total;
                    tj[k] = ok[k] ? w.m : nb - 1;
                    tc[k] = ok[k] ? w.c : kq4 - 1;
                    t[k] = h4[(long long)sh_pr[tj[k]] * kq4 + tc[k]];
                    w.next();
                }
#pragma unroll
                for (int k = 0; k < kDownBatch; ++k) {
                    float a = fmaxf(fmaxf(fabsf(t[k].x), fabsf(t[k].y)),
                                    fmaxf(fabsf(t[k].z), fabsf(t[k].w)));
                    a = ok[k] ? a : 0.f;
#pragma unroll
                    for (int jj = 0; jj < M; ++jj) am[jj] = fmaxf(am[jj], tj[k] == jj ? a : 0.f);
                    if (ok[k]) xl[slot(tj[k], tc[k])] = t[k];
                }
            }
#pragma unroll
            for (int j = 0; j < M; ++j) {
                const float a = wave_max_nonneg(am[j]);
                if (lane == kWave - 1) red.am[j][wave] = a;
            }
            sync_lds();
            if (tid < M) {
                float a = 0.f;
                for (int w = 0; w < kDownWaves; ++w) a = fmaxf(a, red.am[tid][w]);
                sh_e[tid] = xscale_exp(a, kXTarget);
            }
            sync_lds();
            // (each chunk's slot was written by this thread above)
            ChunkWalk w2(tid, kDownBlock, kq4);
            for (int i = tid; i < total; i += kDownBlock, w2.next()) {
                const int j = w2.m, c = w2.c;
                stage_chunk<FMT, M>(p, xl[slot(j, c)], j, c, true, xl, xsum, sh_e[j]);
            }
            sync_lds();
        }

        // ---- stream the share's rows for the batch ----
        float acc[NR][M];
        uint32_t cks[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            cks[r] = 0u;
#pragma unroll
            for (int j = 0; j < M; ++j) acc[r][j] = 0.f;
        }
        auto compute = [&](int q, const uint32_t (&w)[NR][kUnitWords]) {
            const int pass = q / p.upl, ui = q - pass * p.upl;
            const int u = li + ui * p.lg;
            const bool act = u <= u_last;
            const int uc = act ? u : u_last;
            if constexpr (PURE) {
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const uint32_t v = unit_checksum<FMT>(w[r], uc);
                    cks[r] += act ? v : 0u;
                }
            } else {
#pragma unroll
                for (int j = 0; j < M; ++j) {
                    if (j < nb) {
                        float a1[NR][1];
#pragma unroll
                        for (int r = 0; r < NR; ++r) a1[r][0] = acc[r][j];
                        rows_dot<FMT, 1, NR>(w, uc, 0u, xl + j * kq, kq,
                                             (const float2*)xsum + j * k64, k64, a1, act);
#pragma unroll
                        for (int r = 0; r < NR; ++r) acc[r][j] = a1[r][0];
                    }
                    if constexpr (M > 1) __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (ui != p.upl - 1) return;
            // ---- end of a pass: reduce over the row group, last lane writes ----
            const int g = g0 + pass * per_pass + wave * p.rgw + gi;
            const bool last_lane = li == p.lg - 1;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int row = g * RR + r;
                const bool wr = last_lane && g < g1 && row < p.N;
                if constexpr (PURE) {
                    const uint32_t v = group_total(cks[r], p.lg);
                    cks[r] = 0u;
                    if (wr) {
                        unsigned long long pm = pairs;
                        while (pm) {
                            const int pr = __builtin_ctzll(pm);
                            pm &= pm - 1ull;
                            p.cks[(long long)pr * p.N + row] = v;
                        }
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < M; ++j) {
                        if (j < nb) {
                            const float v =
                                __builtin_ldexpf(group_total(acc[r][j], p.lg), -sh_e[j]);
                            acc[r][j] = 0.f;
                            if (wr) p.y0[(long long)sh_pr[j] * p.N + row] = v;
                        }
                    }
                }
            }
        };
        // every wave runs the same number of steps (nsteps, uniform); a
        // step past the end reloads the last one
        for (int q = 0;; q += 2) {
            const bool hb = q + 1 < nsteps;
            load(hb ? q + 1 : q, bufB);
            __builtin_amdgcn_sched_barrier(0);
            compute(q, bufA);
            if (!hb) break;
            const bool hc = q + 2 < nsteps;
            load(hc ? q + 2 : q + 1, bufA);
            __builtin_amdgcn_sched_barrier(0);
            compute(q + 1, bufB);
            if (!hc) break;
        }
        // (the next batch's staging barriers wait for every wave's reads)
    }
}

}  // namespace q4
