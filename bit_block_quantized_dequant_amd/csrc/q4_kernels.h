// q4_kernels.h -- the GEMV, dequant and pure-read kernels of libq4gemv.
//
// One kernel template streams packed weight rows for every GEMV call:
//   * A persistent grid: every wave owns a contiguous, balanced range of
//     "tasks"; one task is one pass of the wave over `rgw` row groups (64/rgw
//     lanes per group, one 64-weight unit per lane per step), and a row group
//     is RR rows of each of NMAT matrices that share the same activations.
//   * The activations of all M token rows are staged once per workgroup in
//     LDS (pre-scaled, swizzled, with per-32-element sums beside them); for
//     the fused RMSNorm call the normalization happens during that staging
//     (trueno-gpu 0.4.11, fused.rs, FusedRmsNormQ4KGemvKernel PHASE 1-2).
//   * The weights of step s+1 are loaded while step s is computed; every
//     weight byte is read from HBM once per call, for all M tokens
//     (inferencelayer 0.2.13, kernel_lab.rs, GEMV_F16S: several activation
//     columns per weight read).
//   * The expert call dedupes the selected experts inside the kernel, so an
//     expert chosen by several tokens is streamed once
//     (inferencelayer 0.2.13, kernel_lab.rs, moe_lab: expert-stacked rows).
//   * PURE instantiations perform the same loads with the same addressing
//     and no arithmetic on x, and write per-row word checksums
//     (inferencelayer 0.2.13, kernel_lab.rs, MOE_PURE_READ).
#pragma once

#include "q4_device.h"

namespace q4 {

constexpr int kBlock = 512;  // threads per workgroup (8 waves)
constexpr int kModeDense = 0;
constexpr int kModeNorm = 1;
constexpr int kModeMoe = 2;
constexpr int kMaxPairs = 64;  // M * top_k limit of the expert call

struct GemvParams {
    const uint8_t* w0;
    const uint8_t* w1;
    float* y0;
    float* y1;
    uint32_t* cks;
    const float* x;
    const float* gamma;
    const int32_t* ids;
    float eps;
    int N;          // rows per matrix (per expert for the expert call)
    int K;
    int top_k;
    int E;
    long long row_bytes;
    int upr;        // units per row = K / 64
    int lg;         // lanes per row group (power of two, <= 64)
    int upl;        // units per lane per row = ceil(upr / lg)
    int rgw;        // row groups per wave pass = 64 / lg
    int nrg;        // row groups per matrix (expert call: padded to a multiple of rgw)
    int ntasks;     // dense calls: total tasks (expert call: computed in the kernel)
    int nwaves;     // waves in the grid
};

// Shared state of the expert call after the in-kernel dedupe.
struct MoeShared {
    int nu;                    // unique valid experts
    int uexp[kMaxPairs];       // their ids, in order of first appearance
    unsigned long long upairs[kMaxPairs];  // (token, slot) pairs that chose each
    unsigned long long invalid;            // pairs with an id outside [0, E)
    unsigned int utok[kMaxPairs];           // tokens that chose each (bit m)
};

// Stage the M activation rows into LDS.  Chunk layout and pre-scaling as in
// q4_device.h; xs receives per-32-element sums (times -8 for Q4_0).  For
// kModeNorm the rows are first RMS-normalized in fp32:
//   r = 1 / sqrt(sum(x^2) / K + eps),  xhat = (x * r) * gamma.
template <int FMT, int M, int MODE>
__device__ __forceinline__ void stage_x(const GemvParams& p, float4* xl, float* xsum,
                                        float* red) {
    const int tid = threadIdx.x;
    const int kq = p.K >> 2;
    const float4* x4 = (const float4*)p.x;
    float rnorm[M];
#pragma unroll
    for (int m = 0; m < M; ++m) rnorm[m] = 1.0f;
    if constexpr (MODE == kModeNorm) {
        const int nw = blockDim.x >> 6;
        const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float ss = 0.f;
            for (int c = tid; c < kq; c += blockDim.x) {
                const float4 v = x4[m * kq + c];
                ss = __builtin_fmaf(v.x, v.x, ss);
                ss = __builtin_fmaf(v.y, v.y, ss);
                ss = __builtin_fmaf(v.z, v.z, ss);
                ss = __builtin_fmaf(v.w, v.w, ss);
            }
            ss = group_sum(ss, kWave);
            if (lane == 0) red[m * 16 + wave] = ss;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float ss = 0.f;
            for (int i = 0; i < nw; ++i) ss += red[m * 16 + i];
            const float ms = ss / (float)p.K;
            rnorm[m] = 1.0f / sqrtf(ms + p.eps);
        }
    }
    const float4* g4 = (const float4*)p.gamma;
    for (int i = tid; i < M * kq; i += blockDim.x) {
        const int m = i / kq;
        const int c = i - m * kq;
        float4 v = x4[i];
        if constexpr (MODE == kModeNorm) {
            const float4 g = g4[c];
            float r = rnorm[0];
#pragma unroll
            for (int mm = 1; mm < M; ++mm)
                if (m == mm) r = rnorm[mm];
            v.x = (v.x * r) * g.x;
            v.y = (v.y * r) * g.y;
            v.z = (v.z * r) * g.z;
            v.w = (v.w * r) * g.w;
        }
        // 8 consecutive lanes hold one 32-element run
        float s = (v.x + v.y) + (v.z + v.w);
        s += __shfl_xor(s, 1, kWave);
        s += __shfl_xor(s, 2, kWave);
        s += __shfl_xor(s, 4, kWave);
        if ((c & 7) == 0) xsum[m * (p.K >> 5) + (c >> 3)] = (FMT == kFmtQ4_0) ? -8.0f * s : s;
        const float sc = elem_is_high<FMT>(4 * c) ? 0x1p20f : 0x1p24f;
        v.x *= sc; v.y *= sc; v.z *= sc; v.w *= sc;
        xl[m * kq + xchunk(c >> 4, c & 15)] = v;
    }
}

// In-kernel dedupe of the expert ids (wave 0); everyone reads it after the
// barrier that follows.
template <int M>
__device__ __forceinline__ void moe_dedupe(const GemvParams& p, MoeShared& sh) {
    const int tid = threadIdx.x;
    if (tid < kWave) {
        const int P = M * p.top_k;
        const bool in = tid < P;
        const int e = in ? p.ids[tid] : -1;
        const bool ok = in && e >= 0 && e < p.E;
        // first appearance of e among the valid pairs?
        bool first = ok;
        for (int t = 0; t < P; ++t) {
            const int et = __shfl(e, t, kWave);
            const bool okt = __shfl((int)ok, t, kWave) != 0;
            if (t < tid && okt && et == e) first = false;
        }
        const unsigned long long fb = __ballot(first);
        const unsigned long long bad = __ballot(in && !ok);
        const int uidx = __popcll(fb & ((1ull << tid) - 1ull));
        unsigned long long pairs = 0;
        unsigned int toks = 0;
        for (int t = 0; t < P; ++t) {
            const int et = __shfl(e, t, kWave);
            const bool okt = __shfl((int)ok, t, kWave) != 0;
            if (okt && et == e) {
                pairs |= 1ull << t;
                toks |= 1u << (t / p.top_k);
            }
        }
        if (first) {
            sh.uexp[uidx] = e;
            sh.upairs[uidx] = pairs;
            sh.utok[uidx] = toks;
        }
        if (tid == 0) {
            sh.nu = __popcll(fb);
            sh.invalid = bad;
        }
    }
}

template <int FMT, int M, int NMAT, int RR, int MODE, bool PURE>
__global__ __launch_bounds__(kBlock) void gemv_kernel(const GemvParams p) {
    extern __shared__ float4 smem[];
    __shared__ MoeShared moe;
    __shared__ float red[8 * 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int gwave = blockIdx.x * (blockDim.x >> 6) + (tid >> 6);
    const int kq = p.K >> 2;
    const int k64 = p.K >> 6;
    float4* xl = smem;
    float* xsum = (float*)(smem + M * kq);

    if constexpr (MODE == kModeMoe) moe_dedupe<M>(p, moe);
    if constexpr (!PURE) stage_x<FMT, M, MODE>(p, xl, xsum, red);
    __syncthreads();

    int ntasks = p.ntasks;
    int tpe = 1;  // tasks per expert (expert call)
    if constexpr (MODE == kModeMoe) {
        tpe = p.nrg / p.rgw;
        ntasks = moe.nu * tpe;
        // rows of pairs with an invalid id: NaN (or an all-ones checksum)
        if (moe.invalid) {
            const int P = M * p.top_k;
            const long long total = (long long)P * p.N;
            const long long stride = (long long)gridDim.x * blockDim.x;
            for (long long i = (long long)blockIdx.x * blockDim.x + tid; i < total; i += stride) {
                const int pr = (int)(i / p.N);
                if ((moe.invalid >> pr) & 1ull) {
                    if constexpr (PURE) {
                        p.cks[i] = 0xFFFFFFFFu;
                        p.cks[total + i] = 0xFFFFFFFFu;
                    } else {
                        p.y0[i] = __builtin_nanf("");
                        p.y1[i] = __builtin_nanf("");
                    }
                }
            }
        }
    }

    const int t0 = (int)(((long long)gwave * ntasks) / p.nwaves);
    const int t1 = (int)(((long long)(gwave + 1) * ntasks) / p.nwaves);
    if (t0 >= t1) return;

    const int gi = lane / p.lg;       // row group of this lane within a pass
    const int li = lane - gi * p.lg;  // lane within its row group
    const uint32_t sel = q4k_sel(li & 3);
    const int nsteps = (t1 - t0) * p.upl;

    // Resolve (task, unit step) -> row base pointers and unit index.
    struct Where {
        const uint8_t* row[NMAT][RR];
        int rowid[RR];  // row index within the matrix (-1: none)
        int u;
        bool active;
        int uexp;  // unique-expert index (expert call)
    };
    auto where = [&](int step) {
        Where wh;
        const int t = t0 + step / p.upl;
        const int ui = step - (step / p.upl) * p.upl;
        wh.u = li + ui * p.lg;
        int rg;
        long long rbase = 0;
        wh.uexp = 0;
        if constexpr (MODE == kModeMoe) {
            wh.uexp = t / tpe;
            rg = (t - wh.uexp * tpe) * p.rgw + gi;
            rbase = (long long)moe.uexp[wh.uexp] * p.N;
        } else {
            rg = t * p.rgw + gi;
        }
        bool any = false;
#pragma unroll
        for (int r = 0; r < RR; ++r) {
            const int row = rg * RR + r;
            const bool ok = row < p.N;
            wh.rowid[r] = ok ? row : -1;
            any |= ok;
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt) {
                const uint8_t* base = mt == 0 ? p.w0 : p.w1;
                wh.row[mt][r] = base + (rbase + (ok ? row : 0)) * p.row_bytes;
            }
        }
        wh.active = any && wh.u < p.upr;
        return wh;
    };

    // rows of a step, matrix-major: row index q = mt * RR + r
    constexpr int NR = NMAT * RR;
    uint32_t cur[NR][kUnitWords];
    uint32_t nxt[NR][kUnitWords];
    auto load = [&](const Where& wh, uint32_t (&dst)[NR][kUnitWords]) {
#pragma unroll
        for (int r = 0; r < RR; ++r)
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt) {
                if (wh.active && wh.rowid[r] >= 0) {
                    load_unit<FMT>(wh.row[mt][r], wh.u, dst[mt * RR + r]);
                } else {
#pragma unroll
                    for (int i = 0; i < kUnitWords; ++i) dst[mt * RR + r][i] = 0u;
                }
            }
    };

    float acc[NR][M];
    uint32_t cks[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) {
        cks[q] = 0u;
#pragma unroll
        for (int m = 0; m < M; ++m) acc[q][m] = 0.f;
    }

    Where wc = where(0);
    load(wc, cur);
    for (int s = 0; s < nsteps; ++s) {
        Where wn = wc;
        if (s + 1 < nsteps) {
            wn = where(s + 1);
            load(wn, nxt);
        }
        // ---- compute step s ----
        if (wc.active) {
            if constexpr (PURE) {
#pragma unroll
                for (int q = 0; q < NR; ++q) cks[q] += unit_checksum<FMT>(cur[q], wc.u);
            } else if constexpr (MODE == kModeMoe) {
                // tokens that chose this expert (uniform across the wave)
                const unsigned int tm = moe.utok[wc.uexp];
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    if ((tm >> m) & 1u) {
                        float a1[NR][1];
#pragma unroll
                        for (int q = 0; q < NR; ++q) a1[q][0] = acc[q][m];
                        rows_dot<FMT, 1, NR>(cur, wc.u, sel, xl + m * kq, kq,
                                             (const float2*)xsum + m * k64, k64, a1);
#pragma unroll
                        for (int q = 0; q < NR; ++q) acc[q][m] = a1[q][0];
                    }
                }
            } else {
                rows_dot<FMT, M, NR>(cur, wc.u, sel, xl, kq, (const float2*)xsum, k64, acc);
            }
        }
        // ---- end of a task: reduce over the row group and write ----
        const int ui = s - (s / p.upl) * p.upl;
        if (ui == p.upl - 1) {
            const float oscale = FMT == kFmtQ4K ? 0x1p24f : 1.0f;
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
                for (int r = 0; r < RR; ++r) {
                    const int q = mt * RR + r;
                    const int row = wc.rowid[r];
                    if constexpr (PURE) {
                        const uint32_t v = group_sum_u32(cks[q], p.lg);
                        cks[q] = 0u;
                        if (li == 0 && row >= 0) {
                            if constexpr (MODE == kModeMoe) {
                                const long long P = (long long)M * p.top_k;
                                unsigned long long pm = moe.upairs[wc.uexp];
                                while (pm) {
                                    const int pr = __builtin_ctzll(pm);
                                    pm &= pm - 1ull;
                                    p.cks[((long long)mt * P + pr) * p.N + row] = v;
                                }
                            } else {
                                p.cks[(long long)mt * p.N + row] = v;
                            }
                        }
                    } else {
#pragma unroll
                        for (int m = 0; m < M; ++m) {
                            const float v = group_sum(acc[q][m], p.lg) * oscale;
                            acc[q][m] = 0.f;
                            if (li == 0 && row >= 0) {
                                float* y = mt == 0 ? p.y0 : p.y1;
                                if constexpr (MODE == kModeMoe) {
                                    unsigned long long pm = moe.upairs[wc.uexp];
                                    while (pm) {
                                        const int pr = __builtin_ctzll(pm);
                                        pm &= pm - 1ull;
                                        if (pr / p.top_k == m) y[(long long)pr * p.N + row] = v;
                                    }
                                } else {
                                    y[(long long)m * p.N + row] = v;
                                }
                            }
                        }
                    }
                }
        }
        // ---- rotate the double buffer ----
#pragma unroll
        for (int q = 0; q < NR; ++q)
#pragma unroll
            for (int i = 0; i < kUnitWords; ++i) cur[q][i] = nxt[q][i];
        wc = wn;
    }
}

// ---------------------------------------------------------------------------
// Dequantization: one lane per 64-weight unit, writing 16 float4.
// Q4_K: w = fma(d*sc, q, -(dmin*m)); d*sc and dmin*m are exact in fp32 (at
// most 17 significant bits), so the single rounding of the fma gives the
// correctly rounded value of d*sc*q - dmin*m.  Q4_0: d*(q-8) is exact.
// ---------------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(float* __restrict__ out,
                                                      const uint8_t* __restrict__ w,
                                                      long long nunits, int upr,
                                                      long long row_bytes) {
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= nunits) return;
    const long long n = gid / upr;
    const int u = (int)(gid - n * upr);
    uint32_t r[kUnitWords];
    load_unit<FMT>(w + n * row_bytes, u, r);
    float4* o = (float4*)(out + n * (long long)upr * kUnitElems + (long long)u * kUnitElems);
    if constexpr (FMT == kFmtQ4K) {
        uint32_t scp, mp;
        q4k_scale_pairs(r[1], r[2], r[3], q4k_sel(u & 3), scp, mp);
        const float d = h_lo(r[0]), dmin = h_hi(r[0]);
        const float ds0 = d * (float)(scp & 0xFFFFu), ds1 = d * (float)(scp >> 16);
        const float dm0 = dmin * (float)(mp & 0xFFFFu), dm1 = dmin * (float)(mp >> 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t q = r[4 + i];
            float4 lo, hi;
            lo.x = __builtin_fmaf(ds0, (float)(q & 15u), -dm0);
            lo.y = __builtin_fmaf(ds0, (float)((q >> 8) & 15u), -dm0);
            lo.z = __builtin_fmaf(ds0, (float)((q >> 16) & 15u), -dm0);
            lo.w = __builtin_fmaf(ds0, (float)((q >> 24) & 15u), -dm0);
            hi.x = __builtin_fmaf(ds1, (float)((q >> 4) & 15u), -dm1);
            hi.y = __builtin_fmaf(ds1, (float)((q >> 12) & 15u), -dm1);
            hi.z = __builtin_fmaf(ds1, (float)((q >> 20) & 15u), -dm1);
            hi.w = __builtin_fmaf(ds1, (float)(q >> 28), -dm1);
            o[i] = lo;
            o[8 + i] = hi;
        }
    } else {
        uint32_t qa[4] = {__builtin_amdgcn_alignbit(r[1], r[0], 16),
                          __builtin_amdgcn_alignbit(r[2], r[1], 16),
                          __builtin_amdgcn_alignbit(r[3], r[2], 16),
                          __builtin_amdgcn_alignbit(r[4], r[3], 16)};
        const float da = h_lo(r[0]), db = h_hi(r[4]);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const float d = half ? db : da;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t q = half ? r[5 + i] : qa[i];
                float4 lo, hi;
                lo.x = d * (float)((int)(q & 15u) - 8);
                lo.y = d * (float)((int)((q >> 8) & 15u) - 8);
                lo.z = d * (float)((int)((q >> 16) & 15u) - 8);
                lo.w = d * (float)((int)((q >> 24) & 15u) - 8);
                hi.x = d * (float)((int)((q >> 4) & 15u) - 8);
                hi.y = d * (float)((int)((q >> 12) & 15u) - 8);
                hi.z = d * (float)((int)((q >> 20) & 15u) - 8);
                hi.w = d * (float)((int)(q >> 28) - 8);
                o[half * 8 + i] = lo;
                o[half * 8 + 4 + i] = hi;
            }
        }
    }
}

}  // namespace q4
