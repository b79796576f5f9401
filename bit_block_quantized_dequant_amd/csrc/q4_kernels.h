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

#ifndef Q4_TASK_ORDER
#define Q4_TASK_ORDER 1
#endif

namespace q4 {

// Threads per workgroup of the VALU GEMV kernel: 256 for single-token calls
// with register-resident activations (512 for longer rows, staged in LDS),
// 512 for dense batched calls; the expert calls 256 at M = 2 .. 4 and 768
// otherwise.  An expert call stages all M token rows in every workgroup: one
// 768-thread workgroup per CU stages them once per CU instead of three
// times, at the same 12 waves per CU.  Measured (E = 64, top-6, K = 2048,
// one box, 768 against 256 threads): M = 1 -5 %, M = 6 and 8 -10 to -12 %,
// but M = 2 .. 4 +3 to +7 %.
constexpr int kBlock = 512;
constexpr int kBlock1 = 256;
#ifndef Q4_XR_MAX_M
#define Q4_XR_MAX_M 2
#endif
constexpr int kXrMaxM = Q4_XR_MAX_M;  // largest batch with register-resident activations
#ifndef Q4_MOE_BLOCK
#define Q4_MOE_BLOCK 0  // 0: by M as above; else every expert call (for measurements)
#endif
constexpr int moe_block(int M) {
    return Q4_MOE_BLOCK > 0 ? Q4_MOE_BLOCK : ((M >= 2 && M <= 4) ? 256 : 768);
}
constexpr int kModeDense = 0;
constexpr int kModeNorm = 1;
constexpr int kModeMoe = 2;
// gate+up calls whose one output is the SiLU-gated product silu(gate) * up
// (dense, and the expert call)
constexpr int kModeSilu = 3;
constexpr int kModeMoeSilu = 4;
// RMSNorm feeding the gate+up pair, with the SiLU-gated product as the output
constexpr int kModeNormSilu = 5;
constexpr bool mode_moe(int mode) { return mode == kModeMoe || mode == kModeMoeSilu; }
constexpr bool mode_silu(int mode) {
    return mode == kModeSilu || mode == kModeMoeSilu || mode == kModeNormSilu;
}
constexpr bool mode_norm(int mode) { return mode == kModeNorm || mode == kModeNormSilu; }
#ifndef Q4_LONGK1_BLOCK
#define Q4_LONGK1_BLOCK 512
#endif
// xr: the single-token kernel with register-resident activations (K <= 4096);
// a single token with longer rows stages them in LDS, in the larger groups.
constexpr int gemv_threads(int M, int mode, bool xr = true) {
    return mode_moe(mode) ? moe_block(M) : (M == 1 ? (xr ? kBlock1 : Q4_LONGK1_BLOCK) : kBlock);
}

// silu(g) * u with silu(g) = g / (1 + exp(-g)), in fp32.  With
// e = exp(-|g|), which never overflows, silu(g) = g / (1 + e) for g >= 0 and
// g e / (1 + e) for g < 0: a few ulp everywhere, down to the subnormal range
// of e (g < -87), where the error stays below (|g| + 1) 2^-148 in absolute.
__device__ __forceinline__ float silu_mul(float g, float u) {
    const float e = expf(-fabsf(g));
    const float s = (g >= 0.0f ? g : g * e) / (1.0f + e);
    return s * u;
}
constexpr int kMaxPairs = 64;  // M * top_k limit of the expert call

// Workgroup barrier for data in LDS only: waits for this wave's LDS
// operations (lgkmcnt(0)), not for its global loads still in flight, which
// __syncthreads would also wait for; so the weight loads issued ahead of the
// activation staging stay in flight across the staging barriers.  LDS is
// coherent within the workgroup; the empty asm statements keep the compiler
// from moving memory operations across the barrier.
__device__ __forceinline__ void sync_lds() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

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
    const uint8_t* sc;  // split-array Q4_0: the f16 scales (w0: the nibble blocks)
    int upr;        // units per row = ceil(K / 64) (the last one half used when K % 64 == 32)
    int lg;         // lanes per row group (power of two, <= 64)
    int upl;        // units per lane per row = ceil(upr / lg)
    int rgw;        // row groups per wave pass = 64 / lg
    int nrg;        // row groups per matrix (expert call: padded to a multiple of rgw)
    int ntasks;     // dense calls: total tasks (expert call: computed in the kernel)
    int nwaves;     // waves in the grid
    int ks;         // batched kernel: waves that split one tile's K range
    int nsl;        // batched kernel: K slices per wave-position group (1: whole rows)
    int msl;        // batched kernel, sliced: staged steps per wave range and slice
    int npg;        // batched kernel, sliced: groups of wave positions staged in turn
    int kp;         // batched kernel, split-K: K parts (one workgroup per tile group and part)
    float* part;    // split-K workspace: partial sums [kp][M][N] (scaled by 2^(e-24))
    int* pexp;      // split-K workspace: each part's token exponents [kp][M]
};

// Shared state of the expert call after the in-kernel dedupe.
struct MoeShared {
    alignas(16) int uexp[kMaxPairs];       // unique valid ids, in order of first appearance
    unsigned long long upairs[kMaxPairs];  // (token, slot) pairs that chose each
    unsigned long long invalid;            // pairs with an id outside [0, E)
    unsigned int utok[kMaxPairs];          // tokens that chose each (bit m)
    int nu;                                // unique valid experts
};

// Stage the M activation rows into LDS.  Chunk layout and pre-scaling as in
// q4_device.h; xs receives per-32-element sums (times -8 for Q4_0).  For
// kModeNorm the rows are first RMS-normalized in fp32:
//   r = 1 / sqrt(sum(x^2) / K + eps),  xhat = (x * r) * gamma,
// with the sum of squares accumulated in fp64 (every square of an fp32 value
// is exact there, and no finite row can overflow it); the mean is rounded to
// fp32 once, as in the definition.
// Every token row m is also scaled by a power of two 2^e_m, chosen so that
// its largest magnitude lies in [2^kXTarget, 2^(kXTarget+1)): the partial
// sums then stay far from both ends of the fp32 range whatever the token's
// own magnitude, and the output is scaled back by 2^-e_m.  Scaling by a
// power of two is exact, so for tokens whose arithmetic never leaves the
// normal fp32 range the result is bit-identical to the unscaled one.
// Split in two so that the first weight loads can be issued in between: the
// global loads of the first NX chunks per thread go out first (the load
// counter is in order, so waiting for them later does not wait for the
// weights); chunks beyond that load in the second half, behind the weights.
// NX is kXReg, or for the expert call the chunks per thread of M tokens of
// K = 2048 (512 chunks each) in its workgroups (longer rows take the tail
// loop).
constexpr int kXReg = 4;
#ifndef Q4_TAIL_BATCH
#define Q4_TAIL_BATCH 4
#endif
constexpr int kTailBatch = Q4_TAIL_BATCH;  // tail chunks per batch of loads (stage_x_finish)
constexpr int xreg_chunks(int M, int mode) {
    return mode_moe(mode) ? (M * 512 + moe_block(M) - 1) / moe_block(M) : kXReg;
}
constexpr int kXTarget = 60;

template <int NX = kXReg>
struct XStage {
    float4 x[NX];
    float4 g[NX];
};

// Per-workgroup scratch of the staging reductions: per token and wave, the
// sum of squares and the largest magnitude (W waves, 8 unless stated).
constexpr int kMaxStageWaves = 8;
static_assert(kBlock / kWave <= kMaxStageWaves && kBlock1 / kWave <= kMaxStageWaves,
              "staging scratch holds 8 waves");
template <int MT, int W = kMaxStageWaves>
struct StageRedT {
    double ss[MT][W];
    float am[MT][W];
    float r[MT];  // per token: the RMSNorm factor
    int e[MT];    // per token: the scale exponent
};
using StageRed = StageRedT<8>;

// Exponent e with amax * 2^e in [2^target, 2^(target+1)), for amax >= 0;
// a zero or non-finite amax leaves the token unscaled (e = 0).
__device__ __forceinline__ int xscale_exp(float amax, int target) {
    if (!(amax > 0.0f) || !(amax < __builtin_inff())) return 0;
    return target - (__builtin_amdgcn_frexp_expf(amax) - 1);
}

// Sum of a double over the whole wave, exact in lane 63: the DPP pattern
// of group_total (q4_device.h) applied to both 32-bit halves.
__device__ __forceinline__ double dpp_add_f64(double v, int ctrl_sel) {
    const unsigned long long b = __builtin_bit_cast(unsigned long long, v);
    int lo = (int)(uint32_t)b, hi = (int)(uint32_t)(b >> 32);
    switch (ctrl_sel) {
        case 0: lo = __builtin_amdgcn_update_dpp(0, lo, 0xB1, 0xF, 0xF, false);
                hi = __builtin_amdgcn_update_dpp(0, hi, 0xB1, 0xF, 0xF, false); break;
        case 1: lo = __builtin_amdgcn_update_dpp(0, lo, 0x4E, 0xF, 0xF, false);
                hi = __builtin_amdgcn_update_dpp(0, hi, 0x4E, 0xF, 0xF, false); break;
        case 2: lo = __builtin_amdgcn_update_dpp(0, lo, 0x141, 0xF, 0xF, false);
                hi = __builtin_amdgcn_update_dpp(0, hi, 0x141, 0xF, 0xF, false); break;
        case 3: lo = __builtin_amdgcn_update_dpp(0, lo, 0x140, 0xF, 0xF, false);
                hi = __builtin_amdgcn_update_dpp(0, hi, 0x140, 0xF, 0xF, false); break;
        case 4: lo = __builtin_amdgcn_update_dpp(0, lo, 0x142, 0xA, 0xF, false);
                hi = __builtin_amdgcn_update_dpp(0, hi, 0x142, 0xA, 0xF, false); break;
        default: lo = __builtin_amdgcn_update_dpp(0, lo, 0x143, 0xC, 0xF, false);
                 hi = __builtin_amdgcn_update_dpp(0, hi, 0x143, 0xC, 0xF, false); break;
    }
    const unsigned long long t = ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
    return v + __builtin_bit_cast(double, t);
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int k = 0; k < 6; ++k) v = dpp_add_f64(v, k);
    return v;
}

// (bs: the kernel's block size, a compile-time constant of every caller, so
// that no load of the dispatch's block size precedes these loads)
// The (token m, chunk c) position of chunk index i = i0 + k * step in rows of
// kq chunks, advanced one step at a time with two divisions up front instead
// of one per step.
struct ChunkWalk {
    int m, c, dm, dc, kq;
    __device__ __forceinline__ ChunkWalk(int i0, int step, int kq_) : kq(kq_) {
        m = i0 / kq;
        c = i0 - m * kq;
        dm = step / kq;
        dc = step - dm * kq;
    }
    __device__ __forceinline__ void next() {
        c += dc;
        m += dm;
        if (c >= kq) {
            c -= kq;
            ++m;
        }
    }
};

template <int MODE, int NX = kXReg>
__device__ __forceinline__ void stage_x_issue(const GemvParams& p, int M, XStage<NX>& st, int bs) {
    const int kq = p.K >> 2;
    const int total = M * kq;
    const float4* x4 = (const float4*)p.x;
    const float4* g4 = (const float4*)p.gamma;
    // (the gamma chunk, i mod K/4, is walked without a division per chunk)
    ChunkWalk w((int)threadIdx.x, bs, mode_norm(MODE) ? kq : 1 << 30);
#pragma unroll
    for (int k = 0; k < NX; ++k) {
        // unconditional (clamped) loads keep the load-counter waits exact
        const int i = (int)threadIdx.x + k * bs;
        st.x[k] = x4[min(i, total - 1)];
        if constexpr (mode_norm(MODE)) {
            st.g[k] = g4[i < total ? w.c : kq - 1];
            w.next();
        }
    }
}

// One float4 chunk of the activations (chunk c of token m, scaled by
// 2^e): its 32-element run sum (over the 8 lanes that hold the run) and its
// pre-scaled, swizzled LDS copy.  Called by every lane; only lanes with
// `store` write (the others hold a clamped duplicate chunk and only take
// part in the lane exchange).
// DEFER: store the chunk and its run sum unscaled (no 2^e, no 2^24 / 2^20);
// the register-resident kernel applies both when it copies its lane's
// activations into registers.
template <int FMT, int M, bool DEFER = false>
__device__ __forceinline__ void stage_chunk(const GemvParams& p, float4 v, int m, int c,
                                            bool store, float4* xl, float* xsum, int e) {
    if constexpr (!DEFER) {
        v.x = __builtin_ldexpf(v.x, e);
        v.y = __builtin_ldexpf(v.y, e);
        v.z = __builtin_ldexpf(v.z, e);
        v.w = __builtin_ldexpf(v.w, e);
    }
    // 8 consecutive lanes hold one 32-element run
    float s = (v.x + v.y) + (v.z + v.w);
    s = dpp_add(s, 0);
    s = dpp_add(s, 1);
    s = dpp_add(s, 2);
    if (store && (c & 7) == 7) xsum[m * 2 * p.upr + (c >> 3)] = (FMT != kFmtQ4K) ? -8.0f * s : s;
    if constexpr (!DEFER) {
        const float sc = elem_is_high<FMT>(4 * c) ? 0x1p20f : 0x1p24f;
        v.x *= sc; v.y *= sc; v.z *= sc; v.w *= sc;
    }
    if (store) xl[m * xrow_chunks(p.upr) + xchunk(c >> 4, c & 15)] = v;
}

// A row whose K is not a multiple of 64 ends in a half unit: its upper 32
// staged activations and their run sum are zero, so the weights past K (the
// padding of a Q4_K row's last super-block, whose nibbles and 6-bit fields
// are finite whatever they hold) add exactly nothing.
template <int M>
__device__ __forceinline__ void stage_pad(const GemvParams& p, float4* xl, float* xsum) {
    if ((p.K & 63) == 0) return;
    const int kq = xrow_chunks(p.upr);
    for (int i = threadIdx.x; i < M * 9; i += blockDim.x) {
        const int m = i / 9, j = i - 9 * m;
        if (j < 8)
            xl[m * kq + xchunk(p.upr - 1, 8 + j)] = make_float4(0.f, 0.f, 0.f, 0.f);
        else
            xsum[m * 2 * p.upr + 2 * p.upr - 1] = 0.f;
    }
}

// TAIL: the call may have more than NX chunks per thread (M * K > NX * 4 *
// blockDim); kernels that cannot are compiled without the extra loops,
// whose load waits would otherwise also cover the weight loads in flight.
// xe[m] receives token m's scale exponent e_m (the same in every thread).
// DEFER (register-resident activations, no RMSNorm): no reduction barrier
// here; the chunks are stored unscaled and each wave's partial maxima are
// left in red.am[m], to be combined after the caller's barrier
// (stage_x_exponent).
template <int FMT, int M, int MODE, bool TAIL, int NX = kXReg, bool DEFER = false, class RED>
__device__ __forceinline__ void stage_x_finish(const GemvParams& p, const XStage<NX>& st,
                                               float4* xl, float* xsum, RED& red,
                                               int (&xe)[M], int bs) {
    static_assert(!DEFER || (M <= kXrMaxM && !mode_norm(MODE)),
                  "deferred scaling: register-resident tokens, no norm");
    const int tid = threadIdx.x;
        const int kq = p.K >> 2;
    const int total = M * kq;
    const float4* x4 = (const float4*)p.x;
    const float4* g4 = (const float4*)p.gamma;
    const int nw = bs >> 6;
    const int wave = tid >> 6, lane = tid & 63;
    double ss[M];
    float am[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        ss[m] = 0.0;
        am[m] = 0.f;
    }
    // sum of squares (RMSNorm) and the largest |x| (|x * gamma| for RMSNorm,
    // whose rows are scaled by r afterwards) of a chunk of token m
    auto acc = [&](float4 v, float4 g, int m, bool valid) {
        double t = 0.0;
        float a;
        if constexpr (mode_norm(MODE)) {
            t = (double)v.x * (double)v.x + (double)v.y * (double)v.y +
                (double)v.z * (double)v.z + (double)v.w * (double)v.w;
            a = fmaxf(fmaxf(fabsf(v.x * g.x), fabsf(v.y * g.y)),
                      fmaxf(fabsf(v.z * g.z), fabsf(v.w * g.w)));
        } else {
            (void)g;
            a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        }
        t = valid ? t : 0.0;
        a = valid ? a : 0.f;
        // selects, not branches (a per-lane branch per token and chunk was
        // compiled as divergent control flow); t, a >= 0, so adding 0 or
        // taking the maximum with 0 leaves the other tokens unchanged
#pragma unroll
        for (int mm = 0; mm < M; ++mm) {
            const bool mine = m == mm;
            if constexpr (mode_norm(MODE)) ss[mm] += mine ? t : 0.0;
            am[mm] = fmaxf(am[mm], mine ? a : 0.f);
        }
    };
    // chunk positions: (mk[k], ck[k]) for the k-th register chunk (the
    // clamped duplicate's for lanes past the end), then the tail's walk
    int mk[NX], ck[NX];
    ChunkWalk wk(tid, bs, kq);
#pragma unroll
    for (int k = 0; k < NX; ++k) {
        const bool valid = tid + k * bs < total;
        mk[k] = valid ? wk.m : M - 1;
        ck[k] = valid ? wk.c : kq - 1;
        wk.next();
    }
#pragma unroll
    for (int k = 0; k < NX; ++k) acc(st.x[k], st.g[k], mk[k], tid + k * bs < total);
    // The tail: chunks beyond the NX in registers, loaded kTailBatch at a
    // time (one wait per batch; a wait for a load issued after the weight
    // loads also waits for those) and kept in their LDS slots unscaled, so
    // that the second pass reads them back from LDS instead of loading them
    // again.  Chunks past the end (whole 32-element runs, as K/4 is a multiple
    // of 8) take part as clamped duplicates and are neither counted nor stored.
    const int kqr = xrow_chunks(p.upr);
    auto slot = [&](int m, int c) { return m * kqr + xchunk(c >> 4, c & 15); };
    if constexpr (TAIL) {
        ChunkWalk wt = wk;
        for (int i0 = tid + NX * bs; i0 < total; i0 += kTailBatch * bs) {
            float4 t[kTailBatch], tg[kTailBatch];
            ChunkWalk wl = wt;
#pragma unroll
            for (int j = 0; j < kTailBatch; ++j) {
                const int i = i0 + j * bs;
                t[j] = x4[min(i, total - 1)];
                tg[j] = make_float4(1.f, 1.f, 1.f, 1.f);
                if constexpr (mode_norm(MODE)) tg[j] = g4[i < total ? wl.c : kq - 1];
                wl.next();
            }
#pragma unroll
            for (int j = 0; j < kTailBatch; ++j) {
                const bool valid = i0 + j * bs < total;
                acc(t[j], tg[j], valid ? wt.m : M - 1, valid);
                if (valid) xl[slot(wt.m, wt.c)] = t[j];
                wt.next();
            }
        }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float a = wave_max_nonneg(am[m]);  // exact in lane 63
        if (lane == kWave - 1) red.am[m][wave] = a;
        if constexpr (mode_norm(MODE)) {
            const double s = wave_sum_f64(ss[m]);
            if (lane == kWave - 1) red.ss[m][wave] = s;
        }
    }
    stage_pad<M>(p, xl, xsum);
    if constexpr (DEFER) {
        (void)nw;
#pragma unroll
        for (int k = 0; k < NX; ++k)
            stage_chunk<FMT, M, true>(p, st.x[k], mk[k], ck[k], tid + k * bs < total, xl, xsum,
                                      0);
        static_assert(!TAIL, "deferred scaling: whole rows in registers");
        return;
    }
    sync_lds();
    // Every thread combines the waves' partials of every token (the same
    // arithmetic, so the same values) and writes the factor and exponent to
    // LDS, where it reads them back by token index: all threads write the
    // same values, so each read returns the thread's own result and no
    // further barrier is needed (a register array indexed at run time would
    // be moved to scratch memory).
    float r1 = 1.0f;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        float a = 0.f;
        double s = 0.0;
        for (int i = 0; i < nw; ++i) {
            a = fmaxf(a, red.am[m][i]);
            if constexpr (mode_norm(MODE)) s += red.ss[m][i];
        }
        float r = 1.0f;
        if constexpr (mode_norm(MODE)) {
            const float ms = (float)(s / (double)p.K);
            r = 1.0f / sqrtf(ms + p.eps);
            a *= r;
        }
        const int e = xscale_exp(a, kXTarget);
        xe[m] = __builtin_amdgcn_readfirstlane(e);
        r1 = r;
        if constexpr (M > 1) {
            red.r[m] = r;
            red.e[m] = e;
        }
    }
    // (one token: the factor and exponent stay in registers)
    auto norm = [&](float4 v, float4 g, int m) {
        if constexpr (mode_norm(MODE)) {
            const float r = M == 1 ? r1 : red.r[m];
            v.x = (v.x * r) * g.x;
            v.y = (v.y * r) * g.y;
            v.z = (v.z * r) * g.z;
            v.w = (v.w * r) * g.w;
        }
        return v;
    };
    auto tok_e = [&](int m) { return M == 1 ? xe[0] : red.e[m]; };
#pragma unroll
    for (int k = 0; k < NX; ++k)
        stage_chunk<FMT, M>(p, norm(st.x[k], st.g[k], mk[k]), mk[k], ck[k], tid + k * bs < total,
                            xl, xsum, tok_e(mk[k]));
    if constexpr (TAIL) {
        // (each chunk's slot was written by this thread in the first pass)
        ChunkWalk wt = wk;
        for (int i0 = tid + NX * bs; i0 < total; i0 += kTailBatch * bs) {
            float4 t[kTailBatch], tg[kTailBatch];
            ChunkWalk wl = wt;
#pragma unroll
            for (int j = 0; j < kTailBatch; ++j) {
                const bool valid = i0 + j * bs < total;
                t[j] = xl[valid ? slot(wl.m, wl.c) : slot(M - 1, kq - 1)];
                tg[j] = make_float4(1.f, 1.f, 1.f, 1.f);
                if constexpr (mode_norm(MODE)) tg[j] = g4[valid ? wl.c : kq - 1];
                wl.next();
            }
#pragma unroll
            for (int j = 0; j < kTailBatch; ++j) {
                const bool valid = i0 + j * bs < total;
                const int m = valid ? wt.m : M - 1, c = valid ? wt.c : kq - 1;
                stage_chunk<FMT, M>(p, norm(t[j], tg[j], m), m, c, valid, xl, xsum, tok_e(m));
                wt.next();
            }
        }
    }
}

// The scale exponent of token m staged with DEFER, from the waves' partial
// maxima (call after the barrier that follows the staging).
template <class RED>
__device__ __forceinline__ int stage_x_exponent(const RED& red, int nwaves, int m) {
    float a = 0.f;
    for (int i = 0; i < nwaves; ++i) a = fmaxf(a, red.am[m][i]);
    return __builtin_amdgcn_readfirstlane(xscale_exp(a, kXTarget));
}

// The expert id of pair (threadIdx.x mod 64), for moe_dedupe; issued ahead
// of other loads so that the dedupe waits for it alone.
template <int M>
__device__ __forceinline__ int moe_load_id(const GemvParams& p) {
    // every wave, unconditionally (clamped): a load under a branch would be
    // merged into its register by a copy that waits for all loads in flight
    return p.ids[min((int)threadIdx.x & (kWave - 1), M * p.top_k - 1)];
}

// In-kernel dedupe of the expert ids (from moe_load_id); wave 0 computes and
// writes the result, and everyone reads it after the barrier that follows.
//   uexp[u]   the u-th unique valid id, in order of first appearance
//   upairs[u] the (token, slot) pairs that chose it (bit m * top_k + s)
//   utok[u]   the tokens that chose it (bit m)
//   nu, invalid: the count of unique valid ids; the pairs with an id outside [0, E)
// Lane t holds pair t's id.  The ids go through LDS (uexp doubles as the
// buffer) and come back as broadcast reads, four at a time, so that every
// lane compares its id with every pair's in plain vector arithmetic: the
// pairs with the same id, and whether an earlier pair has it (then the lane
// is not the expert's first appearance).  Its index among the first
// appearances is a bit count over one ballot.  No lane mask is combined on
// the scalar unit inside the loop: a version that did (one ballot and a
// scalar update per unique expert) spent about 60 ns per expert waiting for
// vector results on the scalar side, and one with a branch per pair about
// 4 us in all before the first weight load.
template <int M>
__device__ __forceinline__ void moe_dedupe(const GemvParams& p, MoeShared& sh, int e_loaded) {
    // every wave waits for its id load here, where it was issued (a load
    // used only under the branch below could be moved into it, behind the
    // activation loads)
    asm volatile("" ::"v"(e_loaded));
    if (threadIdx.x >= kWave) return;  // wave-uniform
    const int lane = threadIdx.x;
    const int P = M * p.top_k;
    const bool in = lane < P;
    const bool ok = in && e_loaded >= 0 && e_loaded < p.E;
    const int ev = ok ? e_loaded : -1;  // -1 (invalid, or no pair) matches no valid id
    const unsigned long long bad = __ballot(in && !ok);
    // (wave 0's LDS operations complete in order: the reads see this write)
    sh.uexp[lane] = ev;
    unsigned long long mine = 0ull;  // the pairs whose id equals this lane's
    uint32_t dup = 0u;               // 1: an earlier pair has this lane's id
    for (int t0 = 0; t0 < P; t0 += 4) {
        const int4 q = *(const int4*)&sh.uexp[t0];  // entries past P hold -1
        const int et[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = t0 + j;
            const uint32_t same = 1u - min((uint32_t)(ev ^ et[j]), 1u);
            mine |= (unsigned long long)same << t;
            dup |= same & ((uint32_t)(t - lane) >> 31);  // t < lane
        }
    }
    const bool first = ok && dup == 0u;
    const unsigned long long fb = __ballot(first);
    const int u = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(fb >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)fb, 0u));
    // the tokens among the pairs (m * top_k < 64 for m < M, as M * top_k <= 64)
    const unsigned long long tkmask = p.top_k >= 64 ? ~0ull : ((1ull << p.top_k) - 1ull);
    unsigned int toks = 0u;
#pragma unroll
    for (int m = 0; m < M; ++m)
        if ((mine >> (m * p.top_k)) & tkmask) toks |= 1u << m;
    if (first) {
        sh.uexp[u] = e_loaded;
        sh.upairs[u] = mine;
        sh.utok[u] = toks;
    }
    if (lane == 0) {
        sh.nu = __popcll(fb);
        sh.invalid = bad;
    }
}

// XR: every lane works on one fixed unit of each row (M <= kXrMaxM tokens,
// K <= 64 units of 64 weights): its 64 activations and two run sums per token
// are copied from LDS into registers once, and the main loop reads no LDS.
template <int FMT, int M, int NMAT, int RR, int MODE, bool PURE, int PF, bool XR, bool TAIL>
__device__ __forceinline__ void gemv_body(const GemvParams& p) {
    static_assert(!XR || (M <= kXrMaxM && !mode_moe(MODE)), "register-resident x: M <= 2");
    extern __shared__ float4 smem[];
    __shared__ MoeShared moe;
    constexpr int NR = NMAT * RR;  // rows of one step, matrix-major: q = mt * RR + r
    constexpr int kBS = gemv_threads(M, MODE, XR);  // the launch's block size (run_plan)
    __shared__ StageRedT<8, (kBS / kWave > kMaxStageWaves ? kBS / kWave : kMaxStageWaves)> red;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the wave index is wave-uniform; say so, so that all task bookkeeping
    // stays in scalar registers and the loops are scalar branches
    const int gwave = __builtin_amdgcn_readfirstlane(blockIdx.x * (kBS >> 6) + (tid >> 6));
    const int kq = xrow_chunks(p.upr);  // LDS float4 chunks per token row
    const int k64 = p.upr;
    float4* xl = smem;
    float* xsum = (float*)(smem + M * kq);

    // ---- the wave's task range ----
    int ntasks = p.ntasks;
    int tpe = 1;  // tasks per expert (expert call)
    // Activation loads go out first (the expert call: right after its ids,
    // so that their latency overlaps the dedupe; the barrier after the
    // dedupe waits for LDS only)
    constexpr int NX = xreg_chunks(M, MODE);
    XStage<NX> xst;
    if constexpr (mode_moe(MODE)) {
        const int eid = moe_load_id<M>(p);
        if constexpr (!PURE) stage_x_issue<MODE, NX>(p, M, xst, kBS);
        moe_dedupe<M>(p, moe, eid);
        sync_lds();
        tpe = p.nrg >> __builtin_ctz(p.rgw);  // (rgw: a power of two dividing nrg)
        ntasks = moe.nu * tpe;
    }
#if Q4_TASK_ORDER == 1
    // strided: wave w takes tasks w, w + W, w + 2W, ... so that all waves
    // sweep one moving window of the weights together
    const int t0 = gwave;
    const int t1 = ntasks;
    const int tstride = p.nwaves;
#else
    // contiguous: wave w takes one balanced range of consecutive tasks
    const int t0 = (int)(((long long)gwave * ntasks) / p.nwaves);
    const int t1 = (int)(((long long)(gwave + 1) * ntasks) / p.nwaves);
    const int tstride = 1;
#endif
    // (lg: a power of two from 4 to 64)
    const int gi = lane >> __builtin_ctz(p.lg);  // row group of this lane within a pass
    const int li = lane & (p.lg - 1);            // lane within its row group
    const uint32_t sel = q4k_sel(li & 3);

    // ---- cursor over (task, unit) steps; advanced without divisions ----
    struct Cursor {
        int t, ui, ue, rgt;
    };
    auto first_cursor = [&]() {
        Cursor c;
        c.t = t0;
        c.ui = 0;
        c.ue = mode_moe(MODE) ? t0 / tpe : 0;
        c.rgt = mode_moe(MODE) ? t0 - c.ue * tpe : t0;
        return c;
    };
    auto next_cursor = [&](Cursor c) {
        if (++c.ui == p.upl) {
            c.ui = 0;
            c.t += tstride;
            c.rgt += tstride;
            if (mode_moe(MODE) && c.rgt >= tpe) {
                c.ue += c.rgt / tpe;
                c.rgt -= (c.rgt / tpe) * tpe;
            }
        }
        return c;
    };
    // first row of this lane's row group
    auto group_row = [&](const Cursor& c) { return (c.rgt * p.rgw + gi) * RR; };
    // Loads are unconditional (a branch around them would make the compiler
    // wait for every outstanding load before each step): lanes past the end of
    // the row re-read the row's last unit and rows past N re-read row N-1;
    // those lines are on their way anyway and the results are never used.
    const int u_last = p.upr - 1;
    // Weight addresses: a wave-uniform 64-bit base (matrix, expert, the
    // task's first row) plus a 32-bit per-lane offset (row inside the task,
    // unit inside the row), so that the loads take the scalar-base form.
    auto unit_off = [&](int u) -> uint32_t {
        return FMT == kFmtQ4K    ? (uint32_t)(u >> 2) * kQ4KBytes
               : FMT == kFmtQ4_0 ? (uint32_t)u * kQ4_0PairBytes
                                 : (uint32_t)u * 32u;
    };
    const int nblk = p.K >> 5;  // split-array Q4_0: blocks per row
    const uint32_t uoff_lane = unit_off(li);
    const uint32_t uoff_last = unit_off(u_last);
    const uint32_t pass_stride = unit_off(p.lg);
    const uint32_t rb = (uint32_t)p.row_bytes;
    auto load = [&](const Cursor& c, uint32_t (&dst)[NR][kUnitWords]) {
        const int u = li + c.ui * p.lg;
        const bool in_row = u <= u_last;
        const uint32_t uoff = in_row ? uoff_lane + c.ui * pass_stride : uoff_last;
        const int g = in_row ? (li & 3) : (u_last & 3);
        const uint32_t qoff = FMT == kFmtQ4K ? uoff + 16u + 32u * (uint32_t)g : uoff;
        const int R0 = c.rgt * p.rgw * RR;  // the task's first row (uniform)
        // (an expert index past the dedupe result, possible only for a wave
        // with no tasks, reads a valid expert instead)
        long long ubase = 0;
        if constexpr (mode_moe(MODE)) {
            const int nu = moe.nu;
            ubase = nu > 0 ? (long long)moe.uexp[min(c.ue, nu - 1)] * p.N : 0ll;
        }
        // The uniform base row is clamped into [0, N-1] (a wave without tasks,
        // or a padded row group of the expert call, may start past N); rows
        // past N then re-read row N-1.
        const int R0c = max(0, min(R0, p.N - 1));
        const long long sbase = (ubase + R0c) * p.row_bytes;
        const int lrow_max = p.N - 1 - R0c;  // >= 0
#pragma unroll
        for (int r = 0; r < RR; ++r) {
            const uint32_t lr = (uint32_t)min(gi * RR + r + (R0 - R0c), lrow_max);
            const uint32_t ro = lr * rb;
            if constexpr (FMT == kFmtQ4_0S) {
                // blocks 2u and 2u + 1 of the row (block B clamped to the
                // row's last block when K % 64 == 32: its activations are 0)
                static_assert(NMAT == 1, "split-array Q4_0: single matrix");
                const int uu = in_row ? u : u_last;
                const uint32_t bA = 2u * (uint32_t)uu;
                const uint32_t bB = (uint32_t)min(2 * uu + 1, nblk - 1);
                const uint32_t srb = 2u * (uint32_t)nblk;
                const uint8_t* sb = p.sc + (ubase + R0c) * (long long)srb;
                load_unit_soa(p.w0 + sbase, ro + 16u * bA, ro + 16u * bB, sb, lr * srb + 2u * bA,
                              lr * srb + 2u * bB, dst[r]);
            } else {
#pragma unroll
                for (int mt = 0; mt < NMAT; ++mt) {
                    const uint8_t* b = (mt == 0 ? p.w0 : p.w1) + sbase;
                    load_unit_at<FMT>(b, ro + uoff, ro + qoff, dst[mt * RR + r]);
                }
            }
        }
    };

    uint32_t bufA[NR][kUnitWords];
    uint32_t bufB[NR][kUnitWords];
    Cursor ca = first_cursor();
    // Activation loads first, then the first weight loads, then the staging
    // arithmetic: the HBM latency of the first step overlaps the staging.
    int xe[M];  // per-token scale exponents of the staged activations
#pragma unroll
    for (int m = 0; m < M; ++m) xe[m] = 0;
    // register-resident single token without RMSNorm: the scale is applied
    // when the lane copies its activations into registers (no extra barrier)
    constexpr bool kDefer = XR && !mode_norm(MODE);
    if constexpr (!PURE && !mode_moe(MODE)) stage_x_issue<MODE, NX>(p, M, xst, kBS);
    load(ca, bufA);  // a wave without tasks reads in-bounds rows it never uses
    if constexpr (!PURE)
        stage_x_finish<FMT, M, MODE, TAIL, NX, kDefer>(p, xst, xl, xsum, red, xe, kBS);
    sync_lds();
    if constexpr (kDefer && !PURE) {
#pragma unroll
        for (int m = 0; m < M; ++m) xe[m] = stage_x_exponent(red, kBS >> 6, m);
    }
    // output scale of token m: 2^(24 - e_m) for Q4_K (whose sums carry the
    // 6-bit scales as sc * 2^-24), 2^-e_m for Q4_0
    int osh[M];
#pragma unroll
    for (int m = 0; m < M; ++m) osh[m] = (FMT == kFmtQ4K ? 24 : 0) - xe[m];
    // the pair bits of one token: top_k consecutive bits (M * top_k <= 64)
    const unsigned long long tkmask = p.top_k >= 64 ? ~0ull : ((1ull << p.top_k) - 1ull);

    if constexpr (mode_moe(MODE)) {
        // rows of pairs with an invalid id: NaN (or an all-ones checksum)
        if (moe.invalid) {
            const int P = M * p.top_k;
            const long long total = (long long)P * p.N;
            const long long stride = (long long)gridDim.x * kBS;
            for (long long i = (long long)blockIdx.x * kBS + tid; i < total; i += stride) {
                const int pr = (int)(i / p.N);
                if ((moe.invalid >> pr) & 1ull) {
                    if constexpr (PURE) {
                        p.cks[i] = 0xFFFFFFFFu;
                        p.cks[total + i] = 0xFFFFFFFFu;
                    } else {
                        p.y0[i] = __builtin_nanf("");
                        if constexpr (!mode_silu(MODE)) p.y1[i] = __builtin_nanf("");
                    }
                }
            }
        }
    }
    if (t0 >= t1) return;

    // register-resident activations of this lane's unit (XR): token m's
    // 16 chunks at xr[16 m ..], its two run sums at xsr[m]
    constexpr int kXrChunks = kUnitChunks - 1;
    float4 xr[XR ? M * kXrChunks : 1];
    float2 xsr[XR ? M : 1];
    if constexpr (XR) {
        const int uc = min(li, p.upr - 1);
#pragma unroll
        for (int m = 0; m < M; ++m) {
#pragma unroll
            for (int c = 0; c < kXrChunks; ++c) xr[m * kXrChunks + c] = xl[m * kq + xchunk(uc, c)];
            xsr[m] = ((const float2*)xsum)[m * k64 + uc];
            if constexpr (kDefer) {
                // 2^e and the 2^24 (2^20 for elements met as high nibbles)
                // pre-scale of the staging, applied here
                const int e = xe[m];
#pragma unroll
                for (int c = 0; c < kXrChunks; ++c) {
                    const int sh = e + (elem_is_high<FMT>(4 * c) ? 20 : 24);
                    float4& v = xr[m * kXrChunks + c];
                    v.x = __builtin_ldexpf(v.x, sh);
                    v.y = __builtin_ldexpf(v.y, sh);
                    v.z = __builtin_ldexpf(v.z, sh);
                    v.w = __builtin_ldexpf(v.w, sh);
                }
                xsr[m].x = __builtin_ldexpf(xsr[m].x, e);
                xsr[m].y = __builtin_ldexpf(xsr[m].y, e);
            }
        }
    }

    float acc[NR][M];
    uint32_t cks[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) {
        cks[q] = 0u;
#pragma unroll
        for (int m = 0; m < M; ++m) acc[q][m] = 0.f;
    }

    // Compute on the loaded data unconditionally (lanes past the end of the
    // row hold a clamped valid unit; their result is dropped by a select, not
    // a branch, so the compiler's load-counter waits stay exact).
    auto compute = [&](const Cursor& c, const uint32_t (&w)[NR][kUnitWords]) {
        const int u = li + c.ui * p.lg;
        const bool act = u <= u_last;
        const int uc = act ? u : u_last;
        if constexpr (PURE) {
#pragma unroll
            for (int q = 0; q < NR; ++q) {
                const uint32_t v = unit_checksum<FMT>(w[q], uc);
                cks[q] += act ? v : 0u;
            }
        } else if constexpr (mode_moe(MODE)) {
            // tokens that chose this expert (uniform across the wave)
            const unsigned int tm = moe.utok[c.ue];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                if ((tm >> m) & 1u) {
                    float a1[NR][1];
#pragma unroll
                    for (int q = 0; q < NR; ++q) a1[q][0] = acc[q][m];
                    rows_dot<FMT, 1, NR>(w, uc, sel, xl + m * kq, kq,
                                         (const float2*)xsum + m * k64, k64, a1, act);
#pragma unroll
                    for (int q = 0; q < NR; ++q) acc[q][m] = a1[q][0];
                }
                if constexpr (M > 1) __builtin_amdgcn_sched_barrier(0);
            }
        } else if constexpr (XR) {
            rows_dot<FMT, M, NR>(w, 0, sel, xr, kXrChunks, xsr, 1, acc, act);
        } else {
            rows_dot<FMT, M, NR>(w, uc, sel, xl, kq, (const float2*)xsum, k64, acc, act);
        }
        if (c.ui != p.upl - 1) return;
        // ---- end of a task: reduce over the row group; its last lane writes ----
        const int r0 = group_row(c);
        const bool last_lane = li == p.lg - 1;
        // expert call: only the tokens that chose the task's expert have
        // totals to reduce and write (wave-uniform), and token m's pairs are
        // bits m * top_k .. of the expert's pair mask
        unsigned int tsel = ~0u;
        unsigned long long upairs = 0ull;
        if constexpr (mode_moe(MODE)) {
            tsel = moe.utok[c.ue];
            upairs = moe.upairs[c.ue];
        }
        auto token_pairs = [&](int m) { return upairs & (tkmask << (m * p.top_k)); };
        if constexpr (mode_silu(MODE) && !PURE) {
            // one output, h = silu(gate) * up: row r's gate total is q = r,
            // its up total q = RR + r, both in this lane
            static_assert(NMAT == 2, "the SiLU-gated product needs the gate and up matrices");
#pragma unroll
            for (int r = 0; r < RR; ++r) {
                const int row = r0 + r;
                const bool wr = last_lane && row < p.N;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    if (!((tsel >> m) & 1u)) continue;
                    const float g = __builtin_ldexpf(group_total(acc[r][m], p.lg), osh[m]);
                    const float u = __builtin_ldexpf(group_total(acc[RR + r][m], p.lg), osh[m]);
                    acc[r][m] = 0.f;
                    acc[RR + r][m] = 0.f;
                    if (wr) {
                        const float h = silu_mul(g, u);
                        if constexpr (mode_moe(MODE)) {
                            unsigned long long pm = token_pairs(m);
                            while (pm) {
                                const int pr = __builtin_ctzll(pm);
                                pm &= pm - 1ull;
                                p.y0[(long long)pr * p.N + row] = h;
                            }
                        } else {
                            p.y0[(long long)m * p.N + row] = h;
                        }
                    }
                }
            }
            return;
        }
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int r = 0; r < RR; ++r) {
                const int q = mt * RR + r;
                const int row = r0 + r;
                const bool wr = last_lane && row < p.N;
                if constexpr (PURE) {
                    const uint32_t v = group_total(cks[q], p.lg);
                    cks[q] = 0u;
                    if (wr) {
                        if constexpr (mode_moe(MODE)) {
                            const long long P = (long long)M * p.top_k;
                            unsigned long long pm = moe.upairs[c.ue];
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
                    float* y = mt == 0 ? p.y0 : p.y1;
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        if (!((tsel >> m) & 1u)) continue;
                        const float v = __builtin_ldexpf(group_total(acc[q][m], p.lg), osh[m]);
                        acc[q][m] = 0.f;
                        if (wr) {
                            if constexpr (mode_moe(MODE)) {
                                unsigned long long pm = token_pairs(m);
                                while (pm) {
                                    const int pr = __builtin_ctzll(pm);
                                    pm &= pm - 1ull;
                                    y[(long long)pr * p.N + row] = v;
                                }
                            } else {
                                y[(long long)m * p.N + row] = v;
                            }
                        }
                    }
                }
            }
    };

    // ---- main loop: PF steps of loads in flight ahead of the computed step ----
    // (a step past the wave's last task reloads the last one, so that every
    // load is unconditional)
    if constexpr (PF == 1) {
        for (;;) {
            const Cursor cb = next_cursor(ca);
            const bool hb = cb.t < t1;
            load(hb ? cb : ca, bufB);
            __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before computing
            compute(ca, bufA);
            if (!hb) break;
            const Cursor cc = next_cursor(cb);
            const bool hc = cc.t < t1;
            load(hc ? cc : cb, bufA);
            __builtin_amdgcn_sched_barrier(0);
            compute(cb, bufB);
            if (!hc) break;
            ca = cc;
        }
    } else {
        // (cursors are selected field by field: a select of whole structs
        // was compiled as a select of their stack addresses and a load)
        auto pick = [](bool c, const Cursor& a, const Cursor& b) {
            Cursor r;
            r.t = c ? a.t : b.t;
            r.ui = c ? a.ui : b.ui;
            r.ue = c ? a.ue : b.ue;
            r.rgt = c ? a.rgt : b.rgt;
            return r;
        };
        uint32_t bufC[NR][kUnitWords];
        Cursor cb = next_cursor(ca);
        Cursor lastv = pick(cb.t < t1, cb, ca);
        load(lastv, bufB);
        for (;;) {
            const Cursor cc = next_cursor(cb);
            lastv = pick(cc.t < t1, cc, lastv);
            load(lastv, bufC);
            __builtin_amdgcn_sched_barrier(0);
            compute(ca, bufA);
            if (!(cb.t < t1)) break;
            const Cursor cd = next_cursor(cc);
            lastv = pick(cd.t < t1, cd, lastv);
            load(lastv, bufA);
            __builtin_amdgcn_sched_barrier(0);
            compute(cb, bufB);
            if (!(cc.t < t1)) break;
            const Cursor ce = next_cursor(cd);
            lastv = pick(ce.t < t1, ce, lastv);
            load(lastv, bufB);
            __builtin_amdgcn_sched_barrier(0);
            compute(cc, bufC);
            if (!(cd.t < t1)) break;
            ca = cd;
            cb = ce;
        }
    }
}

template <int FMT, int M, int NMAT, int RR, int MODE, bool PURE, int PF, bool TAIL, int BS>
__global__ __launch_bounds__(BS) void gemv_kernel(const GemvParams p) {
    gemv_body<FMT, M, NMAT, RR, MODE, PURE, PF, false, TAIL>(p);
}

// The register-resident variant runs up to three 256-thread workgroups per CU
// for one token (as many as its register count lets the occupancy calculator
// place) and one 512-thread group for two tokens.  It is built for at least
// two waves per SIMD, so it may use up to 256 VGPRs where it needs them (two
// tokens' activations take about 245).
template <int FMT, int M, int NMAT, int RR, int MODE, bool PURE, int PF, int BS>
__global__ __launch_bounds__(BS) __attribute__((amdgpu_waves_per_eu(2)))
void gemv_kernel_xr(const GemvParams p) {
    gemv_body<FMT, M, NMAT, RR, MODE, PURE, PF, true, false>(p);
}

// ---------------------------------------------------------------------------
// Reference stream: the fastest way measured on this part to read a byte
// range once, used as the read ceiling of a call of the same byte count.
// Every wave instruction reads 1 KiB contiguous (16 bytes per lane) with the
// non-temporal hint; a wave step is a block of kStreamU such instructions
// (4 KiB), and the next block's loads are issued before the current one is
// summed (two blocks in flight per wave); blocks are strided over all waves
// of a grid of two 256-thread workgroups per CU.  Each block's 32-bit word
// sum (modulo 2^32) is written, which proves every byte was read.  (A sweep
// of launch shapes, bytes in flight per wave and load kinds, including loads
// straight into LDS, found this shape fastest; the hint helps only when each
// instruction consumes whole cache lines.)
// ---------------------------------------------------------------------------
constexpr int kStreamBlock = 256;
constexpr int kStreamU = 4;                         // 1 KiB loads per block
constexpr int kStreamBlockBytes = kStreamU * 1024;  // checksum granule

__device__ __forceinline__ u32x4 ldg16_nt(const uint8_t* p) {
    return __builtin_nontemporal_load((const u32x4*)__builtin_assume_aligned(p, 16));
}

static __global__ __launch_bounds__(kStreamBlock) void stream_read_kernel(
    uint32_t* __restrict__ cks, const uint8_t* __restrict__ w, long long bytes) {
    const int lane = threadIdx.x & 63;
    const int gw =
        __builtin_amdgcn_readfirstlane(blockIdx.x * (kStreamBlock / kWave) + (threadIdx.x >> 6));
    const int nw = gridDim.x * (kStreamBlock / kWave);
    const long long nblk = (bytes + kStreamBlockBytes - 1) / kStreamBlockBytes;
    if (gw >= nblk) return;
    const long long last = bytes - 16;  // bytes is a multiple of 16
    // loads are unconditional: a lane past the end re-reads the last 16
    // bytes and drops them
    auto load = [&](long long b, u32x4 (&r)[kStreamU]) {
#pragma unroll
        for (int i = 0; i < kStreamU; ++i) {
            const long long o = b * kStreamBlockBytes + 1024 * i + 16 * lane;
            r[i] = ldg16_nt(w + (o < last ? o : last));
        }
    };
    auto sum = [&](long long b, const u32x4 (&r)[kStreamU]) {
        uint32_t s = 0;
#pragma unroll
        for (int i = 0; i < kStreamU; ++i) {
            const long long o = b * kStreamBlockBytes + 1024 * i + 16 * lane;
            s += o <= last ? (r[i].x + r[i].y) + (r[i].z + r[i].w) : 0u;
        }
        s = group_total(s, kWave);
        if (lane == kWave - 1) cks[b] = s;
    };
    u32x4 A[kStreamU], B[kStreamU];
    long long b = gw;
    load(b, A);
    for (;;) {
        const long long nb = b + nw;
        const bool hb = nb < nblk;
        load(hb ? nb : b, B);
        __builtin_amdgcn_sched_barrier(0);
        sum(b, A);
        if (!hb) break;
        const long long nc = nb + nw;
        const bool hc = nc < nblk;
        load(hc ? nc : nb, A);
        __builtin_amdgcn_sched_barrier(0);
        sum(nb, B);
        if (!hc) break;
        b = nc;
    }
}

// ---------------------------------------------------------------------------
// Dequantization: one lane per 64-weight unit, writing 16 float4.
// Q4_K: w = fma(d*sc, q, -(dmin*m)); d*sc and dmin*m are exact in fp32 (at
// most 17 significant bits), so the single rounding of the fma gives the
// correctly rounded value of d*sc*q - dmin*m.  Q4_0: d*(q-8) is exact.
// ---------------------------------------------------------------------------
// A Q4_K row whose K is not a multiple of 64 ends in a half unit: only its
// low-nibble sub-block is written (out rows are K floats).
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(float* __restrict__ out,
                                                      const uint8_t* __restrict__ w,
                                                      long long nunits, int upr, int K,
                                                      long long row_bytes) {
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= nunits) return;
    const long long n = gid / upr;
    const int u = (int)(gid - n * upr);
    uint32_t r[kUnitWords];
    load_unit<FMT>(unit_ptr<FMT>(w + n * row_bytes, u), u & 3, r);
    const bool half = (u + 1) * kUnitElems > K;
    float4* o = (float4*)(out + n * (long long)K + (long long)u * kUnitElems);
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
            if (!half) o[8 + i] = hi;
        }
    } else {
        uint32_t qa[4] = {__builtin_amdgcn_alignbit(r[1], r[0], 16),
                          __builtin_amdgcn_alignbit(r[2], r[1], 16),
                          __builtin_amdgcn_alignbit(r[3], r[2], 16),
                          __builtin_amdgcn_alignbit(r[4], r[3], 16)};
        const float da = h_lo(r[0]), db = h_hi(r[4]);
        (void)half;  // (Q4_0 rows are whole units)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const float d = hb ? db : da;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t q = hb ? r[5 + i] : qa[i];
                float4 lo, hi;
                lo.x = d * (float)((int)(q & 15u) - 8);
                lo.y = d * (float)((int)((q >> 8) & 15u) - 8);
                lo.z = d * (float)((int)((q >> 16) & 15u) - 8);
                lo.w = d * (float)((int)((q >> 24) & 15u) - 8);
                hi.x = d * (float)((int)((q >> 4) & 15u) - 8);
                hi.y = d * (float)((int)((q >> 12) & 15u) - 8);
                hi.z = d * (float)((int)((q >> 20) & 15u) - 8);
                hi.w = d * (float)((int)(q >> 28) - 8);
                o[hb * 8 + i] = lo;
                o[hb * 8 + 4 + i] = hi;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Repack of 18-byte Q4_0 blocks into split arrays: one thread per block,
// nine 16-bit loads (the blocks are 2-byte aligned), one 16-bit and one
// 16-byte store.
// ---------------------------------------------------------------------------
static __global__ __launch_bounds__(256) void repack_q4_0_soa_kernel(
    uint16_t* __restrict__ scales, u32x4* __restrict__ quants, const uint8_t* __restrict__ w,
    long long nblocks) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nblocks) return;
    const uint16_t* b = (const uint16_t*)__builtin_assume_aligned(w + 18 * i, 2);
    uint32_t h[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) h[k] = b[k];
    scales[i] = (uint16_t)h[0];
    quants[i] = u32x4{h[1] | (h[2] << 16), h[3] | (h[4] << 16), h[5] | (h[6] << 16),
                      h[7] | (h[8] << 16)};
}

}  // namespace q4
