// q4_host.h -- host side of libq4gemv shared by its translation units:
// argument validation, launch planning and the dispatch from a call to its
// kernel instantiation.
//
// Validation runs before any HIP call, so every refusal path is testable on
// a machine without a GPU.  Launches go through hipLaunchKernel on the
// caller's stream; the library allocates nothing and keeps no per-call state
// (only per-device caches of the compute-unit count, of which kernels have
// had their LDS limit raised and of their occupancy).  Everything here has
// internal linkage: each translation unit that includes it instantiates the
// kernels of its own entry points.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "q4_kernels.h"
#include "q4_mfma.h"
#include "q4_moe_down.h"
#include "q4_router.h"
#include "q4gemv.h"

using namespace q4;

namespace {

constexpr int kMaxDevices = 64;
static_assert(Q4_MAX_MK == kMaxMK, "staging of the batched kernel is sized for Q4_MAX_MK");
static_assert(Q4_MAX_M == kMaxM, "token rows of the batched kernel");

// ---------------------------------------------------------------------------
// Validation (pure host code)
// ---------------------------------------------------------------------------
inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// K granularity of a format: a Q4_K row may end inside its last super-block
// at any multiple of 32 (the rest of that super-block is padding); a Q4_0
// row must hold an even number of 18-byte blocks, so that every row starts
// on a 4-byte boundary for the kernels' word loads; split-array Q4_0 rows
// take any whole number of blocks (their nibble blocks are 16-byte aligned
// and their scales are loaded 16 bits at a time).
inline bool k_ok(int64_t K, int fmt) {
    return K > 0 && K <= INT32_MAX && K % (fmt == kFmtQ4_0 ? 64 : 32) == 0;
}

// Staged columns of a call: K rounded up to whole 64-weight units.
inline int64_t k_units(int64_t K) { return (K + kUnitElems - 1) / kUnitElems; }

// Dense calls: 1 <= M <= Q4_MAX_M.  A single token is staged whole by the
// VALU kernel (K <= Q4_MAX_MK); batches run the matrix-core kernel, which
// stages K in slices when the rows do not fit in LDS at once.
inline int check_dims(int64_t M, int64_t N, int64_t K, int fmt) {
    if (M < 1 || M > Q4_MAX_M) return Q4_ERR_BATCH;
    if (!k_ok(K, fmt) || K > Q4_MAX_K || N < 1 || N > INT32_MAX) return Q4_ERR_SHAPE;
    if (M == 1 && k_units(K) * kUnitElems > Q4_MAX_MK) return Q4_ERR_SHAPE;
    return Q4_OK;
}

// Can the VALU kernel stage this batch whole?
inline bool valu_fits(int64_t M, int64_t K) {
    return M <= 8 && M * k_units(K) * kUnitElems <= Q4_MAX_MK;
}

// Bytes of one weight row: ceil(K/256) super-blocks (Q4_K), K/32 blocks
// (Q4_0), K/32 nibble blocks of 16 bytes (split-array Q4_0; its scales are
// a second array of K/32 f16 per row).
inline long long row_bytes_of(int64_t K, int fmt) {
    return fmt == kFmtQ4K    ? (long long)((K + 255) / 256) * kQ4KBytes
           : fmt == kFmtQ4_0 ? (long long)(K / 32) * 18
                             : (long long)(K / 32) * 16;
}

// ---------------------------------------------------------------------------
// Launch planning
// ---------------------------------------------------------------------------
struct DeviceInfo {
    int cus = 0;
};
inline DeviceInfo g_dev[kMaxDevices];
inline std::mutex g_dev_mu;

inline int device_cus(int* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return Q4_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return Q4_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev[dev].cus == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            return Q4_ERR_HIP;
        g_dev[dev].cus = cus;
    }
    *out = g_dev[dev].cus;
    return Q4_OK;
}

// Optional tuning override of the resident workgroups per CU (read once).
inline int env_int(const char* name, int dflt) {
    const char* s = getenv(name);
    if (!s || !*s) return dflt;
    int v = atoi(s);
    return v > 0 ? v : dflt;
}

inline int pow2ceil(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// LDS bytes of a GEMV workgroup: M rows of ceil(K/64) units of 64 floats
// (17 float4 chunks each) plus two run sums per unit.
inline size_t gemv_lds_bytes(int M, int K, bool pure) {
    if (pure) return 0;
    const size_t upr = (size_t)k_units(K);
    return (size_t)M * upr * 17 * 16 + (size_t)M * upr * 2 * 4;
}

// static shared memory of the batched kernel (its reduction scratch) plus
// margin; the expert call adds its dedupe tables; batches of more than 8
// tokens a larger reduction scratch
constexpr int kMfmaStaticLds = 1024;
constexpr int kMfmaMoeStaticLds = 3072;
constexpr int kMfmaBigStaticLds = 2048;
static_assert(sizeof(StageRedT<8>) + 64 <= kMfmaStaticLds, "static LDS margin");
static_assert(sizeof(StageRedT<16>) + 64 <= kMfmaBigStaticLds, "static LDS margin");

// Resident workgroups per CU that LDS allows (160 KB per CU on gfx950, less
// the static shared state), capped at `mx`.
inline int wg_per_cu(size_t lds, int mx = 2) {
    const size_t cap = 160 * 1024 - 2048;
    int by_lds = lds == 0 ? mx : (int)(cap / lds);
    int w = by_lds < mx ? by_lds : mx;
    static const int override_wg = env_int("Q4GEMV_WG_PER_CU", 0);
    if (override_wg > 0 && override_wg < w) w = override_wg;
    return w < 1 ? 1 : w;
}

// Raise a kernel's dynamic-LDS limit once per device: to 160 KB less
// `reserve` bytes kept for its static shared variables (at least what the
// kernel declares).
inline int allow_big_lds(const void* kern, std::atomic<int>* done, int reserve = 2048) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return Q4_ERR_HIP;
    if (done[dev].load(std::memory_order_acquire)) return Q4_OK;
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, kern) != hipSuccess) return Q4_ERR_HIP;
    if ((long long)fa.sharedSizeBytes > reserve) reserve = (int)fa.sharedSizeBytes;
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       160 * 1024 - reserve);
    if (e != hipSuccess) return Q4_ERR_HIP;
    done[dev].store(1, std::memory_order_release);
    return Q4_OK;
}

// Workgroups of `kern` that can be resident on one CU at once (registers,
// LDS and waves), from the runtime's occupancy calculator; cached per device.
inline int resident_per_cu(const void* kern, int threads, size_t lds, std::atomic<int>* cache) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 1;
    int v = cache[dev].load(std::memory_order_acquire);
    if (v > 0) return v;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, lds) != hipSuccess || n < 1)
        n = 1;
    cache[dev].store(n, std::memory_order_release);
    return n;
}

template <typename Kern>
inline int launch(Kern kern, const GemvParams& p, int blocks, size_t lds, void* stream,
           std::atomic<int>* big_lds_done, int threads = kBlock, int reserve = 2048) {
    if (lds > 64 * 1024) {
        int st = allow_big_lds((const void*)kern, big_lds_done, reserve);
        if (st) return st;
    }
    void* args[] = {(void*)&p};
    hipError_t e = hipLaunchKernel((const void*)kern, dim3(blocks), dim3(threads), args, lds,
                                   (hipStream_t)stream);
    return e == hipSuccess ? Q4_OK : Q4_ERR_HIP;
}

// Fill the work-split fields of p for a call with `rows` rows per matrix
// and RR rows per lane; returns the number of workgroups of `threads`
// threads (at most `wgmax` and `resident` per CU, the second being the
// kernel's occupancy limit).
// Lanes per row group for a row of `upr` 64-weight units: the whole wave
// on one row when the row has at least 64 units, else the power of two that
// covers the row, at least 4 (the group reduction sums whole quads).  Q4GEMV_LG (a power of two from 4 to 64) overrides it for
// measurements; the kernel takes any such width.
// The expert call of 2 to 4 tokens (256-thread workgroups) takes half that
// width (two units per lane and row) where that leaves at least 16 lanes per
// row: E = 64, top-6, K = 2048, M = 4, on one box: 18.4 against 19.3 us
// (seeded ids), 18.4 against 19.4 (SiLU-gated), 20.3 against 20.2 (all ids
// distinct).  With 768-thread groups it was slower (M = 6: 31.7 against
// 28.2 us, M = 8: 37.1 against 36.1).  A single token keeps the dense call's
// width, so that each of its outputs equals q4_0_gemv on that expert bit for
// bit.
// Dense rows of more than 64 units at one or two tokens (activations in LDS)
// take 32 lanes per row: fewer idle lanes in a row's last step (224 units: 7
// steps of 32 lanes against 4 of 64 with the last half idle).  With one row
// per lane (run_m) the 4096 x 14336 Q4_K down-projection measured 10.57
// against 11.66 us at M = 1 and 16.1 against 17.8 at M = 2 (two runs each on
// one box; 16 lanes at M = 1: 14.2 us); eager timings at K = 14336,
// N = 4096, M = 1: gate+up 16.7 against 18.1 us, fused RMSNorm 11.2 against
// 11.8-12.4.  The single-token expert call keeps 64 lanes (E = 16,
// top-4, N = 2048, K = 8192: 32 lanes were 7 % slower, its tasks splitting
// unevenly over the waves), so it equals q4_0_gemv bit for bit only for rows
// of at most 64 units.
inline int choose_lg(int upr, bool moe = false, bool long1 = false) {
    static const int forced = env_int("Q4GEMV_LG", 0);
    if (forced >= 4 && forced <= kWave && (forced & (forced - 1)) == 0) return forced;
    if (long1 && upr > kWave) return 32;
    const int lg = upr >= kWave ? kWave : (upr <= 4 ? 4 : pow2ceil(upr));
    return moe && lg >= 32 ? lg / 2 : lg;
}

inline int plan(GemvParams& p, int M, int K, int rows, int RR, bool moe, int npairs_max, bool pure,
         int cus, int resident, int threads, int wgmax) {
    p.K = K;
    p.upr = (int)k_units(K);
    // The 32-lane groups of long dense rows only where their workgroups
    // (two rows per wave, `threads`-thread groups) fill the CUs evenly: at
    // N = 5120, K = 13824 the 320 groups left 64 CUs with two and were 4-6 %
    // slower than 64 lanes (eager, M = 1 and 2).  The test depends on the
    // shape only, so the gate+up pair decides as its single-matrix calls do.
    bool long_rows = M <= 2 && !moe;
    if (long_rows && p.upr > kWave) {
        const long long need32 = ((rows + 2LL * RR - 1) / (2LL * RR) + threads / kWave - 1) /
                                 (threads / kWave);
        long_rows = need32 % cus == 0 || need32 >= 2LL * cus;
    }
    p.lg = choose_lg(p.upr, moe && M >= 2 && M <= 4, long_rows);
    p.upl = (p.upr + p.lg - 1) / p.lg;
    p.rgw = kWave / p.lg;
    const int nrg = (rows + RR - 1) / RR;
    long long tasks;
    if (moe) {
        p.nrg = (nrg + p.rgw - 1) / p.rgw * p.rgw;
        p.ntasks = 0;
        tasks = (long long)npairs_max * (p.nrg / p.rgw);
    } else {
        p.nrg = nrg;
        p.ntasks = (nrg + p.rgw - 1) / p.rgw;
        tasks = p.ntasks;
    }
    const int wpb = threads / kWave;
    int wgc = wg_per_cu(gemv_lds_bytes(M, K, pure), wgmax);
    if (wgc > resident) wgc = resident;
    // Every CU gets the same number of workgroups (the per-CU load/issue rate
    // is shared by its waves); tasks are then split evenly over all waves.
    static const int bpc_override = env_int("Q4GEMV_BLOCKS_PER_CU", 0);
    const int bpc = bpc_override > 0 ? bpc_override : wgc;
    long long blocks_ll = (long long)cus * bpc;
    const long long need = (tasks + wpb - 1) / wpb;  // no more waves than tasks
    if (blocks_ll > need) blocks_ll = need;
    // At least two steps per wave (a wave with one step has nothing to
    // overlap its loads with), down to one workgroup per CU.
    long long two = (tasks * p.upl / 2 + wpb - 1) / wpb;
    if (two < cus) two = cus;
    if (blocks_ll > two) blocks_ll = two;
    int blocks = (int)(blocks_ll < 1 ? 1 : blocks_ll);
    p.nwaves = blocks * wpb;
    return blocks;
}

#ifndef Q4_RR_SINGLE
#define Q4_RR_SINGLE 2  // rows per lane per step, single-matrix calls
#endif
#ifndef Q4_RR_PAIR
#define Q4_RR_PAIR 1  // rows per lane per step and matrix, two-matrix calls
#endif
#ifndef Q4_RR_MOE
#define Q4_RR_MOE 1  // rows per lane per step and matrix, expert calls
#endif
#ifndef Q4_PREFETCH
#define Q4_PREFETCH 1  // steps of weight loads in flight ahead of the computed one
#endif

// Q4GEMV_XR=0 keeps the activations in LDS also where they fit in registers
// (for comparisons).
inline bool xr_enabled() {
    static const bool on = [] {
        const char* s = getenv("Q4GEMV_XR");
        return !(s && *s && atoi(s) == 0);
    }();
    return on;
}

// RRX > 0 overrides the rows per lane and step (RR).
template <int FMT, int NMAT, int MODE, bool PURE, int M, bool XR, bool TAIL, int RRX = 0>
inline int run_plan(GemvParams& p, int cus, int npairs_max, void* stream) {
    constexpr int RR = RRX > 0 ? RRX
                               : (mode_moe(MODE) ? Q4_RR_MOE : (NMAT == 1 ? Q4_RR_SINGLE : Q4_RR_PAIR));
    // Workgroup shape (measured): dense single-token calls run 256-thread
    // groups, at most two per CU (four were 4 % slower), 512-thread ones for
    // rows over 64 units (the staging then halves per CU); expert calls 256- or
    // 768-thread groups (gemv_threads), as many as their 134-147 VGPRs allow:
    // 12 waves per CU, which beat 8 waves of 512-thread groups by 9-14 %.
    // Dense batched calls on this kernel run two 512-thread groups.
    constexpr int BS = gemv_threads(M, MODE, XR);
    // (three register-resident single-token groups per CU: headline 15.06
    // against 15.17 us, its SiLU form 15.29 against 15.61, the fused RMSNorm
    // call 11.72 against 11.92; three runs on one box)
    constexpr int WGMAX = mode_moe(MODE) ? 4 : (XR && M == 1 ? 3 : 2);
    static std::atomic<int> big_lds_done[kMaxDevices];
    static std::atomic<int> resident[kMaxDevices];
    // a pure-read pass takes the launch shape of the call it mirrors
    auto kern = [](bool pure) {
        if constexpr (XR)
            return pure ? gemv_kernel_xr<FMT, M, NMAT, RR, MODE, true, Q4_PREFETCH, BS>
                        : gemv_kernel_xr<FMT, M, NMAT, RR, MODE, false, Q4_PREFETCH, BS>;
        else
            return pure ? gemv_kernel<FMT, M, NMAT, RR, MODE, true, Q4_PREFETCH, TAIL, BS>
                        : gemv_kernel<FMT, M, NMAT, RR, MODE, false, Q4_PREFETCH, TAIL, BS>;
    };
    const int res = resident_per_cu((const void*)kern(false), BS,
                                    gemv_lds_bytes(M, p.K, false), resident);
    const int blocks =
        plan(p, M, p.K, p.N, RR, mode_moe(MODE), npairs_max, false, cus, res, BS, WGMAX);
    const size_t lds = gemv_lds_bytes(M, p.K, PURE);
    return launch(kern(PURE), p, blocks, lds, stream, big_lds_done, BS);
}

constexpr int kXrTwoMaxRows = 8192;  // single-matrix calls at M = 2 with register-resident x
template <int FMT, int NMAT, int MODE, bool PURE, int M>
inline int run_m(GemvParams& p, int cus, int npairs_max, void* stream) {
    if constexpr (M <= kXrMaxM && !mode_moe(MODE)) {
        // one 64-weight unit per lane per row: at most 64 units (and then
        // the activations need no staging loop beyond the first kXReg chunks).
        // Two tokens hold 128 activations per lane (about 240 VGPRs, one
        // 512-thread workgroup per CU): worth it for short single-matrix calls,
        // whose waves have one or two steps (Q4_0 4096 x 4096: 7.0 -> 6.5 us),
        // not for the gate+up pair of 2 x 14336 rows (19.5 -> 19.7 us).
        const int upr = (int)k_units(p.K);
        const bool two_ok = M == 1 || (NMAT == 1 && p.N <= kXrTwoMaxRows);
        if (two_ok && upr <= kWave && choose_lg(upr) >= upr && xr_enabled()) {
            // A single-matrix call too small to give every CU a task at two
            // rows per lane takes one row per lane: twice the waves for a call
            // that is all latency (Q4_0 K=512 N=256: 3.36 -> 2.88 us; at
            // 4096 x 4096 and up two rows per lane stay faster, 4.9 against
            // 5.2 us).
            if constexpr (M == 1 && NMAT == 1 && Q4_RR_SINGLE != 1) {
                const long long rgw = kWave / choose_lg(upr);
                const long long tasks2 = ((p.N + Q4_RR_SINGLE - 1) / Q4_RR_SINGLE + rgw - 1) / rgw;
                if (tasks2 < cus)
                    return run_plan<FMT, NMAT, MODE, PURE, M, true, false, 1>(p, cus, npairs_max,
                                                                             stream);
            }
            return run_plan<FMT, NMAT, MODE, PURE, M, true, false>(p, cus, npairs_max, stream);
        }
    }
    if ((long long)M * p.K > (long long)xreg_chunks(M, MODE) * 4 * gemv_threads(M, MODE, false)) {
        // long rows at one or two tokens: one row per lane and step (with
        // the 32-lane groups of choose_lg, 10.57 against 11.66 us on the
        // 4096 x 14336 down-projection at M = 1; two rows per lane: 13.56 us)
        if constexpr (M <= 2 && NMAT == 1 && !mode_moe(MODE))
            return run_plan<FMT, NMAT, MODE, PURE, M, false, true, 1>(p, cus, npairs_max, stream);
        return run_plan<FMT, NMAT, MODE, PURE, M, false, true>(p, cus, npairs_max, stream);
    }
    return run_plan<FMT, NMAT, MODE, PURE, M, false, false>(p, cus, npairs_max, stream);
}

// Matrix-core kernel: steps of weight loads each wave keeps in flight, and
// the number of waves per CU the K split aims for.
#ifndef Q4_MFMA_PD_Q4K
#define Q4_MFMA_PD_Q4K 2
#endif
#ifndef Q4_MFMA_PD_Q4_0
#define Q4_MFMA_PD_Q4_0 3
#endif
#ifndef Q4_MFMA_WAVES_PER_CU
#define Q4_MFMA_WAVES_PER_CU 8
#endif

// Waves that split one 16-row tile's K range (1, 2, 4 or 8): the fewest that
// give the CUs at least three quarters of their share of waves, at most one
// per step of the row (gate+up, 1792 tiles: one wave per tile, 16 steps each,
// measured 4 % faster than two waves of 8 steps).  It depends on the matrix
// shape and the CU count only, so a token's result does not depend on the
// batch it is computed in.
inline int mfma_ks(long long ntiles, int steps, int cus) {
    static const int forced = env_int("Q4GEMV_MFMA_KS", 0);
    const long long want = (long long)cus * Q4_MFMA_WAVES_PER_CU;
    int ks = 1;
    while (ks < kMWaves && 2 * ks <= steps && 4 * ntiles * ks < 3 * want) ks *= 2;
    if (forced == 1 || forced == 2 || forced == 4 || forced == 8)
        ks = forced <= steps ? forced : ks;
    return ks;
}

// Batches of at least this many token rows run on the matrix-core kernel
// (at M = 2 the VALU kernel is still below its issue limit and faster).
// Q4GEMV_MFMA=0 sends every batch to the VALU kernel (for comparisons; the
// results differ only by rounding).
#ifndef Q4_MFMA_MIN_M
#define Q4_MFMA_MIN_M 3
#endif
inline bool mfma_enabled() {
    static const bool on = [] {
        const char* s = getenv("Q4GEMV_MFMA");
        return !(s && *s && atoi(s) == 0);
    }();
    return on;
}

inline bool moe_mfma_enabled() {
    static const bool on = [] {
        const char* s = getenv("Q4GEMV_MOE_MFMA");
        return s && *s && atoi(s) != 0;
    }();
    return on;
}

template <int FMT, int NMAT, int MODE, bool PURE, int M, int STG>
inline int run_mfma_launch(GemvParams& p, int cus, int nexperts, int reserve, void* stream) {
    constexpr bool SLICED = STG == kStgSliced;
    constexpr int PD = FMT == kFmtQ4K ? Q4_MFMA_PD_Q4K : Q4_MFMA_PD_Q4_0;
    static std::atomic<int> big_lds_done[kMaxDevices];
    static std::atomic<int> resident[kMaxDevices];
    const int S = msteps(p.K);
    int kse = p.ks;
    while (kse > S) kse >>= 1;  // (the kernel's own clamp)
    const int steps = SLICED ? mslice_regions(kse, p.npg) * p.msl : S;
    // a pure-read pass takes the launch shape of the call it mirrors
    const size_t lds = (size_t)mlayout_steps(FMT, M, steps, PURE).bytes;
    const size_t call_lds = (size_t)mlayout_steps(FMT, M, steps, false).bytes;
    int wgc = wg_per_cu(call_lds);
    if (call_lds > 64 * 1024) {  // the occupancy query needs the raised limit
        static std::atomic<int> big_lds_mirror[kMaxDevices];
        int st = allow_big_lds(
            (const void*)mfma_gemv_kernel<FMT, M, NMAT, MODE, false, PD, STG>, big_lds_mirror,
            reserve);
        if (st) return st;
    }
    const int res = resident_per_cu(
        (const void*)mfma_gemv_kernel<FMT, M, NMAT, MODE, false, PD, STG>, kMBlock, call_lds,
        resident);
    if (wgc > res) wgc = res;
    const long long ntiles_run =
        (MODE == kModeSilu || MODE == kModeNormSilu)
            ? (long long)nexperts * ((p.N + 7) / 8)
            : (long long)NMAT * nexperts * ((p.N + 15) / 16);
    const int TG = kMWaves / p.ks;
    long long blocks = (long long)cus * wgc;
    const long long need = (ntiles_run + TG - 1) / TG;
    if (blocks > need) blocks = need;
    return launch(mfma_gemv_kernel<FMT, M, NMAT, MODE, PURE, PD, STG>, p, (int)blocks, lds,
                  stream, big_lds_done, kMBlock, reserve);
}

template <int FMT, int NMAT, int MODE, bool PURE, int M>
inline int run_mfma_m(GemvParams& p, int cus, int nexperts, void* stream) {
    const int reserve =
        mode_moe(MODE) ? kMfmaMoeStaticLds : (M > 8 ? kMfmaBigStaticLds : kMfmaStaticLds);
    const int budget = 160 * 1024 - reserve;
    // (the expert call: at most nexperts unique experts, each N rows per matrix)
    // (the K split is chosen from the 16-row tile count of the plain call,
    // also for the SiLU-gated call and its 8 + 8-row tiles, so that both
    // accumulate every row alike)
    const long long ntiles = (long long)NMAT * nexperts * ((p.N + 15) / 16);
    const int S = msteps(p.K);
    p.ks = mfma_ks(ntiles, S, cus);
    p.nsl = 1;
    p.msl = S;
    p.npg = 1;
    const bool whole = (long long)M * mpadk(p.K) <= kMaxMK &&
                       mlayout(FMT, M, p.K, false).bytes <= budget;
    if (whole || mode_moe(MODE))  // (expert calls are only sent here whole)
        return run_mfma_launch<FMT, NMAT, MODE, PURE, M, kStgWhole>(p, cus, nexperts, reserve,
                                                                    stream);
    if constexpr (mode_moe(MODE)) {
        return Q4_ERR_SHAPE;
    } else {
        // K slices: the fewest whose staged steps (msl per wave range) fit;
        // past one step per range, wave positions staged in turn
        int kse = p.ks;
        while (kse > S) kse >>= 1;
        const int lmax = (S + kse - 1) / kse;  // longest wave range, in steps
        int nsl = 1, msl = lmax, npg = 1;
        while (mlayout_steps(FMT, M, mslice_regions(kse, npg) * msl, false).bytes > budget) {
            if (msl > 1) {
                ++nsl;
                msl = (lmax + nsl - 1) / nsl;
            } else if (npg < kse) {
                npg *= 2;
            } else {
                return Q4_ERR_SHAPE;
            }
        }
        p.nsl = nsl;
        p.msl = msl;
        p.npg = npg;
        return run_mfma_launch<FMT, NMAT, MODE, PURE, M, kStgSliced>(p, cus, nexperts, reserve,
                                                                     stream);
    }
}

template <int FMT, int NMAT, int MODE, bool PURE>
inline int run(GemvParams& p, int M, int npairs_max, void* stream) {
    int cus = 0;
    int st = device_cus(&cus);
    if (st) return st;
    // batched calls on the matrix cores (also every batch the VALU kernel
    // cannot stage whole); the expert call only on request
    // (Q4GEMV_MOE_MFMA=1: it measured slower than the VALU expert kernel at
    // the E=64, top-6, 1408 x 2048 shape), from M = 2 on, where its
    // activations leave room in LDS for the expert tables
    // (the SiLU-gated expert call always runs the VALU kernel)
    const bool vfits = valu_fits(M, p.K);
    bool use_mfma;
    if constexpr (mode_moe(MODE)) {
        use_mfma = MODE == kModeMoe && moe_mfma_enabled() && M >= 2 &&
                   (long long)M * mpadk(p.K) <= kMaxMK &&
                   mlayout(FMT, M, p.K, false).bytes <= 160 * 1024 - kMfmaMoeStaticLds;
    } else {
        use_mfma = M >= 2 && (!vfits || (M >= Q4_MFMA_MIN_M && mfma_enabled()));
    }
    if constexpr (MODE != kModeMoeSilu) {
    if (use_mfma) {
        const int nexp = mode_moe(MODE) ? npairs_max : 1;
        switch (M) {
            case 2: return run_mfma_m<FMT, NMAT, MODE, PURE, 2>(p, cus, nexp, stream);
            case 3: return run_mfma_m<FMT, NMAT, MODE, PURE, 3>(p, cus, nexp, stream);
            case 4: return run_mfma_m<FMT, NMAT, MODE, PURE, 4>(p, cus, nexp, stream);
            case 5: return run_mfma_m<FMT, NMAT, MODE, PURE, 5>(p, cus, nexp, stream);
            case 6: return run_mfma_m<FMT, NMAT, MODE, PURE, 6>(p, cus, nexp, stream);
            case 7: return run_mfma_m<FMT, NMAT, MODE, PURE, 7>(p, cus, nexp, stream);
            case 8: return run_mfma_m<FMT, NMAT, MODE, PURE, 8>(p, cus, nexp, stream);
        }
        if constexpr (!mode_moe(MODE)) {
            switch (M) {
                case 9: return run_mfma_m<FMT, NMAT, MODE, PURE, 9>(p, cus, nexp, stream);
                case 10: return run_mfma_m<FMT, NMAT, MODE, PURE, 10>(p, cus, nexp, stream);
                case 11: return run_mfma_m<FMT, NMAT, MODE, PURE, 11>(p, cus, nexp, stream);
                case 12: return run_mfma_m<FMT, NMAT, MODE, PURE, 12>(p, cus, nexp, stream);
                case 13: return run_mfma_m<FMT, NMAT, MODE, PURE, 13>(p, cus, nexp, stream);
                case 14: return run_mfma_m<FMT, NMAT, MODE, PURE, 14>(p, cus, nexp, stream);
                case 15: return run_mfma_m<FMT, NMAT, MODE, PURE, 15>(p, cus, nexp, stream);
                case 16: return run_mfma_m<FMT, NMAT, MODE, PURE, 16>(p, cus, nexp, stream);
            }
        }
        return Q4_ERR_BATCH;
    }
    }
    if (!vfits) return Q4_ERR_SHAPE;
    switch (M) {
        case 1: return run_m<FMT, NMAT, MODE, PURE, 1>(p, cus, npairs_max, stream);
        case 2: return run_m<FMT, NMAT, MODE, PURE, 2>(p, cus, npairs_max, stream);
        case 3: return run_m<FMT, NMAT, MODE, PURE, 3>(p, cus, npairs_max, stream);
        case 4: return run_m<FMT, NMAT, MODE, PURE, 4>(p, cus, npairs_max, stream);
        case 5: return run_m<FMT, NMAT, MODE, PURE, 5>(p, cus, npairs_max, stream);
        case 6: return run_m<FMT, NMAT, MODE, PURE, 6>(p, cus, npairs_max, stream);
        case 7: return run_m<FMT, NMAT, MODE, PURE, 7>(p, cus, npairs_max, stream);
        case 8: return run_m<FMT, NMAT, MODE, PURE, 8>(p, cus, npairs_max, stream);
    }
    return Q4_ERR_BATCH;
}

// Expert down-projection: rows per lane group and the lane-group width.
#ifndef Q4_RR_DOWN
#define Q4_RR_DOWN 1
#endif

// Lane-group width that wastes the fewest lanes on a row of `upr` units:
// the widest power of two (64 .. 4) whose last pass over the row leaves at
// most one lane in eight idle, else the one that idles the fewest (rows of
// 22 units, K = 1408: 8 lanes, 3 units each, against 32 lanes with 10 idle).
inline int choose_lg_waste(int upr) {
    static const int forced = env_int("Q4GEMV_LG", 0);
    if (forced >= 4 && forced <= kWave && (forced & (forced - 1)) == 0) return forced;
    int best = 4, best_idle = 1 << 30, best_slots = 1;
    for (int lg = kWave; lg >= 4; lg >>= 1) {
        const int slots = (upr + lg - 1) / lg * lg;
        const int idle = slots - upr;
        if (8 * idle <= slots) return lg;
        if ((long long)idle * best_slots < (long long)best_idle * slots) {
            best = lg;
            best_idle = idle;
            best_slots = slots;
        }
    }
    return best;
}

template <int M, int RR, bool PURE>
inline int run_down_rr(GemvParams& p, int cus, int npairs_max, void* stream) {
    static std::atomic<int> big_lds_done[kMaxDevices];
    static std::atomic<int> resident[kMaxDevices];
    p.upr = (int)k_units(p.K);
    p.lg = choose_lg_waste(p.upr);
    p.upl = (p.upr + p.lg - 1) / p.lg;
    p.rgw = kWave / p.lg;
    p.nrg = (p.N + RR - 1) / RR;
    const size_t lds = PURE ? 0 : down_lds_bytes(M, p.upr);
    const int res = resident_per_cu((const void*)moe_down_kernel<M, RR, false>, kDownBlock,
                                    down_lds_bytes(M, p.upr), resident);
    static const int wgmax = env_int("Q4GEMV_DOWN_WG_PER_CU", 4);
    int wgc = wg_per_cu(down_lds_bytes(M, p.upr), wgmax);
    if (wgc > res) wgc = res;
    // ks workgroups per possible unique expert, so that the grid fills the
    // CUs (at least one workgroup pass over the rows per share)
    const long long per_pass = (long long)kDownWaves * p.rgw;
    long long ks = ((long long)cus * wgc + npairs_max - 1) / npairs_max;
    const long long ks_max = (p.nrg + per_pass - 1) / per_pass;
    if (ks > ks_max) ks = ks_max;
    if (ks < 1) ks = 1;
    p.ks = (int)ks;
    const long long blocks = ks * npairs_max;
    if (blocks > INT32_MAX) return Q4_ERR_SHAPE;
    p.nwaves = (int)blocks * kDownWaves;
    return launch(moe_down_kernel<M, RR, PURE>, p, (int)blocks, lds, stream, big_lds_done,
                  kDownBlock);
}

// Q4GEMV_DOWN_RR=1 or 2 overrides the rows per lane group (measurements).
template <int M, bool PURE>
inline int run_down_m(GemvParams& p, int cus, int npairs_max, void* stream) {
    static const int rr = env_int("Q4GEMV_DOWN_RR", Q4_RR_DOWN);
    if (rr == 2) return run_down_rr<M, 2, PURE>(p, cus, npairs_max, stream);
    return run_down_rr<M, 1, PURE>(p, cus, npairs_max, stream);
}

template <bool PURE>
inline int run_down(GemvParams& p, int M, int npairs_max, void* stream) {
    int cus = 0;
    int st = device_cus(&cus);
    if (st) return st;
    switch (M) {
        case 1: return run_down_m<1, PURE>(p, cus, npairs_max, stream);
        case 2: return run_down_m<2, PURE>(p, cus, npairs_max, stream);
        case 3: return run_down_m<3, PURE>(p, cus, npairs_max, stream);
        case 4: return run_down_m<4, PURE>(p, cus, npairs_max, stream);
        case 5: return run_down_m<5, PURE>(p, cus, npairs_max, stream);
        case 6: return run_down_m<6, PURE>(p, cus, npairs_max, stream);
        case 7: return run_down_m<7, PURE>(p, cus, npairs_max, stream);
        case 8: return run_down_m<8, PURE>(p, cus, npairs_max, stream);
    }
    return Q4_ERR_BATCH;
}

// ---------------------------------------------------------------------------
// Split-K batched GEMV (caller workspace): the partial-sum kernel, then the
// merge kernel, on the caller's stream.  The plan depends on N, K and the CU
// count only (not on M), so every batch of one shape splits alike and a
// token's row does not depend on the batch.
// ---------------------------------------------------------------------------
struct SplitKPlan {
    int kp = 1;       // K parts
    int msl = 0;      // steps per part (staged at once)
    int ngroups = 0;  // tile groups (8 tiles of 16 rows)
    long long part_bytes = 0, exp_bytes = 0, total = 0;
};

inline long long align256(long long v) { return (v + 255) / 256 * 256; }

inline SplitKPlan splitk_plan(int fmt, int64_t M, int64_t N, int64_t K, int cus) {
    SplitKPlan pl;
    const int S = msteps((int)K);
    const long long ntiles = (N + 15) / 16;
    pl.ngroups = (int)((ntiles + kMWaves - 1) / kMWaves);
    static const int forced = env_int("Q4GEMV_SPLITK_KP", 0);
    // about one workgroup per CU (measured: the batched Q4_0 workload at
    // M = 4 / 8 / 16 ran 13.9 / 15.4 / 19.0 us with 8 parts, 19.5 / 21.4 /
    // 25.4 us with 16, 15.2 / 16.5 / 20.9 us with 4)
    long long kp = forced > 0 ? forced : ((long long)cus + pl.ngroups - 1) / pl.ngroups;
    // parts of at most kSplitKOneSteps steps are staged in one pass (up to
    // 64 parts; longer rows keep longer parts)
    const long long kone = (S + kSplitKOneSteps - 1) / kSplitKOneSteps;
    if (forced <= 0 && kone <= 64 && kp < kone) kp = kone;
    if (kp > S) kp = S;
    if (kp < 1) kp = 1;
    // the largest batch's staging of one part must fit in LDS
    for (;;) {
        const int msl = (int)((S + kp - 1) / kp);
        if (mlayout_steps(fmt, kMaxM, msl, false).bytes <= 160 * 1024 - kMfmaBigStaticLds ||
            kp >= S)
            break;
        ++kp;
    }
    pl.kp = (int)kp;
    pl.msl = (int)((S + kp - 1) / kp);
    pl.part_bytes = align256(kp * M * N * 4);
    pl.exp_bytes = align256(kp * M * 4);
    pl.total = pl.exp_bytes + pl.part_bytes;
    return pl;
}

template <int FMT, int M>
inline int run_splitk_m(GemvParams& p, const SplitKPlan& pl, int cus, void* stream) {
    constexpr int PD = FMT == kFmtQ4K ? Q4_MFMA_PD_Q4K : Q4_MFMA_PD_Q4_0;
    constexpr int reserve = M > 8 ? kMfmaBigStaticLds : kMfmaStaticLds;
    static std::atomic<int> big_lds_done[kMaxDevices];
    (void)cus;
    p.ks = 1;
    p.kp = pl.kp;
    p.msl = pl.msl;
    p.nsl = 1;
    p.npg = 1;
    const size_t lds = (size_t)mlayout_steps(FMT, M, pl.msl, false).bytes;
    const long long blocks = (long long)pl.ngroups * pl.kp;
    if (blocks > INT32_MAX) return Q4_ERR_SHAPE;
    int st = launch(mfma_gemv_kernel<FMT, M, 1, kModeDense, false, PD, kStgSplitK>, p,
                    (int)blocks, lds, stream, big_lds_done, kMBlock, reserve);
    if (st) return st;
    const long long outs = (long long)M * p.N;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, p.y0, (const float*)p.part, (const int*)p.pexp,
                       pl.kp, M, p.N);
    return hipGetLastError() == hipSuccess ? Q4_OK : Q4_ERR_HIP;
}

// The split-K call: workspace laid out as [exponents | partials].
template <int FMT>
inline int run_splitk(GemvParams& p, int M, void* ws, int64_t ws_bytes, void* stream) {
    int cus = 0;
    int st = device_cus(&cus);
    if (st) return st;
    const SplitKPlan pl = splitk_plan(FMT, M, p.N, p.K, cus);
    // single tokens and pairs run the VALU kernel, and a plan of one part
    // is the ordinary call: the workspace is not used
    if (M < Q4_MFMA_MIN_M || pl.kp == 1) return run<FMT, 1, kModeDense, false>(p, M, 0, stream);
    if (!ws) return Q4_ERR_NULL;
    if (ws_bytes < pl.total) return Q4_ERR_SHAPE;
    if (!aligned(ws, 256)) return Q4_ERR_ALIGN;
    uint8_t* b = (uint8_t*)ws;
    p.pexp = (int*)b;
    p.part = (float*)(b + pl.exp_bytes);
    switch (M) {
        case 3: return run_splitk_m<FMT, 3>(p, pl, cus, stream);
        case 4: return run_splitk_m<FMT, 4>(p, pl, cus, stream);
        case 5: return run_splitk_m<FMT, 5>(p, pl, cus, stream);
        case 6: return run_splitk_m<FMT, 6>(p, pl, cus, stream);
        case 7: return run_splitk_m<FMT, 7>(p, pl, cus, stream);
        case 8: return run_splitk_m<FMT, 8>(p, pl, cus, stream);
        case 9: return run_splitk_m<FMT, 9>(p, pl, cus, stream);
        case 10: return run_splitk_m<FMT, 10>(p, pl, cus, stream);
        case 11: return run_splitk_m<FMT, 11>(p, pl, cus, stream);
        case 12: return run_splitk_m<FMT, 12>(p, pl, cus, stream);
        case 13: return run_splitk_m<FMT, 13>(p, pl, cus, stream);
        case 14: return run_splitk_m<FMT, 14>(p, pl, cus, stream);
        case 15: return run_splitk_m<FMT, 15>(p, pl, cus, stream);
        case 16: return run_splitk_m<FMT, 16>(p, pl, cus, stream);
    }
    return Q4_ERR_BATCH;
}

inline GemvParams base_params(const void* w0, const void* w1, float* y0, float* y1, const float* x,
                       int64_t N, int64_t K, int fmt) {
    GemvParams p = {};
    p.w0 = (const uint8_t*)w0;
    p.w1 = (const uint8_t*)w1;
    p.y0 = y0;
    p.y1 = y1;
    p.x = x;
    p.N = (int)N;
    p.K = (int)K;
    p.upr = (int)k_units(K);
    p.row_bytes = row_bytes_of(K, fmt);
    return p;
}

// Expert calls: M <= 8 (the decode batch), activations staged whole.
inline int check_moe(int64_t M, int64_t top_k, int64_t E, int64_t N, int64_t K) {
    if (M < 1 || M > 8) return Q4_ERR_BATCH;
    int st = check_dims(M, N, K, kFmtQ4_0);
    if (st) return st;
    if (!valu_fits(M, K)) return Q4_ERR_SHAPE;
    if (E < 1 || E >= (1 << 20) || top_k < 1 || top_k > E || M * top_k > kMaxPairs)
        return Q4_ERR_SHAPE;
    if (E * N > INT32_MAX) return Q4_ERR_SHAPE;
    return Q4_OK;
}

}  // namespace
