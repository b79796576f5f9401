// q4_mfma.h -- matrix-core GEMV kernel for batched calls (M >= 2 token rows;
// the library sends it batches of M >= 3).
//
// With several token rows the fp32 VALU path runs out of issue slots (one
// mixed FMA per weight per token), so the dense batched calls run the
// products on v_mfma_f32_16x16x32_f16 instead:
//
//   D[i][j] = sum_k A[i][k] * B[k][j]   (16 x 16 x 32, fp32 accumulate)
//   lane l holds A[l%16][8(l/16)+t], B[8(l/16)+t][l%16], D[4(l/16)+r][l%16]
//
//   * B = weights.  Column j is row j of a 16-row tile, and the 32 k-slots
//     are the 32 elements of one Q4_0 block or one Q4_K sub-block, which
//     share one scale.  A nibble masked into a 16-bit half in place is the
//     exact f16 subnormal q*2^-24 (low nibble) or 16q*2^-24 (high nibble).
//   * A = activations.  Row i = 2m + h is the high (h = 0) or low (h = 1)
//     f16 part of token m scaled by 2^e_m, e_m chosen so the token's largest
//     magnitude lies in [2^14, 2^15); hi + lo keep ~22 bits of every x.
//     Elements met as high nibbles are staged with a further 2^-4, so every
//     product is exactly q * x * 2^(e_m - 24).
//   * Each lane's D values belong to its own weight row j, so the block
//     scales are applied in the lane that loaded them:
//       Q4_0 (w = d (q - 8)):        y += d * (D - 8 X)
//       Q4_K (w = d sc q - dmin m):  y += d * D - dmin * Dmin, where the
//     6-bit sub-block scales are folded into B (an f16 multiply of the
//     subnormal nibble by sc is exact), so one accumulation runs over all
//     sub-blocks; X are block sums of x, and Dmin = sum_J m_J X_J is one
//     more MFMA per super-block with the sub-block sums as A and the 6-bit
//     mins as B.
//   (Q4_0 layout: inferencelayer 0.2.13, src/bin/kernel_lab.rs, GEMV_F16S;
//    Q4_K layout: trueno-gpu 0.4.11, src/kernels/quantize/fused.rs,
//    FusedRmsNormQ4KGemvKernel::build_ptx, PHASE 3.)
//
// Fragment order.  The 8 k-slots t of lane group c come from 4 nibble
// bytes of each of 2 dwords as (byte 0, 2, 1, 3) -- a mask of the dword and
// a mask of the dword shifted by 8 -- so slot t holds byte slot_byte(t) of
// an 8-byte slice; the 8 elements are the consecutive elements 8p .. 8p+7
// of one "piece" p, whose A fragment for row i sits in LDS slot fslot(i, p).
//   Q4_0 block b, group c:  bytes 8(c&1) .. of its nibbles, low nibbles for
//                           c < 2 (elements 8c ..), high for c >= 2: p = 4b + c
//   Q4_K: see compute() (a lane's slices come from 16-byte loads).
//
// Work split.  A tile is 16 rows of one matrix.  A workgroup is 8 waves in
// groups of KS; each group takes one tile per round and its KS waves split
// the tile's K range, adding their partial sums through LDS at the end of
// the round.  Every wave keeps PD steps of weight loads in flight in a
// register ring, across rounds too.  Order at the start: the activation
// loads, then the first PD steps of weight loads, then the staging
// arithmetic (once per workgroup, RMS-normalized first for the fused call),
// so the staging waits only for the activations.
#pragma once

#include <type_traits>

#include "q4_kernels.h"

namespace q4 {

constexpr int kMBlock = 512;  // threads per workgroup
constexpr int kMWaves = kMBlock / kWave;
static_assert(kMWaves <= kMaxStageWaves, "staging scratch holds 8 waves");
constexpr int kMaxMK = 32768;  // M * K of a call staged whole (register-held pieces)
constexpr int kMPieces = (kMaxMK / 8 + kMBlock - 1) / kMBlock;  // staging pieces per thread
constexpr int kMaxM = 16;  // token rows of the batched kernel: two 8-token A tiles
__host__ __device__ constexpr int mtiles(int M) { return (M + 7) / 8; }

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4m __attribute__((ext_vector_type(4)));

// byte of the 8-byte lane slice that feeds k-slot t
__host__ __device__ constexpr int slot_byte(int t) {
    return (t & 4) | ((t & 1) << 1) | ((t >> 1) & 1);
}

// A step is 256 elements of a row: one Q4_K super-block or eight Q4_0
// blocks, 144 bytes either way.  A row whose K is not a multiple of 256
// ends in a partial step: its activations past K are staged as zeros (a
// Q4_K row's padding is read and multiplied by them; a Q4_0 row's blocks
// past its end are masked, see load() and compute()).
template <int FMT>
struct MStep {
    static constexpr int kElems = 256;
    static constexpr int kBytes = 144;
};
__host__ __device__ inline int msteps(int K) { return (K + 255) / 256; }
__host__ __device__ inline int mpadk(int K) { return msteps(K) * 256; }

// Q4_0 tile-steps (16 rows x 144 bytes) are loaded as 144 contiguous
// 16-byte chunks, 3 per lane, and regrouped through a wave-private LDS copy.
constexpr int kQ40Chunks = 16 * 9;
constexpr int kQ40WaveBytes = kQ40Chunks * 16;

// tokens per row of the Q4_0 block-sum table (M rounded up to even)
__host__ __device__ constexpr int sums_stride(int M) { return M + (M & 1); }

// LDS map (bytes) for M tokens and K columns.
struct MLayout {
    int frag;  // A fragments: 2M rows x (K/8 + 1) pieces x 16 bytes (see fslot)
    int aux;   // Q4_K: Dmin A operand, (K/256) x 4 groups x 2M rows x 2 halves
               // Q4_0: block sums X, (K/32) blocks x sums_stride(M) tokens x fp32
    int exps;  // e_m, 16 ints, then (K-sliced calls) the RMSNorm factors, 16 floats
    int part;  // partial sums, 2 buffers x 8 waves x 64 lanes x float2 per A tile
    int wbuf;  // Q4_0: one tile-step of raw weight bytes per wave
    int bytes;
};

// LDS map for M tokens and `steps` staged 256-column steps (K = 256 steps).
__host__ __device__ inline MLayout mlayout_steps(int fmt, int M, int steps, bool pure) {
    const int K = steps * 256;
    MLayout l;
    l.frag = 0;
    l.aux = pure ? 0 : (K / 8 + 1) * 2 * M * 16;
    l.exps = l.aux + (pure ? 0
                           : (fmt == kFmtQ4K ? (K / 256) * 4 * 2 * M * 4
                                             : (K / 32) * sums_stride(M) * 4));
    l.part = l.exps + 128;
    l.wbuf = l.part + 2 * kMWaves * 64 * 8 * mtiles(M);
    l.bytes = l.wbuf + (fmt != kFmtQ4K ? kMWaves * kQ40WaveBytes : 0);
    return l;
}

// The map of a call that stages its rows whole.
__host__ __device__ inline MLayout mlayout(int fmt, int M, int K0, bool pure) {
    return mlayout_steps(fmt, M, msteps(K0), pure);
}

// 16-byte slot of the A fragment of piece p, row i: rows of K/8 + 1 slots
// (K the staged column count, mpadk of the call's K).
// The odd row length puts the rows a lane group reads 4 banks apart (all 64
// banks for 16 rows), and the staging writes consecutive pieces of a row
// to consecutive slots; both are free of bank conflicts.
__device__ __forceinline__ int fslot(int K, int i, int p) { return i * ((K >> 3) + 1) + p; }


// ---------------------------------------------------------------------------
// Staging of the activations into A fragments.
// ---------------------------------------------------------------------------
// The A fragments of one piece of 8 elements v (token scale 2^e): slot t
// holds element slot_byte(t) scaled by 2^e, 2^(e-4) for a piece met as high
// nibbles; hi = its nearest f16, lo = the f16 of the remainder, which one
// mixed fused multiply-add gives exactly in fp32.  part = the piece's sum
// scaled by 2^e, added in element order (slot_byte is its own inverse); a
// high piece's sum is formed 2^-4 lower and multiplied back by 16, exact
// above the subnormal range.
__device__ __forceinline__ void piece_frag(const float (&v)[8], int e, bool high, h8& hi, h8& lo,
                                           float& part) {
    const int ef = high ? e - 4 : e;
    float xs[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) xs[t] = __builtin_ldexpf(v[slot_byte(t)], ef);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const _Float16 h = (_Float16)xs[t];
        hi[t] = h;
        lo[t] = (_Float16)__builtin_fmaf((float)h, -1.0f, xs[t]);
    }
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += xs[slot_byte(j)];
    part = high ? sum * 16.0f : sum;
}
template <int FMT>
__device__ __forceinline__ bool piece_is_high(int pp) {
    return FMT == kFmtQ4K ? ((pp >> 2) & 1) : ((pp >> 1) & 1);
}

// Per-token largest magnitude of a workgroup's staged pieces, each wave's
// into red.am[m][wave] (0 for tokens it holds no piece of): piece slot k of
// thread tid is piece tid + k * kMBlock of np, of token um[k] (ppt pieces
// per token), with largest magnitude mag(k) (0 for a slot past np).  When
// ppt is a multiple of 64 every slot of a wave lies inside one token, and a
// thread's tokens do not decrease with k: one wave reduction per slot and a
// running maximum over the slots.  Otherwise each token is selected from
// every slot and reduced.  A maximum is exact in any order, so both give the
// same values.
template <int M, int P, typename Red, typename Mag>
__device__ __forceinline__ void piece_maxima(Red& red, const int (&um)[P], int np, int ppt,
                                             Mag mag) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (ppt % kWave == 0) {
        if (lane < M) red.am[lane][wave] = 0.f;
        const int w0 = tid - lane;
        float cur = 0.f;
        int cu = -1;
#pragma unroll
        for (int k = 0; k < P; ++k) {
            if (w0 + k * kMBlock >= np) break;  // (wave-uniform: no piece of this wave)
            const float r = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_max_nonneg(mag(k))),
                                                 kWave - 1));
            const int u = __builtin_amdgcn_readfirstlane(um[k]);
            if (u != cu) {
                if (cu >= 0 && lane == 0) red.am[cu][wave] = cur;
                cu = u;
                cur = r;
            } else {
                cur = fmaxf(cur, r);
            }
        }
        if (cu >= 0 && lane == 0) red.am[cu][wave] = cur;
    } else {
        float am[M];
#pragma unroll
        for (int m = 0; m < M; ++m) am[m] = 0.f;
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const float t = mag(k);
#pragma unroll
            for (int m = 0; m < M; ++m) am[m] = fmaxf(am[m], um[k] == m ? t : 0.f);
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float t = wave_max_nonneg(am[m]);  // am >= 0: largest |x|
            if (lane == kWave - 1) red.am[m][wave] = t;
        }
    }
}

// The activation pieces of one thread (8 consecutive elements each) and
// their tokens, loaded by mstage_issue before the first weight loads: loads
// complete in issue order, so activations loaded after the weights would
// wait for the weights' HBM latency before the staging could start.
template <int P>
struct MStageXT {
    float v[P][8];
    int um[P];
};
using MStageX = MStageXT<kMPieces>;

template <int M>
__device__ __forceinline__ void mstage_issue(const GemvParams& p, MStageX& sx) {
    const int tid = threadIdx.x;
    const int ppt = p.K >> 3;  // pieces per token
    const int np = M * ppt;
    // unconditional loads of clamped pieces keep the load-counter waits exact
#pragma unroll
    for (int k = 0; k < kMPieces; ++k) {
        const int pc = min(tid + k * kMBlock, np - 1);
        int m = 0;
#pragma unroll
        for (int mm = 1; mm < M; ++mm) m += pc >= mm * ppt;
        sx.um[k] = m;
        const float4* src = (const float4*)(p.x + (long long)m * p.K + 8 * (pc - m * ppt));
        const float4 a = src[0], b = src[1];
        sx.v[k][0] = a.x; sx.v[k][1] = a.y; sx.v[k][2] = a.z; sx.v[k][3] = a.w;
        sx.v[k][4] = b.x; sx.v[k][5] = b.y; sx.v[k][6] = b.z; sx.v[k][7] = b.w;
    }
}

template <int FMT, int M, int MODE, typename Red>
__device__ __forceinline__ void mstage(const GemvParams& p, char* lds, const MLayout& ly,
                                       Red& red, MStageX& sx) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ppt = p.K >> 3;  // pieces per token
    const int np = M * ppt;
    const int kp = mpadk(p.K);  // staged columns
    float (&v)[kMPieces][8] = sx.v;
    const int (&um)[kMPieces] = sx.um;
    auto valid = [&](int k) { return tid + k * kMBlock < np; };

    // RMSNorm: r_m = 1 / sqrt(sum(x^2) / K + eps), xhat = (x * r_m) * gamma,
    // the sum of squares in fp64 (exact squares, no overflow for finite x)
    if constexpr (MODE == kModeNorm) {
        double ss[M];
#pragma unroll
        for (int m = 0; m < M; ++m) ss[m] = 0.0;
#pragma unroll
        for (int k = 0; k < kMPieces; ++k) {
            double t = 0.0;
#pragma unroll
            for (int e = 0; e < 8; ++e) t += (double)v[k][e] * (double)v[k][e];
            t = valid(k) ? t : 0.0;
#pragma unroll
            for (int m = 0; m < M; ++m) ss[m] += um[k] == m ? t : 0.0;
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const double t = wave_sum_f64(ss[m]);
            if (lane == kWave - 1) red.ss[m][wave] = t;
        }
        sync_lds();
        float rn[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            double t = 0.0;
            for (int w = 0; w < kMWaves; ++w) t += red.ss[m][w];
            const float ms = (float)(t / (double)p.K);
            rn[m] = 1.0f / sqrtf(ms + p.eps);
        }
#pragma unroll
        for (int k = 0; k < kMPieces; ++k) {
            const int pc = min(tid + k * kMBlock, np - 1);
            const float4* gs = (const float4*)(p.gamma + 8 * (pc - um[k] * ppt));
            const float4 ga = gs[0], gb = gs[1];
            const float g[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
            float r = rn[0];
#pragma unroll
            for (int m = 1; m < M; ++m) r = um[k] == m ? rn[m] : r;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[k][e] = (v[k][e] * r) * g[e];
        }
    }

    // e_m: the token's largest magnitude times 2^e_m lies in [2^14, 2^15)
    // (any finite magnitude: the scale is applied with ldexp, not a
    // constructed power of two)
    {
        piece_maxima<M, kMPieces>(red, um, np, ppt, [&](int k) {
            float t = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) t = fmaxf(t, fabsf(v[k][e]));
            return valid(k) ? t : 0.f;
        });
        sync_lds();
        if (tid < M) {
            float t = 0.f;
            for (int w = 0; w < kMWaves; ++w) t = fmaxf(t, red.am[tid][w]);
            ((int*)(lds + ly.exps))[tid] = xscale_exp(t, 14);
        }
        sync_lds();
    }
    const int* ex = (const int*)(lds + ly.exps);

    // fragments (hi/lo f16 of x 2^e, high-nibble pieces 2^-4 more) and sums
#pragma unroll
    for (int k = 0; k < kMPieces; ++k) {
        const int pc = min(tid + k * kMBlock, np - 1);
        const int m = um[k];
        const int pp = pc - m * ppt;
        h8 hi, lo;
        float part;
        piece_frag(v[k], ex[m], piece_is_high<FMT>(pp), hi, lo, part);
        // the 4 pieces of one 32-element group are 4 consecutive threads
        part = dpp_add(part, 0);
        part = dpp_add(part, 1);
        if (valid(k)) {
            *(h8*)(lds + ly.frag + fslot(kp, 2 * m, pp) * 16) = hi;
            *(h8*)(lds + ly.frag + fslot(kp, 2 * m + 1, pp) * 16) = lo;
            if ((pp & 3) == 0) {
                const int g32 = pp >> 2;  // Q4_0 block / Q4_K sub-block index
                if constexpr (FMT != kFmtQ4K) {
                    ((float*)(lds + ly.aux))[g32 * sums_stride(M) + m] = part;
                } else {
                    // Dmin A operand: group c = J/2 of super-block sb holds
                    // the sums of sub-blocks 2c (half 0) and 2c+1 (half 1),
                    // scaled by 2^-5 to stay inside the f16 range
                    const int sb = g32 >> 3, J = g32 & 7;
                    const float xs = part * 0.03125f;
                    const _Float16 h = (_Float16)xs;
                    const _Float16 l = (_Float16)(xs - (float)h);
                    _Float16* a = (_Float16*)(lds + ly.aux);
                    const int base = ((sb * 4 + (J >> 1)) * 2 * M + 2 * m) * 2 + (J & 1);
                    a[base] = h;
                    a[base + 2] = l;
                }
            }
        }
    }
    // columns K .. kp of a partial last step: zero fragments and zero sums
    const int padp = (kp - p.K) >> 3;  // padded pieces per token
    for (int i = tid; i < M * padp; i += kMBlock) {
        const int m = i / padp;
        const int pp = ppt + (i - m * padp);
        const h8 z = (h8)((_Float16)0.0f);
        *(h8*)(lds + ly.frag + fslot(kp, 2 * m, pp) * 16) = z;
        *(h8*)(lds + ly.frag + fslot(kp, 2 * m + 1, pp) * 16) = z;
        if ((pp & 3) == 0) {
            const int g32 = pp >> 2;
            if constexpr (FMT != kFmtQ4K) {
                ((float*)(lds + ly.aux))[g32 * sums_stride(M) + m] = 0.f;
            } else {
                const int sb = g32 >> 3, J = g32 & 7;
                _Float16* a = (_Float16*)(lds + ly.aux);
                const int base = ((sb * 4 + (J >> 1)) * 2 * M + 2 * m) * 2 + (J & 1);
                a[base] = (_Float16)0.0f;
                a[base + 2] = (_Float16)0.0f;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// K-sliced staging (calls whose activations do not fit in LDS at once).
// Wave position sl of a tile group owns the steps [sl S / KS, (sl + 1) S / KS)
// of a row, as in a call staged whole.  The positions form npg groups
// staged in turn; for each group, nsl slices hold the s-th of nsl equal
// sub-ranges of each of its positions' ranges, each position's in a region
// of msl steps (local step region * msl + j).  A wave therefore meets its
// own steps in the same order as in a call staged whole (the same
// rounding, bit for bit); it idles in the other groups' slices (npg > 1
// only where even one step per position does not fit in LDS).
// ---------------------------------------------------------------------------
struct MSlice {
    int S, KS, npg, nsl, msl;
    __device__ __forceinline__ int nslices() const { return npg * nsl; }
    // sub-range [a, b) of wave position sl in slice `slice` and its region
    // (empty when sl is not in the slice's group)
    __device__ __forceinline__ void range(int sl, int slice, int& a, int& b, int& reg) const {
        const int g = slice / nsl, s = slice - g * nsl;
        const int p0 = g * KS / npg, p1 = (g + 1) * KS / npg;
        a = b = reg = 0;
        if (sl < p0 || sl >= p1) return;
        reg = sl - p0;
        const int s0 = sl * S / KS, L = (sl + 1) * S / KS - s0;
        a = s0 + s * L / nsl;
        b = s0 + (s + 1) * L / nsl;
    }
    // the wave position of region `reg` in slice `slice` (-1: none)
    __device__ __forceinline__ int position(int reg, int slice) const {
        const int g = slice / nsl;
        const int p = g * KS / npg + reg;
        return p < (g + 1) * KS / npg ? p : -1;
    }
};
// Regions (positions) per group: the staged steps of a slice are regions * msl.
__host__ __device__ inline int mslice_regions(int KS, int npg) { return (KS + npg - 1) / npg; }

// Per-token factors from whole rows read from global memory: the RMSNorm
// factor r_m (fp64 sum of squares) and the exponent e_m with
// max_k |x_hat[m,k]| 2^e_m in [2^14, 2^15), into the exps region.
// A batch of kMBatch activation pieces (8 floats each) per thread: pieces
// i0 + j * kMBlock of the M token rows of x, columns c0 + 8 * (piece within
// the row), loaded together so that the thread waits once per batch, not once
// per piece (a wait for a load issued after the weight loads also waits for
// those).  Pieces past np load the last piece and have ok = false.  w walks
// the (token, piece) positions (rows of ppr pieces) without divisions.
constexpr int kMBatch = 4;
struct MPieces {
    float v[kMBatch][8];
    int m[kMBatch];  // token (the last for pieces past np)
    int c[kMBatch];  // piece within the token's row
    bool ok[kMBatch];
};
template <int M>
__device__ __forceinline__ void mpiece_batch(const GemvParams& p, int i0, int np, int ppr, int c0,
                                             ChunkWalk& w, MPieces& b) {
#pragma unroll
    for (int j = 0; j < kMBatch; ++j) {
        b.ok[j] = i0 + j * kMBlock < np;
        b.m[j] = b.ok[j] ? w.m : M - 1;
        b.c[j] = b.ok[j] ? w.c : ppr - 1;
        const float4* src =
            (const float4*)(p.x + (long long)b.m[j] * p.K + c0 + 8 * b.c[j]);
        const float4 x0 = src[0], x1 = src[1];
        b.v[j][0] = x0.x; b.v[j][1] = x0.y; b.v[j][2] = x0.z; b.v[j][3] = x0.w;
        b.v[j][4] = x1.x; b.v[j][5] = x1.y; b.v[j][6] = x1.z; b.v[j][7] = x1.w;
        w.next();
    }
}
// gamma for the pieces of a batch
__device__ __forceinline__ void mpiece_gamma(const GemvParams& p, const MPieces& b, int c0,
                                             float (&g)[kMBatch][8]) {
#pragma unroll
    for (int j = 0; j < kMBatch; ++j) {
        const float4* gs = (const float4*)(p.gamma + c0 + 8 * b.c[j]);
        const float4 ga = gs[0], gb = gs[1];
        g[j][0] = ga.x; g[j][1] = ga.y; g[j][2] = ga.z; g[j][3] = ga.w;
        g[j][4] = gb.x; g[j][5] = gb.y; g[j][6] = gb.z; g[j][7] = gb.w;
    }
}

template <int M, int MODE, typename Red>
__device__ __forceinline__ void mstage_factors(const GemvParams& p, char* lds, const MLayout& ly,
                                               Red& red) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ppt = p.K >> 3;  // pieces of 8 per token
    const int np = M * ppt;
    int* ex = (int*)(lds + ly.exps);
    float* rn = (float*)(lds + ly.exps) + 16;
    if constexpr (MODE == kModeNorm) {
        double ss[M];
#pragma unroll
        for (int m = 0; m < M; ++m) ss[m] = 0.0;
        ChunkWalk w(tid, kMBlock, ppt);
        for (int i0 = tid; i0 < np; i0 += kMBatch * kMBlock) {
            MPieces b;
            mpiece_batch<M>(p, i0, np, ppt, 0, w, b);
#pragma unroll
            for (int j = 0; j < kMBatch; ++j) {
                double t = 0.0;
#pragma unroll
                for (int e = 0; e < 8; ++e) t += (double)b.v[j][e] * (double)b.v[j][e];
                t = b.ok[j] ? t : 0.0;
#pragma unroll
                for (int mm = 0; mm < M; ++mm) ss[mm] += b.m[j] == mm ? t : 0.0;
            }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const double t = wave_sum_f64(ss[m]);
            if (lane == kWave - 1) red.ss[m][wave] = t;
        }
        sync_lds();
        if (tid < M) {
            double t = 0.0;
            for (int w = 0; w < kMWaves; ++w) t += red.ss[tid][w];
            const float ms = (float)(t / (double)p.K);
            rn[tid] = 1.0f / sqrtf(ms + p.eps);
        }
        sync_lds();
    }
    float am[M];
#pragma unroll
    for (int m = 0; m < M; ++m) am[m] = 0.f;
    ChunkWalk w(tid, kMBlock, ppt);
    for (int i0 = tid; i0 < np; i0 += kMBatch * kMBlock) {
        MPieces b;
        mpiece_batch<M>(p, i0, np, ppt, 0, w, b);
        float g[kMBatch][8];
        if constexpr (MODE == kModeNorm) mpiece_gamma(p, b, 0, g);
#pragma unroll
        for (int j = 0; j < kMBatch; ++j) {
            float t = 0.f;
            if constexpr (MODE == kModeNorm) {
                const float r = rn[b.m[j]];
#pragma unroll
                for (int e = 0; e < 8; ++e) t = fmaxf(t, fabsf((b.v[j][e] * r) * g[j][e]));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) t = fmaxf(t, fabsf(b.v[j][e]));
            }
            t = b.ok[j] ? t : 0.f;
#pragma unroll
            for (int mm = 0; mm < M; ++mm) am[mm] = fmaxf(am[mm], b.m[j] == mm ? t : 0.f);
        }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float t = wave_max_nonneg(am[m]);
        if (lane == kWave - 1) red.am[m][wave] = t;
    }
    sync_lds();
    if (tid < M) {
        float t = 0.f;
        for (int w = 0; w < kMWaves; ++w) t = fmaxf(t, red.am[tid][w]);
        ex[tid] = xscale_exp(t, 14);
    }
    sync_lds();
}

// Stage slice s: the fragments (and sums) of every staged step of every
// token, with the factors of mstage_factors; columns past K are zero.
template <int FMT, int M, int MODE>
__device__ __forceinline__ void mstage_slice(const GemvParams& p, char* lds, const MLayout& ly,
                                             const MSlice& sc, int s) {
    const int tid = threadIdx.x;
    const int kst = mslice_regions(sc.KS, sc.npg) * sc.msl * 256;  // staged columns
    const int ppl = kst >> 3;              // staged pieces per token
    const int np = M * ppl;
    const int* ex = (const int*)(lds + ly.exps);
    const float* rn = (const float*)(lds + ly.exps) + 16;
    // (a 32-element group's 4 pieces are 4 consecutive threads, all active
    // together: ppl and the block size are multiples of 4).  Pieces are
    // loaded kMBatch at a time, unconditionally (a piece that is not staged,
    // or lies past K, loads the row's first piece and is staged as zeros).
    ChunkWalk w(tid, kMBlock, ppl);
    for (int i0 = tid; i0 < np; i0 += kMBatch * kMBlock) {
        float v[kMBatch][8], g[kMBatch][8];
        int mj[kMBatch], plj[kMBatch];
        bool stj[kMBatch], ldj[kMBatch];
#pragma unroll
        for (int j = 0; j < kMBatch; ++j) {
            const bool ok = i0 + j * kMBlock < np;
            const int m = ok ? w.m : M - 1;
            const int pl = ok ? w.c : ppl - 1;
            w.next();
            const int ls = pl >> 5, pin = pl & 31;
            const int rg = ls / sc.msl, jj = ls - rg * sc.msl;
            const int sl = sc.position(rg, s);
            int a = 0, b = 0, reg = 0;
            if (sl >= 0) sc.range(sl, s, a, b, reg);
            const bool staged = ok && jj < b - a;  // (a region's unused tail is never read)
            const int col = (a + jj) * 256 + pin * 8;
            const bool ld = staged && col < p.K;
            const int colc = ld ? col : 0;
            const float4* src = (const float4*)(p.x + (long long)m * p.K + colc);
            const float4 x0 = src[0], x1 = src[1];
            v[j][0] = x0.x; v[j][1] = x0.y; v[j][2] = x0.z; v[j][3] = x0.w;
            v[j][4] = x1.x; v[j][5] = x1.y; v[j][6] = x1.z; v[j][7] = x1.w;
            if constexpr (MODE == kModeNorm) {
                const float4* gs = (const float4*)(p.gamma + colc);
                const float4 ga = gs[0], gb = gs[1];
                g[j][0] = ga.x; g[j][1] = ga.y; g[j][2] = ga.z; g[j][3] = ga.w;
                g[j][4] = gb.x; g[j][5] = gb.y; g[j][6] = gb.z; g[j][7] = gb.w;
            }
            mj[j] = m;
            plj[j] = pl;
            stj[j] = staged;
            ldj[j] = ld;
        }
#pragma unroll
        for (int j = 0; j < kMBatch; ++j) {
            const int m = mj[j], pl = plj[j], pin = pl & 31;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[j][e] = ldj[j] ? v[j][e] : 0.f;
            if constexpr (MODE == kModeNorm) {
                const float r = rn[m];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[j][e] = (v[j][e] * r) * g[j][e];
            }
            h8 hi, lo;
            float part;
            piece_frag(v[j], ex[m], piece_is_high<FMT>(pin), hi, lo, part);
            part = dpp_add(part, 0);
            part = dpp_add(part, 1);
            if (stj[j]) {
                *(h8*)(lds + ly.frag + fslot(kst, 2 * m, pl) * 16) = hi;
                *(h8*)(lds + ly.frag + fslot(kst, 2 * m + 1, pl) * 16) = lo;
                if ((pl & 3) == 0) {
                    const int g32 = pl >> 2;  // local block / sub-block index
                    if constexpr (FMT != kFmtQ4K) {
                        ((float*)(lds + ly.aux))[g32 * sums_stride(M) + m] = part;
                    } else {
                        const int sb = g32 >> 3, J = g32 & 7;
                        const float xs = part * 0.03125f;
                        const _Float16 h = (_Float16)xs;
                        const _Float16 l = (_Float16)(xs - (float)h);
                        _Float16* ap = (_Float16*)(lds + ly.aux);
                        const int base = ((sb * 4 + (J >> 1)) * 2 * M + 2 * m) * 2 + (J & 1);
                        ap[base] = h;
                        ap[base + 2] = l;
                    }
                }
            }
        }
    }
}

// Split-K: the exponents of one K part, from its columns [c0, c1) only
// (max_k |x[m,k]| 2^e_m in [2^14, 2^15) over the part; a part whose
// columns are all zero gets kNoExp, which the merge ignores).
constexpr int kNoExp = 1 << 20;
template <int M, typename Red>
__device__ __forceinline__ void mstage_part_factors(const GemvParams& p, char* lds,
                                                    const MLayout& ly, Red& red, int c0, int c1) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ppr = (min(c1, p.K) - c0) >> 3;  // pieces of 8 per token in the part
    const int np = M * ppr;
    int* ex = (int*)(lds + ly.exps);
    float am[M];
#pragma unroll
    for (int m = 0; m < M; ++m) am[m] = 0.f;
    ChunkWalk w(tid, kMBlock, ppr);
    for (int i0 = tid; i0 < np; i0 += kMBatch * kMBlock) {
        MPieces b;
        mpiece_batch<M>(p, i0, np, ppr, c0, w, b);
#pragma unroll
        for (int j = 0; j < kMBatch; ++j) {
            float t = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) t = fmaxf(t, fabsf(b.v[j][e]));
            t = b.ok[j] ? t : 0.f;
#pragma unroll
            for (int mm = 0; mm < M; ++mm) am[mm] = fmaxf(am[mm], b.m[j] == mm ? t : 0.f);
        }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float t = wave_max_nonneg(am[m]);
        if (lane == kWave - 1) red.am[m][wave] = t;
    }
    sync_lds();
    if (tid < M) {
        float t = 0.f;
        for (int w = 0; w < kMWaves; ++w) t = fmaxf(t, red.am[tid][w]);
        ex[tid] = t > 0.f ? xscale_exp(t, 14) : kNoExp;
    }
    sync_lds();
}

// Split-K staging in one pass, for a part of at most kSplitKOneSteps steps:
// its M * ppt <= 128 M pieces fit in P = ceil(M / 4) pieces per thread,
// a count fixed at compile time so that the loads stay unconditional (a
// load under a branch is merged into its register by a copy, which waits
// for every load in flight).  Piece pp of token m covers columns c0 + 8 pp
// .. of the row; pieces past K (in the row's partial last step) are loaded
// clamped and staged as zeros.  The loads go out before the weight loads
// (mstage_issue's reason).
constexpr int kSplitKOneSteps = 4;
template <int M>
__host__ __device__ constexpr int part_pieces() { return (M + 3) / 4; }

template <int M, int P>
__device__ __forceinline__ void mstage_part_issue(const GemvParams& p, int c0, int ppt,
                                                  MStageXT<P>& sx) {
    const int tid = threadIdx.x;
    const int np = M * ppt;
#pragma unroll
    for (int k = 0; k < P; ++k) {
        const int pc = min(tid + k * kMBlock, np - 1);
        int m = 0;
#pragma unroll
        for (int mm = 1; mm < M; ++mm) m += pc >= mm * ppt;
        sx.um[k] = m;
        const int col = min(c0 + 8 * (pc - m * ppt), p.K - 8);
        const float4* src = (const float4*)(p.x + (long long)m * p.K + col);
        const float4 a = src[0], b = src[1];
        sx.v[k][0] = a.x; sx.v[k][1] = a.y; sx.v[k][2] = a.z; sx.v[k][3] = a.w;
        sx.v[k][4] = b.x; sx.v[k][5] = b.y; sx.v[k][6] = b.z; sx.v[k][7] = b.w;
    }
}

// The part's exponents (kNoExp for a token with no nonzero element in the
// part) and its fragments and sums, in the layout of mstage_slice (region
// width kst columns, local piece and group indices).
template <int FMT, int M, int P, typename Red>
__device__ __forceinline__ void mstage_part_finish(const GemvParams& p, char* lds,
                                                   const MLayout& ly, Red& red, MStageXT<P>& sx,
                                                   int c0, int ppt, int kst) {
    const int tid = threadIdx.x;
    const int np = M * ppt;
    float (&v)[P][8] = sx.v;
    const int (&um)[P] = sx.um;
    auto valid = [&](int k) { return tid + k * kMBlock < np; };
    int* ex = (int*)(lds + ly.exps);
#pragma unroll
    for (int k = 0; k < P; ++k) {
        const int pc = min(tid + k * kMBlock, np - 1);
        if (c0 + 8 * (pc - um[k] * ppt) >= p.K) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[k][e] = 0.f;
        }
    }
    {
        piece_maxima<M, P>(red, um, np, ppt, [&](int k) {
            float t = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) t = fmaxf(t, fabsf(v[k][e]));
            return valid(k) ? t : 0.f;
        });
        sync_lds();
        if (tid < M) {
            float t = 0.f;
            for (int w = 0; w < kMWaves; ++w) t = fmaxf(t, red.am[tid][w]);
            ex[tid] = t > 0.f ? xscale_exp(t, 14) : kNoExp;
        }
        sync_lds();
    }
#pragma unroll
    for (int k = 0; k < P; ++k) {
        const int pc = min(tid + k * kMBlock, np - 1);
        const int m = um[k];
        const int pp = pc - m * ppt;
        h8 hi, lo;
        float part;
        piece_frag(v[k], ex[m], piece_is_high<FMT>(pp), hi, lo, part);
        // the 4 pieces of one 32-element group are 4 consecutive threads
        // (ppt is a multiple of 32)
        part = dpp_add(part, 0);
        part = dpp_add(part, 1);
        if (valid(k)) {
            *(h8*)(lds + ly.frag + fslot(kst, 2 * m, pp) * 16) = hi;
            *(h8*)(lds + ly.frag + fslot(kst, 2 * m + 1, pp) * 16) = lo;
            if ((pp & 3) == 0) {
                const int g32 = pp >> 2;
                if constexpr (FMT != kFmtQ4K) {
                    ((float*)(lds + ly.aux))[g32 * sums_stride(M) + m] = part;
                } else {
                    const int sb = g32 >> 3, J = g32 & 7;
                    const float xs = part * 0.03125f;
                    const _Float16 h = (_Float16)xs;
                    const _Float16 l = (_Float16)(xs - (float)h);
                    _Float16* a = (_Float16*)(lds + ly.aux);
                    const int base = ((sb * 4 + (J >> 1)) * 2 * M + 2 * m) * 2 + (J & 1);
                    a[base] = h;
                    a[base + 2] = l;
                }
            }
        }
    }
}

// The merge of split-K partial sums: y[m, row] = sum over parts q (in
// order) of part[q][m][row] brought to the common scale 2^(24 - e*), e* the
// smallest exponent of the token's parts (the part of largest magnitude);
// parts with no nonzero column are skipped.
static __global__ __launch_bounds__(256) void splitk_reduce_kernel(
    float* __restrict__ y, const float* __restrict__ part, const int* __restrict__ pexp, int kp,
    int M, int N) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long long)M * N) return;
    const int m = (int)(i / N), row = (int)(i - (long long)m * N);
    const int* pe = pexp + m;
    const float* pp = part + (long long)m * N + row;
    const long long qs = (long long)M * N;  // part stride
    // parts in chunks of 8 whose loads all go out before their use; with
    // at most 8 parts, exponents and partials in one round trip
    constexpr int U = 8;
    if (kp <= U) {
        int e[U];
        float v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const bool ok = j < kp;
            e[j] = ok ? pe[j * M] : kNoExp;
            v[j] = ok ? pp[j * qs] : 0.f;
        }
        int emin = kNoExp;
#pragma unroll
        for (int j = 0; j < U; ++j) emin = min(emin, e[j]);
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < U; ++j)
            if (e[j] != kNoExp) sum += __builtin_ldexpf(v[j], emin - e[j]);
        y[i] = emin == kNoExp ? 0.f : __builtin_ldexpf(sum, 24 - emin);
        return;
    }
    int emin = kNoExp;
    for (int q0 = 0; q0 < kp; q0 += U) {
        int e[U];
#pragma unroll
        for (int j = 0; j < U; ++j) e[j] = q0 + j < kp ? pe[(q0 + j) * M] : kNoExp;
#pragma unroll
        for (int j = 0; j < U; ++j) emin = min(emin, e[j]);
    }
    float sum = 0.f;
    for (int q0 = 0; q0 < kp; q0 += U) {
        int e[U];
        float v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const bool ok = q0 + j < kp;
            e[j] = ok ? pe[(q0 + j) * M] : kNoExp;
            v[j] = ok ? pp[(q0 + j) * qs] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < U; ++j)
            if (e[j] != kNoExp) sum += __builtin_ldexpf(v[j], emin - e[j]);
    }
    y[i] = emin == kNoExp ? 0.f : __builtin_ldexpf(sum, 24 - emin);
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
// Expert call: the in-kernel dedupe (per unique expert, the (token, slot)
// pairs that chose it; a token may list one expert in several slots).
struct MfmaMoe {
    MoeShared d;
};
struct MfmaNoMoe {};

// Split-K: the tile group g and K part q of workgroup b of T.  Workgroups
// are dispatched to the 8 XCDs in turn (b % 8), each with its own L2; the
// roles are dealt so that XCD x takes a contiguous run of (group, part)
// pairs, i.e. the consecutive parts of a group mostly share one L2 (the
// 144-byte blocks of a row do not end on cache lines, so two parts that
// meet inside a line would each fetch it).  A bijection for any T: XCD x
// holds T / 8 workgroups, one more when x < T % 8.
constexpr int kXcds = 8;
__host__ __device__ inline void splitk_role(int b, int T, int kp, int& g, int& q) {
    const int per = T / kXcds, rem = T - per * kXcds;
    const int x = b % kXcds, i = b / kXcds;
    const int L = x * per + (x < rem ? x : rem) + i;
    g = L / kp;
    q = L - g * kp;
}

// Staging of the batched kernel: whole rows, K slices, or (split-K) one K
// part per workgroup, whose partial sums splitk_reduce_kernel merges.
constexpr int kStgWhole = 0;
constexpr int kStgSliced = 1;
constexpr int kStgSplitK = 2;

template <int FMT, int M, int NMAT, int MODE, bool PURE, int PD, int STG>
__global__ __launch_bounds__(kMBlock) void mfma_gemv_kernel(const GemvParams p) {
    constexpr bool SLICED = STG == kStgSliced;
    constexpr bool SPLITK = STG == kStgSplitK;
    static_assert(M >= 2 && M <= kMaxM, "batched kernel");
    static_assert(!mode_moe(MODE) || (M <= 8 && STG == kStgWhole), "expert call: M <= 8, whole rows");
    static_assert(!SPLITK || (MODE == kModeDense && NMAT == 1 && !PURE),
                  "split-K: single-matrix GEMV");
    constexpr int NT = mtiles(M);  // A tiles of 8 tokens
    using St = MStep<FMT>;
    extern __shared__ float4 smem4[];
    char* lds = (char*)smem4;
    __shared__ StageRedT<(M > 8 ? 16 : 8)> red;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = msteps(p.K);
    // Q4_0: blocks of the row (a partial last step has fewer than 8), and
    // the largest byte offset of a 16-byte chunk inside the last step
    const int nblk = p.K >> 5;
    const uint32_t last_end = (uint32_t)(18 * (nblk - 8 * (S - 1)));  // bytes of the row in it
    const uint32_t last_col = last_end - 16;
    // Q4_K: elements of the row in its last super-block
    const int klast = p.K - 256 * (S - 1);
    // waves per tile (1, 2, 4 or 8), at most S so that every wave has steps
    // (a wave without steps would skip the end-of-round reduction)
    int KS = p.ks;
    while (KS > S) KS >>= 1;
    // staged steps: the whole row, (K-sliced) KS regions of msl steps, or
    // (split-K, KS = 1) one part of msl steps
    const int staged_steps = SLICED ? mslice_regions(KS, p.npg) * p.msl : (SPLITK ? p.msl : S);
    const MLayout ly = mlayout_steps(FMT, M, staged_steps, PURE);
    const int kst = staged_steps * 256;  // staged columns
    const int TG = kMWaves / KS;      // tiles per workgroup and round
    const int grp = wave / KS, sl = wave - grp * KS;
    const int jrow = lane & 15;  // tile row of this lane's B column and D values
    const int c = lane >> 4;     // k group
    const int st0 = sl * S / KS, st1 = (sl + 1) * S / KS;  // st1 > st0 as KS <= S
    constexpr bool kMoe = mode_moe(MODE);
    // SiLU-gated gate+up: a tile is 8 rows of the gate matrix (columns
    // 0-7) and the same 8 rows of the up matrix (columns 8-15), so that a
    // row's two totals meet in one 16-lane row of the wave
    constexpr bool kPair = MODE == kModeSilu || MODE == kModeNormSilu;
    static_assert(!mode_silu(MODE) || (kPair && NMAT == 2 && FMT == kFmtQ4K),
                  "matrix-core SiLU epilogue: dense Q4_K gate+up only");
    constexpr int kTileShift = kPair ? 3 : 4;
    const int tpm = (p.N + (1 << kTileShift) - 1) >> kTileShift;  // tiles per matrix (per
                                                                   // expert for the expert call)
    __shared__ std::conditional_t<kMoe, MfmaMoe, MfmaNoMoe> moe;
    int nu = 1;  // matrices of NMAT: 1, or the unique selected experts
    if constexpr (kMoe) {
        moe_dedupe<M>(p, moe.d, moe_load_id<M>(p));
        __syncthreads();
        // outputs of pairs with an invalid id: NaN (or all-ones checksums)
        if (moe.d.invalid) {
            const int P = M * p.top_k;
            const long long total = (long long)P * p.N;
            for (long long i = (long long)blockIdx.x * kMBlock + threadIdx.x; i < total;
                 i += (long long)gridDim.x * kMBlock) {
                const int pr = (int)(i / p.N);
                if ((moe.d.invalid >> pr) & 1ull) {
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
        __syncthreads();
        nu = __builtin_amdgcn_readfirstlane(moe.d.nu);
    }
    const int per_mat = nu * tpm;  // tiles per matrix
    const int ntiles = (kPair ? 1 : NMAT) * per_mat;
    if (ntiles == 0) return;  // (expert call with no valid id: all waves)
    const int per_round = gridDim.x * TG;
    const int nrounds = (ntiles + per_round - 1) / per_round;
    const uint32_t rb = (uint32_t)p.row_bytes;
    // tile t: matrix mt, unique expert u (0 unless expert call), first row row0
    struct Tile {
        int mt, u, row0;
        long long ebase;  // first row of the expert
    };
    auto tile_at = [&](int t) {
        Tile T;
        T.mt = (NMAT == 2 && !kPair) ? (t >= per_mat ? 1 : 0) : 0;
        const int rem = t - T.mt * per_mat;
        T.u = kMoe ? rem / tpm : 0;
        T.row0 = (rem - T.u * tpm) << kTileShift;
        T.ebase = 0;
        if constexpr (kMoe)
            T.ebase = (long long)__builtin_amdgcn_readfirstlane(moe.d.uexp[T.u]) * p.N;
        return T;
    };

    // weight registers of one step (12 dwords in both formats)
    struct WR {
        uint32_t v[12];
    };
    // Q4_0: this lane's three chunks of a tile-step (row, byte offset)
    int q0chunk[3], q0row[3];
    uint32_t q0col[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        q0chunk[k] = min(lane + kWave * k, kQ40Chunks - 1);
        q0row[k] = q0chunk[k] / 9;
        q0col[k] = (uint32_t)(q0chunk[k] - 9 * q0row[k]) * 16u;
    }
    // Loads past the wave's last step, and those of a group without a tile
    // in the last round, are not consumed: they go to the group's own
    // last-round tile with every lane on one address (spread over the chip,
    // one cache line per instruction) and stay unconditional.
    auto load = [&](int r, int st, WR& w) {
        const int rr = min(r, nrounds - 1);
        // (split-K: workgroup b serves tile group b / kp, one tile per wave)
        int sg = 0, sq = 0;
        if constexpr (SPLITK) splitk_role((int)blockIdx.x, (int)gridDim.x, p.kp, sg, sq);
        const int traw = SPLITK ? sg * TG + grp
                                : (rr * (int)gridDim.x + (int)blockIdx.x) * TG + grp;
        const bool idle = SPLITK ? (r > 0 || traw >= ntiles) : (r >= nrounds || traw >= ntiles);
        const Tile T = tile_at(min(traw, ntiles - 1));
        const int row0 = T.row0;
        const bool up = kPair ? jrow >= 8 : T.mt != 0;
        const uint8_t* base = (up ? p.w1 : p.w0) + (T.ebase + row0) * p.row_bytes;
        const uint32_t lr = (uint32_t)min(kPair ? (jrow & 7) : jrow, p.N - 1 - row0);
        const uint32_t off = idle ? 0u : lr * rb + (uint32_t)st * St::kBytes;
        if constexpr (FMT == kFmtQ4K) {
            // header, then 16 bytes of each 64-byte half of the nibbles:
            // lane group c takes bytes 16c .. 16c+15 of half h (chunk 2h +
            // c/2, bytes 16(c&1) ..)
            const uint32_t co = idle ? 0u : 16u * (uint32_t)c;
            const u32x4 h = ldg16(base + off);
            const u32x4 q0 = ldg16(base + off + co + 16);
            const u32x4 q1 = ldg16(base + off + co + 80);
            w.v[0] = h.x; w.v[1] = h.y; w.v[2] = h.z; w.v[3] = h.w;
            w.v[4] = q0.x; w.v[5] = q0.y; w.v[6] = q0.z; w.v[7] = q0.w;
            w.v[8] = q1.x; w.v[9] = q1.y; w.v[10] = q1.z; w.v[11] = q1.w;
        } else if constexpr (FMT == kFmtQ4_0S) {
            // split arrays: chunks lane and lane + 64 of the tile-step's 16
            // rows x 8 nibble blocks (row ch / 8, block ch % 8; blocks past
            // the row's end re-read its last block, whose scale is masked),
            // and the same rows' 8 f16 scales each, two per lane
            const uint32_t nb = (uint32_t)nblk;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int ch = lane + kWave * k;
                const uint32_t ro = (uint32_t)min(ch >> 3, p.N - 1 - row0);
                const uint32_t gb = (uint32_t)min(st * 8 + (ch & 7), nblk - 1);
                const uint32_t qo = idle ? 0u : ro * rb + 16u * gb;
                const u32x4 v = ldg16(base + qo);
                w.v[4 * k] = v.x; w.v[4 * k + 1] = v.y; w.v[4 * k + 2] = v.z; w.v[4 * k + 3] = v.w;
                const uint8_t* sb = p.sc + (T.ebase + row0) * (long long)(2u * nb);
                const uint32_t so2 = idle ? 0u : ro * 2u * nb + 2u * gb;
                w.v[8 + k] = *(const uint16_t*)__builtin_assume_aligned(sb + so2, 2);
            }
        } else {
            // chunks lane, lane + 64, lane + 128 (clamped) of the tile-step:
            // chunk ch is bytes 16 (ch % 9) .. of the step's 144 bytes of
            // tile row ch / 9
            // (in a partial last step, a chunk that would cross the row's
            // end is loaded from the row's last 16 bytes instead, and
            // gather() moves its words back into place; chunks past the end
            // load the same bytes, and their blocks are masked)
            const uint32_t so = (uint32_t)st * St::kBytes;
            const bool part = st == S - 1;
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const uint32_t ro = (uint32_t)min(q0row[k], p.N - 1 - row0) * rb;
                const uint32_t col = part ? min(q0col[k], last_col) : q0col[k];
                const uint32_t o = idle ? 0u : ro + so + col;
                const u32x4 v = ldg16(base + o);
                w.v[4 * k] = v.x; w.v[4 * k + 1] = v.y; w.v[4 * k + 2] = v.z; w.v[4 * k + 3] = v.w;
            }
        }
    };

    // A fragment of piece pp for this lane in tile t (rows i >= 2M repeat
    // row 2M-1)
    int i_lane[NT];
    const char* arow[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        i_lane[t] = min(16 * t + jrow, 2 * M - 1);
        arow[t] = lds + ly.frag + fslot(kst, i_lane[t], 0) * 16;
    }
    auto afrag = [&](int t, int pp) { return *(const h8*)(arow[t] + pp * 16); };

    // Q4_0: write the tile-step to this wave's LDS copy and read back, per
    // block pair k (36 bytes, words 0..8 at word 9k of row jrow): words
    // 2h..2h+2 (the lane's bytes of block A), 5+2h, 6+2h (block B) and word
    // 4 (h = 0) or word 0 (h = 1), the scale the others lack; h = c & 1.
    // LDS operations of one wave are performed in order, so the reads see
    // the writes, and the next step's writes follow this step's reads.
    struct WQ {
        uint32_t v[4][6];
    };
    char* wb = lds + ly.wbuf + wave * kQ40WaveBytes;
    auto gather = [&](const WR& w, int st, WQ& q) {
        if constexpr (FMT == kFmtQ4_0S) {
            // split arrays: the copy holds the 16 rows' nibble blocks (row r,
            // block b at 16 (8r + b)), then their scales (at 2048 + 2 (8r + b));
            // per block pair k this lane reads its 8 bytes of blocks 2k and
            // 2k + 1 (bytes 8 (c & 1) ..) and the pair's two scales
            (void)st;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int ch = lane + kWave * k;
                *(u32x4*)(wb + ch * 16) =
                    u32x4{w.v[4 * k], w.v[4 * k + 1], w.v[4 * k + 2], w.v[4 * k + 3]};
                *(uint16_t*)(wb + 2048 + ch * 2) = (uint16_t)w.v[8 + k];
            }
            __asm__ volatile("" ::: "memory");
            const int hh = c & 1;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t* pa = (const uint32_t*)(wb + jrow * 128 + 32 * k + 8 * hh);
                q.v[k][0] = pa[0];
                q.v[k][1] = pa[1];
                q.v[k][2] = pa[4];
                q.v[k][3] = pa[5];
                q.v[k][4] = *(const uint32_t*)(wb + 2048 + jrow * 16 + 4 * k);
                q.v[k][5] = 0u;
            }
            __asm__ volatile("" ::: "memory");
            return;
        }
        const bool part = st == S - 1;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const uint32_t a0 = w.v[4 * k], a1 = w.v[4 * k + 1], a2 = w.v[4 * k + 2],
                           a3 = w.v[4 * k + 3];
            // a chunk loaded from the row's last 16 bytes (see load()):
            // word i of the chunk is word i + sh of what was loaded
            const int sh = part ? max(0, (int)(q0col[k] + 16u) - (int)last_end) >> 2 : 0;
            const uint32_t b0 = sh == 0 ? a0 : sh == 1 ? a1 : sh == 2 ? a2 : a3;
            const uint32_t b1 = sh == 0 ? a1 : sh == 1 ? a2 : a3;
            const uint32_t b2 = sh == 0 ? a2 : a3;
            *(u32x4*)(wb + q0chunk[k] * 16) = u32x4{b0, b1, b2, a3};
        }
        __asm__ volatile("" ::: "memory");
        const uint32_t* wd = (const uint32_t*)wb + jrow * 36;
        const int hh = c & 1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t* pa = wd + 9 * k + 2 * hh;
            q.v[k][0] = pa[0];
            q.v[k][1] = pa[1];
            q.v[k][2] = pa[2];
            q.v[k][3] = pa[5];
            q.v[k][4] = pa[6];
            q.v[k][5] = wd[9 * k + 4 - 4 * hh];
        }
        __asm__ volatile("" ::: "memory");
    };

    // step st of the row (for the masks of a partial last step), staged at
    // local step stl (its fragments and sums)
    auto compute = [&](const WR& w, int st, int stl, float2 (&y)[NT]) {
        if constexpr (FMT == kFmtQ4K) {
            // Lane group c holds, of half h (h = 0, 1), the 16 bytes
            // 16(c&1) .. of chunk g = 2h + c/2: low nibbles of sub-block
            // J = 2g, high nibbles of J = 2g + 1.  MFMA (h, n, s) takes the
            // nibbles n of bytes 8s .. 8s+7 (s = 0, 1): piece
            // p = 8g + 4n + 2(c&1) + s of the row.  The sub-block scale goes
            // into B: (q * 2^-24) * sc is the exact subnormal q*sc*2^-24
            // (q*sc <= 945), and for an in-place high nibble
            // (16q * 2^-24) * sc is exact too (its A piece carries 2^-4).
            const uint32_t h1 = w.v[1], h2 = w.v[2], h3 = w.v[3];
            const uint32_t qq = (uint32_t)(c >> 1);
            const uint32_t sc_lo = h1 & 0x3F3F3F3Fu;  // sub-blocks 0..3
            const uint32_t sc_hi = (h3 & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u);  // 4..7
            // scales of sub-blocks 2g, 2g + 1 for g = qq (half 0) and 2 + qq
            // (half 1), each as an f16 pair (sc, sc)
            uint32_t scp[2][2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const uint32_t sb = (hh ? sc_hi : sc_lo) >> (16u * qq);
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const float f = (float)((sb >> (8 * n)) & 0xFFu);
                    scp[hh][n] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f, f));
                }
            }
            typedef _Float16 h2v __attribute__((ext_vector_type(2)));
            auto pmul = [](uint32_t a, uint32_t b) {
                return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2v, a) *
                                                        __builtin_bit_cast(h2v, b));
            };
            f4 acc0[NT], acc1[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                acc0[t] = (f4)(0.f);
                acc1[t] = (f4)(0.f);
            }
            const int pbase = stl * 32 + 8 * (int)qq + 2 * (c & 1);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                for (int sidx = 0; sidx < 2; ++sidx) {
                    const uint32_t d0 = w.v[4 + 4 * hh + 2 * sidx], d1 = w.v[5 + 4 * hh + 2 * sidx];
                    const uint32_t d08 = d0 >> 8, d18 = d1 >> 8;
                    const u32x4m blo = {pmul(d0 & 0x000F000Fu, scp[hh][0]),
                                        pmul(d08 & 0x000F000Fu, scp[hh][0]),
                                        pmul(d1 & 0x000F000Fu, scp[hh][0]),
                                        pmul(d18 & 0x000F000Fu, scp[hh][0])};
                    const u32x4m bhi = {pmul(d0 & 0x00F000F0u, scp[hh][1]),
                                        pmul(d08 & 0x00F000F0u, scp[hh][1]),
                                        pmul(d1 & 0x00F000F0u, scp[hh][1]),
                                        pmul(d18 & 0x00F000F0u, scp[hh][1])};
                    const int pp = pbase + 16 * hh + sidx;
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        acc0[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            afrag(t, pp), __builtin_bit_cast(h8, blo), acc0[t], 0, 0, 0);
                        acc1[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            afrag(t, pp + 4), __builtin_bit_cast(h8, bhi), acc1[t], 0, 0, 0);
                    }
                }
            }
            uint32_t scq, mp;
            q4k_scale_pairs(h1, h2, h3, q4k_sel(c), scq, mp);
            (void)scq;
            const u32x4m bmin = {mp, 0u, 0u, 0u};
            const float d = h_lo(w.v[0]), dmin32 = h_hi(w.v[0]) * 32.0f;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint32_t am =
                    *(const uint32_t*)(lds + ly.aux + ((stl * 4 + c) * 2 * M + i_lane[t]) * 4);
                const u32x4m amin = {am, 0u, 0u, 0u};
                const f4 Dm = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    __builtin_bit_cast(h8, amin), __builtin_bit_cast(h8, bmin), (f4)(0.f), 0, 0,
                    0);
                f4 tt;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    tt[r] = __builtin_fmaf(-dmin32, Dm[r], d * (acc0[t][r] + acc1[t][r]));
                y[t].x += tt[0] + tt[1];
                y[t].y += tt[2] + tt[3];
            }
        } else {
            WQ q;
            gather(w, st, q);
            const uint32_t hsel = (uint32_t)(c & 1);
            const uint32_t mask = c >= 2 ? 0x00F000F0u : 0x000F000Fu;
            constexpr int MP = sums_stride(M);
            const float* xsum[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t)
                xsum[t] = (const float*)(lds + ly.aux) + min(8 * t + 2 * c, MP - 2);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                uint32_t qa0, qa1, b0, b1;
                float dA, dB;
                const int blk0 = st * 8 + 2 * k;  // block index of block A in the row
                if constexpr (FMT == kFmtQ4_0S) {
                    qa0 = q.v[k][0];
                    qa1 = q.v[k][1];
                    b0 = q.v[k][2];
                    b1 = q.v[k][3];
                    dA = h_lo(q.v[k][4]);
                    dB = h_hi(q.v[k][4]);
                } else {
                    const uint32_t a0 = q.v[k][0], a1 = q.v[k][1], a2 = q.v[k][2];
                    const uint32_t z = q.v[k][5];
                    b0 = q.v[k][3];
                    b1 = q.v[k][4];
                    qa0 = __builtin_amdgcn_alignbit(a1, a0, 16);
                    qa1 = __builtin_amdgcn_alignbit(a2, a1, 16);
                    dA = h_lo(hsel ? z : a0);
                    dB = h_hi(hsel ? a2 : z);
                }
                // blocks past the row's end (partial last step) hold other
                // bytes: their scales are masked (their activations are 0)
                dA = blk0 < nblk ? dA : 0.f;
                dB = blk0 + 1 < nblk ? dB : 0.f;
                const u32x4m ba = {qa0 & mask, (qa0 >> 8) & mask, qa1 & mask, (qa1 >> 8) & mask};
                const u32x4m bb = {b0 & mask, (b0 >> 8) & mask, b1 & mask, (b1 >> 8) & mask};
                const int blk = stl * 8 + 2 * k;  // local block index of block A
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const f4 DA = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        afrag(t, blk * 4 + c), __builtin_bit_cast(h8, ba), (f4)(0.f), 0, 0, 0);
                    const f4 DB = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        afrag(t, blk * 4 + 4 + c), __builtin_bit_cast(h8, bb), (f4)(0.f), 0, 0,
                        0);
                    const float2 XA = *(const float2*)(xsum[t] + blk * MP);
                    const float2 XB = *(const float2*)(xsum[t] + (blk + 1) * MP);
                    // d (D - 8 X 2^-24): X holds sums of x 2^e, D carries 2^(e-24)
                    y[t].x = __builtin_fmaf(dA, __builtin_fmaf(-0x1p-21f, XA.x, DA[0] + DA[1]),
                                            y[t].x);
                    y[t].y = __builtin_fmaf(dA, __builtin_fmaf(-0x1p-21f, XA.y, DA[2] + DA[3]),
                                            y[t].y);
                    y[t].x = __builtin_fmaf(dB, __builtin_fmaf(-0x1p-21f, XB.x, DB[0] + DB[1]),
                                            y[t].x);
                    y[t].y = __builtin_fmaf(dB, __builtin_fmaf(-0x1p-21f, XB.y, DB[2] + DB[3]),
                                            y[t].y);
                }
            }
        }
    };

    // word checksum of the step's bytes, each word counted by one lane
    // (the words a call reads: in a Q4_K row's last super-block, the nibble
    // chunks that hold no element < K are left out; in a Q4_0 row, the
    // masked blocks past its end)
    auto checksum = [&](const WR& w, int st) {
        uint32_t s = 0;
        if constexpr (FMT == kFmtQ4K) {
            const bool last = st == S - 1;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int g = 2 * hh + (c >> 1);  // nibble chunk of these words
                uint32_t t = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) t += w.v[4 + 4 * hh + i];
                s += (!last || 64 * g < klast) ? t : 0u;
            }
            if (c == 0) s += w.v[0] + w.v[1] + w.v[2] + w.v[3];
        } else {
            // lane group 0: words 0,1 (a), 5,6 (b), 4 (z); group 1: 2,3 (a), 7,8 (b)
            WQ q;
            gather(w, st, q);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                uint32_t t = q.v[k][0] + q.v[k][1] + q.v[k][3] + q.v[k][4];
                if (c == 0) t += q.v[k][5];
                s += (c < 2 && st * 8 + 2 * k < nblk) ? t : 0u;
            }
        }
        return s;
    };

    // End of round r: add the KS partial sums of the group's tile and write.
    auto finish = [&](int r, float2 (&y)[NT], uint32_t cks, int buf) {
        float2* part = (float2*)(lds + ly.part) + buf * kMWaves * 64 * NT;
        if constexpr (PURE) y[0].x = __builtin_bit_cast(float, cks);
#pragma unroll
        for (int t = 0; t < NT; ++t) part[(wave * 64 + lane) * NT + t] = y[t];
        __syncthreads();
        const int t = (r * (int)gridDim.x + (int)blockIdx.x) * TG + grp;
        if (sl == 0 && t < ntiles) {
            const Tile T = tile_at(t);
            const int mt = T.mt;
            const int row = T.row0 + jrow;
            if constexpr (PURE) {
                uint32_t tot = cks;
                for (int k = 1; k < KS; ++k)
                    tot += __builtin_bit_cast(uint32_t, part[((wave + k) * 64 + lane) * NT].x);
                tot += __shfl_xor(tot, 16, kWave);
                tot += __shfl_xor(tot, 32, kWave);
                if (c == 0 && row < p.N) {
                    if constexpr (kMoe) {
                        // every (token, slot) pair that chose this expert
                        const long long P = (long long)M * p.top_k;
                        unsigned long long pm = moe.d.upairs[T.u];
                        while (pm) {
                            const int pr = __builtin_ctzll(pm);
                            pm &= pm - 1ull;
                            p.cks[((long long)mt * P + pr) * p.N + row] = tot;
                        }
                    } else {
                        p.cks[(long long)mt * p.N + row] = tot;
                    }
                }
            } else {
                const int* ex = (const int*)(lds + ly.exps);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    float2 tot = y[t];
                    for (int k = 1; k < KS; ++k) {
                        const float2 o = part[((wave + k) * 64 + lane) * NT + t];
                        tot.x += o.x;
                        tot.y += o.y;
                    }
                    if constexpr (kPair) {
                        // columns j and j + 8 hold row row0 + j of gate and of up
                        const float ux = __shfl_xor(tot.x, 8, kWave);
                        const float uy = __shfl_xor(tot.y, 8, kWave);
                        const int prow = T.row0 + (jrow & 7);
                        if (jrow < 8 && prow < p.N) {
#pragma unroll
                            for (int hm = 0; hm < 2; ++hm) {
                                const int m = 8 * t + 2 * c + hm;
                                if (m < M) {
                                    const int sm = 24 - ex[m];
                                    const float g = __builtin_ldexpf(hm ? tot.y : tot.x, sm);
                                    const float u = __builtin_ldexpf(hm ? uy : ux, sm);
                                    p.y0[(long long)m * p.N + prow] = silu_mul(g, u);
                                }
                            }
                        }
                        continue;
                    }
                    float* yo = mt ? p.y1 : p.y0;
                    if (row < p.N) {
#pragma unroll
                        for (int hm = 0; hm < 2; ++hm) {
                            const int m = 8 * t + 2 * c + hm;
                            if (m < M) {
                                const float v = __builtin_ldexpf(hm ? tot.y : tot.x, 24 - ex[m]);
                                if constexpr (kMoe) {
                                    // output [token, slot, row] for every slot in which
                                    // token m chose this expert
                                    // (token m's pairs: bits m * top_k .. of the mask)
                                    const unsigned long long tk =
                                        p.top_k >= 64 ? ~0ull : ((1ull << p.top_k) - 1ull);
                                    unsigned long long pm =
                                        moe.d.upairs[T.u] & (tk << (m * p.top_k));
                                    while (pm) {
                                        const int pr = __builtin_ctzll(pm);
                                        pm &= pm - 1ull;
                                        yo[(long long)pr * p.N + row] = v;
                                    }
                                } else {
                                    yo[(long long)m * p.N + row] = v;
                                }
                            }
                        }
                    }
                }
            }
        }
    };

    if constexpr (SPLITK) {
        // ---- split-K: this workgroup's tile group and K part; each wave
        // one tile (KS = 1) over the part's steps; partial sums in the
        // part's own scale to the workspace (a second kernel merges them:
        // the kernel boundary makes every part visible, with no device-scope
        // fence, which on this part writes back a whole L2) ----
        int g, kp;
        splitk_role((int)blockIdx.x, (int)gridDim.x, p.kp, g, kp);
        const MSlice sc{S, 1, 1, p.kp, p.msl};
        int a, b, reg;
        sc.range(0, kp, a, b, reg);
        // one pass over the part's activations (parts of at most
        // kSplitKOneSteps steps; the call-uniform choice), else two passes
        // from global memory
        const int ppt = (b - a) * 32;
        const bool one = p.msl <= kSplitKOneSteps;
        constexpr int PP = part_pieces<M>();
        MStageXT<PP> sx;
        if (one) mstage_part_issue<M, PP>(p, a * 256, ppt, sx);
        __builtin_amdgcn_sched_barrier(0);  // the activation loads go out first
        // two steps of weights in flight, the first two before the staging;
        // every load is unconditional (a step past the part is an idle load
        // of one cache line) and the loop is counted, so that no load is
        // merged into its registers by a copy that would wait for it
        WR wa, wb;
        auto sk_load = [&](int st, WR& w) { load(st < b ? 0 : 1, min(st, b - 1), w); };
        sk_load(a, wa);
        sk_load(a + 1, wb);
        __builtin_amdgcn_sched_barrier(0);
        if (one) {
            mstage_part_finish<FMT, M, PP>(p, lds, ly, red, sx, a * 256, ppt, p.msl * 256);
        } else {
            mstage_part_factors<M>(p, lds, ly, red, a * 256, b * 256);
            mstage_slice<FMT, M, kModeDense>(p, lds, ly, sc, kp);
        }
        sync_lds();
        float2 y[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) y[t] = make_float2(0.f, 0.f);
        const int nst = b - a;  // >= 1: parts are never empty (kp <= S)
        for (int i = 0; i < (nst >> 1); ++i) {
            const int st = a + 2 * i;
            compute(wa, st, st - a, y);
            sk_load(st + 2, wa);
            __builtin_amdgcn_sched_barrier(0);
            compute(wb, st + 1, st + 1 - a, y);
            sk_load(st + 3, wb);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (nst & 1) compute(wa, b - 1, nst - 1, y);
        // partial sums of this wave's tile (lane group c: tokens 8t + 2c + hm)
        const int t_wave = g * TG + grp;
        const int* ex = (const int*)(lds + ly.exps);
        if (t_wave < ntiles) {
            const int row = (t_wave << 4) + jrow;
            if (row < p.N) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int hm = 0; hm < 2; ++hm) {
                        const int m = 8 * t + 2 * c + hm;
                        if (m < M)
                            p.part[((long long)kp * M + m) * p.N + row] = hm ? y[t].y : y[t].x;
                    }
            }
        }
        if ((int)threadIdx.x < M) p.pexp[kp * M + threadIdx.x] = ex[threadIdx.x];
        return;  // (splitk_reduce_kernel, launched next on the stream, merges the parts)
    } else if constexpr (SLICED) {
        // ---- K-sliced: per round, the slices one after another; in each,
        // the wave computes its sub-range (the first step's loads issued
        // ahead of the staging).  Every wave meets the same barriers: two
        // per slice (none for a pure read) and finish()'s one per round. ----
        const MSlice sc{S, KS, p.npg, p.nsl, p.msl};
        if constexpr (!PURE) mstage_factors<M, mode_norm(MODE) ? kModeNorm : kModeDense>(p, lds, ly, red);
        int buf = 0;
        for (int r = 0; r < nrounds; ++r) {
            float2 y[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) y[t] = make_float2(0.f, 0.f);
            uint32_t cks = 0;
            for (int s = 0; s < sc.nslices(); ++s) {
                int a, b, reg;
                sc.range(sl, s, a, b, reg);
                const int lbase = reg * sc.msl - a;  // local step of step st: st + lbase
                WR wa, wb;
                if (a < b) load(r, a, wa);
                if constexpr (!PURE) {
                    sync_lds();  // every wave is done with the previous slice
                    mstage_slice<FMT, M, mode_norm(MODE) ? kModeNorm : kModeDense>(p, lds, ly,
                                                                                 sc, s);
                    sync_lds();
                }
                for (int st = a; st < b; st += 2) {
                    const bool hb = st + 1 < b;
                    if (hb) load(r, st + 1, wb);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (PURE) cks += checksum(wa, st);
                    else compute(wa, st, st + lbase, y);
                    if (!hb) break;
                    if (st + 2 < b) load(r, st + 2, wa);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (PURE) cks += checksum(wb, st + 1);
                    else compute(wb, st + 1, st + 1 + lbase, y);
                }
            }
            finish(r, y, cks, buf);
            buf ^= 1;
        }
        return;
    } else {
    // Ring of PD steps in flight.  The wave's steps, round after round, are
    // (r, st0) .. (r, st1 - 1); slot j of the ring is consumed and reloaded
    // in place, PD steps ahead (past the last round the tile index clamps,
    // so the loads stay unconditional and the load-counter waits exact).
    WR w[PD];
    int lr = 0, ls = st0;
    MStageX sx;
    if constexpr (!PURE) mstage_issue<M>(p, sx);
    __builtin_amdgcn_sched_barrier(0);  // the activation loads go out first
#pragma unroll
    for (int j = 0; j < PD; ++j) {
        load(lr, ls, w[j]);
        if (++ls == st1) {
            ls = st0;
            ++lr;
        }
    }
    if constexpr (!PURE) mstage<FMT, M, mode_norm(MODE) ? kModeNorm : kModeDense>(p, lds, ly, red, sx);
    sync_lds();

    const int n = nrounds * (st1 - st0);
    int cs = st0, cr = 0, buf = 0;
    float2 y[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) y[t] = make_float2(0.f, 0.f);
    uint32_t cks = 0;
    for (int base = 0; base < n; base += PD) {
#pragma unroll
        for (int j = 0; j < PD; ++j) {
            const bool act = base + j < n;  // wave-uniform
            if (act) {
                if constexpr (PURE) {
                    cks += checksum(w[j], cs);
                } else {
                    compute(w[j], cs, cs, y);
                }
            }
            load(lr, ls, w[j]);
            if (++ls == st1) {
                ls = st0;
                ++lr;
            }
            if (act && ++cs == st1) {
                cs = st0;
                finish(cr, y, cks, buf);
                ++cr;
                buf ^= 1;
#pragma unroll
                for (int t = 0; t < NT; ++t) y[t] = make_float2(0.f, 0.f);
                cks = 0;
            }
        }
    }
    }
}

}  // namespace q4
