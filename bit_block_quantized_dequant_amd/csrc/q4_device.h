// q4_device.h -- device-side building blocks of libq4gemv (gfx950, wave64).
//
// Block formats (little-endian):
//   Q4_0: 18 bytes per 32 weights: f16 d, then 16 bytes whose low nibble j is
//         element j and high nibble element j+16; w = d*(q-8)
//         (inferencelayer 0.2.13, src/bin/kernel_lab.rs, GEMV_F16S WGSL).
//   Q4_K: 144 bytes per 256 weights: f16 d, f16 dmin, 12 bytes of packed 6-bit
//         scales/mins, 128 nibble bytes in 64-element chunks (32 low nibbles,
//         then 32 high nibbles); w = d*sc*q - dmin*m
//         (trueno-gpu 0.4.11, src/kernels/quantize/fused.rs,
//          FusedRmsNormQ4KGemvKernel::build_ptx, PHASE 3).
//
// The unit of work of one lane is 64 consecutive weights of one row:
//   Q4_K: chunk g of super-block s (unit u = 4s + g): its 32 nibble bytes
//         hold sub-block 2g in the low nibbles and 2g+1 in the high nibbles;
//         the 16-byte super-block header is loaded beside them.
//   Q4_0: the block pair (2u, 2u+1): 36 bytes, 9 dword-aligned words.
//
// Arithmetic trick (exact): a nibble q masked into the low bits of a 16-bit
// half is the f16 subnormal q * 2^-24, and a nibble masked in place in the
// high half of a byte is 16q * 2^-24.  v_fma_mix_f32 converts such a half to
// fp32 exactly inside the fused multiply-add, so one instruction does
// convert + multiply + accumulate.  The activations are staged pre-scaled by
// 2^24 (elements met as low nibbles) or 2^20 (high nibbles), which makes
// every product exactly q * x.  The 6-bit Q4_K scales and mins are used the
// same way (value sc * 2^-24), so Q4_K row sums come out scaled by 2^-24 and
// are multiplied by 2^24 once at the end; powers of two are exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

constexpr int kWave = 64;
constexpr int kFmtQ4_0 = 0;
constexpr int kFmtQ4K = 1;
// Q4_0 in split arrays (inferencelayer 0.2.13, kernel_lab.rs, GEMV_F16S:
// `scales: array<f16>`, `quants: array<vec4<u32>>`): an f16 scale per block
// in one array, the block's 16 nibble bytes in another.
constexpr int kFmtQ4_0S = 2;

constexpr int kUnitElems = 64;      // weights per lane unit
constexpr int kQ4KBytes = 144;      // Q4_K super-block
constexpr int kQ4_0PairBytes = 36;  // two Q4_0 blocks
constexpr int kUnitWords = 12;      // registers per loaded unit (Q4_0 uses 9)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte global load from a 4-byte aligned address (Q4_0 pairs sit at a
// 36-byte stride, so only dword alignment is guaranteed).
#ifndef Q4_NT_LOADS
#define Q4_NT_LOADS 0
#endif
__device__ __forceinline__ u32x4 ldg16(const uint8_t* p) {
#if Q4_NT_LOADS
    typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
    const u32x4a4 t = __builtin_nontemporal_load((const u32x4a4*)__builtin_assume_aligned(p, 4));
    return u32x4{t.x, t.y, t.z, t.w};
#else
    const uint32_t* q = (const uint32_t*)__builtin_assume_aligned(p, 4);
    u32x4 v;
    __builtin_memcpy(&v, q, 16);
    return v;
#endif
}

__device__ __forceinline__ uint32_t ldg4(const uint8_t* p) {
    return *(const uint32_t*)__builtin_assume_aligned(p, 4);
}

// The low / high 16-bit half of a word taken as f16 and widened exactly.
__device__ __forceinline__ float h_lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float h_hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// ---------------------------------------------------------------------------
// Unit loads.  Q4_K: `p` is the super-block, g the 32-byte nibble chunk (the
// 16-byte header is loaded beside it); Q4_0: `p` is the block pair.
// ---------------------------------------------------------------------------
template <int FMT>
__device__ __forceinline__ void load_unit(const uint8_t* p, int g, uint32_t (&r)[kUnitWords]) {
    if constexpr (FMT == kFmtQ4K) {
        const uint8_t* qs = p + 16 + 32 * g;
        u32x4 h = ldg16(p);
        u32x4 a = ldg16(qs);
        u32x4 b = ldg16(qs + 16);
        r[0] = h.x; r[1] = h.y; r[2] = h.z; r[3] = h.w;
        r[4] = a.x; r[5] = a.y; r[6] = a.z; r[7] = a.w;
        r[8] = b.x; r[9] = b.y; r[10] = b.z; r[11] = b.w;
    } else {
        (void)g;
        u32x4 a = ldg16(p);
        u32x4 b = ldg16(p + 16);
        r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
        r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
        r[8] = ldg4(p + 32);
    }
}

// Same, as a base plus 32-bit offsets: Q4_K header at base + ho and its
// 32 nibble bytes at base + qo; Q4_0 pair at base + ho (qo unused).
template <int FMT>
__device__ __forceinline__ void load_unit_at(const uint8_t* base, uint32_t ho, uint32_t qo,
                                             uint32_t (&r)[kUnitWords]) {
    if constexpr (FMT == kFmtQ4K) {
        u32x4 h = ldg16(base + ho);
        u32x4 a = ldg16(base + qo);
        u32x4 b = ldg16(base + qo + 16);
        r[0] = h.x; r[1] = h.y; r[2] = h.z; r[3] = h.w;
        r[4] = a.x; r[5] = a.y; r[6] = a.z; r[7] = a.w;
        r[8] = b.x; r[9] = b.y; r[10] = b.z; r[11] = b.w;
    } else {
        (void)qo;
        const uint8_t* p = base + ho;
        u32x4 a = ldg16(p);
        u32x4 b = ldg16(p + 16);
        r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
        r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
        r[8] = ldg4(p + 32);
    }
}

// Split-array Q4_0 unit: blocks A and B's 16 nibble bytes (words 0-3, 4-7;
// both 16-byte aligned) and their f16 scales (2-byte aligned) packed into
// word 8 (A low, B high).
__device__ __forceinline__ void load_unit_soa(const uint8_t* qbase, uint32_t qa, uint32_t qb,
                                              const uint8_t* sbase, uint32_t sa, uint32_t sb,
                                              uint32_t (&r)[kUnitWords]) {
    const u32x4 a = ldg16(qbase + qa);
    const u32x4 b = ldg16(qbase + qb);
    const uint32_t da = *(const uint16_t*)__builtin_assume_aligned(sbase + sa, 2);
    const uint32_t db = *(const uint16_t*)__builtin_assume_aligned(sbase + sb, 2);
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
    r[8] = da | (db << 16);
}

// Unit u of a row: the super-block (Q4_K) or block pair (Q4_0) it lives in.
template <int FMT>
__device__ __forceinline__ const uint8_t* unit_ptr(const uint8_t* row, int u) {
    return FMT == kFmtQ4K ? row + (u >> 2) * kQ4KBytes : row + u * kQ4_0PairBytes;
}

// ---------------------------------------------------------------------------
// Q4_K scale/min pairs of the two sub-blocks (2g, 2g+1) a lane works on, as
// two f16-subnormal halves (value v * 2^-24) each.  Header words: h1 = S[0..3],
// h2 = S[4..7], h3 = S[8..11].
//   sub-blocks 0-3: sc = S[j] & 63, m = S[j+4] & 63
//   sub-blocks 4-7: sc = (S[j+4] & 15) | (S[j-4] >> 6) << 4,
//                   m  = (S[j+4] >> 4) | (S[j]   >> 6) << 4
// `sel` = 0x0C000C00 | 2g | (2g+1) << 16 picks bytes 2g, 2g+1 out of the
// eight bytes {high-group word, low-group word} into the two halves.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t q4k_sel(int g) {
    return 0x0C000C00u | (uint32_t)(2 * g) | ((uint32_t)(2 * g + 1) << 16);
}

__device__ __forceinline__ void q4k_scale_pairs(uint32_t h1, uint32_t h2, uint32_t h3,
                                                uint32_t sel, uint32_t& scp, uint32_t& mp) {
    const uint32_t lo4 = 0x0F0F0F0Fu;
    // sub-blocks 4-7: low nibble from S[8..11], bits 4-5 from the top of S[0..7]
    uint32_t sc_hi = (lo4 & h3) | (~lo4 & (h1 >> 2));
    uint32_t m_hi = (lo4 & (h3 >> 4)) | (~lo4 & (h2 >> 2));
    scp = __builtin_amdgcn_perm(sc_hi, h1, sel) & 0x003F003Fu;
    mp = __builtin_amdgcn_perm(m_hi, h2, sel) & 0x003F003Fu;
}

// ---------------------------------------------------------------------------
// Nibble dot products.  One word q of nibble bytes b0..b3 feeds
//   lo: low nibbles  of b0,b1,b2,b3 against xa = x[e], x[e+1], x[e+2], x[e+3]
//   hi: high nibbles of b0,b1,b2,b3 against xb (the elements they encode).
// xa / xb are staged pre-scaled (2^24 / 2^20), so each product is q * x.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void nib_dot(uint32_t q, const float4& xa, const float4& xb,
                                        float& slo, float& shi) {
    const uint32_t t0 = q & 0x000F000Fu;  // low nibbles of b0, b2
    const uint32_t t1 = q & 0x00F000F0u;  // high nibbles of b0, b2 (times 16)
    const uint32_t q8 = q >> 8;
    const uint32_t t2 = q8 & 0x000F000Fu;  // low nibbles of b1, b3
    const uint32_t t3 = q8 & 0x00F000F0u;  // high nibbles of b1, b3 (times 16)
    slo = __builtin_fmaf(h_lo(t0), xa.x, slo);
    shi = __builtin_fmaf(h_lo(t1), xb.x, shi);
    slo = __builtin_fmaf(h_hi(t0), xa.z, slo);
    shi = __builtin_fmaf(h_hi(t1), xb.z, shi);
    slo = __builtin_fmaf(h_lo(t2), xa.y, slo);
    shi = __builtin_fmaf(h_lo(t3), xb.y, shi);
    slo = __builtin_fmaf(h_hi(t2), xa.w, slo);
    shi = __builtin_fmaf(h_hi(t3), xb.w, shi);
}

// LDS layout of the staged activations: per token row, unit u's 16 float4
// chunks at u*17 .. u*17+15 (one chunk of padding per unit).  Lanes reading
// the same chunk of consecutive units are 272 bytes apart, i.e. 4 banks
// apart, so 16 of them hit 16 different bank groups; and a chunk's offset
// from the lane's unit base is a compile-time constant (an immediate in the
// LDS instruction, no address arithmetic per step).
constexpr int kUnitChunks = 17;
__device__ __forceinline__ int xchunk(int u, int c) { return u * kUnitChunks + c; }
__device__ __forceinline__ int xrow_chunks(int upr) { return upr * kUnitChunks; }

// Is element e (within its row) met as a high nibble?  Q4_K: elements 32..63
// of each 64-element chunk; Q4_0: elements 16..31 of each 32-element block.
template <int FMT>
__device__ __forceinline__ bool elem_is_high(int e) {
    return FMT == kFmtQ4K ? (e & 32) != 0 : (e & 16) != 0;
}

// ---------------------------------------------------------------------------
// One unit of NR rows against M token rows of staged activations.  Every
// activation chunk is read from LDS once and used for all NR rows.
//   xl  : LDS chunks of token 0 (token m at xl + m * kq, kq = xrow_chunks(K))
//   xs  : LDS per-32-run sums of token 0, as float2 per unit (token m at
//         xs + m * (K/64)); Q4_K: plain sums X; Q4_0: -8 * X.
// acc[r][m] accumulates row r's dot product with token m (Q4_K: scaled by
// 2^-24); with act == false the accumulators are left as they were (a lane
// past the end of its row computes on a clamped duplicate and drops it).  For M > 1 a scheduling fence after each nibble word keeps the
// compiler from hoisting all 16*M chunk reads at once (register pressure).
// ---------------------------------------------------------------------------
template <int FMT, int M, int NR>
__device__ __forceinline__ void rows_dot(const uint32_t (&w)[NR][kUnitWords], int u,
                                         uint32_t sel, const float4* __restrict__ xl, int kq,
                                         const float2* __restrict__ xs, int k64,
                                         float (&acc)[NR][M], bool act = true) {
    const float4* xu = xl + u * kUnitChunks;
    if constexpr (FMT == kFmtQ4K) {
        float s0[NR][M], s1[NR][M];
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) { s0[r][m] = 0.f; s1[r][m] = 0.f; }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float4 xa = xu[m * kq + i];
                const float4 xb = xu[m * kq + 8 + i];
#pragma unroll
                for (int r = 0; r < NR; ++r) nib_dot(w[r][4 + i], xa, xb, s0[r][m], s1[r][m]);
            }
            if constexpr (M > 1) __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            uint32_t scp, mp;
            q4k_scale_pairs(w[r][1], w[r][2], w[r][3], sel, scp, mp);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float2 X = xs[m * k64 + u];
                float t = __builtin_fmaf(h_lo(scp), s0[r][m], 0.0f);
                t = __builtin_fmaf(h_hi(scp), s1[r][m], t);
                float v = __builtin_fmaf(h_lo(mp), X.x, 0.0f);
                v = __builtin_fmaf(h_hi(mp), X.y, v);
                float a = __builtin_fmaf(h_lo(w[r][0]), t, acc[r][m]);
                a = __builtin_fmaf(-h_hi(w[r][0]), v, a);
                acc[r][m] = act ? a : acc[r][m];
            }
        }
    } else {
        // 18-byte blocks: block A = bytes 0..17 (d in w0.lo, nibbles
        // shifted by two bytes), block B = bytes 18..35 (d in w4.hi,
        // nibbles in w5..w8).  Split arrays: nibbles in w0..w3 and w4..w7,
        // scales in w8.
        constexpr bool kSoa = FMT == kFmtQ4_0S;
        uint32_t qa[NR][4];
        float a0[NR][M], a1[NR][M], b0[NR][M], b1[NR][M];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            if constexpr (kSoa) {
                qa[r][0] = w[r][0];
                qa[r][1] = w[r][1];
                qa[r][2] = w[r][2];
                qa[r][3] = w[r][3];
            } else {
                qa[r][0] = __builtin_amdgcn_alignbit(w[r][1], w[r][0], 16);
                qa[r][1] = __builtin_amdgcn_alignbit(w[r][2], w[r][1], 16);
                qa[r][2] = __builtin_amdgcn_alignbit(w[r][3], w[r][2], 16);
                qa[r][3] = __builtin_amdgcn_alignbit(w[r][4], w[r][3], 16);
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float2 X8 = xs[m * k64 + u];  // (-8 * X_A, -8 * X_B)
                a0[r][m] = X8.x; a1[r][m] = 0.f;
                b0[r][m] = X8.y; b1[r][m] = 0.f;
            }
        }
        // nibble word i: block A (words 0-3, chunks i and 4+i) or block B
        // (words 4-7, chunks 8+i' and 12+i')
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int ca = i < 4 ? i : 4 + i;  // low-nibble chunk; high = ca + 4
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float4 xlo = xu[m * kq + ca];
                const float4 xhi = xu[m * kq + ca + 4];
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    if (i < 4)
                        nib_dot(qa[r][i], xlo, xhi, a0[r][m], a1[r][m]);
                    else
                        nib_dot(w[r][kSoa ? i : 1 + i], xlo, xhi, b0[r][m], b1[r][m]);
                }
            }
            if constexpr (M > 1) __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float dA = h_lo(w[r][kSoa ? 8 : 0]);
                const float dB = h_hi(w[r][kSoa ? 8 : 4]);
                float a = __builtin_fmaf(dA, a0[r][m] + a1[r][m], acc[r][m]);
                a = __builtin_fmaf(dB, b0[r][m] + b1[r][m], a);
                acc[r][m] = act ? a : acc[r][m];
            }
    }
}

// Sum of the words a pure-read pass attributes to this unit: every Q4_0
// word; for Q4_K the nibble words, plus the header once per super-block
// (by the lane holding chunk 0).
template <int FMT>
__device__ __forceinline__ uint32_t unit_checksum(const uint32_t (&w)[kUnitWords], int u) {
    uint32_t s = 0;
    if constexpr (FMT == kFmtQ4K) {
#pragma unroll
        for (int i = 4; i < 12; ++i) s += w[i];
        if ((u & 3) == 0) s += w[0] + w[1] + w[2] + w[3];
    } else {
#pragma unroll
        for (int i = 0; i < 9; ++i) s += w[i];
    }
    return s;
}

// Sum over aligned groups of `width` lanes (power of two, 4 <= width <= 64)
// with DPP lane moves: xor 1 and 2 (quad_perm), 4 (row_half_mirror) and 8
// (row_mirror) leave every lane of a 16-lane row with the row's sum;
// row_bcast:15 then adds row 0's total into row 1 (and row 2's into row 3)
// and row_bcast:31 adds lanes 0-31's total into rows 2 and 3.  The group's
// total is exact in its LAST lane (li == width - 1) for every width; other
// lanes may hold partial sums.  The addition order is fixed by the width
// alone, so equal inputs give bit-equal results in every kernel.
template <typename T>
__device__ __forceinline__ T dpp_add(T v, int ctrl_sel) {
    int iv = __builtin_bit_cast(int, v);
    int t;
    switch (ctrl_sel) {
        case 0: t = __builtin_amdgcn_update_dpp(0, iv, 0xB1, 0xF, 0xF, false); break;   // quad xor 1
        case 1: t = __builtin_amdgcn_update_dpp(0, iv, 0x4E, 0xF, 0xF, false); break;   // quad xor 2
        case 2: t = __builtin_amdgcn_update_dpp(0, iv, 0x141, 0xF, 0xF, false); break;  // half mirror
        case 3: t = __builtin_amdgcn_update_dpp(0, iv, 0x140, 0xF, 0xF, false); break;  // mirror
        case 4: t = __builtin_amdgcn_update_dpp(0, iv, 0x142, 0xA, 0xF, false); break;  // bcast 15
        default: t = __builtin_amdgcn_update_dpp(0, iv, 0x143, 0xC, 0xF, false); break; // bcast 31
    }
    return v + __builtin_bit_cast(T, t);
}

// Largest value of a whole wave of NON-NEGATIVE floats, exact in lane 63:
// the same DPP pattern as group_total with max in place of the sum (lanes a
// row operation does not write read 0, which max ignores for v >= 0).
__device__ __forceinline__ float wave_max_nonneg(float v) {
    auto mx = [](float a, int t) { return fmaxf(a, __builtin_bit_cast(float, t)); };
    const int iv0 = __builtin_bit_cast(int, v);
    v = mx(v, __builtin_amdgcn_update_dpp(0, iv0, 0xB1, 0xF, 0xF, false));  // quad xor 1
    v = mx(v, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v = mx(v, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    v = mx(v, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    v = mx(v, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
    v = mx(v, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
    return v;
}

template <typename T>
__device__ __forceinline__ T group_total(T v, int width) {
    v = dpp_add(v, 0);
    v = dpp_add(v, 1);
    if (width > 4) v = dpp_add(v, 2);
    if (width > 8) v = dpp_add(v, 3);
    if (width > 16) v = dpp_add(v, 4);
    if (width > 32) v = dpp_add(v, 5);
    return v;
}

}  // namespace q4
