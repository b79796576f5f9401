// q4gemv.hip -- libq4gemv entry points: status text, version, the expert router, the
// dequantization calls and the split-array repack
// (declared in include/q4gemv.h; validation and launch planning in q4_host.h).
#include "q4_host.h"

extern "C" {

const char* q4_strerror(int status) {
    switch (status) {
        case Q4_OK: return "ok";
        case Q4_ERR_NULL: return "a required pointer is NULL";
        case Q4_ERR_SHAPE: return "N, K, E, top_k or M*K outside the supported limits";
        case Q4_ERR_BATCH: return "batch M outside [1, 16] (dense calls) or [1, 8] (expert calls, router)";
        case Q4_ERR_ALIGN: return "pointer not aligned (weights and x: 16 bytes; others: 4)";
        case Q4_ERR_ARG: return "invalid argument";
        case Q4_ERR_HIP: return "the HIP runtime refused the launch";
    }
    return "unknown status";
}

int q4_version(void) { return 1; }

int moe_router_q4_0(int32_t* ids, float* weights, const void* w_router, const float* x,
                    int64_t M, int64_t E, int64_t K, int64_t top_k, int normalize,
                    void* stream) {
    if (!ids || !weights || !w_router || !x) return Q4_ERR_NULL;
    if (M < 1 || M > 8) return Q4_ERR_BATCH;
    if (!k_ok(K, kFmtQ4_0) || K > kRouterMaxK) return Q4_ERR_SHAPE;
    if (E < 1 || E > kRouterMaxE || top_k < 1 || top_k > E || top_k > kRouterMaxTopK)
        return Q4_ERR_SHAPE;
    if (normalize != 0 && normalize != 1) return Q4_ERR_ARG;
    if (!aligned(w_router, 16) || !aligned(x, 16) || !aligned(ids, 4) || !aligned(weights, 4))
        return Q4_ERR_ALIGN;
    const size_t lds = router_lds_bytes((int)K, (int)E);
    if (lds > 64 * 1024) {
        static std::atomic<int> big_lds_done[kMaxDevices];
        int st = allow_big_lds((const void*)router_kernel, big_lds_done);
        if (st) return st;
    }
    hipLaunchKernelGGL(router_kernel, dim3((unsigned)M), dim3(kRouterBlock), lds,
                       (hipStream_t)stream, ids, weights, (const uint8_t*)w_router, x, (int)E,
                       (int)K, (int)top_k, normalize);
    return hipGetLastError() == hipSuccess ? Q4_OK : Q4_ERR_HIP;
}

int dequant_q4k(float* out, const void* w, int64_t N, int64_t K, void* stream) {
    if (!out || !w) return Q4_ERR_NULL;
    if (!k_ok(K, kFmtQ4K) || N < 1 || N > INT32_MAX) return Q4_ERR_SHAPE;
    if (!aligned(w, 16) || !aligned(out, 16)) return Q4_ERR_ALIGN;
    const long long upr = k_units(K);
    const long long nunits = (long long)N * upr;
    const long long blocks = (nunits + 255) / 256;
    if (blocks > INT32_MAX) return Q4_ERR_SHAPE;
    hipLaunchKernelGGL(dequant_kernel<kFmtQ4K>, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, out, (const uint8_t*)w, nunits, (int)upr, (int)K,
                       row_bytes_of(K, kFmtQ4K));
    return hipGetLastError() == hipSuccess ? Q4_OK : Q4_ERR_HIP;
}

int dequant_q4_0(float* out, const void* w, int64_t N, int64_t K, void* stream) {
    if (!out || !w) return Q4_ERR_NULL;
    if (!k_ok(K, kFmtQ4_0) || N < 1 || N > INT32_MAX) return Q4_ERR_SHAPE;
    if (!aligned(w, 16) || !aligned(out, 16)) return Q4_ERR_ALIGN;
    const long long upr = k_units(K);
    const long long nunits = (long long)N * upr;
    const long long blocks = (nunits + 255) / 256;
    if (blocks > INT32_MAX) return Q4_ERR_SHAPE;
    hipLaunchKernelGGL(dequant_kernel<kFmtQ4_0>, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, out, (const uint8_t*)w, nunits, (int)upr, (int)K,
                       row_bytes_of(K, kFmtQ4_0));
    return hipGetLastError() == hipSuccess ? Q4_OK : Q4_ERR_HIP;
}

int q4_0_repack_soa(void* scales, void* quants, const void* w, int64_t N, int64_t K,
                    void* stream) {
    if (!scales || !quants || !w) return Q4_ERR_NULL;
    if (!k_ok(K, kFmtQ4_0S) || K > Q4_MAX_K || N < 1 || N > INT32_MAX) return Q4_ERR_SHAPE;
    if (!aligned(w, 2) || !aligned(scales, 2) || !aligned(quants, 16)) return Q4_ERR_ALIGN;
    const long long nblocks = (long long)N * (K / 32);
    const long long blocks = (nblocks + 255) / 256;
    if (blocks > INT32_MAX) return Q4_ERR_SHAPE;
    hipLaunchKernelGGL(repack_q4_0_soa_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, (uint16_t*)scales, (u32x4*)quants,
                       (const uint8_t*)w, nblocks);
    return hipGetLastError() == hipSuccess ? Q4_OK : Q4_ERR_HIP;
}

}  // extern "C"
