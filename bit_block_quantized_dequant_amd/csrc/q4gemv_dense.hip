// q4gemv_dense.hip -- libq4gemv entry points: the single-matrix GEMV calls (Q4_0, Q4_K,
// RMSNorm + Q4_K, split-array Q4_0)
// (declared in include/q4gemv.h; validation and launch planning in q4_host.h).
#include "q4_host.h"

extern "C" {

int q4_0_gemv(float* y, const void* w, const float* x, int64_t M, int64_t N, int64_t K,
              void* stream) {
    if (!y || !w || !x) return Q4_ERR_NULL;
    int st = check_dims(M, N, K, kFmtQ4_0);
    if (st) return st;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return Q4_ERR_ALIGN;
    GemvParams p = base_params(w, w, y, y, x, N, K, kFmtQ4_0);
    return run<kFmtQ4_0, 1, kModeDense, false>(p, (int)M, 0, stream);
}

int q4k_gemv(float* y, const void* w, const float* x, int64_t M, int64_t N, int64_t K,
             void* stream) {
    if (!y || !w || !x) return Q4_ERR_NULL;
    int st = check_dims(M, N, K, kFmtQ4K);
    if (st) return st;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return Q4_ERR_ALIGN;
    GemvParams p = base_params(w, w, y, y, x, N, K, kFmtQ4K);
    return run<kFmtQ4K, 1, kModeDense, false>(p, (int)M, 0, stream);
}

int fused_rmsnorm_q4k_gemv(float* y, const void* w, const float* x, const float* gamma,
                           float eps, int64_t M, int64_t N, int64_t K, void* stream) {
    if (!y || !w || !x || !gamma) return Q4_ERR_NULL;
    int st = check_dims(M, N, K, kFmtQ4K);
    if (st) return st;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(gamma, 16) || !aligned(y, 4))
        return Q4_ERR_ALIGN;
    if (!(eps >= 0.0f) || !isfinite(eps)) return Q4_ERR_ARG;
    GemvParams p = base_params(w, w, y, y, x, N, K, kFmtQ4K);
    p.gamma = gamma;
    p.eps = eps;
    return run<kFmtQ4K, 1, kModeNorm, false>(p, (int)M, 0, stream);
}

int q4_0_gemv_soa(float* y, const void* scales, const void* quants, const float* x, int64_t M,
                  int64_t N, int64_t K, void* stream) {
    if (!y || !scales || !quants || !x) return Q4_ERR_NULL;
    int st = check_dims(M, N, K, kFmtQ4_0S);
    if (st) return st;
    if (!aligned(quants, 16) || !aligned(scales, 2) || !aligned(x, 16) || !aligned(y, 4))
        return Q4_ERR_ALIGN;
    GemvParams p = base_params(quants, quants, y, y, x, N, K, kFmtQ4_0S);
    p.sc = (const uint8_t*)scales;
    return run<kFmtQ4_0S, 1, kModeDense, false>(p, (int)M, 0, stream);
}

}  // extern "C"
