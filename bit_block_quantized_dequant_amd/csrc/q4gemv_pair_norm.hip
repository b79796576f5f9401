// q4gemv_pair_norm.hip -- libq4gemv entry points: RMSNorm feeding the gate+up pair, and its SiLU-gated single output
// (declared in include/q4gemv.h; validation and launch planning in q4_host.h).
#include "q4_host.h"

extern "C" {

int fused_rmsnorm_gate_up_q4k_gemv(float* gate, float* up, const void* w_gate,
                                   const void* w_up, const float* x, const float* gamma,
                                   float eps, int64_t M, int64_t N, int64_t K, void* stream) {
    if (!gate || !up || !w_gate || !w_up || !x || !gamma) return Q4_ERR_NULL;
    int st = check_dims(M, N, K, kFmtQ4K);
    if (st) return st;
    if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(x, 16) || !aligned(gamma, 16) ||
        !aligned(gate, 4) || !aligned(up, 4))
        return Q4_ERR_ALIGN;
    if (!(eps >= 0.0f) || !isfinite(eps)) return Q4_ERR_ARG;
    GemvParams p = base_params(w_gate, w_up, gate, up, x, N, K, kFmtQ4K);
    p.gamma = gamma;
    p.eps = eps;
    return run<kFmtQ4K, 2, kModeNorm, false>(p, (int)M, 0, stream);
}

int fused_rmsnorm_gate_up_silu_q4k_gemv(float* h, const void* w_gate, const void* w_up,
                                        const float* x, const float* gamma, float eps,
                                        int64_t M, int64_t N, int64_t K, void* stream) {
    if (!h || !w_gate || !w_up || !x || !gamma) return Q4_ERR_NULL;
    int st = check_dims(M, N, K, kFmtQ4K);
    if (st) return st;
    if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(x, 16) || !aligned(gamma, 16) ||
        !aligned(h, 4))
        return Q4_ERR_ALIGN;
    if (!(eps >= 0.0f) || !isfinite(eps)) return Q4_ERR_ARG;
    GemvParams p = base_params(w_gate, w_up, h, nullptr, x, N, K, kFmtQ4K);
    p.gamma = gamma;
    p.eps = eps;
    return run<kFmtQ4K, 2, kModeNormSilu, false>(p, (int)M, 0, stream);
}

}  // extern "C"
