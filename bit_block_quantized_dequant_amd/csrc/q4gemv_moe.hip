// q4gemv_moe.hip -- libq4gemv entry points: the expert-selected gate/up calls
// and the expert down-projection
// (declared in include/q4gemv.h; validation and launch planning in q4_host.h).
#include "q4_host.h"

extern "C" {

int moe_q4_gemv(float* gate, float* up, const void* w_gate, const void* w_up, const float* x,
                const int32_t* ids, int64_t M, int64_t top_k, int64_t E, int64_t N, int64_t K,
                void* stream) {
    if (!gate || !up || !w_gate || !w_up || !x || !ids) return Q4_ERR_NULL;
    int st = check_moe(M, top_k, E, N, K);
    if (st) return st;
    if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(x, 16) || !aligned(gate, 4) ||
        !aligned(up, 4) || !aligned(ids, 4))
        return Q4_ERR_ALIGN;
    GemvParams p = base_params(w_gate, w_up, gate, up, x, N, K, kFmtQ4_0);
    p.ids = ids;
    p.top_k = (int)top_k;
    p.E = (int)E;
    const int umax = (int)(M * top_k < E ? M * top_k : E);
    return run<kFmtQ4_0, 2, kModeMoe, false>(p, (int)M, umax, stream);
}

int moe_q4_gemv_silu(float* h, const void* w_gate, const void* w_up, const float* x,
                     const int32_t* ids, int64_t M, int64_t top_k, int64_t E, int64_t N,
                     int64_t K, void* stream) {
    if (!h || !w_gate || !w_up || !x || !ids) return Q4_ERR_NULL;
    int st = check_moe(M, top_k, E, N, K);
    if (st) return st;
    if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(x, 16) || !aligned(h, 4) ||
        !aligned(ids, 4))
        return Q4_ERR_ALIGN;
    GemvParams p = base_params(w_gate, w_up, h, nullptr, x, N, K, kFmtQ4_0);
    p.ids = ids;
    p.top_k = (int)top_k;
    p.E = (int)E;
    const int umax = (int)(M * top_k < E ? M * top_k : E);
    return run<kFmtQ4_0, 2, kModeMoeSilu, false>(p, (int)M, umax, stream);
}

int moe_q4_gemv_down(float* y, const void* w_down, const float* h, const int32_t* ids,
                     int64_t M, int64_t top_k, int64_t E, int64_t N, int64_t K, void* stream) {
    if (!y || !w_down || !h || !ids) return Q4_ERR_NULL;
    int st = check_moe(M, top_k, E, N, K);
    if (st) return st;
    if (!aligned(w_down, 16) || !aligned(h, 16) || !aligned(y, 4) || !aligned(ids, 4))
        return Q4_ERR_ALIGN;
    GemvParams p = base_params(w_down, w_down, y, nullptr, h, N, K, kFmtQ4_0);
    p.ids = ids;
    p.top_k = (int)top_k;
    p.E = (int)E;
    const int umax = (int)(M * top_k < E ? M * top_k : E);
    return run_down<false>(p, (int)M, umax, stream);
}

}  // extern "C"
