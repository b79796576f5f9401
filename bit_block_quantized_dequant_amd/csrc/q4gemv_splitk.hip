// q4gemv_splitk.hip -- libq4gemv entry points: the split-K batched GEMV
// (caller workspace) and its workspace query (declared in include/q4gemv.h;
// validation and launch planning in q4_host.h).
#include "q4_host.h"

namespace {

template <int FMT>
int splitk_call(float* y, const void* w, const float* x, int64_t M, int64_t N, int64_t K,
                void* ws, int64_t ws_bytes, void* stream) {
    if (!y || !w || !x) return Q4_ERR_NULL;
    int st = check_dims(M, N, K, FMT);
    if (st) return st;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return Q4_ERR_ALIGN;
    GemvParams p = base_params(w, w, y, y, x, N, K, FMT);
    return run_splitk<FMT>(p, (int)M, ws, ws_bytes, stream);
}

}  // namespace

extern "C" {

int q4_splitk_workspace(int format, int64_t M, int64_t N, int64_t K, int64_t* bytes) {
    if (!bytes) return Q4_ERR_NULL;
    if (format != Q4_FORMAT_Q4_0 && format != Q4_FORMAT_Q4K) return Q4_ERR_ARG;
    const int fmt = format == Q4_FORMAT_Q4K ? kFmtQ4K : kFmtQ4_0;
    int st = check_dims(M, N, K, fmt);
    if (st) return st;
    int cus = 0;
    st = device_cus(&cus);
    if (st) return st;
    const SplitKPlan pl = splitk_plan(fmt, M, N, K, cus);
    *bytes = (M < Q4_MFMA_MIN_M || pl.kp == 1) ? 0 : pl.total;
    return Q4_OK;
}

int q4_0_gemv_splitk(float* y, const void* w, const float* x, int64_t M, int64_t N, int64_t K,
                     void* workspace, int64_t workspace_bytes, void* stream) {
    return splitk_call<kFmtQ4_0>(y, w, x, M, N, K, workspace, workspace_bytes, stream);
}

int q4k_gemv_splitk(float* y, const void* w, const float* x, int64_t M, int64_t N, int64_t K,
                    void* workspace, int64_t workspace_bytes, void* stream) {
    return splitk_call<kFmtQ4K>(y, w, x, M, N, K, workspace, workspace_bytes, stream);
}

}  // extern "C"
