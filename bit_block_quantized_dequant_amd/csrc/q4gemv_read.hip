// q4gemv_read.hip -- libq4gemv entry points: the pure-read bandwidth ceiling
// (declared in include/q4gemv.h; validation and launch planning in q4_host.h).
#include "q4_host.h"

extern "C" {

int q4_pure_read(uint32_t* checksum, int kernel_id, const void* w0, const void* w1,
                 const int32_t* ids, int64_t M, int64_t top_k, int64_t E, int64_t N, int64_t K,
                 void* stream) {
    if (kernel_id < Q4_READ_Q4_0_GEMV || kernel_id > Q4_READ_MOE_DOWN) return Q4_ERR_ARG;
    if (!checksum || !w0) return Q4_ERR_NULL;
    if (kernel_id == Q4_READ_STREAM) {
        if (K <= 0 || K % 256 != 0 || N < 1 || N > INT32_MAX) return Q4_ERR_SHAPE;
        if (!aligned(w0, 16) || !aligned(checksum, 4)) return Q4_ERR_ALIGN;
        int cus = 0;
        int st = device_cus(&cus);
        if (st) return st;
        const long long bytes = N * (K / 256) * (long long)kQ4KBytes;
        const long long nblk = (bytes + kStreamBlockBytes - 1) / kStreamBlockBytes;
        static std::atomic<int> resident[kMaxDevices];
        int wgc = resident_per_cu((const void*)stream_read_kernel, kStreamBlock, 0, resident);
        if (wgc > 2) wgc = 2;  // two workgroups per CU (measured fastest)
        long long blocks = (long long)cus * wgc;
        const long long need = (nblk + kStreamBlock / kWave - 1) / (kStreamBlock / kWave);
        if (blocks > need) blocks = need;
        hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kStreamBlock), 0,
                           (hipStream_t)stream, checksum, (const uint8_t*)w0, bytes);
        return hipGetLastError() == hipSuccess ? Q4_OK : Q4_ERR_HIP;
    }
    if ((kernel_id == Q4_READ_GATE_UP || kernel_id == Q4_READ_MOE) && !w1) return Q4_ERR_NULL;
    const bool moe = kernel_id == Q4_READ_MOE || kernel_id == Q4_READ_MOE_DOWN;
    if (moe && !ids) return Q4_ERR_NULL;
    const int fmt = (kernel_id == Q4_READ_Q4_0_GEMV || moe) ? kFmtQ4_0 : kFmtQ4K;
    int st = moe ? check_moe(M, top_k, E, N, K) : check_dims(M, N, K, fmt);
    if (st) return st;
    if (!aligned(w0, 16) || (w1 && !aligned(w1, 16)) || !aligned(checksum, 4) ||
        (ids && !aligned(ids, 4)))
        return Q4_ERR_ALIGN;
    GemvParams p = base_params(w0, w1 ? w1 : w0, nullptr, nullptr, nullptr, N, K, fmt);
    p.cks = checksum;
    switch (kernel_id) {
        case Q4_READ_Q4_0_GEMV: return run<kFmtQ4_0, 1, kModeDense, true>(p, (int)M, 0, stream);
        case Q4_READ_Q4K_GEMV: return run<kFmtQ4K, 1, kModeDense, true>(p, (int)M, 0, stream);
        case Q4_READ_GATE_UP: return run<kFmtQ4K, 2, kModeDense, true>(p, (int)M, 0, stream);
        case Q4_READ_MOE: {
            p.ids = ids;
            p.top_k = (int)top_k;
            p.E = (int)E;
            const int umax = (int)(M * top_k < E ? M * top_k : E);
            return run<kFmtQ4_0, 2, kModeMoe, true>(p, (int)M, umax, stream);
        }
        case Q4_READ_MOE_DOWN: {
            p.ids = ids;
            p.top_k = (int)top_k;
            p.E = (int)E;
            const int umax = (int)(M * top_k < E ? M * top_k : E);
            return run_down<true>(p, (int)M, umax, stream);
        }
    }
    return Q4_ERR_ARG;
}

}  // extern "C"
