// q4gemv_noalloc.hip -- libq4gemv entry point: the split-K batched Q4_0 GEMV
// with a library-held workspace, for callers that cannot allocate (declared
// in include/q4gemv.h; the kernels and their planning are q4_0_gemv_splitk's,
// in q4_mfma.h and q4_host.h).
#include "q4_host.h"

namespace {

// The workspace: one file-scope device array, one copy per GPU for the life
// of the process.  In host code its name is not a device address; the
// address comes from hipGetSymbolAddress, once per device, with that device
// current, at the entry point's first call there, and only that address is
// used afterwards.  The workspace holds nothing between calls (the kernels
// write every word they read), so nothing in it has to start at zero.
constexpr long long kScratchBytes = 8ll << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return Q4_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return Q4_ERR_HIP;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return Q4_OK;
}

}  // namespace

extern "C" {

long long q4_noalloc_scratch_bytes(void) { return kScratchBytes; }

int q4_0_gemv_splitk_noalloc(float* y, const void* w, const float* x, int64_t M, int64_t N,
                             int64_t K, void* stream) {
    if (!y || !w || !x) return Q4_ERR_NULL;
    int st = check_dims(M, N, K, kFmtQ4_0);
    if (st) return st;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return Q4_ERR_ALIGN;
    int cus = 0;
    st = device_cus(&cus);
    if (st) return st;
    const SplitKPlan pl = splitk_plan(kFmtQ4_0, M, N, K, cus);
    const bool splits = M >= Q4_MFMA_MIN_M && pl.kp > 1;
    if (splits && pl.total > kScratchBytes) return Q4_ERR_SHAPE;
    void* ws = nullptr;
    if (splits) {
        st = scratch_address(&ws);
        if (st) return st;
    }
    GemvParams p = base_params(w, w, y, y, x, N, K, kFmtQ4_0);
    return run_splitk<kFmtQ4_0>(p, (int)M, ws, splits ? kScratchBytes : 0, stream);
}

}  // extern "C"
