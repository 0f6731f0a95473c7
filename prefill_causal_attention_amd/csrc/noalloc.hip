// pca_rms_norm_qkv_proj_noalloc: the RMSNorm-folded QKV projection with the
// per-row 1/rms workspace in a fixed device array of this library instead of
// a caller-owned buffer, for callers that cannot allocate device memory.
//
// The array below lives in the library's code object; each GPU the library
// runs on holds its own copy, at its own address, until the process ends.
// Host code never uses the array's name as an address: on first use on a
// device (that device current) its device address is looked up once with
// hipGetSymbolAddress and kept per device, and only that address is handed to
// the kernels.  No call here allocates or frees memory.
//
// Every call on one GPU shares that GPU's array: the statistics kernel writes
// rows [0, M) before the GEMM reads them (both on the caller's stream), so
// nothing has to start at zero, but two calls whose work overlaps in time on
// one GPU (different streams, or different host threads) race on it.
#include <mutex>

#include "pca_abi.hpp"
#include "pca_internal.hpp"

namespace {

static __device__ __align__(256) float scratch[PCA_NOALLOC_MAX_ROWS];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once found

// Device address of the current device's copy of `scratch`.
pca_status scratch_of_current_device(float** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return pca::abi_error(PCA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return pca::abi_error(PCA_ERR_UNSUPPORTED, "device index %d beyond the %d the library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return pca::abi_error(PCA_ERR_HIP, "hipGetSymbolAddress of the static workspace on device %d: %s", dev,
                                  hipGetErrorString(e));
        g_scratch[dev] = static_cast<float*>(p);
    }
    *out = g_scratch[dev];
    return PCA_OK;
}

}  // namespace

extern "C" pca_status pca_rms_norm_qkv_proj_noalloc(const pca_bf16* x, int64_t ldx, const pca_bf16* w_t,
                                                    int64_t ldw, float eps, pca_bf16* y, int64_t ldy, int64_t M,
                                                    int64_t N, int64_t K, void* stream) {
    pca_status st = pca::rms_norm_qkv_proj_check(x, ldx, w_t, ldw, eps, y, ldy, M, N, K);
    if (st != PCA_OK) return st;
    if (M > PCA_NOALLOC_MAX_ROWS)
        return pca::abi_error(PCA_ERR_UNSUPPORTED, "M = %lld rows exceed the static workspace of %d rows",
                              (long long)M, PCA_NOALLOC_MAX_ROWS);
    float* ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != PCA_OK) return st;
    return pca::rms_norm_qkv_proj_launch(x, ldx, w_t, ldw, eps, ws, y, ldy, M, N, K, stream);
}
