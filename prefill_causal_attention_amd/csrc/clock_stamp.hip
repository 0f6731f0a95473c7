// pca_clock_stamp: the shader-clock cycle counter and the 100 MHz real-time
// counter of every XCD, read on the device in stream order.  Two stamps
// around a stretch of work give each XCD's average shader clock over it
// (cycles / seconds), which is what the MFMA peak of the chip scales with.
#include "pca.h"
#include "pca_abi.hpp"
#include "pca_internal.hpp"

namespace {

constexpr int kStampBlocks = 64;   // round-robin dispatch gives every XCD several of them

// Each block's first lane writes (XCC id, s_memtime, s_memrealtime) at its
// own slot; out has 3 * kStampBlocks entries.
__global__ __launch_bounds__(64) void clock_stamp_kernel(uint64_t* out) {
    if (threadIdx.x != 0) return;
    // hardware register XCC_ID (id 20), bits [3:0]: the XCD the wave runs on
    const uint32_t xcc = (uint32_t)__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xFu;
    const uint64_t cyc = __builtin_amdgcn_s_memtime();
    const uint64_t rt = __builtin_amdgcn_s_memrealtime();
    out[3 * blockIdx.x + 0] = xcc;
    out[3 * blockIdx.x + 1] = cyc;
    out[3 * blockIdx.x + 2] = rt;
}

}  // namespace

extern "C" pca_status pca_clock_stamp(uint64_t* out, void* stream) {
    if (out == nullptr || ((uintptr_t)out & 7u))
        return pca::abi_error(PCA_ERR_INVALID_ARG, "out must be an 8-byte aligned device buffer of %d uint64",
                              3 * kStampBlocks);
    hipLaunchKernelGGL(clock_stamp_kernel, dim3(kStampBlocks), dim3(64), 0, (hipStream_t)stream, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return pca::abi_error(PCA_ERR_HIP, "clock_stamp launch: %s", hipGetErrorString(e));
    return PCA_OK;
}
