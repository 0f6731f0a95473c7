// pca_clock_stamp: the shader-clock cycle counters and the 100 MHz real-time
// counter, read on the device in stream order by blocks spread over every CU.
// Two stamps around a stretch of work give each XCD's average shader clock
// over it (cycles / seconds), which is what the MFMA peak of the chip scales
// with.  The cycle counter a wave reads (s_memtime) belongs to its part of the
// chip, and counters of different shader engines of one XCD do not agree, so
// the two stamps are paired per CU (its hardware location), never across.
#include "pca.h"
#include "pca_abi.hpp"
#include "pca_internal.hpp"

namespace {

constexpr int kStampBlocks = 1024;   // several per CU, so every CU stamps both times
constexpr int kStampWords = 4;

// Each block's first lane writes, at out[4 b .. 4 b + 3]: the XCC id, the
// wave's HW_ID register (shader engine, array and CU in bits 8-15),
// s_memtime and s_memrealtime.
__global__ __launch_bounds__(64) void clock_stamp_kernel(uint64_t* out) {
    if (threadIdx.x != 0) return;
    // hardware register XCC_ID (id 20), bits [3:0]: the XCD the wave runs on
    const uint32_t xcc = (uint32_t)__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xFu;
    // hardware register HW_ID (id 4), all 32 bits
    const uint32_t hwid = (uint32_t)__builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);
    const uint64_t cyc = __builtin_amdgcn_s_memtime();
    const uint64_t rt = __builtin_amdgcn_s_memrealtime();
    uint64_t* o = out + (size_t)kStampWords * blockIdx.x;
    o[0] = xcc;
    o[1] = hwid;
    o[2] = cyc;
    o[3] = rt;
}

}  // namespace

extern "C" pca_status pca_clock_stamp(uint64_t* out, void* stream) {
    if (out == nullptr || ((uintptr_t)out & 7u))
        return pca::abi_error(PCA_ERR_INVALID_ARG, "out must be an 8-byte aligned device buffer of %d uint64",
                              kStampWords * kStampBlocks);
    hipLaunchKernelGGL(clock_stamp_kernel, dim3(kStampBlocks), dim3(64), 0, (hipStream_t)stream, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return pca::abi_error(PCA_ERR_HIP, "clock_stamp launch: %s", hipGetErrorString(e));
    return PCA_OK;
}
