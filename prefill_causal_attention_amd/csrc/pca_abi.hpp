// Host-side pieces of the C ABI shared between its source files: the
// thread-local error message and the checks and launch of the RMSNorm-folded
// projection, which two entry points share (one with a caller-owned
// workspace, one with the library's static workspace).
#pragma once

#include <stdint.h>

#include "pca.h"

namespace pca {

// Records the message for pca_last_error() and returns st.
pca_status abi_error(pca_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Every argument check of the RMSNorm-folded projection except its workspace.
pca_status rms_norm_qkv_proj_check(const pca_bf16* x, int64_t ldx, const pca_bf16* w_t, int64_t ldw, float eps,
                                   pca_bf16* y, int64_t ldy, int64_t M, int64_t N, int64_t K);

// Row statistics into inv_rms[M], then the GEMM scaled by them (arguments checked).
pca_status rms_norm_qkv_proj_launch(const pca_bf16* x, int64_t ldx, const pca_bf16* w_t, int64_t ldw, float eps,
                                    float* inv_rms, pca_bf16* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                    void* stream);

}  // namespace pca
