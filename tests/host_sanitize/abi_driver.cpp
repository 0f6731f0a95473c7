// Host-only driver for the C ABI's argument handling, built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer together with the library's
// host source (the checks and argument packing of every entry point).  The
// kernel launchers are replaced by stubs that only count calls and keep the
// last arguments, so no GPU is needed: every valid call must reach exactly
// one launcher with the arguments the header promises, every invalid call
// none.  Device addresses are fake and never dereferenced.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <climits>

#include "pca.h"
#include "pca_internal.hpp"

namespace pca {
static int g_launches = 0;
static GemmArgs g_gemm;
static AttnArgs g_attn;
static KvWriteArgs g_kv;
hipError_t launch_kv_write_bf16(const KvWriteArgs& a, hipStream_t) { ++g_launches; g_kv = a; return hipSuccess; }
hipError_t launch_kv_write_fp8(const KvWriteArgs& a, hipStream_t) { ++g_launches; g_kv = a; return hipSuccess; }
hipError_t launch_e4m3_encode(const float*, uint8_t*, int64_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_qkv_gemm(const GemmArgs& a, hipStream_t) { ++g_launches; g_gemm = a; return hipSuccess; }
hipError_t launch_gemm_fp8(const Fp8GemmArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_quantize_rows(const uint16_t*, int64_t, int, int, uint8_t*, int64_t, float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_quantize_heads(const uint16_t*, int64_t, int64_t, int, int, float, uint8_t*, int64_t, uint8_t*,
                                 int64_t, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_rms_stats(const uint16_t*, int64_t, int, int, float, float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_attention(const AttnArgs& a, hipStream_t) { ++g_launches; g_attn = a; return hipSuccess; }
}  // namespace pca

static int g_fail = 0, g_checks = 0;

#define EXPECT(cond, ...)                                                        \
    do {                                                                         \
        ++g_checks;                                                              \
        if (!(cond)) {                                                           \
            ++g_fail;                                                            \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);                 \
            fprintf(stderr, __VA_ARGS__);                                        \
            fprintf(stderr, " (last error: %s)\n", pca_last_error());            \
        }                                                                        \
    } while (0)

// status of one call, and how many launches it made
#define CALL(expect_status, expect_launches, expr)                                                          \
    do {                                                                                                    \
        const int before = pca::g_launches;                                                                 \
        const pca_status st = (expr);                                                                       \
        EXPECT(st == (expect_status), "%s -> %d, want %d", #expr, (int)st, (int)(expect_status));           \
        EXPECT(pca::g_launches - before == (expect_launches), "%s launched %d kernels, want %d", #expr,    \
               pca::g_launches - before, (int)(expect_launches));                                           \
        if ((expect_status) != PCA_OK) EXPECT(pca_last_error()[0] != '\0', "%s: empty error message", #expr); \
    } while (0)

static pca_bf16* B(uintptr_t a) { return (pca_bf16*)a; }
static const uintptr_t A1 = 0x100000, A2 = 0x200000, A3 = 0x300000, A4 = 0x400000, A5 = 0x500000;

static void layout_checks() {
    pca_kv_layout_t l;
    CALL(PCA_OK, 0, pca_kv_layout(32, 8, 128, 16, PCA_DTYPE_BF16, &l));
    EXPECT(l.qkv_ld == 6144 && l.k_off == 4096 && l.v_off == 5120 && l.kv_bytes_per_token_layer == 4096, "GQA layout");
    CALL(PCA_OK, 0, pca_kv_layout(40, 8, 128, 16, PCA_DTYPE_FP8_E4M3, &l));
    EXPECT(l.scale_slot_stride == 8 && l.scale_bytes_per_token_layer == 64 && l.page_bytes == 16 * 8 * 128, "fp8 layout");
    // extreme sizes: the overflow guard must answer before any product overflows
    const int big[] = {1, 7, 128, 1 << 20, INT_MAX / 2, INT_MAX};
    for (int a : big)
        for (int b : big)
            for (int hd : big) {
                const pca_status st = pca_kv_layout(a, b, hd, 16, PCA_DTYPE_BF16, &l);
                ++g_checks;
                if (st == PCA_OK) EXPECT(l.qkv_ld == ((int64_t)a + 2 * (int64_t)b) * hd, "qkv_ld %d %d %d", a, b, hd);
            }
    CALL(PCA_ERR_INVALID_ARG, 0, pca_kv_layout(INT_MAX, 1, INT_MAX, INT_MAX, PCA_DTYPE_FP8_E4M3, &l));
    CALL(PCA_ERR_INVALID_ARG, 0, pca_kv_layout(-1, 1, 128, 16, PCA_DTYPE_BF16, &l));
    CALL(PCA_ERR_UNSUPPORTED, 0, pca_kv_layout(8, 2, 128, 16, (pca_dtype)9, &l));
    CALL(PCA_ERR_INVALID_ARG, 0, pca_kv_layout(8, 2, 128, 16, PCA_DTYPE_BF16, nullptr));
}

static void gemm_checks() {
    CALL(PCA_OK, 1, pca_qkv_proj(B(A1), 4096, B(A2), 4096, B(A3), 6144, 8192, 6144, 4096, nullptr));
    EXPECT(pca::g_gemm.M == 8192 && pca::g_gemm.N == 6144 && pca::g_gemm.K == 4096 && pca::g_gemm.kv_mode == 0 &&
               pca::g_gemm.res == nullptr && pca::g_gemm.row_scale == nullptr,
           "qkv_proj args");
    const int64_t sizes[] = {-1, 0, 1, 7, 8, INT32_MAX, (int64_t)INT32_MAX + 1, INT64_MAX / 4};
    for (int64_t M : sizes)
        for (int64_t K : sizes) {
            const int before = pca::g_launches;
            const pca_status st = pca_qkv_proj(B(A1), K > 8 ? K : 8, B(A2), K > 8 ? K : 8, B(A3), 64, M, 64, K, nullptr);
            ++g_checks;
            EXPECT((st == PCA_OK) == (pca::g_launches == before + 1), "launch iff OK (M=%lld K=%lld)", (long long)M,
                   (long long)K);
        }
    CALL(PCA_ERR_INVALID_ARG, 0, pca_qkv_proj(nullptr, 64, B(A2), 64, B(A3), 64, 4, 4, 64, nullptr));
    CALL(PCA_ERR_INVALID_ARG, 0, pca_qkv_proj(B(A1), INT64_MAX, B(A2), 64, B(A3), 64, 4, 4, 64, nullptr));
    CALL(PCA_ERR_INVALID_ARG, 0, pca_qkv_proj(B(A1), 64, B(A2), 64, B(A3), INT64_MIN, 4, 4, 64, nullptr));
    // residual: in place and separate, partial overlap refused
    CALL(PCA_OK, 1, pca_out_proj_residual(B(A1), 4096, B(A2), 4096, B(A4), 4096, B(A4), 4096, 64, 4096, 4096, nullptr));
    EXPECT(pca::g_gemm.res == B(A4) && pca::g_gemm.ldr == 4096, "residual args");
    CALL(PCA_ERR_INVALID_ARG, 0,
         pca_out_proj_residual(B(A1), 4096, B(A2), 4096, B(A4 + 64), 4096, B(A4), 4096, 64, 4096, 4096, nullptr));
    CALL(PCA_ERR_INVALID_ARG, 0,
         pca_out_proj_residual(B(A1), 64, B(A2), 64, B(A4), INT64_MAX, B(A5), 64, 4, 64, 64, nullptr));
    CALL(PCA_ERR_INVALID_ARG, 0,
         pca_out_proj_residual(B(A1), 64, B(A2), 64, B(A4), INT64_MAX / 16 * 8, B(A5), 64, 4, 64, 64, nullptr));
    CALL(PCA_ERR_UNSUPPORTED, 0,
         pca_qkv_proj(B(A1), INT64_MAX / 16 * 8, B(A2), 64, B(A3), 64, 4, 64, 64, nullptr));
    // RMSNorm: the statistics kernel and the GEMM (two launches)
    CALL(PCA_OK, 2, pca_rms_norm_qkv_proj(B(A1), 4096, B(A2), 4096, 1e-6f, (float*)A5, B(A3), 6144, 8192, 6144, 4096,
                                          nullptr));
    EXPECT(pca::g_gemm.row_scale == (float*)A5, "row scale");
    CALL(PCA_ERR_INVALID_ARG, 0,
         pca_rms_norm_qkv_proj(B(A1), 64, B(A2), 64, -0.0f - 1.0f, (float*)A5, B(A3), 64, 4, 64, 64, nullptr));
    // fp8 operands
    CALL(PCA_OK, 1, pca_quantize_rows_fp8(B(A1), 4096, 8192, 4096, (uint8_t*)A2, 4096, (float*)A3, nullptr));
    CALL(PCA_ERR_INVALID_ARG, 0, pca_quantize_rows_fp8(B(A1), 4096, INT64_MAX, 4096, (uint8_t*)A2, 4096, (float*)A3, nullptr));
    CALL(PCA_OK, 1, pca_qkv_proj_fp8((uint8_t*)A1, 4096, (float*)A2, (uint8_t*)A3, 4096, (float*)A4, B(A5), 6144, 8192,
                                     6144, 4096, nullptr));
    CALL(PCA_ERR_INVALID_ARG, 0, pca_qkv_proj_fp8((uint8_t*)A1, 4096, (float*)A2, (uint8_t*)A3, 4096, (float*)A4, B(A5),
                                                  6144, INT64_MAX, 6144, 4096, nullptr));
}

static void attention_checks() {
    const int32_t* cu = (const int32_t*)A5;
    CALL(PCA_OK, 1, pca_prefill_attention(B(A1), B(A2), B(A3), 6144, 6144, 6144, nullptr, 1, 8192, 8192, 32, 8, 128,
                                          0.088f, 1, B(A4), 4096, nullptr));
    EXPECT(pca::g_attn.window == 0 && pca::g_attn.block_table == nullptr && pca::g_attn.n_kv_head == 8, "attention args");
    CALL(PCA_OK, 1, pca_prefill_attention_window(B(A1), B(A2), B(A3), 6144, 6144, 6144, cu, 16, 4096, 27808, 32, 8, 128,
                                                 0.088f, 1, 1024, B(A4), 4096, nullptr));
    EXPECT(pca::g_attn.window == 1024 && pca::g_attn.num_seqs == 16, "window args");
    // split key ranges: the workspace is checked before any launch
    const int64_t wsb = pca_prefill_attention_splitkv_workspace(1, 2048, 32, 32, 128);
    EXPECT(wsb == 4096 + 256LL * 2 * 8 * 64 * 66 * 4, "split workspace bytes %lld", (long long)wsb);
    EXPECT(pca_prefill_attention_splitkv_workspace(1, 2048, 32, 7, 128) == -1 && pca_last_error()[0] != '\0',
           "split workspace of invalid sizes");
    EXPECT(pca_prefill_attention_splitkv_workspace(0, 2048, 32, 8, 128) == -1, "split workspace, no sequences");
    CALL(PCA_OK, 1, pca_prefill_attention_splitkv(B(A1), B(A2), B(A3), 12288, 12288, 12288, nullptr, 1, 2048, 2048, 32,
                                                  32, 128, 0.088f, 1, B(A4), 4096, (void*)0x10000000, wsb, nullptr));
    EXPECT(pca::g_attn.split_ws == (void*)0x10000000 && pca::g_attn.window == 0, "split args");
    CALL(PCA_ERR_INVALID_ARG, 0, pca_prefill_attention_splitkv(B(A1), B(A2), B(A3), 12288, 12288, 12288, nullptr, 1,
                                                               2048, 2048, 32, 32, 128, 0.088f, 1, B(A4), 4096,
                                                               nullptr, wsb, nullptr));
    CALL(PCA_ERR_INVALID_ARG, 0, pca_prefill_attention_splitkv(B(A1), B(A2), B(A3), 12288, 12288, 12288, nullptr, 1,
                                                               2048, 2048, 32, 32, 128, 0.088f, 1, B(A4), 4096,
                                                               (void*)0x10000080, wsb, nullptr));
    CALL(PCA_ERR_INVALID_ARG, 0, pca_prefill_attention_splitkv(B(A1), B(A2), B(A3), 12288, 12288, 12288, nullptr, 1,
                                                               2048, 2048, 32, 32, 128, 0.088f, 1, B(A4), 4096,
                                                               (void*)0x10000000, wsb - 1, nullptr));
    CALL(PCA_ERR_INVALID_ARG, 0, pca_prefill_attention_splitkv(B(A1), B(A2), B(A3), 12288, 12288, 12288, nullptr, 1,
                                                               2048, 2048, 32, 32, 128, 0.088f, 1, B(A4), 4096,
                                                               (void*)0x10000000, -1, nullptr));
    CALL(PCA_OK, 1, pca_prefill_attention(B(A1), B(A2), B(A3), 6144, 6144, 6144, nullptr, 1, 8192, 8192, 32, 8, 128,
                                          0.088f, 1, B(A4), 4096, nullptr));
    EXPECT(pca::g_attn.split_ws == nullptr, "plain attention: no split workspace");
    CALL(PCA_OK, 0, pca_prefill_attention(nullptr, nullptr, nullptr, 64, 64, 64, nullptr, 1, 0, 0, 1, 1, 64, 0.1f, 1,
                                          nullptr, 64, nullptr));
    CALL(PCA_ERR_INVALID_ARG, 0, pca_prefill_attention(B(A1), B(A2), B(A3), 6144, 6144, 6144, nullptr, 1, INT_MAX,
                                                       INT64_MAX, 32, 8, 128, 0.088f, 1, B(A4), 4096, nullptr));
    // views past 2 GiB, with strides and lengths whose byte products overflow int64
    CALL(PCA_ERR_UNSUPPORTED, 0, pca_prefill_attention(B(A1), B(A2), B(A3), 6144, 6144, 6144, (const int32_t*)A5, 2,
                                                       INT_MAX, INT64_MAX, 32, 8, 128, 0.088f, 1, B(A4), 4096, nullptr));
    CALL(PCA_ERR_UNSUPPORTED, 0, pca_prefill_attention(B(A1), B(A2), B(A3), INT64_MAX / 16 * 8, 6144, 6144, nullptr, 1,
                                                       64, 64, 32, 8, 128, 0.088f, 1, B(A4), 4096, nullptr));
    CALL(PCA_ERR_UNSUPPORTED, 0, pca_prefill_attention_fp8qk(B(A1), 6144, (uint8_t*)A2, INT64_MAX / 32 * 16, (uint8_t*)A3,
                                                             8, B(A3), 6144, nullptr, 1, 64, 64, 32, 8, 128, 0.088f, 1,
                                                             B(A4), 4096, nullptr));
    CALL(PCA_ERR_INVALID_ARG, 0, pca_prefill_attention(B(A1), B(A2), B(A3), INT64_MAX, 6144, 6144, nullptr, 1, 64, 64,
                                                       INT_MAX, 1, 128, 0.088f, 1, B(A4), 4096, nullptr));
    CALL(PCA_ERR_INVALID_ARG, 0, pca_prefill_attention_window(B(A1), B(A2), B(A3), 6144, 6144, 6144, nullptr, 1, 64, 64,
                                                              32, 8, 128, 0.088f, 1, INT_MIN, B(A4), 4096, nullptr));
    // fp8 scores
    CALL(PCA_OK, 1, pca_prefill_attention_fp8qk(B(A1), 6144, (uint8_t*)A2, 1024, (uint8_t*)A3, 8, B(A3), 6144, nullptr, 1,
                                                8192, 8192, 32, 8, 128, 0.088f, 1, B(A4), 4096, nullptr));
    EXPECT(pca::g_attn.k8 == (const uint8_t*)A2 && pca::g_attn.ldke == 8, "fp8qk args");
    CALL(PCA_OK, 1, pca_quantize_heads_fp8(B(A1), 6144, 8192, 8, 128, 1.0f, (uint8_t*)A2, 1024, (uint8_t*)A3, 8, nullptr));
    CALL(PCA_ERR_UNSUPPORTED, 0, pca_quantize_heads_fp8(B(A1), 6144, INT64_MAX, 8, 128, 1.0f, (uint8_t*)A2, 1024,
                                                        (uint8_t*)A3, 8, nullptr));
    // paged: the pools' byte size and page count reach the kernel arguments
    CALL(PCA_OK, 1, pca_prefill_attention_paged(B(A1), 4096, cu, 8, 512, 4096, cu, 8192, cu, 512, 16,
                                                PCA_DTYPE_FP8_E4M3, (void*)A2, (void*)A3, (float*)A4, (float*)A5, 4096,
                                                32, 8, 128, 0.088f, 1, B(A4), 4096, nullptr));
    EXPECT(pca::g_attn.num_pages == 4096 && pca::g_attn.pool_bytes == 4096LL * 16 * 8 * 128 &&
               pca::g_attn.k_scale == (const float*)A4,
           "paged fp8 args");
    CALL(PCA_OK, 1, pca_prefill_attention_paged(B(A1), 4096, cu, 8, 512, 4096, cu, 8192, cu, 512, 16, PCA_DTYPE_BF16,
                                                (void*)A2, (void*)A3, nullptr, nullptr, 4096, 32, 8, 128, 0.088f, 1,
                                                B(A4), 4096, nullptr));
    EXPECT(pca::g_attn.pool_bytes == 4096LL * 16 * 8 * 128 * 2 && pca::g_attn.k_scale == nullptr, "paged bf16 args");
    EXPECT(pca::g_attn.window == 0, "paged call has no window");
    CALL(PCA_OK, 1, pca_prefill_attention_paged_window(B(A1), 4096, cu, 8, 512, 4096, cu, 8192, cu, 512, 16,
                                                       PCA_DTYPE_BF16, (void*)A2, (void*)A3, nullptr, nullptr, 4096,
                                                       32, 8, 128, 0.088f, 1, 1024, B(A4), 4096, nullptr));
    EXPECT(pca::g_attn.window == 1024 && pca::g_attn.block_table == cu, "paged window args");
    CALL(PCA_ERR_INVALID_ARG, 0, pca_prefill_attention_paged_window(B(A1), 4096, cu, 8, 512, 4096, cu, 8192, cu, 512,
                                                                    16, PCA_DTYPE_BF16, (void*)A2, (void*)A3, nullptr,
                                                                    nullptr, 4096, 32, 8, 128, 0.088f, 1, INT_MIN,
                                                                    B(A4), 4096, nullptr));
    CALL(PCA_ERR_UNSUPPORTED, 0, pca_prefill_attention_paged(B(A1), 4096, cu, 8, 512, 4096, cu, INT_MAX, cu, INT_MAX, 16,
                                                             PCA_DTYPE_BF16, (void*)A2, (void*)A3, nullptr, nullptr,
                                                             INT64_MAX / 16, 32, 8, 128, 0.088f, 1, B(A4), 4096,
                                                             nullptr));
}

static void kv_checks() {
    const int32_t* bt = (const int32_t*)A5;
    CALL(PCA_OK, 1, pca_kv_cache_write(B(A1), B(A2), 6144, 6144, nullptr, 1, 8192, bt, 512, 8, 128, 16, PCA_DTYPE_BF16,
                                       (void*)A3, (void*)A4, nullptr, nullptr, 512, nullptr));
    EXPECT(pca::g_kv.num_pages == 512 && pca::g_kv.total_tokens == 8192, "kv args");
    CALL(PCA_OK, 1, pca_kv_cache_write(B(A1), B(A2), 7168, 7168, nullptr, 1, 32768, bt, 2048, 8, 128, 16,
                                       PCA_DTYPE_FP8_E4M3, (void*)A3, (void*)A4, (float*)A3, (float*)A4, 2048, nullptr));
    CALL(PCA_ERR_UNSUPPORTED, 0, pca_kv_cache_write(B(A1), B(A2), 6144, 6144, nullptr, 1, INT64_MAX / 2, bt, 512, 8, 128,
                                                    16, PCA_DTYPE_BF16, (void*)A3, (void*)A4, nullptr, nullptr, 512,
                                                    nullptr));
    CALL(PCA_ERR_UNSUPPORTED, 0, pca_kv_cache_write(B(A1), B(A2), 6144, 6144, nullptr, 1, 64, bt, 4, 8, 128, 16,
                                                    PCA_DTYPE_BF16, (void*)A3, (void*)A4, nullptr, nullptr, INT64_MAX,
                                                    nullptr));
    // fused write: every valid combination is one launch
    CALL(PCA_OK, 1, pca_qkv_proj_kv_write(B(A1), 4096, B(A2), 4096, B(A3), 6144, 8192, 4096, 32, 8, 128, nullptr, 1, bt,
                                          512, 16, PCA_DTYPE_BF16, (void*)A4, (void*)A5, nullptr, nullptr, 512, nullptr));
    EXPECT(pca::g_gemm.kv_mode == 1 && pca::g_gemm.k_col0 == 4096 && pca::g_gemm.v_col0 == 5120, "fused args");
    CALL(PCA_ERR_INVALID_ARG, 0, pca_qkv_proj_kv_write(B(A1), 4096, B(A2), 4096, B(A3), 6144, 8192, 4096, INT_MAX, 8,
                                                       128, nullptr, 1, bt, 512, 16, PCA_DTYPE_BF16, (void*)A4,
                                                       (void*)A5, nullptr, nullptr, 512, nullptr));
    CALL(PCA_OK, 1, pca_e4m3_encode((const float*)A1, (uint8_t*)A2, INT64_MAX, nullptr));
    CALL(PCA_ERR_INVALID_ARG, 0, pca_e4m3_encode((const float*)A1, (uint8_t*)A2, INT64_MIN, nullptr));
}

int main() {
    layout_checks();
    gemm_checks();
    attention_checks();
    kv_checks();
    printf("%s: %d checks, %d failures, %d launches\n", g_fail ? "FAILED" : "OK", g_checks, g_fail, pca::g_launches);
    return g_fail ? 1 : 0;
}
