// C ABI of libpca: host-side validation, then kernel launch on the caller's stream.
// Every check runs before any enqueue, so a call that fails leaves device
// memory untouched.  See include/pca.h for the contract of each call.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "pca.h"
#include "pca_abi.hpp"
#include "pca_internal.hpp"

#include <atomic>

namespace pca {

int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = -1;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n > 0 ? n : 0;
}

}  // namespace pca

namespace {

thread_local char g_err[512] = "";

pca_status vfail(pca_status st, const char* fmt, va_list ap) {
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    return st;
}

pca_status fail(pca_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vfail(st, fmt, ap);
    va_end(ap);
    return st;
}

pca_status ok() {
    g_err[0] = '\0';
    return PCA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool supported_head_dim(int hd) { return hd == 32 || hd == 64 || hd == 128; }

constexpr int64_t kMaxBufferBytes = int64_t(1) << 31;   // buffer-resource offsets stay below 2^31

// a * b * c for non-negative factors, or INT64_MAX when the product does not
// fit in int64 (so a size check against any bound refuses it)
int64_t sat_mul(int64_t a, int64_t b, int64_t c = 1) {
    int64_t r;
    if (a < 0 || b < 0 || c < 0) return INT64_MAX;
    if (__builtin_mul_overflow(a, b, &r) || __builtin_mul_overflow(r, c, &r)) return INT64_MAX;
    return r;
}

// true when a view of `rows` rows of stride `ld` elements of `elem` bytes
// reaches 2 GiB (the reach of one buffer resource)
bool view_too_big(int64_t rows, int64_t ld, int64_t elem) { return sat_mul(rows, ld, elem) >= kMaxBufferBytes; }

pca_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(PCA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// sizes of one packed-sequence batch: cu_seqlens may be null only for one sequence
pca_status check_batch(const int32_t* cu, int num_seqs, int64_t total_tokens) {
    if (num_seqs < 1) return fail(PCA_ERR_INVALID_ARG, "num_seqs must be >= 1 (got %d)", num_seqs);
    if (cu == nullptr && num_seqs != 1)
        return fail(PCA_ERR_INVALID_ARG, "cu_seqlens is NULL but num_seqs = %d (must be 1)", num_seqs);
    if (total_tokens < 0) return fail(PCA_ERR_INVALID_ARG, "total_tokens must be >= 0");
    if (cu != nullptr && ((uintptr_t)cu & 3u))
        return fail(PCA_ERR_INVALID_ARG, "cu_seqlens must be 4-byte aligned");
    return PCA_OK;
}

// Shape checks of a GEMM call; fills the GEMM part of `a` (no fused write).
pca_status check_gemm(const pca_bf16* x, int64_t ldx, const pca_bf16* w_t, int64_t ldw, pca_bf16* y, int64_t ldy,
                      int64_t M, int64_t N, int64_t K, pca::GemmArgs& a) {
    if (!x || !w_t || !y) return fail(PCA_ERR_INVALID_ARG, "null pointer (x=%p w_t=%p y=%p)", x, w_t, y);
    if (!aligned16(x) || !aligned16(w_t) || !aligned16(y))
        return fail(PCA_ERR_INVALID_ARG, "x, w_t and y must be 16-byte aligned");
    if (M < 1 || N < 1 || K < 8 || K % 8 != 0)
        return fail(PCA_ERR_INVALID_ARG, "need M >= 1, N >= 1, K >= 8 and K %% 8 == 0 (M=%lld N=%lld K=%lld)",
                    (long long)M, (long long)N, (long long)K);
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
        return fail(PCA_ERR_INVALID_ARG, "M, N, K must fit in int32");
    if (ldx < K || ldw < K || ldy < N || ldx % 8 || ldw % 8 || ldy % 8)
        return fail(PCA_ERR_INVALID_ARG, "leading dimensions must be >= the row width and multiples of 8 "
                    "(ldx=%lld ldw=%lld ldy=%lld)", (long long)ldx, (long long)ldw, (long long)ldy);
    if (view_too_big(256, ldx, 2) || view_too_big(256, ldw, 2))
        return fail(PCA_ERR_UNSUPPORTED, "row stride too large for a 256-row tile view");
    // the grid holds one workgroup per 128 x 256 tile at most
    if ((M + 127) / 128 * ((N + 255) / 256) > INT32_MAX)
        return fail(PCA_ERR_UNSUPPORTED, "M x N too large for one launch (M=%lld N=%lld)", (long long)M, (long long)N);
    memset(&a, 0, sizeof(a));
    a.x = x; a.ldx = ldx; a.w = w_t; a.ldw = ldw; a.y = y; a.ldy = ldy;
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.kv_mode = 0;
    return PCA_OK;
}

// Checks of the page-pool side of a KV-cache write (shared by the separate
// and the fused write).
pca_status check_kv_cache(const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens,
                          const int32_t* block_table, int max_pages_per_seq, int n_kv_head, int head_dim,
                          int page_size, pca_dtype cache_dtype, void* k_cache, void* v_cache,
                          float* k_scale, float* v_scale, int64_t num_pages) {
    if (!block_table || !k_cache || !v_cache) return fail(PCA_ERR_INVALID_ARG, "null block_table, k_cache or v_cache");
    if (!aligned16(k_cache) || !aligned16(v_cache))
        return fail(PCA_ERR_INVALID_ARG, "k_cache and v_cache must be 16-byte aligned");
    if ((uintptr_t)block_table & 3u) return fail(PCA_ERR_INVALID_ARG, "block_table must be 4-byte aligned");
    if (page_size != 16) return fail(PCA_ERR_UNSUPPORTED, "page_size must be 16 (got %d)", page_size);
    pca_status st = check_batch(cu_seqlens, num_seqs, total_tokens);
    if (st != PCA_OK) return st;
    if (max_pages_per_seq < 1 || num_pages < 1)
        return fail(PCA_ERR_INVALID_ARG, "max_pages_per_seq and num_pages must be >= 1");
    if (num_pages > INT32_MAX / page_size)
        return fail(PCA_ERR_UNSUPPORTED, "num_pages * page_size must be below 2^31 (num_pages=%lld)", (long long)num_pages);
    if (cache_dtype == PCA_DTYPE_BF16) {
        if (k_scale || v_scale) return fail(PCA_ERR_INVALID_ARG, "k_scale/v_scale must be NULL for a bf16 cache");
    } else if (cache_dtype == PCA_DTYPE_FP8_E4M3) {
        if (!k_scale || !v_scale) return fail(PCA_ERR_INVALID_ARG, "fp8 cache needs k_scale and v_scale");
        if (((uintptr_t)k_scale & 3u) || ((uintptr_t)v_scale & 3u))
            return fail(PCA_ERR_INVALID_ARG, "k_scale/v_scale must be 4-byte aligned");
    } else {
        return fail(PCA_ERR_UNSUPPORTED, "unknown cache dtype %d", (int)cache_dtype);
    }
    if (n_kv_head <= 0 || sat_mul(total_tokens, 2, sat_mul(n_kv_head, head_dim) / 8) >= (int64_t(1) << 31))
        return fail(PCA_ERR_UNSUPPORTED, "batch too large (total_tokens * n_kv_head * head_dim)");
    return PCA_OK;
}

}  // namespace

namespace pca {

pca_status abi_error(pca_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vfail(st, fmt, ap);
    va_end(ap);
    return st;
}

pca_status rms_norm_qkv_proj_check(const pca_bf16* x, int64_t ldx, const pca_bf16* w_t, int64_t ldw, float eps,
                                   pca_bf16* y, int64_t ldy, int64_t M, int64_t N, int64_t K) {
    GemmArgs a;
    const pca_status st = check_gemm(x, ldx, w_t, ldw, y, ldy, M, N, K, a);
    if (st != PCA_OK) return st;
    if (!(eps >= 0.0f) || eps > 1e30f) return fail(PCA_ERR_INVALID_ARG, "eps must be finite and >= 0");
    return PCA_OK;
}

pca_status rms_norm_qkv_proj_launch(const pca_bf16* x, int64_t ldx, const pca_bf16* w_t, int64_t ldw, float eps,
                                    float* inv_rms, pca_bf16* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                    void* stream) {
    GemmArgs a;
    pca_status st = check_gemm(x, ldx, w_t, ldw, y, ldy, M, N, K, a);
    if (st != PCA_OK) return st;
    a.row_scale = inv_rms;
    st = hip_status(launch_rms_stats(x, ldx, (int)M, (int)K, eps, inv_rms, (hipStream_t)stream), "rms stats launch");
    if (st != PCA_OK) return st;
    return hip_status(launch_qkv_gemm(a, (hipStream_t)stream), "rms_norm_qkv_proj launch");
}

}  // namespace pca

extern "C" {

const char* pca_last_error(void) { return g_err; }

const char* pca_version(void) { return "pca 0.1.0 gfx950"; }

pca_status pca_kv_layout(int n_head, int n_kv_head, int head_dim, int page_size,
                         pca_dtype cache_dtype, pca_kv_layout_t* out) {
    if (out == nullptr) return fail(PCA_ERR_INVALID_ARG, "out is NULL");
    if (n_head <= 0 || n_kv_head <= 0 || head_dim <= 0 || page_size <= 0)
        return fail(PCA_ERR_INVALID_ARG, "sizes must be positive (n_head=%d n_kv_head=%d head_dim=%d page_size=%d)",
                    n_head, n_kv_head, head_dim, page_size);
    if (n_head % n_kv_head != 0)
        return fail(PCA_ERR_INVALID_ARG, "n_head (%d) must be a multiple of n_kv_head (%d)", n_head, n_kv_head);
    int64_t eb;
    if (cache_dtype == PCA_DTYPE_BF16) eb = 2;
    else if (cache_dtype == PCA_DTYPE_FP8_E4M3) eb = 1;
    else return fail(PCA_ERR_UNSUPPORTED, "unknown cache dtype %d", (int)cache_dtype);
    const int64_t hd = head_dim, nq = n_head, nk = n_kv_head, ps = page_size;
    // all products below stay far from int64 overflow for int inputs: (2^31)^3 < 2^94 is not,
    // so bound the largest one explicitly
    if ((nq + 2 * nk) > (int64_t(1) << 40) / hd || ps * nk > (int64_t(1) << 40) / hd)
        return fail(PCA_ERR_INVALID_ARG, "layout sizes overflow");
    memset(out, 0, sizeof(*out));
    out->qkv_ld = (nq + 2 * nk) * hd;
    out->q_off = 0;
    out->k_off = nq * hd;
    out->v_off = (nq + nk) * hd;
    out->head_stride = hd;
    out->page_size = ps;
    out->pool_page_stride = ps * nk * hd;
    out->pool_slot_stride = nk * hd;
    out->pool_head_stride = hd;
    out->scale_page_stride = eb == 1 ? ps * nk : 0;
    out->scale_slot_stride = eb == 1 ? nk : 0;
    out->elem_bytes = eb;
    out->kv_bytes_per_token_layer = 2 * nk * hd * eb;
    out->scale_bytes_per_token_layer = eb == 1 ? 2 * nk * 4 : 0;
    out->page_bytes = ps * nk * hd * eb;
    return ok();
}

pca_status pca_qkv_proj(const pca_bf16* x, int64_t ldx, const pca_bf16* w_t, int64_t ldw,
                        pca_bf16* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* stream) {
    pca::GemmArgs a;
    pca_status st = check_gemm(x, ldx, w_t, ldw, y, ldy, M, N, K, a);
    if (st != PCA_OK) return st;
    return hip_status(pca::launch_qkv_gemm(a, (hipStream_t)stream), "qkv_proj launch");
}

pca_status pca_quantize_rows_fp8(const pca_bf16* x, int64_t ldx, int64_t M, int64_t K, uint8_t* q, int64_t ldq,
                                 float* scales, void* stream) {
    if (!x || !q || !scales) return fail(PCA_ERR_INVALID_ARG, "null x, q or scales");
    if (!aligned16(x) || !aligned16(q) || ((uintptr_t)scales & 3u))
        return fail(PCA_ERR_INVALID_ARG, "x and q must be 16-byte aligned, scales 4-byte aligned");
    if (M < 1 || K < 16 || K % 16 != 0 || M > INT32_MAX || K > INT32_MAX)
        return fail(PCA_ERR_INVALID_ARG, "need M >= 1 and K >= 16, K %% 16 == 0 (M=%lld K=%lld)", (long long)M, (long long)K);
    if (ldx < K || ldq < K || ldx % 8 || ldq % 16)
        return fail(PCA_ERR_INVALID_ARG, "ldx >= K (multiple of 8) and ldq >= K (multiple of 16) required");
    return hip_status(pca::launch_quantize_rows(x, ldx, (int)M, (int)K, q, ldq, scales, (hipStream_t)stream),
                      "quantize_rows_fp8 launch");
}

pca_status pca_qkv_proj_fp8(const uint8_t* xq, int64_t ldxq, const float* sx, const uint8_t* wq, int64_t ldwq,
                            const float* sw, pca_bf16* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* stream) {
    if (!xq || !sx || !wq || !sw || !y) return fail(PCA_ERR_INVALID_ARG, "null xq, sx, wq, sw or y");
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || ((uintptr_t)sx & 3u) || ((uintptr_t)sw & 3u))
        return fail(PCA_ERR_INVALID_ARG, "xq, wq, y must be 16-byte aligned, sx and sw 4-byte aligned");
    if (M < 1 || N < 1 || K < 16 || K % 16 != 0)
        return fail(PCA_ERR_INVALID_ARG, "need M >= 1, N >= 1, K >= 16 and K %% 16 == 0 (M=%lld N=%lld K=%lld)",
                    (long long)M, (long long)N, (long long)K);
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return fail(PCA_ERR_INVALID_ARG, "M, N, K must fit in int32");
    if (ldxq < K || ldwq < K || ldy < N || ldxq % 16 || ldwq % 16 || ldy % 8)
        return fail(PCA_ERR_INVALID_ARG, "ldxq, ldwq >= K (multiples of 16), ldy >= N (multiple of 8) required");
    if (view_too_big(256, ldxq, 1) || view_too_big(256, ldwq, 1))
        return fail(PCA_ERR_UNSUPPORTED, "row stride too large for a 256-row tile view");
    if ((M + 255) / 256 * ((N + 255) / 256) > INT32_MAX)
        return fail(PCA_ERR_UNSUPPORTED, "M x N too large for one launch (M=%lld N=%lld)", (long long)M, (long long)N);
    pca::Fp8GemmArgs a;
    a.x = xq; a.ldx = ldxq; a.sx = sx; a.w = wq; a.ldw = ldwq; a.sw = sw; a.y = y; a.ldy = ldy;
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    return hip_status(pca::launch_gemm_fp8(a, (hipStream_t)stream), "qkv_proj_fp8 launch");
}

pca_status pca_rms_norm_qkv_proj(const pca_bf16* x, int64_t ldx, const pca_bf16* w_t, int64_t ldw, float eps,
                                 float* inv_rms, pca_bf16* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                 void* stream) {
    pca_status st = pca::rms_norm_qkv_proj_check(x, ldx, w_t, ldw, eps, y, ldy, M, N, K);
    if (st != PCA_OK) return st;
    if (!inv_rms || ((uintptr_t)inv_rms & 3u)) return fail(PCA_ERR_INVALID_ARG, "inv_rms must be a 4-byte aligned device buffer");
    return pca::rms_norm_qkv_proj_launch(x, ldx, w_t, ldw, eps, inv_rms, y, ldy, M, N, K, stream);
}

pca_status pca_out_proj_residual(const pca_bf16* o, int64_t ldo, const pca_bf16* w_t, int64_t ldw,
                                 const pca_bf16* res, int64_t ldr, pca_bf16* out, int64_t ldout,
                                 int64_t M, int64_t N, int64_t K, void* stream) {
    pca::GemmArgs a;
    pca_status st = check_gemm(o, ldo, w_t, ldw, out, ldout, M, N, K, a);
    if (st != PCA_OK) return st;
    if (!res) return fail(PCA_ERR_INVALID_ARG, "null res");
    if (!aligned16(res) || ldr < N || ldr % 8)
        return fail(PCA_ERR_INVALID_ARG, "res must be 16-byte aligned with ldr >= N and a multiple of 8");
    if (res != out) {
        // res may be out itself (in-place residual update) but must not partly overlap it;
        // extents in bytes, refused when they do not fit (addresses compared as integers)
        auto extent = [](int64_t rows, int64_t ld, int64_t width) -> int64_t {
            const int64_t e = sat_mul(rows - 1, ld);
            return e >= INT64_MAX / 4 ? INT64_MAX : (e + width) * 2;
        };
        const int64_t rb = extent(M, ldr, N), ob = extent(M, ldout, N);
        if (rb == INT64_MAX || ob == INT64_MAX) return fail(PCA_ERR_INVALID_ARG, "res or out extent overflows");
        const uintptr_t r0 = (uintptr_t)res, o0 = (uintptr_t)out;
        if (r0 < o0 + (uint64_t)ob && o0 < r0 + (uint64_t)rb)
            return fail(PCA_ERR_INVALID_ARG, "res overlaps out without being out");
    } else if (ldr != ldout) {
        return fail(PCA_ERR_INVALID_ARG, "in-place residual needs ldr == ldout");
    }
    a.res = res;
    a.ldr = ldr;
    return hip_status(pca::launch_qkv_gemm(a, (hipStream_t)stream), "out_proj_residual launch");
}

pca_status pca_qkv_proj_kv_write(const pca_bf16* x, int64_t ldx, const pca_bf16* w_t, int64_t ldw,
                                 pca_bf16* y, int64_t ldy, int64_t M, int64_t K,
                                 int n_head, int n_kv_head, int head_dim,
                                 const int32_t* cu_seqlens, int num_seqs,
                                 const int32_t* block_table, int max_pages_per_seq, int page_size,
                                 pca_dtype cache_dtype, void* k_cache, void* v_cache,
                                 float* k_scale, float* v_scale, int64_t num_pages, void* stream) {
    if (n_head <= 0 || n_kv_head <= 0 || n_head % n_kv_head != 0)
        return fail(PCA_ERR_INVALID_ARG, "need n_head, n_kv_head > 0 and n_head %% n_kv_head == 0 (%d, %d)",
                    n_head, n_kv_head);
    if (!supported_head_dim(head_dim))
        return fail(PCA_ERR_UNSUPPORTED, "head_dim %d not supported (32, 64 or 128)", head_dim);
    const int64_t N = ((int64_t)n_head + 2 * (int64_t)n_kv_head) * head_dim;
    pca::GemmArgs a;
    pca_status st = check_gemm(x, ldx, w_t, ldw, y, ldy, M, N, K, a);
    if (st != PCA_OK) return st;
    st = check_kv_cache(cu_seqlens, num_seqs, M, block_table, max_pages_per_seq, n_kv_head, head_dim,
                        page_size, cache_dtype, k_cache, v_cache, k_scale, v_scale, num_pages);
    if (st != PCA_OK) return st;
    const int64_t nkc = (int64_t)n_kv_head * head_dim;
    if (cache_dtype == PCA_DTYPE_FP8_E4M3 && (((int64_t)n_head * head_dim) % 128 != 0 || nkc % 128 != 0))
        return fail(PCA_ERR_UNSUPPORTED, "fused fp8 write needs n_head*head_dim and n_kv_head*head_dim to be "
                    "multiples of 128 (got %d*%d, %d*%d)", n_head, head_dim, n_kv_head, head_dim);
    a.kv_mode = cache_dtype == PCA_DTYPE_BF16 ? 1 : 2;
    a.k_col0 = n_head * head_dim;
    a.v_col0 = (int)(a.k_col0 + nkc);
    a.kv.k = nullptr; a.kv.v = nullptr; a.kv.ldk = 0; a.kv.ldv = 0;
    a.kv.cu_seqlens = cu_seqlens; a.kv.num_seqs = num_seqs; a.kv.total_tokens = M;
    a.kv.block_table = block_table; a.kv.max_pages_per_seq = max_pages_per_seq;
    a.kv.n_kv_head = n_kv_head; a.kv.head_dim = head_dim; a.kv.page_size = page_size;
    a.kv.k_cache = k_cache; a.kv.v_cache = v_cache; a.kv.k_scale = k_scale; a.kv.v_scale = v_scale;
    a.kv.num_pages = num_pages;
    return hip_status(pca::launch_qkv_gemm(a, (hipStream_t)stream), "qkv_proj_kv_write launch");
}

pca_status pca_prefill_attention(const pca_bf16* q, const pca_bf16* k, const pca_bf16* v,
                                 int64_t ldq, int64_t ldk, int64_t ldv,
                                 const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                                 int64_t total_tokens, int n_head, int n_kv_head, int head_dim,
                                 float scale, int causal, pca_bf16* o, int64_t ldo, void* stream) {
    return pca_prefill_attention_window(q, k, v, ldq, ldk, ldv, cu_seqlens, num_seqs, max_seqlen, total_tokens,
                                        n_head, n_kv_head, head_dim, scale, causal, 0, o, ldo, stream);
}

namespace {
// the token-major attention calls: plain, sliding window, split key ranges
pca_status prefill_attention_impl(const pca_bf16* q, const pca_bf16* k, const pca_bf16* v,
                                  int64_t ldq, int64_t ldk, int64_t ldv,
                                  const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                                  int64_t total_tokens, int n_head, int n_kv_head, int head_dim,
                                  float scale, int causal, int window, void* split_ws, int64_t split_ws_bytes,
                                  pca_bf16* o, int64_t ldo, void* stream) {
    if (window < 0) return fail(PCA_ERR_INVALID_ARG, "window must be >= 0 (0: no window), got %d", window);
    if (total_tokens == 0 && num_seqs >= 1 && causal == 1) return ok();   // empty batch: nothing to read or write
    if (!q || !k || !v || !o) return fail(PCA_ERR_INVALID_ARG, "null q, k, v or o");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(PCA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
    if (causal != 1) return fail(PCA_ERR_INVALID_ARG, "only causal attention (causal = 1) is provided");
    if (n_head <= 0 || n_kv_head <= 0 || n_head % n_kv_head != 0)
        return fail(PCA_ERR_INVALID_ARG, "need n_head, n_kv_head > 0 and n_head %% n_kv_head == 0 (%d, %d)",
                    n_head, n_kv_head);
    if (!supported_head_dim(head_dim))
        return fail(PCA_ERR_UNSUPPORTED, "head_dim %d not supported (32, 64 or 128)", head_dim);
    pca_status st = check_batch(cu_seqlens, num_seqs, total_tokens);
    if (st != PCA_OK) return st;
    if (!(scale > 0.0f) || scale != scale || scale > 1e30f) return fail(PCA_ERR_INVALID_ARG, "scale must be finite and > 0");
    if (ldq < (int64_t)n_head * head_dim || ldk < (int64_t)n_kv_head * head_dim ||
        ldv < (int64_t)n_kv_head * head_dim || ldo < (int64_t)n_head * head_dim ||
        ldq % 8 || ldk % 8 || ldv % 8 || ldo % 8)
        return fail(PCA_ERR_INVALID_ARG, "row strides must cover the heads and be multiples of 8 "
                    "(ldq=%lld ldk=%lld ldv=%lld ldo=%lld)", (long long)ldq, (long long)ldk, (long long)ldv, (long long)ldo);
    if (total_tokens == 0) return ok();
    if (max_seqlen < 1 || (cu_seqlens == nullptr && max_seqlen < total_tokens))
        return fail(PCA_ERR_INVALID_ARG, "max_seqlen must be >= 1 and cover the sequence (got %d)", max_seqlen);
    // each sequence is read through its own buffer view, which must stay below 2 GiB
    const int64_t longest = cu_seqlens ? (max_seqlen < total_tokens ? max_seqlen : total_tokens) : total_tokens;
    if (view_too_big(longest, ldq, 2) || view_too_big(longest, ldk, 2) || view_too_big(longest, ldv, 2))
        return fail(PCA_ERR_UNSUPPORTED, "per-sequence q/k/v views beyond 2 GiB are not supported");
    pca::AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q; a.k = k; a.v = v; a.ldq = ldq; a.ldk = ldk; a.ldv = ldv;
    a.cu_seqlens = cu_seqlens; a.num_seqs = num_seqs; a.max_seqlen = max_seqlen;
    a.total_tokens = total_tokens; a.n_head = n_head; a.n_kv_head = n_kv_head; a.head_dim = head_dim;
    a.scale = scale; a.o = o; a.ldo = ldo;
    a.window = window;
    if (split_ws_bytes >= 0) {
        if (!split_ws) return fail(PCA_ERR_INVALID_ARG, "null workspace");
        if ((uintptr_t)split_ws & 255u) return fail(PCA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
        const int64_t need = pca::attention_split_workspace(num_seqs, max_seqlen, n_head, n_kv_head, head_dim);
        if (split_ws_bytes < need)
            return fail(PCA_ERR_INVALID_ARG, "workspace of %lld bytes, %lld needed", (long long)split_ws_bytes,
                        (long long)need);
        a.split_ws = split_ws;
    }
    return hip_status(pca::launch_attention(a, (hipStream_t)stream), "prefill_attention launch");
}
}  // namespace

pca_status pca_prefill_attention_window(const pca_bf16* q, const pca_bf16* k, const pca_bf16* v,
                                        int64_t ldq, int64_t ldk, int64_t ldv,
                                        const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                                        int64_t total_tokens, int n_head, int n_kv_head, int head_dim,
                                        float scale, int causal, int window, pca_bf16* o, int64_t ldo,
                                        void* stream) {
    return prefill_attention_impl(q, k, v, ldq, ldk, ldv, cu_seqlens, num_seqs, max_seqlen, total_tokens, n_head,
                                  n_kv_head, head_dim, scale, causal, window, nullptr, -1, o, ldo, stream);
}

int64_t pca_prefill_attention_splitkv_workspace(int num_seqs, int max_seqlen, int n_head, int n_kv_head,
                                                int head_dim) {
    if (num_seqs < 1 || max_seqlen < 1 || n_head <= 0 || n_kv_head <= 0 || n_head % n_kv_head != 0 ||
        !supported_head_dim(head_dim)) {
        fail(PCA_ERR_INVALID_ARG, "need num_seqs, max_seqlen >= 1, n_head %% n_kv_head == 0 and head_dim "
             "32, 64 or 128 (%d, %d, %d, %d, %d)", num_seqs, max_seqlen, n_head, n_kv_head, head_dim);
        return -1;
    }
    return pca::attention_split_workspace(num_seqs, max_seqlen, n_head, n_kv_head, head_dim);
}

pca_status pca_prefill_attention_splitkv(const pca_bf16* q, const pca_bf16* k, const pca_bf16* v,
                                         int64_t ldq, int64_t ldk, int64_t ldv,
                                         const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                                         int64_t total_tokens, int n_head, int n_kv_head, int head_dim,
                                         float scale, int causal, pca_bf16* o, int64_t ldo,
                                         void* workspace, int64_t workspace_bytes, void* stream) {
    if (workspace_bytes < 0) return fail(PCA_ERR_INVALID_ARG, "workspace_bytes must be >= 0");
    return prefill_attention_impl(q, k, v, ldq, ldk, ldv, cu_seqlens, num_seqs, max_seqlen, total_tokens, n_head,
                                  n_kv_head, head_dim, scale, causal, 0, workspace, workspace_bytes, o, ldo,
                                  stream);
}

pca_status pca_prefill_attention_fp8qk(const pca_bf16* q, int64_t ldq, const uint8_t* k_codes, int64_t ldk,
                                       const uint8_t* k_exps, int64_t lde, const pca_bf16* v, int64_t ldv,
                                       const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                                       int64_t total_tokens, int n_head, int n_kv_head, int head_dim,
                                       float scale, int causal, pca_bf16* o, int64_t ldo, void* stream) {
    if (total_tokens == 0 && num_seqs >= 1 && causal == 1) return ok();   // empty batch: nothing to read or write
    if (!q || !k_codes || !k_exps || !v || !o) return fail(PCA_ERR_INVALID_ARG, "null q, k_codes, k_exps, v or o");
    if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v) || !aligned16(o) || ((uintptr_t)k_exps & 3u))
        return fail(PCA_ERR_INVALID_ARG, "q, k_codes, v and o must be 16-byte aligned, k_exps 4-byte aligned");
    if (causal != 1) return fail(PCA_ERR_INVALID_ARG, "only causal attention (causal = 1) is provided");
    if (n_head <= 0 || n_kv_head <= 0 || n_head % n_kv_head != 0)
        return fail(PCA_ERR_INVALID_ARG, "need n_head, n_kv_head > 0 and n_head %% n_kv_head == 0 (%d, %d)",
                    n_head, n_kv_head);
    if (head_dim != 128) return fail(PCA_ERR_UNSUPPORTED, "fp8 score operands need head_dim 128 (got %d)", head_dim);
    pca_status st = check_batch(cu_seqlens, num_seqs, total_tokens);
    if (st != PCA_OK) return st;
    if (!(scale > 0.0f) || scale != scale || scale > 1e30f) return fail(PCA_ERR_INVALID_ARG, "scale must be finite and > 0");
    if (ldq < (int64_t)n_head * head_dim || ldk < (int64_t)n_kv_head * head_dim || lde < n_kv_head ||
        ldv < (int64_t)n_kv_head * head_dim || ldo < (int64_t)n_head * head_dim ||
        ldq % 8 || ldk % 16 || lde % 4 || ldv % 8 || ldo % 8)
        return fail(PCA_ERR_INVALID_ARG, "row strides must cover the heads; ldq, ldv, ldo multiples of 8, ldk of 16, lde of 4 "
                    "(ldq=%lld ldk=%lld lde=%lld ldv=%lld ldo=%lld)", (long long)ldq, (long long)ldk, (long long)lde,
                    (long long)ldv, (long long)ldo);
    if (total_tokens == 0) return ok();
    if (max_seqlen < 1 || (cu_seqlens == nullptr && max_seqlen < total_tokens))
        return fail(PCA_ERR_INVALID_ARG, "max_seqlen must be >= 1 and cover the sequence (got %d)", max_seqlen);
    const int64_t longest = cu_seqlens ? (max_seqlen < total_tokens ? max_seqlen : total_tokens) : total_tokens;
    if (view_too_big(longest, ldq, 2) || view_too_big(longest, ldk, 1) || view_too_big(longest, lde, 1) ||
        view_too_big(longest, ldv, 2))
        return fail(PCA_ERR_UNSUPPORTED, "per-sequence q/k/v views beyond 2 GiB are not supported");
    pca::AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q; a.v = v; a.ldq = ldq; a.ldv = ldv;
    a.k8 = k_codes; a.ldk8 = ldk; a.kex = k_exps; a.ldke = lde;
    a.cu_seqlens = cu_seqlens; a.num_seqs = num_seqs; a.max_seqlen = max_seqlen;
    a.total_tokens = total_tokens; a.n_head = n_head; a.n_kv_head = n_kv_head; a.head_dim = head_dim;
    a.scale = scale; a.o = o; a.ldo = ldo;
    return hip_status(pca::launch_attention(a, (hipStream_t)stream), "prefill_attention_fp8qk launch");
}

namespace {
pca_status prefill_attention_paged_impl(const pca_bf16* q, int64_t ldq, const int32_t* cu_seqlens_q, int num_seqs,
                                        int max_seqlen_q, int64_t total_q, const int32_t* ctx_lens, int max_ctx_len,
                                        const int32_t* block_table, int max_pages_per_seq, int page_size,
                                        pca_dtype cache_dtype, const void* k_cache, const void* v_cache,
                                        const float* k_scale, const float* v_scale, int64_t num_pages,
                                        int n_head, int n_kv_head, int head_dim, float scale, int causal, int window,
                                        pca_bf16* o, int64_t ldo, void* stream) {
    if (window < 0) return fail(PCA_ERR_INVALID_ARG, "window must be >= 0 (0: no window), got %d", window);
    if (total_q == 0 && num_seqs >= 1 && causal == 1) return ok();   // empty batch: nothing to read or write
    if (!q || !o || !k_cache || !v_cache || !block_table || !ctx_lens)
        return fail(PCA_ERR_INVALID_ARG, "null q, o, k_cache, v_cache, block_table or ctx_lens");
    if (!aligned16(q) || !aligned16(o) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PCA_ERR_INVALID_ARG, "q, o, k_cache and v_cache must be 16-byte aligned");
    if (((uintptr_t)block_table & 3u) || ((uintptr_t)ctx_lens & 3u))
        return fail(PCA_ERR_INVALID_ARG, "block_table and ctx_lens must be 4-byte aligned");
    if (causal != 1) return fail(PCA_ERR_INVALID_ARG, "only causal attention (causal = 1) is provided");
    if (n_head <= 0 || n_kv_head <= 0 || n_head % n_kv_head != 0)
        return fail(PCA_ERR_INVALID_ARG, "need n_head, n_kv_head > 0 and n_head %% n_kv_head == 0 (%d, %d)",
                    n_head, n_kv_head);
    if (!supported_head_dim(head_dim))
        return fail(PCA_ERR_UNSUPPORTED, "head_dim %d not supported (32, 64 or 128)", head_dim);
    if (page_size != 16) return fail(PCA_ERR_UNSUPPORTED, "page_size must be 16 (got %d)", page_size);
    int64_t elem;
    if (cache_dtype == PCA_DTYPE_BF16) {
        if (k_scale || v_scale) return fail(PCA_ERR_INVALID_ARG, "k_scale/v_scale must be NULL for a bf16 cache");
        elem = 2;
    } else if (cache_dtype == PCA_DTYPE_FP8_E4M3) {
        if (!k_scale || !v_scale) return fail(PCA_ERR_INVALID_ARG, "an fp8 cache needs k_scale and v_scale");
        if (((uintptr_t)k_scale & 3u) || ((uintptr_t)v_scale & 3u))
            return fail(PCA_ERR_INVALID_ARG, "k_scale/v_scale must be 4-byte aligned");
        elem = 1;
    } else {
        return fail(PCA_ERR_UNSUPPORTED, "unknown cache dtype %d", (int)cache_dtype);
    }
    pca_status st = check_batch(cu_seqlens_q, num_seqs, total_q);
    if (st != PCA_OK) return st;
    if (!(scale > 0.0f) || scale != scale || scale > 1e30f) return fail(PCA_ERR_INVALID_ARG, "scale must be finite and > 0");
    if (ldq < (int64_t)n_head * head_dim || ldo < (int64_t)n_head * head_dim || ldq % 8 || ldo % 8)
        return fail(PCA_ERR_INVALID_ARG, "ldq/ldo must cover n_head*head_dim and be multiples of 8");
    if (max_pages_per_seq < 1 || num_pages < 1)
        return fail(PCA_ERR_INVALID_ARG, "max_pages_per_seq and num_pages must be >= 1");
    if (total_q == 0) return ok();
    if (max_seqlen_q < 1 || (cu_seqlens_q == nullptr && max_seqlen_q < total_q))
        return fail(PCA_ERR_INVALID_ARG, "max_seqlen_q must be >= 1 and cover the chunk (got %d)", max_seqlen_q);
    if (max_ctx_len < max_seqlen_q || (int64_t)max_ctx_len > (int64_t)max_pages_per_seq * page_size)
        return fail(PCA_ERR_INVALID_ARG, "max_ctx_len (%d) must be >= max_seqlen_q and <= max_pages_per_seq * page_size",
                    max_ctx_len);
    const int64_t pool_bytes = sat_mul(num_pages, page_size, sat_mul(n_kv_head, head_dim, elem));
    if (pool_bytes >= kMaxBufferBytes) return fail(PCA_ERR_UNSUPPORTED, "page pools of 2 GiB or more are not supported");
    // LDS: 4 bf16 tiles (+ 4 fp8 staging tiles) + the staged block-table row
    const int64_t lds = 4 * 64 * (int64_t)head_dim * (elem == 1 ? 3 : 2) + (((int64_t)max_ctx_len + 15) / 16 + 3) / 4 * 16;
    if (lds > 160 * 1024) return fail(PCA_ERR_UNSUPPORTED, "max_ctx_len %d too long for the staged block table", max_ctx_len);
    const int64_t longest = cu_seqlens_q ? (max_seqlen_q < total_q ? max_seqlen_q : total_q) : total_q;
    if (view_too_big(longest, ldq, 2)) return fail(PCA_ERR_UNSUPPORTED, "per-sequence q views beyond 2 GiB");
    pca::AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q; a.k = (const uint16_t*)k_cache; a.v = (const uint16_t*)v_cache; a.ldq = ldq;
    a.cu_seqlens = cu_seqlens_q; a.num_seqs = num_seqs; a.max_seqlen = max_seqlen_q;
    a.total_tokens = total_q; a.n_head = n_head; a.n_kv_head = n_kv_head; a.head_dim = head_dim;
    a.scale = scale; a.o = o; a.ldo = ldo;
    a.block_table = block_table; a.max_pages_per_seq = max_pages_per_seq; a.ctx_lens = ctx_lens;
    a.max_ctx = max_ctx_len; a.pool_bytes = pool_bytes; a.num_pages = num_pages;
    a.k_scale = elem == 1 ? k_scale : nullptr; a.v_scale = elem == 1 ? v_scale : nullptr;
    a.window = window;
    return hip_status(pca::launch_attention(a, (hipStream_t)stream), "prefill_attention_paged launch");
}
}  // namespace

pca_status pca_prefill_attention_paged(const pca_bf16* q, int64_t ldq, const int32_t* cu_seqlens_q, int num_seqs,
                                       int max_seqlen_q, int64_t total_q, const int32_t* ctx_lens, int max_ctx_len,
                                       const int32_t* block_table, int max_pages_per_seq, int page_size,
                                       pca_dtype cache_dtype, const void* k_cache, const void* v_cache,
                                       const float* k_scale, const float* v_scale, int64_t num_pages,
                                       int n_head, int n_kv_head, int head_dim, float scale, int causal,
                                       pca_bf16* o, int64_t ldo, void* stream) {
    return prefill_attention_paged_impl(q, ldq, cu_seqlens_q, num_seqs, max_seqlen_q, total_q, ctx_lens, max_ctx_len,
                                        block_table, max_pages_per_seq, page_size, cache_dtype, k_cache, v_cache,
                                        k_scale, v_scale, num_pages, n_head, n_kv_head, head_dim, scale, causal, 0, o,
                                        ldo, stream);
}

pca_status pca_prefill_attention_paged_window(const pca_bf16* q, int64_t ldq, const int32_t* cu_seqlens_q,
                                              int num_seqs, int max_seqlen_q, int64_t total_q,
                                              const int32_t* ctx_lens, int max_ctx_len, const int32_t* block_table,
                                              int max_pages_per_seq, int page_size, pca_dtype cache_dtype,
                                              const void* k_cache, const void* v_cache, const float* k_scale,
                                              const float* v_scale, int64_t num_pages, int n_head, int n_kv_head,
                                              int head_dim, float scale, int causal, int window, pca_bf16* o,
                                              int64_t ldo, void* stream) {
    return prefill_attention_paged_impl(q, ldq, cu_seqlens_q, num_seqs, max_seqlen_q, total_q, ctx_lens, max_ctx_len,
                                        block_table, max_pages_per_seq, page_size, cache_dtype, k_cache, v_cache,
                                        k_scale, v_scale, num_pages, n_head, n_kv_head, head_dim, scale, causal,
                                        window, o, ldo, stream);
}

pca_status pca_kv_cache_write(const pca_bf16* k, const pca_bf16* v, int64_t ldk, int64_t ldv,
                              const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens,
                              const int32_t* block_table, int max_pages_per_seq,
                              int n_kv_head, int head_dim, int page_size, pca_dtype cache_dtype,
                              void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              int64_t num_pages, void* stream) {
    if (total_tokens == 0 && num_seqs >= 1) return ok();   // empty batch: nothing to read or write
    if (!k || !v) return fail(PCA_ERR_INVALID_ARG, "null k or v");
    if (!aligned16(k) || !aligned16(v)) return fail(PCA_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
    if (n_kv_head <= 0) return fail(PCA_ERR_INVALID_ARG, "n_kv_head must be > 0");
    if (!supported_head_dim(head_dim))
        return fail(PCA_ERR_UNSUPPORTED, "head_dim %d not supported (32, 64 or 128)", head_dim);
    if (ldk < (int64_t)n_kv_head * head_dim || ldv < (int64_t)n_kv_head * head_dim || ldk % 8 || ldv % 8)
        return fail(PCA_ERR_INVALID_ARG, "ldk/ldv must cover n_kv_head*head_dim and be multiples of 8");
    pca_status st = check_kv_cache(cu_seqlens, num_seqs, total_tokens, block_table, max_pages_per_seq, n_kv_head,
                                   head_dim, page_size, cache_dtype, k_cache, v_cache, k_scale, v_scale, num_pages);
    if (st != PCA_OK) return st;
    if (total_tokens == 0) return ok();
    pca::KvWriteArgs a;
    a.k = k; a.v = v; a.ldk = ldk; a.ldv = ldv;
    a.cu_seqlens = cu_seqlens; a.num_seqs = num_seqs; a.total_tokens = total_tokens;
    a.block_table = block_table; a.max_pages_per_seq = max_pages_per_seq;
    a.n_kv_head = n_kv_head; a.head_dim = head_dim; a.page_size = page_size;
    a.k_cache = k_cache; a.v_cache = v_cache; a.k_scale = k_scale; a.v_scale = v_scale;
    a.num_pages = num_pages;
    hipError_t e = cache_dtype == PCA_DTYPE_BF16 ? pca::launch_kv_write_bf16(a, (hipStream_t)stream)
                                                 : pca::launch_kv_write_fp8(a, (hipStream_t)stream);
    return hip_status(e, "kv_cache_write launch");
}

pca_status pca_quantize_heads_fp8(const pca_bf16* x, int64_t ldx, int64_t T, int n_heads, int head_dim, float prescale,
                                  uint8_t* codes, int64_t ldc, uint8_t* exps, int64_t lde, void* stream) {
    if (T == 0) return ok();
    if (T < 0 || n_heads < 1) return fail(PCA_ERR_INVALID_ARG, "need T >= 0 and n_heads >= 1");
    if (!x || !codes || !exps) return fail(PCA_ERR_INVALID_ARG, "null x, codes or exps");
    if (!supported_head_dim(head_dim))
        return fail(PCA_ERR_UNSUPPORTED, "head_dim %d not supported (32, 64 or 128)", head_dim);
    if (!aligned16(x) || ((uintptr_t)codes & 7u))
        return fail(PCA_ERR_INVALID_ARG, "x must be 16-byte aligned, codes 8-byte aligned");
    const int64_t w = (int64_t)n_heads * head_dim;
    if (ldx < w || ldx % 8 || ldc < w || ldc % 8 || lde < n_heads)
        return fail(PCA_ERR_INVALID_ARG, "ldx, ldc >= n_heads*head_dim (multiples of 8) and lde >= n_heads required");
    if (!(prescale > 0.0f && prescale <= 3.40282347e38f)) return fail(PCA_ERR_INVALID_ARG, "prescale must be finite and > 0");
    if (sat_mul(T, w) / 8 >= (int64_t(1) << 40)) return fail(PCA_ERR_UNSUPPORTED, "input too large");
    return hip_status(pca::launch_quantize_heads(x, ldx, T, n_heads, head_dim, prescale, codes, ldc, exps, lde,
                                                 (hipStream_t)stream),
                      "quantize_heads_fp8 launch");
}

pca_status pca_e4m3_encode(const float* x, uint8_t* codes, int64_t n, void* stream) {
    if (n == 0) return ok();
    if (n < 0) return fail(PCA_ERR_INVALID_ARG, "n must be >= 0 (n=%lld)", (long long)n);
    if (!x || !codes) return fail(PCA_ERR_INVALID_ARG, "null x or codes");
    if (!aligned16(x) || ((uintptr_t)codes & 3u))
        return fail(PCA_ERR_INVALID_ARG, "x must be 16-byte aligned, codes 4-byte aligned");
    return hip_status(pca::launch_e4m3_encode(x, codes, n, (hipStream_t)stream), "e4m3_encode launch");
}

}  // extern "C"
