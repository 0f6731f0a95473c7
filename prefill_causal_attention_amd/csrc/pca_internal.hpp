// Internal launch entry points of libpca (host side).  Arguments have been
// validated by the C ABI layer (pca_api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pca {

struct KvWriteArgs {
    const uint16_t* k;
    const uint16_t* v;
    int64_t ldk, ldv;
    const int32_t* cu_seqlens;   // may be null: one sequence
    int num_seqs;
    int64_t total_tokens;
    const int32_t* block_table;
    int max_pages_per_seq;
    int n_kv_head, head_dim, page_size;
    void* k_cache;
    void* v_cache;
    float* k_scale;
    float* v_scale;
    int64_t num_pages;
    int wave_lookup = 0;          // separate KV write only: slots looked up per wave (set by its launcher)
};

hipError_t launch_kv_write_bf16(const KvWriteArgs& a, hipStream_t s);
hipError_t launch_kv_write_fp8(const KvWriteArgs& a, hipStream_t s);
// q[i] = E4M3 code of x[i] (RNE, saturating), i < n
hipError_t launch_e4m3_encode(const float* x, uint8_t* q, int64_t n, hipStream_t s);

struct GemmArgs {
    const uint16_t* x;
    int64_t ldx;
    const uint16_t* w;   // (N, K) row-major
    int64_t ldw;
    uint16_t* y;
    int64_t ldy;
    int M, N, K;
    // optional KV-cache write of y's K and V columns from the epilogue
    int kv_mode;          // 0: none, 1: bf16 cache, 2: fp8 E4M3 cache
    int k_col0, v_col0;   // first K / V column of y; each range is n_kv_head * head_dim wide
    KvWriteArgs kv;       // cache side (kv.k, kv.v, kv.ldk, kv.ldv unused; tokens are y's rows)
    // optional residual: y = x w^T + res (res may be y itself)
    const uint16_t* res;
    int64_t ldr;
    // optional per-row scale of the product (RMSNorm's 1 / rms): y[m] = row_scale[m] * (x w^T)[m]
    const float* row_scale;
};

hipError_t launch_qkv_gemm(const GemmArgs& a, hipStream_t s);

// fp8 GEMM: y[m, n] = RNE_bf16(sx[m] * sw[n] * sum_k dec(x[m, k]) dec(w[n, k])), E4M3 codes
struct Fp8GemmArgs {
    const uint8_t* x;
    int64_t ldx;
    const float* sx;
    const uint8_t* w;   // (N, K) row-major codes
    int64_t ldw;
    const float* sw;
    uint16_t* y;
    int64_t ldy;
    int M, N, K;
};

hipError_t launch_gemm_fp8(const Fp8GemmArgs& a, hipStream_t s);

// Row-wise E4M3 quantisation (absmax scale per row), the fp8 KV cache's rule
hipError_t launch_quantize_rows(const uint16_t* x, int64_t ldx, int M, int K, uint8_t* q, int64_t ldq, float* scales,
                                hipStream_t s);

// Per-(token, head) E4M3 rows of x * prescale with power-of-two scales
// (codes (T, H*hd) stride ldq, scale bytes e + 127 (T, H) stride lde)
hipError_t launch_quantize_heads(const uint16_t* x, int64_t ldx, int64_t T, int H, int hd, float prescale, uint8_t* q,
                                 int64_t ldq, uint8_t* ex, int64_t lde, hipStream_t s);

// inv_rms[m] = 1 / sqrt(mean_k x[m, k]^2 + eps) for the M rows of x (K columns)
hipError_t launch_rms_stats(const uint16_t* x, int64_t ldx, int M, int K, float eps, float* inv_rms, hipStream_t s);

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    int64_t ldq, ldk, ldv;
    const int32_t* cu_seqlens;   // may be null: one sequence
    int num_seqs;
    int max_seqlen;
    int64_t total_tokens;
    int n_head, n_kv_head, head_dim;
    float scale;
    uint16_t* o;
    int64_t ldo;
    // paged K/V (a chunk over a cached prefix); block_table == null: k, v are
    // token-major rows of the chunk itself
    const int32_t* block_table;   // [num_seqs][max_pages_per_seq]
    int max_pages_per_seq;
    const int32_t* ctx_lens;      // [num_seqs] keys per sequence (prefix + chunk)
    int max_ctx;
    int64_t pool_bytes;           // bytes of the K (and of the V) pool, < 2^31
    int64_t num_pages;            // pages per pool (block-table entries outside [0, num_pages) read zeros)
    int window;                   // > 0: sliding window of that many keys (row r sees r - window < c <= r)
    const float* k_scale;         // paged fp8 pools: per-(slot, kv head) scales; null for bf16 pools
    const float* v_scale;
    // fp8 score operands (k unused): K as E4M3 codes (token rows, stride ldk8
    // bytes) with power-of-two scale bytes (token rows of n_kv, stride ldke);
    // Q is quantised inside the kernel
    const uint8_t* k8;
    int64_t ldk8;
    const uint8_t* kex;
    int64_t ldke;
    // split key ranges for shallow grids: a zeroed-once workspace of at least
    // attention_split_workspace(...) bytes (null: never split)
    void* split_ws;
};

hipError_t launch_attention(const AttnArgs& a, hipStream_t s);

// Split-key-range workspace.  One slot per task group (8 waves of 32 query
// rows that share a kv head), at most kSplitMaxSlots of them when the split
// runs: first the slots' 4-byte arrival counters, in a block of fixed size
// (so calls of different sizes on one workspace never write partial results
// where another size keeps counters), then per slot two chunks' partials of
// 8 waves x 64 lanes x (head_dim / 2 accumulators + reference + half-row sum)
// fp32.
constexpr int64_t kSplitMaxSlots = 1024;
constexpr int64_t kSplitCounterBytes = kSplitMaxSlots * 4;
inline int64_t attention_split_slots(int num_seqs, int max_seqlen, int n_head, int n_kv_head) {
    const int64_t G = n_head / n_kv_head;
    const int64_t ntg = (G * ((max_seqlen + 31) / 32) + 7) / 8;
    return (int64_t)num_seqs * n_kv_head * ntg;
}
inline int64_t attention_split_workspace(int num_seqs, int max_seqlen, int n_head, int n_kv_head, int head_dim) {
    int64_t slots = attention_split_slots(num_seqs, max_seqlen, n_head, n_kv_head);
    if (slots > kSplitMaxSlots) slots = kSplitMaxSlots;   // more never split
    return kSplitCounterBytes + slots * 2 * 8 * 64 * (head_dim / 2 + 2) * 4;
}

// Compute units of the current device (looked up once per device; 0 if
// unknown).  Grids deeper than one workgroup per CU launch one per CU and
// loop over their work.
int device_cus();

}  // namespace pca
