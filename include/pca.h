/*
 * pca.h -- C ABI of libpca, the prefill attention-unit path on MI355X (gfx950).
 *
 * The path is the prefill forward of one decoder layer's attention unit as the
 * "Prefill decoder-layer attention data flow" article (hncyxsy.com/news/270449)
 * lays it out: one fused QKV projection GEMM (§1.2, §2.1, §4.1), the head
 * split by stride (§2.2), causal attention with online softmax and GQA head
 * sharing (§2.3, §3.1-§3.4, §4.3), the heads flattened back to (s, h) (§3.3),
 * and the write of K/V into a paged KV cache (§4.2; the paging follows
 * "Prefill vs decode tuning notes" (hncyxsy.com/news/227904) §3.4, its fp8
 * storage §3.3, and the 16-token block size of "Decoding LLM inference
 * latency: prefill bottlenecks" (lnwmold.com/news/496245) §3.3).
 *
 * Conventions shared by every call:
 *  - Pointers marked "device" are HIP device addresses; the caller allocates
 *    and owns every buffer.  The library allocates nothing and keeps no state
 *    besides a thread-local error message.
 *  - Compute calls are asynchronous: they validate their arguments on the
 *    host, enqueue kernels on `stream` (a hipStream_t; NULL = the null
 *    stream) and return.  Validation happens before any enqueue, so a call
 *    that returns an error has not touched device memory.
 *  - bf16 values travel as their 16-bit storage pattern (pca_bf16).
 *  - Device pointers must be 16-byte aligned; leading dimensions (row
 *    strides, in elements) must be multiples of 8 and at least the row width.
 *  - Errors: PCA_ERR_INVALID_ARG for a null or misaligned pointer, a size
 *    out of range or an inconsistent shape; PCA_ERR_UNSUPPORTED for a
 *    head_dim, page size or dtype the kernels are not built for;
 *    PCA_ERR_HIP when the launch itself fails.  pca_last_error() describes
 *    the last failure on the calling thread.
 */
#ifndef PCA_H
#define PCA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t pca_bf16;

typedef enum pca_status {
    PCA_OK = 0,
    PCA_ERR_INVALID_ARG = 1,
    PCA_ERR_UNSUPPORTED = 2,
    PCA_ERR_HIP = 3
} pca_status;

typedef enum pca_dtype {
    PCA_DTYPE_BF16 = 0,      /* 2 bytes per element                              */
    PCA_DTYPE_FP8_E4M3 = 1   /* OCP E4M3 (max 448, no inf), 1 byte per element   */
} pca_dtype;

/* Offsets and strides of the head split and of the page pools.  All strides
 * and offsets are in elements; the *_bytes fields are bytes. */
typedef struct pca_kv_layout_t {
    int64_t qkv_ld;             /* row width of the fused projection output: (n_head + 2 n_kv) hd */
    int64_t q_off;              /* first column of Q in that row: 0                                */
    int64_t k_off;              /* first column of K: n_head * hd                                  */
    int64_t v_off;              /* first column of V: (n_head + n_kv) * hd                         */
    int64_t head_stride;        /* columns between consecutive heads: hd                           */
    int64_t page_size;          /* token slots per page                                            */
    int64_t pool_page_stride;   /* elements per page: page_size * n_kv * hd                        */
    int64_t pool_slot_stride;   /* elements per slot: n_kv * hd                                    */
    int64_t pool_head_stride;   /* elements per kv head within a slot: hd                          */
    int64_t scale_page_stride;  /* fp8 only: scales per page, page_size * n_kv (else 0)            */
    int64_t scale_slot_stride;  /* fp8 only: scales per slot, n_kv (else 0)                        */
    int64_t elem_bytes;         /* 2 for bf16, 1 for fp8                                           */
    int64_t kv_bytes_per_token_layer;    /* 2 * n_kv * hd * elem_bytes (K and V)                  */
    int64_t scale_bytes_per_token_layer; /* fp8: 2 * n_kv * 4 (K and V scales), else 0            */
    int64_t page_bytes;         /* bytes of one page of one pool                                   */
} pca_kv_layout_t;

/*
 * pca_kv_layout -- pure host arithmetic, no device work.
 *   Byte accounting follows the data-flow article §3.4 (K and V, per kv head,
 *   per token: 16 KB for 32 kv heads and 4 KB for 8 at head_dim 128, 2-byte
 *   elements) and the tuning notes §3.1 (2 x layers x heads x head_dim x
 *   tokens x bytes).  The column offsets are the head split of the article's
 *   §2.2: the fused row is [Q | K | V], each head a run of head_dim columns.
 *   n_head % n_kv_head must be 0.  `out` is a host pointer owned by the
 *   caller.  Returns PCA_ERR_INVALID_ARG for non-positive or inconsistent
 *   sizes and on int64 overflow, PCA_ERR_UNSUPPORTED for an unknown dtype.
 */
pca_status pca_kv_layout(int n_head, int n_kv_head, int head_dim, int page_size,
                         pca_dtype cache_dtype, pca_kv_layout_t* out);

/*
 * pca_qkv_proj -- y[M, N] = x[M, K] * w_t[N, K]^T, bf16 in, fp32
 *   accumulation, one round-to-nearest-even to bf16 out.
 *   This is the single fused QKV GEMM of the data-flow article (§2.1, §4.1):
 *   the three projections in one (h, 3h) -- for GQA (h, (n_head+2 n_kv) hd)
 *   -- weight, so the activation is read from HBM once.  The weight is passed
 *   pre-transposed, (N, K) row-major, as the article's §5.1 advises doing
 *   once at load time so the GEMM reads both operands along K.
 *   x:   device, M rows of K elements, row stride ldx (>= K).
 *   w_t: device, N rows of K elements, row stride ldw (>= K).
 *   y:   device, M rows of N elements, row stride ldy (>= N); must not
 *        overlap x or w_t.
 *   M, N >= 1 (any value); K >= 8 and a multiple of 8.
 */
pca_status pca_qkv_proj(const pca_bf16* x, int64_t ldx, const pca_bf16* w_t, int64_t ldw,
                        pca_bf16* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                        void* stream);

/*
 * pca_quantize_rows_fp8 -- row-wise OCP E4M3 quantisation for fp8 GEMM
 *   operands ("Prefill vs decode tuning notes" (hncyxsy.com/news/227904) §2.3:
 *   FP8 inputs, wider accumulation), with the fp8 KV cache's rule: for each
 *   row r, amax = max|x[r, :]|, scales[r] = amax / 448,
 *   q[r, k] = E4M3_RNE_saturate(x[r, k] * (448 / amax)), binary32 RN steps;
 *   amax == 0 gives scale 0 and codes of +-0.
 *   x: device bf16, M rows of K elements (stride ldx); q: device uint8, M rows
 *   (stride ldq, a multiple of 16); scales: device float[M].  K >= 16 and a
 *   multiple of 16.  Use it on the activations (rows = tokens) and, once at
 *   load time, on the pre-transposed weight (rows = output features).
 */
pca_status pca_quantize_rows_fp8(const pca_bf16* x, int64_t ldx, int64_t M, int64_t K, uint8_t* q, int64_t ldq,
                                 float* scales, void* stream);

/*
 * pca_qkv_proj_fp8 -- the fused QKV projection on fp8 operands (tuning notes
 *   §2.3):  y[m, n] = RNE_bf16(sx[m] * sw[n] * sum_k dec(xq[m, k]) * dec(wq[n, k]))
 *   with fp32 accumulation on gfx950's fp8 matrix cores (twice the bf16 rate).
 *   xq, sx: the rows of x from pca_quantize_rows_fp8; wq, sw: the rows of
 *   w^T (N, K) likewise.  y: device bf16, M rows of N (stride ldy).  K >= 16
 *   and a multiple of 16; ldxq, ldwq multiples of 16.
 */
pca_status pca_qkv_proj_fp8(const uint8_t* xq, int64_t ldxq, const float* sx, const uint8_t* wq, int64_t ldwq,
                            const float* sw, pca_bf16* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * pca_rms_norm_qkv_proj -- the layer's input RMSNorm folded into the fused
 *   QKV projection.  The data-flow article's §2.1 normalises the layer input
 *   before the (h, 3h) projection; here the normalised activations are never
 *   written: y[m, :] = inv_rms[m] * (x[m, :] * w_t^T) with
 *   inv_rms[m] = 1 / sqrt(mean_k x[m, k]^2 + eps), applied to the fp32
 *   accumulators before the single bf16 rounding.  The norm's gain g acts on
 *   the K axis and is folded into the weight at load time, like the
 *   transpose: w_t[n, k] = RNE_bf16(W[k, n] * g[k]).
 *   x, w_t, y, M, N, K: as for pca_qkv_proj.
 *   eps: >= 0.  inv_rms: device float[M], a caller-owned workspace that
 *        receives 1/rms per row (the library allocates nothing).
 */
pca_status pca_rms_norm_qkv_proj(const pca_bf16* x, int64_t ldx, const pca_bf16* w_t, int64_t ldw, float eps,
                                 float* inv_rms, pca_bf16* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                 void* stream);

/* Rows the static workspace of pca_rms_norm_qkv_proj_noalloc holds (1 MiB of fp32). */
#define PCA_NOALLOC_MAX_ROWS 262144

/*
 * pca_rms_norm_qkv_proj_noalloc -- pca_rms_norm_qkv_proj for callers that
 *   cannot allocate device memory (code under HIP graph capture, tight
 *   serving loops, harnesses that forbid hipMalloc): the same result, with
 *   the per-row 1/rms workspace taken from a fixed device array inside the
 *   library (PCA_NOALLOC_MAX_ROWS floats per GPU, held until the process
 *   ends) instead of an inv_rms argument.  The call itself allocates and
 *   frees nothing.  Arguments and errors as pca_rms_norm_qkv_proj; M beyond
 *   PCA_NOALLOC_MAX_ROWS is PCA_ERR_UNSUPPORTED.  All calls on one GPU share
 *   its array (it keeps the last call's 1/rms values): calls whose work
 *   overlaps in time on one GPU (other streams or host threads) race and must
 *   be serialised by the caller.
 */
pca_status pca_rms_norm_qkv_proj_noalloc(const pca_bf16* x, int64_t ldx, const pca_bf16* w_t, int64_t ldw,
                                         float eps, pca_bf16* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                         void* stream);

/*
 * pca_out_proj_residual -- the output projection and residual add that close
 *   the attention unit: out = res + o * w_t^T.  The data-flow article's §2.1
 *   writes the layer as residual = input, ..., attend, residual += attention
 *   output; §3.3 lays the heads out as (s, n_head*head_dim) precisely so that
 *   the output projection W_o reads them as one matrix.  Same GEMM as
 *   pca_qkv_proj (fp32 accumulation); the residual is added to the fp32
 *   accumulators and the sum rounded once to bf16 (RNE).
 *   o:   device, M rows of K elements (the attention output, K = n_head*hd).
 *   w_t: device, W_o pre-transposed to (N, K), N = h.
 *   res: device, M rows of N elements, row stride ldr; may be out itself
 *        (with ldr == ldout) for an in-place update, else must not overlap it.
 *   out: device, M rows of N elements, row stride ldout.
 *   Sizes and strides as for pca_qkv_proj.
 */
pca_status pca_out_proj_residual(const pca_bf16* o, int64_t ldo, const pca_bf16* w_t, int64_t ldw,
                                 const pca_bf16* res, int64_t ldr, pca_bf16* out, int64_t ldout,
                                 int64_t M, int64_t N, int64_t K, void* stream);

/*
 * pca_qkv_proj_kv_write -- pca_qkv_proj with the KV-cache write done by the
 *   GEMM's epilogue.  The data-flow article's §4.2 notes that the projection
 *   output can be scattered into its cache blocks by the kernel that produces
 *   it, and that a separate copy pass is waste: here the GEMM tiles that
 *   produce K and V columns also store them into their page slots, so the
 *   separate pass (which re-reads K and V from y) disappears.
 *   Result: y as from pca_qkv_proj (bit for bit), with
 *        N = (n_head + 2 n_kv_head) * head_dim and the [Q | K | V] column
 *        order of pca_kv_layout; and the pools (and fp8 scales) exactly as
 *        pca_kv_cache_write would leave them for k = y + k_off, v = y + v_off
 *        (row stride ldy), total_tokens = M.
 *   x, w_t, y, M, K: as for pca_qkv_proj.
 *   cu_seqlens, num_seqs, block_table, max_pages_per_seq, page_size,
 *   cache_dtype, k_cache, v_cache, k_scale, v_scale, num_pages: as for
 *        pca_kv_cache_write (tokens are the M rows of y).
 *   n_head, n_kv_head: > 0, n_head a multiple of n_kv_head; head_dim 32, 64
 *        or 128.  For an fp8 cache, n_head*head_dim and n_kv_head*head_dim
 *        must be multiples of 128 (else PCA_ERR_UNSUPPORTED): each 128-column
 *        slab of a GEMM tile then holds whole heads of one of K or V.
 */
pca_status pca_qkv_proj_kv_write(const pca_bf16* x, int64_t ldx, const pca_bf16* w_t, int64_t ldw,
                                 pca_bf16* y, int64_t ldy, int64_t M, int64_t K,
                                 int n_head, int n_kv_head, int head_dim,
                                 const int32_t* cu_seqlens, int num_seqs,
                                 const int32_t* block_table, int max_pages_per_seq, int page_size,
                                 pca_dtype cache_dtype, void* k_cache, void* v_cache,
                                 float* k_scale, float* v_scale, int64_t num_pages, void* stream);

/*
 * pca_prefill_attention -- causal GQA attention over packed sequences.
 *   For sequence b, query head i (kv head g = i / (n_head / n_kv_head)) and
 *   position r:  o[r, i] = sum_{c <= r} softmax_c(q[r, i] . k[c, g] * scale) v[c, g]
 *   (data-flow article §2.3, §3.1, §3.2; GQA sharing §3.4).  The kernel is
 *   the fused blockwise form (§3.2, §4.3): scores and probabilities live only
 *   in registers, the softmax runs online per kv tile, and the causal mask is
 *   control flow -- kv tiles after a query tile are never visited.
 *   q, k, v: device, token-major rows; head h of token t starts at
 *        q + t*ldq + h*head_dim (likewise k, v with kv heads).  They may be
 *        strided views into one fused projection output (use the offsets
 *        from pca_kv_layout).
 *   cu_seqlens: device int32[num_seqs + 1], cu[0] = 0, non-decreasing,
 *        cu[num_seqs] = total_tokens; sequence b is tokens [cu[b], cu[b+1]).
 *        NULL means one sequence of total_tokens (num_seqs must be 1).
 *        Entries are clamped to [0, total_tokens] on the device, so a bad
 *        table cannot cause out-of-bounds access (it gives wrong output).
 *   max_seqlen: >= the longest sequence; rows of longer sequences past
 *        max_seqlen are not written.
 *   head_dim: 32, 64 or 128 (else PCA_ERR_UNSUPPORTED).  causal must be 1.
 *   o:   device, bf16, (total_tokens, n_head*head_dim) with row stride ldo;
 *        head i of token t at o + t*ldo + i*head_dim (heads flattened back
 *        to (s, h), §3.3).  Must not overlap q, k, v.
 *   total_tokens == 0 (with num_seqs >= 1) is a no-op and accepts NULL buffers.
 */
pca_status pca_prefill_attention(const pca_bf16* q, const pca_bf16* k, const pca_bf16* v,
                                 int64_t ldq, int64_t ldk, int64_t ldv,
                                 const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                                 int64_t total_tokens, int n_head, int n_kv_head, int head_dim,
                                 float scale, int causal, pca_bf16* o, int64_t ldo,
                                 void* stream);

/*
 * pca_prefill_attention_window -- pca_prefill_attention with a sliding window
 *   ("Decoding LLM inference latency" (lnwmold.com/news/496245) §4.1: each
 *   token attends only to its W most recent positions, O(n W) work instead of
 *   O(n^2)).  Row r of a sequence sees keys c with r - window < c <= r (window
 *   keys, itself included); kv tiles wholly before a wave's window are never
 *   visited.  window == 0 means no window (exactly pca_prefill_attention);
 *   window < 0 is PCA_ERR_INVALID_ARG.  Every other argument as for
 *   pca_prefill_attention.
 */
pca_status pca_prefill_attention_window(const pca_bf16* q, const pca_bf16* k, const pca_bf16* v,
                                        int64_t ldq, int64_t ldk, int64_t ldv,
                                        const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                                        int64_t total_tokens, int n_head, int n_kv_head, int head_dim,
                                        float scale, int causal, int window, pca_bf16* o, int64_t ldo,
                                        void* stream);

/*
 * pca_prefill_attention_splitkv -- pca_prefill_attention for shallow grids,
 *   with the key range of long query blocks split over two workgroups (the
 *   data-flow article §5.2: a grid that fills the compute units about once
 *   leaves many idle while the longest tiles finish).  When the launch has at
 *   most one task group (8 waves of 32 query rows sharing a kv head) per
 *   workgroup slot of the device, and its units (sequence, kv head) spread
 *   evenly over the 8 XCDs, task groups with more than three quarters of the
 *   longest sequence's 64-key tiles (at least 8 tiles in it) run as two
 *   chunks, tiles [0, n/2) and [n/2, n).  Each chunk stores its partial result (fp32 accumulators,
 *   reference and row sums) in the workspace; the chunk that finishes second
 *   merges the two in chunk order and writes o.  Otherwise the call runs
 *   pca_prefill_attention unchanged (bitwise the same output).
 *   The output is deterministic, but a split row sums its keys in a
 *   different order than pca_prefill_attention, so the two differ by
 *   rounding; it also depends on the launch (a sequence alone and inside a
 *   batch may differ by rounding).
 *   workspace: device memory of at least
 *        pca_prefill_attention_splitkv_workspace(...) bytes, 256-byte aligned,
 *        owned by the caller, ZEROED ONCE before its first use; every call
 *        leaves its counters zero again.  Calls that share a workspace must
 *        not overlap (one stream, or ordered).
 *   Every other argument as for pca_prefill_attention.  Errors: a null or
 *   misaligned workspace, or workspace_bytes below the needed size, is
 *   PCA_ERR_INVALID_ARG (before any launch).
 */
pca_status pca_prefill_attention_splitkv(const pca_bf16* q, const pca_bf16* k, const pca_bf16* v,
                                         int64_t ldq, int64_t ldk, int64_t ldv,
                                         const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                                         int64_t total_tokens, int n_head, int n_kv_head, int head_dim,
                                         float scale, int causal, pca_bf16* o, int64_t ldo,
                                         void* workspace, int64_t workspace_bytes, void* stream);

/*
 * pca_prefill_attention_splitkv_workspace -- bytes of the workspace for
 *   pca_prefill_attention_splitkv with these sizes: 4 KiB of arrival
 *   counters (at the same place for every size, so one workspace serves calls
 *   of different sizes), then, per task group slot (num_seqs * n_kv_head *
 *   ceil(G * ceil(max_seqlen / 32) / 8) of them, G = n_head / n_kv_head, at
 *   most 1024: larger launches are never split), two chunks' partial results
 *   of 32 * (32 * head_dim + 128) bytes each (264 KiB per slot at head_dim
 *   128).  Returns -1 for invalid sizes (num_seqs or
 *   max_seqlen < 1, n_head not a multiple of n_kv_head, head_dim not 32, 64
 *   or 128), with the reason in pca_last_error().
 */
int64_t pca_prefill_attention_splitkv_workspace(int num_seqs, int max_seqlen, int n_head, int n_kv_head,
                                                int head_dim);

/*
 * pca_prefill_attention_paged -- causal GQA attention of a prefill chunk over
 *   its sequence's cached prefix.  Chunked prefill ("Prefill vs decode tuning
 *   notes" (hncyxsy.com/news/227904) §2.1; "Decoding LLM inference latency"
 *   (lnwmold.com/news/496245) §3.3 runs it with 512-token chunks over 16-token
 *   blocks) processes a long prompt a chunk at a time, keeping the earlier
 *   chunks' K/V in the paged cache.  The chunk's own K/V must already be in
 *   the cache (pca_kv_cache_write or pca_qkv_proj_kv_write): all keys are read
 *   from the pools through the block table.
 *   For sequence b, chunk rows are q rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *   (Lq of them) and its keys are cache positions 0 .. ctx_lens[b]-1, so row r
 *   sits at position P + r with P = ctx_lens[b] - Lq and sees keys c <= P + r:
 *        o[r, i] = sum_{c <= P + r} softmax_c(q[r, i] . k[c, g] * scale) v[c, g].
 *   q, o: as for pca_prefill_attention (token-major, row strides ldq, ldo).
 *   cu_seqlens_q: device int32[num_seqs + 1] over the chunk rows (NULL = one
 *        sequence of total_q rows); max_seqlen_q >= the longest chunk.
 *   ctx_lens: device int32[num_seqs], keys per sequence (prefix + chunk);
 *        clamped on the device to [Lq, max_pages_per_seq * 16].
 *        max_ctx_len >= every ctx_lens[b] (sizes the staged block-table row).
 *   block_table, max_pages_per_seq, page_size (16), cache_dtype, k_cache,
 *        v_cache, k_scale, v_scale, num_pages: the pools of pca_kv_cache_write.
 *        An fp8 cache is dequantised on load (tuning notes §3.3): each tile
 *        of E4M3 codes is decoded, multiplied by its (token, kv head) scale
 *        and rounded to bf16 on chip before the matrix products; k_scale and
 *        v_scale must then be given (NULL for a bf16 cache).  Each pool must
 *        be smaller than 2 GiB.
 *        A block-table entry outside [0, num_pages) makes its 16 keys (and,
 *        for fp8, their scales) read as zeros: the output is then not that of
 *        any real cache, but no access leaves the K, V or scale pools (each
 *        is read through a buffer view of exactly its own size).
 *   head_dim 32, 64 or 128; causal must be 1.
 */
pca_status pca_prefill_attention_paged(const pca_bf16* q, int64_t ldq, const int32_t* cu_seqlens_q, int num_seqs,
                                       int max_seqlen_q, int64_t total_q, const int32_t* ctx_lens, int max_ctx_len,
                                       const int32_t* block_table, int max_pages_per_seq, int page_size,
                                       pca_dtype cache_dtype, const void* k_cache, const void* v_cache,
                                       const float* k_scale, const float* v_scale, int64_t num_pages,
                                       int n_head, int n_kv_head, int head_dim, float scale, int causal,
                                       pca_bf16* o, int64_t ldo, void* stream);

/*
 * pca_prefill_attention_paged_window -- pca_prefill_attention_paged with a
 *   sliding window ("Decoding LLM inference latency" (lnwmold.com/news/496245)
 *   §4.1): chunk row r at position P + r sees the cached keys c with
 *   P + r - window < c <= P + r, so a chunk over a long prefix reads only
 *   the last window keys before each row; kv tiles wholly before a wave's
 *   window are never requested.  window == 0 means no window (exactly
 *   pca_prefill_attention_paged); window < 0 is PCA_ERR_INVALID_ARG.  Every
 *   other argument, and the errors, as for pca_prefill_attention_paged.
 */
pca_status pca_prefill_attention_paged_window(const pca_bf16* q, int64_t ldq, const int32_t* cu_seqlens_q,
                                              int num_seqs, int max_seqlen_q, int64_t total_q,
                                              const int32_t* ctx_lens, int max_ctx_len, const int32_t* block_table,
                                              int max_pages_per_seq, int page_size, pca_dtype cache_dtype,
                                              const void* k_cache, const void* v_cache, const float* k_scale,
                                              const float* v_scale, int64_t num_pages, int n_head, int n_kv_head,
                                              int head_dim, float scale, int causal, int window, pca_bf16* o,
                                              int64_t ldo, void* stream);

/*
 * pca_kv_cache_write -- scatter each token's K and V into its page slot.
 *   Token position p of sequence b goes to page block_table[b*max_pages_per_seq
 *   + p / page_size], slot p % page_size (data-flow article §4.2,
 *   "per-block contiguous"; tuning notes §3.4).  Pools are
 *   [num_pages][page_size][n_kv_head][head_dim]; slots no token maps to are
 *   left untouched.
 *   k, v: device bf16, token-major rows (row strides ldk, ldv); kv head j of
 *        token t at k + t*ldk + j*head_dim.
 *   cu_seqlens: as for pca_prefill_attention (NULL = one sequence).
 *   block_table: device int32[num_seqs][max_pages_per_seq].  Entries outside
 *        [0, num_pages) and positions past max_pages_per_seq*page_size are
 *        skipped on the device (never written out of bounds).
 *   page_size: 16 (else PCA_ERR_UNSUPPORTED).  head_dim: 32, 64 or 128.
 *   num_pages * page_size < 2^31 (else PCA_ERR_UNSUPPORTED).
 *   cache_dtype PCA_DTYPE_BF16: k_cache, v_cache are bf16 pools, a bit copy;
 *        k_scale and v_scale must be NULL.
 *   cache_dtype PCA_DTYPE_FP8_E4M3 (tuning notes §3.3): k_cache, v_cache are
 *        uint8 pools of E4M3 codes and k_scale, v_scale are device fp32 pools
 *        [num_pages][page_size][n_kv_head].  For each (token, kv head) row x
 *        of K (and of V): amax = max|x|, scale = amax / 448,
 *        code = E4M3_RNE_saturate(x * (448 / amax)), every step in binary32
 *        round-to-nearest; amax == 0 gives scale 0 and codes of +-0.
 *   total_tokens == 0 (with num_seqs >= 1) is a no-op and accepts NULL buffers.
 */
pca_status pca_kv_cache_write(const pca_bf16* k, const pca_bf16* v, int64_t ldk, int64_t ldv,
                              const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens,
                              const int32_t* block_table, int max_pages_per_seq,
                              int n_kv_head, int head_dim, int page_size, pca_dtype cache_dtype,
                              void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              int64_t num_pages, void* stream);

/*
 * pca_quantize_heads_fp8 -- per-(token, head) E4M3 rows with power-of-two
 *   scales, the operand form of pca_prefill_attention_fp8qk (tuning notes
 *   §2.3: FP8 inputs, wider accumulation).  For token t and head h, with
 *   y = RN32(x[t, h, :] * prescale) and amax = max|y|: e is the smallest
 *   integer in [-127, 127] with amax * 2^-e <= 448 (amax == 0: e = -127),
 *   codes[t, h, :] = E4M3_RNE(y * 2^-e) (an exact scaling, so one rounding)
 *   and exps[t, h] = e + 127 (the OCP microscaling E8M0 byte: 2^(byte-127)).
 *   x: device bf16, T rows, head h of row t at x + t*ldx + h*head_dim
 *      (ldx >= n_heads*head_dim, a multiple of 8; 16-byte aligned) -- e.g.
 *      the K columns of the fused projection output.
 *   codes: device uint8, same layout with row stride ldc (multiple of 8,
 *      8-byte aligned).  exps: device uint8, T rows of n_heads, stride lde.
 *   head_dim: 32, 64 or 128.  prescale: finite, > 0 (1 for K).  T == 0 is a
 *   no-op.
 */
pca_status pca_quantize_heads_fp8(const pca_bf16* x, int64_t ldx, int64_t T, int n_heads, int head_dim, float prescale,
                                  uint8_t* codes, int64_t ldc, uint8_t* exps, int64_t lde, void* stream);

/*
 * pca_prefill_attention_fp8qk -- pca_prefill_attention with fp8 operands for
 *   the scores (tuning notes §2.3: FP8 inputs with wider accumulation, the
 *   softmax kept in higher precision).  K arrives as pca_quantize_heads_fp8
 *   output (prescale 1): codes k_codes (T rows, stride ldk bytes, a multiple
 *   of 16; head j of token t at k_codes + t*ldk + j*128) and scale bytes
 *   k_exps (T rows of n_kv_head, stride lde: a multiple of 4, k_exps 4-byte
 *   aligned).  Q (bf16, as for
 *   pca_prefill_attention) is quantised inside with the same rule after the
 *   factor c = RN32(scale * RN32(log2 e)): per (token, head), codes of
 *   RN32(q * c) * 2^-e.  The scores are exact products of the dequantised
 *   operands accumulated in fp32 (in log2 units), the softmax is taken in
 *   base 2 with fp32 exp2 and sums, P is rounded to bf16 for P.V with V in
 *   bf16, and o gets the normalised rows as bf16 (same layout as
 *   pca_prefill_attention).  head_dim must be 128 (else PCA_ERR_UNSUPPORTED);
 *   other arguments and errors as pca_prefill_attention.
 */
pca_status pca_prefill_attention_fp8qk(const pca_bf16* q, int64_t ldq, const uint8_t* k_codes, int64_t ldk,
                                       const uint8_t* k_exps, int64_t lde, const pca_bf16* v, int64_t ldv,
                                       const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                                       int64_t total_tokens, int n_head, int n_kv_head, int head_dim,
                                       float scale, int causal, pca_bf16* o, int64_t ldo, void* stream);

/*
 * pca_e4m3_encode -- codes[i] = E4M3_RNE_saturate(x[i]) for i < n: the OCP
 *   E4M3 encoder behind every fp8 result of this library (the KV cache of the
 *   tuning notes §3.3 and the fp8 operands of §2.3), as a plain elementwise op
 *   (e.g. for values already divided by a caller's own scale).  Round to
 *   nearest even; finite magnitudes above 448 give the largest normal code
 *   (0x7E, or 0xFE when negative); the sign bit is kept (-0 gives 0x80).
 *   NaN inputs give unspecified codes.
 *   x: device float[n], 16-byte aligned; codes: device uint8[n], 4-byte
 *   aligned, must not overlap x.  n == 0 is a no-op (NULL buffers allowed).
 */
pca_status pca_e4m3_encode(const float* x, uint8_t* codes, int64_t n, void* stream);

/*
 * pca_clock_stamp -- measurement utility: enqueues on `stream` a small kernel
 *   whose 1024 one-wave blocks each write, at out[4*b .. 4*b+3], the XCD it
 *   ran on (hardware XCC id), its HW_ID register (shader engine, array and CU
 *   in bits 8-15), the shader-clock cycle counter it reads (s_memtime) and
 *   the 100 MHz real-time counter (s_memrealtime).  Two stamps around a
 *   stretch of work give, per CU present in both, the average shader clock
 *   over it (cycles over seconds), the clock the MFMA peak scales with (the
 *   published dense peaks assume 2.4 GHz).  Cycle counters of different
 *   shader engines do not agree, so only stamps of one CU may be paired.
 *   out: device uint64[4096], 8-byte aligned.
 */
pca_status pca_clock_stamp(uint64_t* out, void* stream);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* pca_last_error(void);

/* Library version string, e.g. "pca 0.1.0 gfx950". */
const char* pca_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PCA_H */
