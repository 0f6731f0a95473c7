// Paged KV-cache write (bf16 copy, or fp8 E4M3 with per-(token, kv head) scales).
//
// Placement: token position p of sequence b goes to page
// block_table[b][p / page_size], slot p % page_size; pools are
// [page][slot][kv_head][head_dim] ("per-block contiguous" layout of the
// prefill data-flow article (hncyxsy.com/news/270449) §4.2, with the page
// table of the prefill/decode tuning notes (hncyxsy.com/news/227904) §3.4).
// The fp8 form follows the tuning notes §3.3 (1 byte per element), encoded as
// OCP E4M3 with an absmax scale per (token, kv head).
//
// HBM-bound: every byte is read once and written once.  One token's K (or V)
// for all kv heads is a contiguous run both in the fused projection row and in
// its page slot, so the copy is a set of contiguous 16-byte chunks.  A block
// takes 1024 consecutive chunks (4 per thread, lanes on consecutive chunks so
// each wave instruction covers 1 KiB of contiguous memory), resolves the
// page slot of the few tokens it touches once into LDS, then moves the data.
#include "pca_device.hpp"
#include "pca_internal.hpp"

namespace pca {

namespace {

constexpr int kThreads = 256;
constexpr int kItems = 4;
constexpr int kChunksPerBlock = kThreads * kItems;

// Largest b with cu[b] <= t (cu = null: single sequence).
__device__ inline int find_seq(const int32_t* cu, int num_seqs, int64_t t) {
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Slot index (page * page_size + slot) of token t, or -1 if the token maps to
// no valid slot (outside every sequence, past the block table, or a page
// number outside [0, num_pages)).
__device__ inline int64_t token_slot(const KvWriteArgs& a, int64_t t) {
    int b = 0;
    int64_t start = 0, end = a.total_tokens;
    if (a.cu_seqlens != nullptr) {
        b = find_seq(a.cu_seqlens, a.num_seqs, t);
        start = a.cu_seqlens[b];
        end = a.cu_seqlens[b + 1];
    }
    if (t < start || t >= end) return -1;
    int64_t pos = t - start;
    int64_t pidx = pos / a.page_size;
    if (pidx >= a.max_pages_per_seq) return -1;
    int32_t page = a.block_table[(int64_t)b * a.max_pages_per_seq + pidx];
    if (page < 0 || (int64_t)page >= a.num_pages) return -1;
    return (int64_t)page * a.page_size + (pos % a.page_size);
}

// Resolve the slots of tokens [first, first + ntok) into LDS.
__device__ inline void resolve_slots(const KvWriteArgs& a, int64_t first, int ntok, int64_t* slots) {
    for (int i = threadIdx.x; i < ntok; i += kThreads) {
        int64_t t = first + i;
        slots[i] = (t < a.total_tokens) ? token_slot(a, t) : -1;
    }
    __syncthreads();
}

__global__ __launch_bounds__(kThreads) void kv_write_bf16_kernel(KvWriteArgs a) {
    // chunks per token per tensor (K or V): n_kv * head_dim / 8
    const uint32_t C = (uint32_t)(a.n_kv_head * a.head_dim / 8);
    const uint32_t C2 = 2 * C;
    const uint32_t first_chunk = blockIdx.x * (uint32_t)kChunksPerBlock;
    const int64_t first_tok = first_chunk / C2;
    const int ntok = (int)((first_chunk + kChunksPerBlock - 1) / C2 - first_tok + 1);
    __shared__ int64_t slots[kChunksPerBlock / 8 + 2];
    resolve_slots(a, first_tok, ntok, slots);

    const uint32_t total_chunks = (uint32_t)a.total_tokens * C2;
    u32x4_t val[kItems];
    int64_t dst[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        uint32_t id = first_chunk + i * kThreads + threadIdx.x;
        dst[i] = -1;
        if (id < total_chunks) {
            uint32_t tok = id / C2;
            uint32_t rem = id - tok * C2;
            bool is_v = rem >= C;
            uint32_t c = is_v ? rem - C : rem;
            const uint16_t* src = (is_v ? a.v + (int64_t)tok * a.ldv : a.k + (int64_t)tok * a.ldk) + c * 8;
            val[i] = *reinterpret_cast<const u32x4_t*>(src);
            int64_t slot = slots[tok - first_tok];
            if (slot >= 0) dst[i] = (is_v ? 1 : 0) | ((slot * (int64_t)C + c) << 1);
        }
    }
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        if (dst[i] >= 0) {
            uint16_t* pool = (dst[i] & 1) ? (uint16_t*)a.v_cache : (uint16_t*)a.k_cache;
            *reinterpret_cast<u32x4_t*>(pool + (dst[i] >> 1) * 8) = val[i];
        }
    }
}

// OCP E4M3 encoding of a binary32 value, round to nearest even, finite
// overflow saturating to +-448; the sign bit is copied from y.
__device__ inline uint32_t e4m3_rne_sat(float y) {
    uint32_t u = __builtin_bit_cast(uint32_t, y);
    uint32_t sign = (u >> 24) & 0x80u;
    float a = __builtin_fabsf(y);
    uint32_t code;
    if (a >= 448.0f) {
        code = 0x7Eu;
    } else if (a < 0.015625f) {                       // below 2^-6: subnormal step 2^-9
        code = (uint32_t)__builtin_rintf(a * 512.0f);  // exact scaling, rint = ties to even
    } else {
        uint32_t ua = __builtin_bit_cast(uint32_t, a);
        uint32_t r = (ua + 0x7FFFFu + ((ua >> 20) & 1u)) >> 20;   // keep 3 mantissa bits, RNE
        code = r - (120u << 3);                                    // exponent bias 127 -> 7
        if (code > 0x7Eu) code = 0x7Eu;
    }
    return sign | code;
}

__global__ __launch_bounds__(kThreads) void kv_write_fp8_kernel(KvWriteArgs a) {
    const uint32_t R = (uint32_t)(a.head_dim / 8);          // lanes per (token, kv head) row
    const uint32_t C = (uint32_t)a.n_kv_head * R;
    const uint32_t C2 = 2 * C;
    const uint32_t first_chunk = blockIdx.x * (uint32_t)kChunksPerBlock;
    const int64_t first_tok = first_chunk / C2;
    const int ntok = (int)((first_chunk + kChunksPerBlock - 1) / C2 - first_tok + 1);
    __shared__ int64_t slots[kChunksPerBlock / 8 + 2];
    resolve_slots(a, first_tok, ntok, slots);

    const uint32_t total_chunks = (uint32_t)a.total_tokens * C2;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        // whole rows of R lanes stay inside one pass (R divides 256), so the
        // shuffles below always pair lanes of the same row
        uint32_t id = first_chunk + i * kThreads + threadIdx.x;
        bool live = id < total_chunks;
        uint32_t tok = live ? id / C2 : 0;
        uint32_t rem = id - tok * C2;
        bool is_v = rem >= C;
        uint32_t c = is_v ? rem - C : rem;
        u32x4_t w = {0u, 0u, 0u, 0u};
        if (live) {
            const uint16_t* src = (is_v ? a.v + (int64_t)tok * a.ldv : a.k + (int64_t)tok * a.ldk) + c * 8;
            w = *reinterpret_cast<const u32x4_t*>(src);
        }
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = bf16_lo(w[j]);
            x[2 * j + 1] = bf16_hi(w[j]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[j]));
        for (uint32_t m = 1; m < R; m <<= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, (int)m));
        // binary32 round-to-nearest division (no fast-math): scale = amax / 448, inv = 448 / amax
        float scale = amax / 448.0f;
        float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) lo |= e4m3_rne_sat(x[j] * inv) << (8 * j);
#pragma unroll
        for (int j = 0; j < 4; ++j) hi |= e4m3_rne_sat(x[4 + j] * inv) << (8 * j);
        if (live) {
            int64_t slot = slots[tok - first_tok];
            if (slot >= 0) {
                uint8_t* pool = is_v ? (uint8_t*)a.v_cache : (uint8_t*)a.k_cache;
                u32x2_t out = {lo, hi};
                *reinterpret_cast<u32x2_t*>(pool + slot * (int64_t)C * 8 + c * 8) = out;
                if (c % R == 0) {
                    float* sp = is_v ? a.v_scale : a.k_scale;
                    sp[slot * a.n_kv_head + c / R] = scale;
                }
            }
        }
    }
}

uint32_t num_blocks(const KvWriteArgs& a) {
    uint64_t chunks = (uint64_t)a.total_tokens * 2 * (uint64_t)(a.n_kv_head * a.head_dim / 8);
    return (uint32_t)((chunks + kChunksPerBlock - 1) / kChunksPerBlock);
}

}  // namespace

hipError_t launch_kv_write_bf16(const KvWriteArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(kv_write_bf16_kernel, dim3(num_blocks(a)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_kv_write_fp8(const KvWriteArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(kv_write_fp8_kernel, dim3(num_blocks(a)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace pca
