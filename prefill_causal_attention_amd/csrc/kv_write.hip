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
// each wave instruction covers 1 KiB of contiguous memory): it issues all its
// loads first, resolves the page slot of the few tokens it touches into LDS
// while they are in flight, then stores.  Loads and stores are non-temporal:
// the data is touched once.
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

    // the data loads go out first; the page-slot lookups (a dependent chain of
    // small loads) overlap them
    const uint32_t total_chunks = (uint32_t)a.total_tokens * C2;
    u32x4_t val[kItems];
    uint32_t tok[kItems], cc[kItems];
    bool isv[kItems], live[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const uint32_t id = first_chunk + i * kThreads + threadIdx.x;
        live[i] = id < total_chunks;
        tok[i] = live[i] ? id / C2 : 0;
        const uint32_t rem = id - tok[i] * C2;
        isv[i] = rem >= C;
        cc[i] = isv[i] ? rem - C : rem;
        if (live[i]) {
            const uint16_t* src = (isv[i] ? a.v + (int64_t)tok[i] * a.ldv : a.k + (int64_t)tok[i] * a.ldk) + cc[i] * 8;
            val[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src));
        }
    }
    resolve_slots(a, first_tok, ntok, slots);
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        if (!live[i]) continue;
        const int64_t slot = slots[tok[i] - first_tok];
        if (slot < 0) continue;
        uint16_t* pool = isv[i] ? (uint16_t*)a.v_cache : (uint16_t*)a.k_cache;
        __builtin_nontemporal_store(val[i], reinterpret_cast<u32x4_t*>(pool + (slot * (int64_t)C + cc[i]) * 8));
    }
}

// OCP E4M3 encoding of a binary32 value, round to nearest even, finite
// overflow saturating to +-448; the sign bit is copied from y.  Branch-free:
// below 2^-6 the code is the subnormal count rint(|y| * 2^9) (exact scaling,
// ties to even); from there the 3 kept mantissa bits are rounded to nearest
// even in the integer domain and the exponent rebiased from 127 to 7.
__device__ inline uint32_t e4m3_rne_sat(float y) {
    const uint32_t u = __builtin_bit_cast(uint32_t, y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = __builtin_fabsf(y);
    const uint32_t ua = u & 0x7FFFFFFFu;
    const uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);
    const uint32_t nrm = ((ua + 0x7FFFFu + ((ua >> 20) & 1u)) >> 20) - (120u << 3);
    uint32_t code = a < 0.015625f ? sub : nrm;
    code = (a >= 448.0f || code > 0x7Eu) ? 0x7Eu : code;
    return sign | code;
}

// max over the R-lane group (R = 4, 8 or 16, aligned) holding one (token, kv
// head) row, with DPP lane permutes inside 16-lane rows: swap neighbours, swap
// pairs, mirror halves of 8, mirror the 16
template <int R>
__device__ inline float group_max(float v) {
    v = __builtin_fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
    v = __builtin_fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
    if constexpr (R >= 8)
        v = __builtin_fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
    if constexpr (R >= 16)
        v = __builtin_fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
    return v;
}

template <int R>
__global__ __launch_bounds__(kThreads) void kv_write_fp8_kernel(KvWriteArgs a) {
    const uint32_t C = (uint32_t)a.n_kv_head * R;            // chunks per token per tensor
    const uint32_t C2 = 2 * C;
    const uint32_t first_chunk = blockIdx.x * (uint32_t)kChunksPerBlock;
    const int64_t first_tok = first_chunk / C2;
    const int ntok = (int)((first_chunk + kChunksPerBlock - 1) / C2 - first_tok + 1);
    __shared__ int64_t slots[kChunksPerBlock / 8 + 2];

    // data loads first, page-slot lookups overlapping them
    const uint32_t total_chunks = (uint32_t)a.total_tokens * C2;
    u32x4_t w[kItems];
    uint32_t tok[kItems], cc[kItems];
    bool isv[kItems], live[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        // whole rows of R lanes stay inside one pass (R divides 256)
        const uint32_t id = first_chunk + i * kThreads + threadIdx.x;
        live[i] = id < total_chunks;
        tok[i] = live[i] ? id / C2 : 0;
        const uint32_t rem = id - tok[i] * C2;
        isv[i] = rem >= C;
        cc[i] = isv[i] ? rem - C : rem;
        w[i] = u32x4_t{0u, 0u, 0u, 0u};
        if (live[i]) {
            const uint16_t* src = (isv[i] ? a.v + (int64_t)tok[i] * a.ldv : a.k + (int64_t)tok[i] * a.ldk) + cc[i] * 8;
            w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src));
        }
    }
    resolve_slots(a, first_tok, ntok, slots);
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = bf16_lo(w[i][j]);
            x[2 * j + 1] = bf16_hi(w[i][j]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[j]));
        amax = group_max<R>(amax);
        // binary32 round-to-nearest division (no fast-math): scale = amax / 448, inv = 448 / amax
        const float scale = amax / 448.0f;
        const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) lo |= e4m3_rne_sat(x[j] * inv) << (8 * j);
#pragma unroll
        for (int j = 0; j < 4; ++j) hi |= e4m3_rne_sat(x[4 + j] * inv) << (8 * j);
        if (!live[i]) continue;
        const int64_t slot = slots[tok[i] - first_tok];
        if (slot < 0) continue;
        uint8_t* pool = isv[i] ? (uint8_t*)a.v_cache : (uint8_t*)a.k_cache;
        __builtin_nontemporal_store(u32x2_t{lo, hi}, reinterpret_cast<u32x2_t*>(pool + slot * (int64_t)C * 8 + cc[i] * 8));
        if (cc[i] % R == 0) {
            float* sp = isv[i] ? a.v_scale : a.k_scale;
            sp[slot * a.n_kv_head + cc[i] / R] = scale;
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
    switch (a.head_dim / 8) {
        case 4: hipLaunchKernelGGL(kv_write_fp8_kernel<4>, dim3(num_blocks(a)), dim3(kThreads), 0, s, a); break;
        case 8: hipLaunchKernelGGL(kv_write_fp8_kernel<8>, dim3(num_blocks(a)), dim3(kThreads), 0, s, a); break;
        case 16: hipLaunchKernelGGL(kv_write_fp8_kernel<16>, dim3(num_blocks(a)), dim3(kThreads), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pca
