// Device helpers shared by the kernels that write the paged KV cache: the
// page-slot lookup of a token and the row maxima over lane groups (the E4M3
// encoder itself sits with the other device helpers).
//
// Placement: token position p of sequence b goes to page
// block_table[b][p / page_size], slot p % page_size (prefill data-flow article
// (hncyxsy.com/news/270449) §4.2; page table of the prefill/decode tuning
// notes (hncyxsy.com/news/227904) §3.4).  The fp8 form is the tuning notes'
// 1-byte storage (§3.3), encoded as OCP E4M3.
#pragma once

#include "pca_device.hpp"
#include "pca_internal.hpp"

namespace pca {

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

// max over the L-lane group (L = 1, 2, 4, 8 or 16, aligned) of non-negative
// binary32 values passed as their bit patterns, whose integer order is their
// value order; the unsigned max takes each DPP lane permute as an operand.
template <int L>
__device__ inline uint32_t group_umax(uint32_t v) {
    if constexpr (L >= 2) v = __builtin_elementwise_max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    if constexpr (L >= 4) v = __builtin_elementwise_max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    if constexpr (L >= 8) v = __builtin_elementwise_max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    if constexpr (L >= 16) v = __builtin_elementwise_max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    return v;
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

}  // namespace pca
