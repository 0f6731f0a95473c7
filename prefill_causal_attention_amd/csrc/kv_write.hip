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
// each wave instruction covers 1 KiB of contiguous memory).  When every block
// is resident at once, a block issues all its loads first, resolves the page
// slot of the few tokens it touches into LDS while they are in flight, then
// stores; deeper grids (and a wave's 64 chunks within one token) instead look
// the slots up per wave with scalar loads ahead of the data loads.  Loads and
// stores are non-temporal: the data is touched once.
#include "kv_common.hpp"

namespace pca {

namespace {

constexpr int kThreads = 256;
constexpr int kItems = 4;
constexpr int kChunksPerBlock = kThreads * kItems;

// Resolve the slots of tokens [first, first + ntok) into LDS.  Slot indices
// fit in int32: the host keeps num_pages * page_size below 2^31.
__device__ inline void resolve_slots(const KvWriteArgs& a, int64_t first, int ntok, int32_t* slots) {
    for (int i = threadIdx.x; i < ntok; i += kThreads) {
        int64_t t = first + i;
        slots[i] = (t < a.total_tokens) ? (int32_t)token_slot(a, t) : -1;
    }
    __syncthreads();
}

template <bool PW>
__global__ __launch_bounds__(kThreads) void kv_write_bf16_kernel(KvWriteArgs a) {
    // chunks per token per tensor (K or V): n_kv * head_dim / 8
    const uint32_t C = (uint32_t)(a.n_kv_head * a.head_dim / 8);
    const uint32_t C2 = 2 * C;
    const uint32_t first_chunk = blockIdx.x * (uint32_t)kChunksPerBlock;
    const int64_t first_tok = first_chunk / C2;
    const int ntok = (int)((first_chunk + kChunksPerBlock - 1) / C2 - first_tok + 1);
    __shared__ int32_t slots[kChunksPerBlock / 8 + 2];
    const uint32_t total_chunks = (uint32_t)a.total_tokens * C2;

    // wave_lookup (the launcher sets it when C2 % 64 == 0, so the 64 chunks a
    // wave instruction covers belong to one token, and the grid takes more
    // than one round of resident blocks): each wave looks its items' slots up
    // itself with scalar loads before its data loads -- no block barrier, and
    // the lookups do not queue behind the data.  Otherwise the block resolves
    // its tokens' slots into LDS while its data loads are in flight, which is
    // faster when every block starts at once (the lookup latency would then
    // delay the whole launch).
    constexpr bool per_wave = PW;
    [[maybe_unused]] int32_t wslot[kItems];
    if constexpr (per_wave) {
        const uint32_t wfirst = first_chunk + (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x & ~63u);
#pragma unroll
        for (int i = 0; i < kItems; ++i) {
            const uint32_t t = (uint32_t)__builtin_amdgcn_readfirstlane((int)(min(wfirst + i * kThreads, total_chunks - 1) / C2));
            wslot[i] = (int32_t)token_slot(a, t);
        }
    }
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
    if constexpr (!per_wave) resolve_slots(a, first_tok, ntok, slots);
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        if (!live[i]) continue;
        const int32_t slot = per_wave ? wslot[i] : slots[tok[i] - first_tok];
        if (slot < 0) continue;
        uint16_t* pool = isv[i] ? (uint16_t*)a.v_cache : (uint16_t*)a.k_cache;
        __builtin_nontemporal_store(val[i], reinterpret_cast<u32x4_t*>(pool + ((uint64_t)(uint32_t)slot * C + cc[i]) * 8));
    }
}

// R = head_dim / 8 lanes hold one (token, kv head) row of K or V.  The row's
// amax is a max over those lanes; the divisions that follow are the same on
// all of them, so lane q of every quad divides for item q only (a quad lies
// inside one row group, R >= 4) and the quad exchanges the results by DPP:
// two divisions per lane instead of two per item.
template <int R, bool PW>
__global__ __launch_bounds__(kThreads) void kv_write_fp8_kernel(KvWriteArgs a) {
    static_assert(kItems == 4 && R >= 4, "one item per quad lane");
    const uint32_t C = (uint32_t)a.n_kv_head * R;            // chunks per token per tensor
    const uint32_t C2 = 2 * C;
    const uint32_t first_chunk = blockIdx.x * (uint32_t)kChunksPerBlock;
    const int64_t first_tok = first_chunk / C2;
    const int ntok = (int)((first_chunk + kChunksPerBlock - 1) / C2 - first_tok + 1);
    __shared__ int32_t slots[kChunksPerBlock / 8 + 2];
    const uint32_t total_chunks = (uint32_t)a.total_tokens * C2;

    // slots per wave with scalar loads, or per block in LDS, chosen as in the
    // bf16 write
    constexpr bool per_wave = PW;
    [[maybe_unused]] int32_t wslot[kItems];
    if constexpr (per_wave) {
        const uint32_t wfirst = first_chunk + (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x & ~63u);
#pragma unroll
        for (int i = 0; i < kItems; ++i) {
            const uint32_t t = (uint32_t)__builtin_amdgcn_readfirstlane((int)(min(wfirst + i * kThreads, total_chunks - 1) / C2));
            wslot[i] = (int32_t)token_slot(a, t);
        }
    }
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
    if constexpr (!per_wave) resolve_slots(a, first_tok, ntok, slots);

    float x[kItems][8];
    float amax[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[i][2 * j] = bf16_lo(w[i][j]);
            x[i][2 * j + 1] = bf16_hi(w[i][j]);
        }
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(x[i][j]));
        amax[i] = __builtin_bit_cast(float, group_umax<R>(__builtin_bit_cast(uint32_t, m)));
    }
    // binary32 round-to-nearest divisions (no fast-math): scale = amax / 448, inv = 448 / amax
    const uint32_t q = threadIdx.x & 3u;
    const float am = q == 0 ? amax[0] : q == 1 ? amax[1] : q == 2 ? amax[2] : amax[3];
    const float inv_q = am > 0.0f ? 448.0f / am : 0.0f;
    float inv[kItems];
    inv[0] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, inv_q), 0x00, 0xF, 0xF, false));
    inv[1] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, inv_q), 0x55, 0xF, 0xF, false));
    inv[2] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, inv_q), 0xAA, 0xF, 0xF, false));
    inv[3] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, inv_q), 0xFF, 0xF, 0xF, false));
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const uint32_t lo = e4m3x4(x[i][0] * inv[i], x[i][1] * inv[i], x[i][2] * inv[i], x[i][3] * inv[i]);
        const uint32_t hi = e4m3x4(x[i][4] * inv[i], x[i][5] * inv[i], x[i][6] * inv[i], x[i][7] * inv[i]);
        if (!live[i]) continue;
        const int32_t slot = per_wave ? wslot[i] : slots[tok[i] - first_tok];
        if (slot < 0) continue;
        uint8_t* pool = isv[i] ? (uint8_t*)a.v_cache : (uint8_t*)a.k_cache;
        __builtin_nontemporal_store(u32x2_t{lo, hi},
                                    reinterpret_cast<u32x2_t*>(pool + ((uint64_t)(uint32_t)slot * C + cc[i]) * 8));
    }
    // the scale of item q's row, stored by the lane at offset q inside the row
    if ((threadIdx.x & (R - 1)) < 4) {
        const bool lv = q == 0 ? live[0] : q == 1 ? live[1] : q == 2 ? live[2] : live[3];
        const uint32_t tq = q == 0 ? tok[0] : q == 1 ? tok[1] : q == 2 ? tok[2] : tok[3];
        const bool vq = q == 0 ? isv[0] : q == 1 ? isv[1] : q == 2 ? isv[2] : isv[3];
        const uint32_t cq = q == 0 ? cc[0] : q == 1 ? cc[1] : q == 2 ? cc[2] : cc[3];
        if (lv) {
            const int32_t slot = per_wave ? (q == 0 ? wslot[0] : q == 1 ? wslot[1] : q == 2 ? wslot[2] : wslot[3])
                                          : slots[tq - first_tok];
            if (slot >= 0) {
                float* sp = vq ? a.v_scale : a.k_scale;
                sp[(uint64_t)(uint32_t)slot * a.n_kv_head + cq / R] = am / 448.0f;
            }
        }
    }
}

// Elementwise E4M3 encoding of binary32 values (the encoder of every fp8
// producer here), four values per thread with one 16-byte load and one
// 4-byte store; a grid-stride loop covers any n.
__global__ __launch_bounds__(256) void e4m3_encode_kernel(const float* x, uint8_t* q, int64_t n) {
    const int64_t n4 = n / 4;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(x) + i);
        __builtin_nontemporal_store(e4m3x4(v[0], v[1], v[2], v[3]), reinterpret_cast<uint32_t*>(q) + i);
    }
    if (blockIdx.x == 0 && threadIdx.x < n - n4 * 4) {
        const int64_t i = n4 * 4 + threadIdx.x;
        q[i] = (uint8_t)(e4m3x4(x[i], 0.0f, 0.0f, 0.0f) & 0xFFu);
    }
}

uint32_t num_blocks(const KvWriteArgs& a) {
    uint64_t chunks = (uint64_t)a.total_tokens * 2 * (uint64_t)(a.n_kv_head * a.head_dim / 8);
    return (uint32_t)((chunks + kChunksPerBlock - 1) / kChunksPerBlock);
}

// per-wave slot lookups: a wave's 64 chunks must lie in one token (2 * n_kv *
// head_dim / 8 a multiple of 64), and the grid must be deeper than the 8
// resident blocks per CU (measured: T = 32768 fp8 +4-5%, T = 8192 bf16 -20%
// when every block starts at once)
KvWriteArgs with_lookup_mode(const KvWriteArgs& a) {
    KvWriteArgs b = a;
    const int64_t c2 = 2 * (int64_t)a.n_kv_head * a.head_dim / 8;
    const int ncu = device_cus();
    b.wave_lookup = c2 % 64 == 0 && ncu > 0 && (int64_t)num_blocks(a) > 8 * (int64_t)ncu ? 1 : 0;
    return b;
}

}  // namespace

hipError_t launch_kv_write_bf16(const KvWriteArgs& a0, hipStream_t s) {
    const KvWriteArgs a = with_lookup_mode(a0);
    if (a.wave_lookup)
        hipLaunchKernelGGL(kv_write_bf16_kernel<true>, dim3(num_blocks(a)), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(kv_write_bf16_kernel<false>, dim3(num_blocks(a)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_kv_write_fp8(const KvWriteArgs& a0, hipStream_t s) {
    const KvWriteArgs a = with_lookup_mode(a0);
    const dim3 grid(num_blocks(a)), block(kThreads);
    switch ((a.head_dim / 8) * 2 + (a.wave_lookup ? 1 : 0)) {
        case 8: hipLaunchKernelGGL((kv_write_fp8_kernel<4, false>), grid, block, 0, s, a); break;
        case 9: hipLaunchKernelGGL((kv_write_fp8_kernel<4, true>), grid, block, 0, s, a); break;
        case 16: hipLaunchKernelGGL((kv_write_fp8_kernel<8, false>), grid, block, 0, s, a); break;
        case 17: hipLaunchKernelGGL((kv_write_fp8_kernel<8, true>), grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL((kv_write_fp8_kernel<16, false>), grid, block, 0, s, a); break;
        case 33: hipLaunchKernelGGL((kv_write_fp8_kernel<16, true>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_e4m3_encode(const float* x, uint8_t* q, int64_t n, hipStream_t s) {
    const int64_t blocks = (n / 4 + 255) / 256;
    const uint32_t grid = (uint32_t)(blocks < 1 ? 1 : (blocks > 16384 ? 16384 : blocks));
    hipLaunchKernelGGL(e4m3_encode_kernel, dim3(grid), dim3(256), 0, s, x, q, n);
    return hipGetLastError();
}

}  // namespace pca
