// Shared pieces of the two MFMA GEMMs (bf16 and fp8 operands): tile
// geometry, the LDS swizzle, inline-asm LDS reads, the barrier, the
// XCD-aware tile order and wave-uniform buffer resources.  Both kernels keep
// K steps of 128 bytes per operand row (64 bf16 or 128 fp8 elements), so
// their DMA and LDS layouts are byte-identical.
#pragma once

#include "pca_device.hpp"

#include <utility>

namespace pca {
namespace gemm {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int BM = 256, BN = 256;
// (both GEMMs run eight waves of 128 (n) x 64 (m) and keep their wave
// constants in their own files)
constexpr int ROWB = 128;                     // bytes per tile row (one K step: 64 bf16 or 128 fp8)
constexpr int TILE_B = 256 * ROWB;            // 32 KiB: one operand tile
constexpr int STAGE_B = 2 * TILE_B;           // W tile, then X tile
constexpr int LDS_BYTES = 2 * STAGE_B;        // 128 KiB
constexpr int DMA_PER_TILE = TILE_B / 1024;   // 32 one-KiB DMA blocks per operand tile
constexpr int kGroupM = 8;
constexpr uint32_t kOob = 0x80000000u;        // an offset past every buffer: loads return 0

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ inline int swz(int row) { return (row >> 1) & 7; }

// s_waitcnt immediate waiting for vmcnt <= n only (gfx9 encoding: vmcnt in
// bits [15:14] and [3:0]; expcnt 7 and lgkmcnt 15 mean "no wait")
constexpr int vmcnt_imm(int n) { return ((n & 0x30) << 10) | (n & 0xF) | 0x0F70; }
static_assert(vmcnt_imm(0) == 0x0F70 && vmcnt_imm(16) == 0x4F70, "s_waitcnt encoding");

template <int OFF>
__device__ __forceinline__ u32x4_t lds_read_b128(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "DS offset field is 16 bits");
    u32x4_t r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
    return r;
}

// Workgroup barrier with no implied waits: the operand DMA of the next K step
// stays in flight across it.  All LDS reads are inline asm retired by explicit
// lgkmcnt waits, and the DMA by explicit vmcnt waits, before a barrier that
// needs them; the memory clobber and scheduling barriers pin the order.
__device__ __forceinline__ void wg_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Tile of grid position `id` in a tiles_m x tiles_n grid (see tile_coords).
__device__ inline void tile_coords_id(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    // XCD x runs positions x, x + 8, ...: it gets the contiguous range of
    // the total / 8 tiles (one more for the first total % 8 XCDs) from
    // x * (total / 8) + min(x, total % 8)
    const int per = total / kNumXcd, rem = total % kNumXcd, x = id % kNumXcd;
    id = x * per + min(x, rem) + id / kNumXcd;
    int per_group = kGroupM * tiles_n;
    int group = id / per_group;
    int first_m = group * kGroupM;
    int gsize = min(tiles_m - first_m, kGroupM);
    int in_group = id - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

__device__ inline void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
    tile_coords_id((int)blockIdx.x, tiles_m, tiles_n, tm, tn);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int64_t bytes) {
    const uint64_t b = (uint64_t)p;
    const uint64_t ub = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    return make_rsrc((const void*)ub, (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes));
}

// Grid shape (the data-flow article's §5.2 "wave" effect: a grid of 384
// tiles on 256 CUs takes two rounds for one and a half rounds of work).  A
// 128-row tile costs about 0.6 of a 256-row one (per-tile start-up and
// epilogue, half the operand reuse).
//  * A grid whose 128-row tiles all fit in one round of the CUs runs on them:
//    1024 x 6144 x 4096 has 96 tiles of 256 rows, which leave 160 CUs idle,
//    and runs 1.37-1.45x faster as 192 tiles of 128 rows.
//  * A grid of 256-row tiles whose last round is at most half full keeps the
//    full rounds in 256-row tiles (whole column strips) and turns the rest
//    into one round of 128-row tiles: 2048 x 12288 x 4096 is one round of 256
//    tiles of 256 rows plus 256 tiles of 128 rows (1.10x faster than 384
//    tiles of 256 rows, whose second round is half idle; 3000 x 6144 x 4096:
//    1.19x).  Only for grids of at most kMaxMixedRounds full rounds: 27808 x
//    6144 x 4096 (ten full rounds and a fifth) measured 2% slower mixed.
//  * Otherwise 256-row tiles throughout (a grid of only 128-row tiles
//    measured 16-22% slower than 256-row tiles on every multi-round shape).
// (Measured on the bf16 GEMM; the fp8 GEMM, with the same tiles, follows the
// same plan: 2048 x 12288 x 4096 +10%, 1024 x 6144 x 4096 +30%.)
constexpr int64_t kMaxMixedRounds = 3;

struct TilePlan {
    int bmt;       // 256, 128, or 0: split_n strips of 256-row tiles, then 128-row tiles
    int tiles;
    int split_n;
};

inline TilePlan plan_tiles(int64_t M, int64_t N, int64_t ncu) {
    const int64_t tn = (N + BN - 1) / BN, tm256 = (M + 255) / 256, tm128 = (M + 127) / 128;
    const int64_t t256 = tm256 * tn, t128 = tm128 * tn;
    if (ncu > 0) {
        if (t256 < t128 && t128 <= ncu) return {128, (int)t128, 0};
        const int64_t full = t256 / ncu * ncu;               // tiles of the full rounds
        if (full > 0 && full < t256 && full <= kMaxMixedRounds * ncu) {
            const int64_t n1 = full / tm256;                 // strips of 256-row tiles within them
            const int64_t small = tm128 * (tn - n1);
            if (n1 >= 1 && n1 < tn && small <= ncu) return {0, (int)(tm256 * n1 + small), (int)n1};
        }
    }
    return {256, (int)t256, 0};
}

}  // namespace gemm
}  // namespace pca
