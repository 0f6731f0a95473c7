// Fused QKV projection: y[M, N] = x[M, K] * w[N, K]^T (bf16 in, fp32 accumulate,
// bf16 RNE out).
//
// One GEMM with the Q, K and V weights concatenated, so the activation is read
// from HBM once (prefill data-flow article (hncyxsy.com/news/270449) §2.1 and
// §4.1); the weight arrives pre-transposed to (N, K) so both operands are read
// along K (§5.1).
//
// gfx950 design.
//  * Workgroup tile 256 x 256 (M x N), K step 64, eight waves, two per SIMD
//    (waves w and w + 4 share one), each a 64 (m) x 128 (n) sub-tile of
//    2 x 4 v_mfma_f32_32x32x16_bf16 blocks with its 128 fp32 accumulators per
//    lane in registers.  While one wave of a SIMD waits on its LDS operand
//    reads, the workgroup barrier or its DMA, the other issues MFMAs (one wave
//    per SIMD with a 128 x 128 sub-tile each measured 4-10% slower on every
//    projection shape, although it reads a third fewer LDS bytes per MFMA).
//    The wave computes the transposed product (MFMA rows = n, columns = m), so
//    each lane's accumulator holds 4 consecutive n of one m.  Grids too small
//    to fill the CUs, and the last round of short grids, use 128 x 256 tiles
//    instead (waves of 32 x 128); see plan_tiles.
//  * Operand tiles go from HBM/L2 straight into LDS with buffer_load ... lds
//    (no register staging, no LDS stores), double-buffered: the tiles of K
//    step kt + 2 are requested as soon as step kt's tiles are no longer read,
//    so each load has a whole K step of matrix work to land.  Only waves 0-3
//    (one per SIMD) request tiles: the CU accepts these requests at about 64
//    bytes per clock, so the 64 KiB of a K step keeps a requesting wave waiting
//    at its DMA instructions for ~600-1000 cycles.  Requested by every wave,
//    right after the barrier, that wait held both waves of each SIMD off the
//    matrix cores at once; now the other wave of the SIMD issues MFMAs through
//    it (+4-7% on the projection shapes, the same bits).  Rows of 64
//    elements (8 chunks of 16 bytes) are stored with chunk c of row r at
//    c ^ ((r >> 1) & 7): the 16 rows a 16-lane group of a ds_read_b128 touches
//    then cover all 64 banks once.
//  * The 32 MFMAs of a wave's K step run as one fixed sequence; the 6 operand
//    reads of each 16-key step are issued one step ahead as inline asm and
//    retired by explicit lgkmcnt waits, and scheduling barriers keep the
//    order.  (Deeper DMA pipelines -- 4 or 5 stages of 32-wide K steps -- and
//    operand reads two steps ahead measured slower or equal.)
//  * Ragged M, N read zeros through the buffer-resource range check, a ragged
//    K tail through an out-of-range offset.
//  * Tile order: consecutive workgroup ids go round-robin to the 8 XCDs, so
//    the id is first remapped so that each XCD owns one contiguous range of
//    tiles, which is then walked in groups of 8 M-tiles: the tiles resident on
//    one XCD at a time share A rows and B columns in that XCD's L2.
#include "gemm_common.hpp"
#include "kv_common.hpp"

#include <utility>

namespace pca {

namespace {

using namespace gemm;

constexpr int BKK = 64;                       // bf16 elements per K step (ROWB bytes)
constexpr int kWavesG = 8;                    // two waves per SIMD
constexpr int kThreadsG = kWavesG * 64;
constexpr int FNg = 4;                        // 32 x 32 blocks per wave along n: 128 columns
constexpr int kDmaWaves = 4;                  // waves 0..3 request every operand tile
constexpr int DMA_W_PER_WAVE = DMA_PER_TILE / kDmaWaves;   // 1 KiB DMA blocks of the W tile per requesting wave

// Wait until at most N LDS reads are outstanding; the fragments pass through
// the asm so their consumers stay after the wait (6 or 5 fragments per step).
template <int N>
__device__ __forceinline__ void lds_wait_f(u32x4_t (&f)[6]) {
    asm volatile("s_waitcnt lgkmcnt(%6)"
                 : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]), "+v"(f[5])
                 : "n"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait_f(u32x4_t (&f)[5]) {
    asm volatile("s_waitcnt lgkmcnt(%5)" : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]) : "n"(N));
}

// KV = 0: plain GEMM; 1 / 2: the epilogue also writes y's K and V columns
// into the bf16 / fp8 page pools.  RES: y = x w^T + res, the residual added
// to the fp32 accumulators before the single bf16 rounding.  RS: the fp32
// accumulators of row m are scaled by row_scale[m] before that rounding.
// BMT: rows of x per tile, 256 (waves of 64 x 128) or 128 (waves of 32 x 128).
// One workgroup computes output tile (tm, tn).
template <int KV, bool RES, bool RS, int BMT>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, int tm, int tn) {
    constexpr int FMg = BMT / 128;                    // 32 x 32 blocks per wave along m
    constexpr int WMR = 32 * FMg;                     // x rows per wave
    constexpr int NF = FNg + FMg;                     // operand fragments per 16-key step
    constexpr int DMA_X_PER_WAVE = BMT * ROWB / 1024 / kDmaWaves;   // 1 KiB DMA blocks of the x tile per requesting wave
    extern __shared__ __align__(16) uint16_t smem[];
    lds_char_t* lds = (lds_char_t*)smem;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;     // wave position: 4 (m) x 2 (n)
    const int r32 = lane & 31, half = lane >> 5;

    const int m0 = tm * BMT, n0 = tn * BN;
    const int rows_x = min(BMT, a.M - m0), rows_w = min(BN, a.N - n0);
    const int nk = (a.K + BKK - 1) / BKK;

    // DMA lane offsets (bytes from the tile's first row at the current K step)
    // of the requesting waves 0..3 (the others compute them too, unused):
    // block b of a wave covers rows 8b .. 8b + 7; lane l writes physical chunk
    // l % 8 of row 8b + l / 8, i.e. fetches logical chunk (l % 8) ^ swz(row).
    // (sized for the 256-row tile: a lambda capturing an array whose size
    // depends on BMT leaves the host side without the kernel's stub)
    uint32_t offx[DMA_W_PER_WAVE], offw[DMA_W_PER_WAVE];
    int lchx[DMA_W_PER_WAVE], lchw[DMA_W_PER_WAVE];
    static_assert(DMA_X_PER_WAVE <= DMA_W_PER_WAVE, "x tile has at most 256 rows");
#pragma unroll
    for (int i = 0; i < DMA_W_PER_WAVE; ++i) {
        const int row = ((wave & (kDmaWaves - 1)) * DMA_W_PER_WAVE + i) * 8 + lane / 8;
        lchw[i] = (lane % 8) ^ swz(row);
        offw[i] = (uint32_t)(((int64_t)row * a.ldw + lchw[i] * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < DMA_X_PER_WAVE; ++i) {
        const int row = ((wave & (kDmaWaves - 1)) * DMA_X_PER_WAVE + i) * 8 + lane / 8;
        lchx[i] = (lane % 8) ^ swz(row);
        offx[i] = (uint32_t)(((int64_t)row * a.ldx + lchx[i] * 8) * 2);
    }
    auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
        const int k0 = kt * BKK;
        const bool tail = k0 + BKK > a.K;        // uniform: last step of a ragged K
        const __amdgpu_buffer_rsrc_t rw =
            uniform_rsrc(a.w + (int64_t)n0 * a.ldw + k0, (int64_t)rows_w * a.ldw * 2 - (int64_t)k0 * 2);
        const __amdgpu_buffer_rsrc_t rx =
            uniform_rsrc(a.x + (int64_t)m0 * a.ldx + k0, (int64_t)rows_x * a.ldx * 2 - (int64_t)k0 * 2);
        lds_char_t* dst = lds + stage * STAGE_B;
        if (wave >= kDmaWaves) return;                    // uniform per wave
#pragma unroll
        for (int i = 0; i < DMA_W_PER_WAVE; ++i) {
            const int blk = wave * DMA_W_PER_WAVE + i;
            const bool oob = tail && (k0 + lchw[i] * 8 >= a.K);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)(dst + blk * 1024), 16,
                                                     oob ? kOob : offw[i], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < DMA_X_PER_WAVE; ++i) {
            const int blk = wave * DMA_X_PER_WAVE + i;
            const bool oob = tail && (k0 + lchx[i] * 8 >= a.K);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(dst + TILE_B + blk * 1024), 16,
                                                     oob ? kOob : offx[i], 0, 0, 0);
        }
    };

    // operand read addresses: both operands read row (block*32 + r32), logical
    // chunk ks*2 + half; the swizzle depends only on r32, so one address per
    // (stage, ks) serves every block through the immediate offset
    uint32_t waddr[4], xaddr[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const uint32_t base = (uint32_t)(uintptr_t)lds + r32 * ROWB + (((ks * 2 + half) ^ swz(r32)) * 16);
        waddr[ks] = base + wn * 128 * ROWB;
        xaddr[ks] = base + wm * WMR * ROWB;
    }

    f32x16_t acc[FNg][FMg];
#pragma unroll
    for (int i = 0; i < FNg; ++i)
#pragma unroll
        for (int j = 0; j < FMg; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // NF operand fragments of 16-key step ks: W blocks i (rows wn*128 + i*32),
    // X blocks j (rows wm*WMR + j*32)
    auto read_step = [&](uint32_t soff, auto KSc, u32x4_t (&f)[NF]) __attribute__((always_inline)) {
        constexpr int ks = decltype(KSc)::value;
        const uint32_t wa = waddr[ks] + soff, xa = xaddr[ks] + soff;
        static_for<FNg>([&](auto Ic) {
            constexpr int i = decltype(Ic)::value;
            f[i] = lds_read_b128<i * 32 * ROWB>(wa);
        });
        static_for<FMg>([&](auto Jc) {
            constexpr int j = decltype(Jc)::value;
            f[FNg + j] = lds_read_b128<TILE_B + j * 32 * ROWB>(xa);
        });
    };
    auto mfmas = [&](const u32x4_t (&f)[NF]) __attribute__((always_inline)) {
        static_for<FNg * FMg>([&](auto Ic) {
            constexpr int i = decltype(Ic)::value / FMg, j = decltype(Ic)::value % FMg;
            acc[i][j] = mfma32x32x16(as_bf16x8(f[i]), as_bf16x8(f[FNg + j]), acc[i][j]);
        });
        __builtin_amdgcn_sched_barrier(0);
    };

    // Software pipeline over K steps with two LDS stages and one barrier per
    // step.  The operands of 16-key step ks + 1 are read while ks runs on the
    // matrix cores.  The barrier of step kt sits after the wave's last LDS read
    // of stage kt & 1 and before that step's last 8 MFMAs: past it, step
    // kt + 1's tiles are visible (every wave waited for its own loads first)
    // and stage kt & 1 is free, so the first operands of step kt + 1 are read
    // and step kt + 2's tiles requested while those 8 MFMAs run.
    issue(0, 0);
    if (1 < nk) issue(1, 1);
    if (1 < nk) __builtin_amdgcn_s_waitcnt(vmcnt_imm(DMA_W_PER_WAVE + DMA_X_PER_WAVE));   // step 0 only
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    wg_barrier();
    u32x4_t f[2][NF];
    read_step(0u, std::integral_constant<int, 0>{}, f[0]);
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        const uint32_t soff = (uint32_t)(st * STAGE_B);
        static_for<3>([&](auto KSc) {
            constexpr int ks = decltype(KSc)::value;
            read_step(soff, std::integral_constant<int, ks + 1>{}, f[(ks + 1) & 1]);
            lds_wait_f<NF>(f[ks & 1]);
            mfmas(f[ks & 1]);
        });
        lds_wait_f<0>(f[1]);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // this wave's loads of step kt + 1
        wg_barrier();
        if (kt + 1 < nk) read_step(soff ^ (uint32_t)STAGE_B, std::integral_constant<int, 0>{}, f[0]);
        if (kt + 2 < nk) issue(kt + 2, st);
        mfmas(f[1]);
    }

    // Epilogue.  The accumulators hold, per block (i, j), column m = r32 and
    // rows n = g*8 + half*4 + 0..3 -- 8-byte runs spread over 32 rows of y per
    // store instruction.  Each wave instead stages its WMR x 128 bf16 tile in
    // LDS (token-major, 16-byte chunks XOR-swizzled by row so neither the
    // 32-row writes nor the row reads collide on banks) and writes it back as
    // full rows: 16 lanes x 16 bytes = one 256-byte run of a y row per lane
    // group, four rows per store instruction.
    wg_barrier();                                        // every wave is done with the operand stages
    lds_char_t* stg = lds + wave * (WMR * 256);          // this wave's staging rows
    const int c = lane & 15;                             // the lane's 16-byte chunk of a row: columns c*8 .. c*8+7
    const int n = n0 + wn * 128 + c * 8;
    const int m_lo = m0 + wm * WMR;
    if constexpr (RES) {
        // the residual sub-tile goes into the staging area first, row by row
        // (coalesced 16-byte loads), and is added to the accumulators below.
        // The loads go out eight at a time through a buffer resource over
        // rows m_lo .. M - 1 (rows past M read 0), so one wait covers eight
        // (loaded one by one behind per-row branches, each load was waited
        // for on its own: 2-4% slower).  A lane whose 8 columns cross N
        // (ragged N only) reads them one by one.
        if (n + 7 < a.N) {
            const int64_t rows_left = a.M > m_lo ? (int64_t)(a.M - m_lo) : 0;
            const __amdgpu_buffer_rsrc_t rr =
                uniform_rsrc(a.res + (int64_t)m_lo * a.ldr, min<int64_t>(rows_left * a.ldr * 2, 0x7FFFFFFF));
#pragma unroll
            for (int r0 = 0; r0 < WMR / 4; r0 += 8) {
                u32x4_t rv[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int ml = (r0 + k) * 4 + (lane >> 4);
                    rv[k] = __builtin_amdgcn_raw_buffer_load_b128(rr, (uint32_t)(((int64_t)ml * a.ldr + n) * 2), 0, 0);
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int ml = (r0 + k) * 4 + (lane >> 4);
                    *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(stg + ml * 256 + ((c ^ (ml & 15)) * 16)) =
                        rv[k];
                }
            }
        } else {
            for (int r = 0; r < WMR / 4; ++r) {
                const int ml = r * 4 + (lane >> 4);
                const int m = m_lo + ml;
                u32x4_t rv = {0u, 0u, 0u, 0u};
                if (m < a.M) {
                    const uint16_t* src = a.res + (int64_t)m * a.ldr + n;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < a.N) rv[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
                }
                *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(stg + ml * 256 + ((c ^ (ml & 15)) * 16)) = rv;
            }
        }
    }
    // RMSNorm folded in: the row scale multiplies the fp32 accumulators (the
    // norm's gain is folded into the weight's K axis at load time)
#pragma unroll
    for (int j = 0; j < FMg; ++j) {
        [[maybe_unused]] float rsc = 1.0f;
        if constexpr (RS) {
            const int m = m_lo + j * 32 + r32;
            if (m < a.M) rsc = a.row_scale[m];
        }
#pragma unroll
        for (int i = 0; i < FNg; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int ml = j * 32 + r32, ci = i * 4 + g;
                __attribute__((address_space(3))) u32x2_t* slot =
                    reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>(stg + ml * 256 + ((ci ^ (ml & 15)) * 16) + half * 8);
                float t0 = acc[i][j][g * 4 + 0], t1 = acc[i][j][g * 4 + 1];
                float t2 = acc[i][j][g * 4 + 2], t3 = acc[i][j][g * 4 + 3];
                if constexpr (RS) {
                    t0 *= rsc; t1 *= rsc; t2 *= rsc; t3 *= rsc;
                }
                if constexpr (RES) {
                    const u32x2_t rr = *slot;                // this lane's own 4 residual values
                    t0 += bf16_lo(rr[0]); t1 += bf16_hi(rr[0]);
                    t2 += bf16_lo(rr[1]); t3 += bf16_hi(rr[1]);
                }
                *slot = u32x2_t{pack_bf16x2(t0, t1), pack_bf16x2(t2, t3)};
            }
    }

    // fused KV-cache write: where the lane's 8 columns go (the data-flow
    // article's §4.2 point -- the projection output goes straight into its
    // page slot, no second pass over K and V).  The cache receives exactly
    // the bf16 values stored to y, so it equals a separate pca_kv_cache_write
    // of y.
    [[maybe_unused]] const KvWriteArgs& kv = a.kv;
    [[maybe_unused]] int kv_sel = -1, kvh = 0, dcol = 0;   // 0: K, 1: V; kv head and first d of the chunk
    [[maybe_unused]] int slot_lo = -1;                     // page slot of token m_lo + lane
    if constexpr (KV != 0) {
        const int hd = kv.head_dim, nkc = kv.n_kv_head * hd;
        int col = -1;
        if (n >= a.k_col0 && n < a.k_col0 + nkc) { kv_sel = 0; col = n - a.k_col0; }
        else if (n >= a.v_col0 && n < a.v_col0 + nkc) { kv_sel = 1; col = n - a.v_col0; }
        if (col >= 0) { kvh = col / hd; dcol = col - kvh * hd; }
        // only waves whose columns touch K or V look up page slots
        const int nw0 = n0 + wn * 128, nw1 = min(nw0 + 128, a.N);
        if ((nw0 < a.k_col0 + nkc && nw1 > a.k_col0) || (nw0 < a.v_col0 + nkc && nw1 > a.v_col0)) {
            if (lane < WMR && m_lo + lane < a.M) slot_lo = (int)token_slot(kv, m_lo + lane);

        }
    }

#pragma unroll 4
    for (int r = 0; r < WMR / 4; ++r) {
        const int ml = r * 4 + (lane >> 4);
        const u32x4_t v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
            stg + ml * 256 + ((c ^ (ml & 15)) * 16));
        const int m = m_lo + ml;
        [[maybe_unused]] int slot = -1;
        if constexpr (KV != 0)   // the slot of row ml sits in lane ml of slot_lo
            slot = __builtin_amdgcn_ds_bpermute((ml & 63) * 4, slot_lo);
        if (m >= a.M) continue;
        uint16_t* dst = a.y + (int64_t)m * a.ldy + n;
        if (n + 7 < a.N) {
            *reinterpret_cast<u32x4_t*>(dst) = v;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < a.N) dst[e] = (uint16_t)((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        }
        if constexpr (KV == 1) {
            if (kv_sel >= 0 && slot >= 0) {
                uint16_t* pool = kv_sel == 0 ? (uint16_t*)kv.k_cache : (uint16_t*)kv.v_cache;
                *reinterpret_cast<u32x4_t*>(pool + ((int64_t)slot * kv.n_kv_head + kvh) * kv.head_dim + dcol) = v;
            }
        } else if constexpr (KV == 2) {
            // fp8: the wave's 128 columns are whole heads of K or of V (the
            // host checks that both ranges start on a multiple of 128 and span
            // a multiple of 128), so kv_sel is uniform over the wave and a
            // (token, kv head) row is hd / 8 consecutive lanes of a 16-lane
            // row group.  Codes come from the bf16 values, as for a separate
            // write from y.
            if (kv_sel >= 0) {
                float x[8];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    x[2 * t] = bf16_lo(v[t]);
                    x[2 * t + 1] = bf16_hi(v[t]);
                }
                float amax = 0.0f;
#pragma unroll
                for (int t = 0; t < 8; ++t) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[t]));
                const int hd = kv.head_dim;
                amax = hd == 128 ? group_max<16>(amax) : hd == 64 ? group_max<8>(amax) : group_max<4>(amax);
                if (slot >= 0) {
                    // binary32 round-to-nearest division (no fast-math): scale = amax / 448, inv = 448 / amax
                    const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
                    const uint32_t lo = e4m3x4(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
                    const uint32_t hi = e4m3x4(x[4] * inv, x[5] * inv, x[6] * inv, x[7] * inv);
                    const int64_t row = (int64_t)slot * kv.n_kv_head + kvh;
                    uint8_t* pool = kv_sel == 0 ? (uint8_t*)kv.k_cache : (uint8_t*)kv.v_cache;
                    *reinterpret_cast<u32x2_t*>(pool + row * hd + dcol) = u32x2_t{lo, hi};
                    if (dcol == 0) (kv_sel == 0 ? kv.k_scale : kv.v_scale)[row] = amax / 448.0f;
                }
            }
        }
    }
}

// The grid: BMT 256 or 128, tiles of that height over the whole output; BMT
// 0, the first split_n column strips (BN wide) in 256-row tiles, then the
// rest of N in 128-row tiles, the 256-row tiles first in dispatch order.
template <int KV, bool RES, bool RS, int BMT>
__global__ __launch_bounds__(kThreadsG) __attribute__((amdgpu_waves_per_eu(2, 2)))
void qkv_gemm_kernel(GemmArgs a, int split_n) {
    const int tiles_n = (a.N + BN - 1) / BN;
    int tm, tn;
    if constexpr (BMT != 0) {
        tile_coords_id((int)blockIdx.x, (a.M + BMT - 1) / BMT, tiles_n, tm, tn);
        gemm_tile<KV, RES, RS, BMT>(a, tm, tn);
    } else {
        const int tm256 = (a.M + 255) / 256, big = tm256 * split_n;
        if ((int)blockIdx.x < big) {
            tile_coords_id((int)blockIdx.x, tm256, split_n, tm, tn);
            gemm_tile<KV, RES, RS, 256>(a, tm, tn);
        } else {
            tile_coords_id((int)blockIdx.x - big, (a.M + 127) / 128, tiles_n - split_n, tm, tn);
            gemm_tile<KV, RES, RS, 128>(a, tm, tn + split_n);
        }
    }
}

}  // namespace

namespace {

// One wave per row: 16-byte loads along the row, fp32 sum of squares, a
// cross-lane reduction, then 1 / sqrt(mean + eps) (IEEE division and square
// root, no fast-math).  HBM-bound: reads x once.  The loads go out eight at a
// time (4096 elements of the row per batch) before any of them is summed, so
// a wave has 128 bytes per lane in flight instead of waiting on each load;
// each lane still adds its elements in row order.
__global__ __launch_bounds__(256) void rms_stats_kernel(const uint16_t* x, int64_t ldx, int M, int K, float eps,
                                                        float* inv_rms) {
    constexpr int NB = 8;
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;                                   // uniform per wave
    const uint16_t* row = x + (int64_t)m * ldx;
    float acc = 0.0f;
    for (int k0 = lane * 8; k0 < K; k0 += NB * 512) {     // K is a multiple of 8
        u32x4_t v[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int k = k0 + i * 512;
            v[i] = k < K ? *reinterpret_cast<const u32x4_t*>(row + k) : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float lo = bf16_lo(v[i][t]), hi = bf16_hi(v[i][t]);
                acc = __builtin_fmaf(lo, lo, acc);
                acc = __builtin_fmaf(hi, hi, acc);
            }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) inv_rms[m] = 1.0f / __builtin_sqrtf(acc / (float)K + eps);
}

template <int KV, bool RES, bool RS, int BMT>
hipError_t launch_tiles(const GemmArgs& a, int tiles, int split_n, hipStream_t s) {
    static const hipError_t attr = hipFuncSetAttribute((const void*)qkv_gemm_kernel<KV, RES, RS, BMT>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((qkv_gemm_kernel<KV, RES, RS, BMT>), dim3(tiles), dim3(kThreadsG), LDS_BYTES, s, a, split_n);
    return hipGetLastError();
}

template <int KV, bool RES, bool RS>
hipError_t launch_kv(const GemmArgs& a, hipStream_t s) {
    const TilePlan t = plan_tiles(a.M, a.N, device_cus());
    if (t.bmt == 128) return launch_tiles<KV, RES, RS, 128>(a, t.tiles, 0, s);
    if (t.bmt == 0) return launch_tiles<KV, RES, RS, 0>(a, t.tiles, t.split_n, s);
    return launch_tiles<KV, RES, RS, 256>(a, t.tiles, 0, s);
}

}  // namespace

hipError_t launch_qkv_gemm(const GemmArgs& a, hipStream_t s) {
    if (a.res != nullptr)
        return a.kv_mode == 0 && a.row_scale == nullptr ? launch_kv<0, true, false>(a, s) : hipErrorInvalidValue;
    if (a.row_scale != nullptr) return a.kv_mode == 0 ? launch_kv<0, false, true>(a, s) : hipErrorInvalidValue;
    switch (a.kv_mode) {
        case 0: return launch_kv<0, false, false>(a, s);
        case 1: return launch_kv<1, false, false>(a, s);
        case 2: return launch_kv<2, false, false>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rms_stats(const uint16_t* x, int64_t ldx, int M, int K, float eps, float* inv_rms, hipStream_t s) {
    hipLaunchKernelGGL(rms_stats_kernel, dim3((uint32_t)((M + 3) / 4)), dim3(256), 0, s, x, ldx, M, K, eps, inv_rms);
    return hipGetLastError();
}

}  // namespace pca
