// Causal GQA flash-attention forward for prefill, gfx950.
//
// Computes, per packed sequence, query head i (kv head g = i / G) and row r,
//   o[r, i] = sum_{c <= r} softmax_c(q[r, i] . k[c, g] * scale) v[c, g]
// as the fused blockwise form of the prefill data-flow article
// (hncyxsy.com/news/270449): scores QK^T scaled by 1/sqrt(head_dim) (§3.1),
// online softmax with a running max and exp-sum per row and rescaling of the
// partial output when the max moves (§3.2), the causal mask as control flow
// over kv tiles (§3.1, §4.3), GQA sharing of one K/V head by G query heads
// (§3.4), and heads written straight into the flattened (s, n_head*hd) output
// (§3.3).  Scores never leave registers.
//
// gfx950 mapping.
//  * A wave owns 32 query rows of one head.  A workgroup is 8 waves that
//    share one kv head (and so every K/V tile in LDS), one workgroup per CU:
//    two waves per SIMD, waves w and w + 4 on the same SIMD.  For G = 4 the
//    workgroup is 4 query heads x 64 consecutive rows.
//  * Ping-pong between the two waves of a SIMD.  Waves 0-3 (group A) and
//    4-7 (group B) alternate two phases per kv tile, switching at a
//    workgroup barrier: the matrix phase (O += P V for this tile, then the
//    scores of the next tile) and the softmax phase (max, exponentials, sums,
//    packing of P).  While one wave of a SIMD is in its matrix phase the
//    other is in its softmax, so the MFMA pipe and the VALU work at the same
//    time; the matrix-phase wave runs at raised priority so its MFMAs issue
//    as soon as the pipe frees.  (Within one wave, transcendental VALU work
//    overlaps poorly with that wave's own MFMAs; across two waves it
//    overlaps almost completely.)
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the 32x32 accumulator then holds, in each
//    lane, 16 keys of ONE query (the lane's column).  Row max and row sum are
//    lane-local plus one exchange between the wave's two 32-lane halves
//    (v_permlane32_swap, no LDS traffic), and the accumulator is
//    already the B operand of the second product O^T = V^T P^T once
//    converted to bf16 -- no cross-lane shuffle of P.
//  * K runs one tile ahead of V (the matrix phase of tile j needs K_{j+1}
//    and V_j): K and V have separate LDS double buffers, and the tiles
//    K_{j+2}, V_{j+1} are in flight during tile j.  They go from HBM/L2
//    straight into LDS with buffer_load ... lds (no register staging).  Rows
//    are stored key-major with the 16-byte chunks of each row XOR-swizzled
//    by the row index, so that the K operand reads (ds_read_b128, 16 rows per
//    16 lanes) and the V operand reads hit all 64 banks once.  V^T comes out
//    of LDS with the gfx950 transpose read ds_read_b64_tr_b16: each 16-lane
//    group returns, for 16 consecutive d, 4 keys per lane -- the A-operand
//    layout of O^T = V^T P^T, in the same key order the S^T accumulator hands
//    to the B operand (within 16 keys: 0-3, 8-11 | 4-7, 12-15).
//  * Q stays in registers (B operand of S^T) for the whole kv loop; the O^T
//    accumulator (fp32) likewise.
//  * scale*log2(e) is folded into Q once (before its bf16 rounding), and
//    each score chain starts from the accumulator value -R, R the row's
//    reference max in log2 units: the MFMA hands over s*c - R and the
//    softmax of a tile is one exp2 and one add per score, plus the packing
//    of P to bf16 (m, l, P in fp32; P rounded to bf16 only as the MFMA
//    operand).  A row moves R up to its tile max only on the wave's first
//    tile and when its tile sum of p passes 2^12; only then are the max, the
//    rescale of O and l and the -R accumulator refreshed, behind one branch.
//  * The causal rule: a wave skips kv tiles that start after its last query,
//    and masks per element only on tiles that reach past its first query.
//    Workgroups are ordered heaviest-first (rank-major when every workgroup
//    takes one task group, unit-major with the longest sequence first when
//    workgroups take a heavy and a light one), and units (sequence, kv head)
//    go round-robin over the 8 XCDs (workgroup ids are dispatched that way),
//    so one unit's K/V stays in one XCD's L2 and, with 8 kv heads, every XCD
//    gets one kv head of every sequence.
#include "pca_device.hpp"
#include "pca_internal.hpp"

#include <cstring>

#include <utility>

namespace pca {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int kWaves = 8;               // per workgroup; waves w and w + 4 share a SIMD
constexpr int kThreads = kWaves * 64;
constexpr int BQ = 32;                  // query rows per wave
constexpr int BK = 64;                  // keys per kv tile
constexpr float kSumLimit = 4096.0f;    // a row's reference moves when its tile sum of p exceeds this
constexpr int kVmcnt0 = 0x0F70;         // s_waitcnt vmcnt(0), other counters unconstrained

template <int HD>
struct Cfg {
    static constexpr int NC = HD / 8;                    // 16-byte chunks per key row
    static constexpr int ROWB = HD * 2;                  // bytes per key row
    static constexpr int TILE = BK * ROWB;               // bytes of one K (or V) tile
    static constexpr int KBUF0 = 0, KBUF1 = TILE;        // K double buffer
    static constexpr int VBUF0 = 2 * TILE, VBUF1 = 3 * TILE;   // V double buffer
    static constexpr int LDS_BYTES = 4 * TILE;
    static constexpr int RPI = 1024 / ROWB;              // key rows per 1 KiB DMA block
    static constexpr int NBLK = TILE / 1024;             // 1 KiB DMA blocks per tile
    static constexpr int DMA_ITERS = (NBLK + kWaves - 1) / kWaves;
    static constexpr int DCH = HD / 16;                  // k16 steps over head_dim
    static constexpr int DB = HD / 32;                   // 32-row blocks of O^T
    // fp8 pages: a tile of E4M3 codes (1 byte each) is staged behind the bf16
    // buffers and converted into them by the wave that loaded it
    static constexpr int T8 = BK * HD;                   // bytes of one fp8 tile
    static constexpr int NB8 = T8 / 1024;                // 1 KiB DMA blocks per fp8 tile (<= 8 waves)
    static constexpr int RPI8 = 1024 / HD;               // key rows per fp8 block
    static constexpr int F8K0 = 4 * TILE, F8K1 = F8K0 + T8, F8V0 = F8K0 + 2 * T8, F8V1 = F8K0 + 3 * T8;
    static constexpr int LDS_FP8 = 4 * TILE + 4 * T8;
    static_assert(VBUF1 + 3 * 16 * ROWB < 65536, "V reads use 16-bit DS immediate offsets");
};

// Physical 16-byte chunk of logical chunk c in key row r is c ^ swz(r): the
// keys of 16 consecutive rows are all distinct (K reads), and so are the
// physical chunks of 4 consecutive rows x 4 consecutive chunks (V transpose
// reads), for head_dim 128.
template <int HD>
__device__ inline int swz(int r) { return ((r & 3) * 4 + ((r >> 2) & 3)) & (Cfg<HD>::NC - 1); }

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ inline uint32_t lds_addr(const lds_char_t* p) { return (uint32_t)(uintptr_t)p; }

// Workgroup barrier with no implied waits.  __syncthreads (and any fence on
// LDS) makes the compiler wait for every outstanding global load, because the
// K/V DMA writes LDS; here the DMA must stay in flight across half-steps.  No
// fence is needed: every LDS read of the kernel is inline asm retired by an
// explicit lgkmcnt wait before its data is used, and the DMA is retired by an
// explicit vmcnt wait before the barrier that publishes it.  The memory
// clobber and the scheduling barriers keep the compiler from moving anything
// across.
__device__ __forceinline__ void wg_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// ds_read_b64_tr_b16 as inline asm.  Issued through the builtin, the read
// carries no alias information, and the compiler then waits for every
// outstanding global->LDS DMA (the next kv tiles, which target the other
// buffers) before it; as asm its completion is tracked by lds_wait.
template <int OFF>
__device__ __forceinline__ u32x2_t lds_read_tr16(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "DS offset field is 16 bits");
    u32x2_t r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
    return r;
}

// ds_read_b128 as inline asm, for the same reason: all LDS reads of the
// matrix phase are issued and retired under explicit control.
template <int OFF>
__device__ __forceinline__ u32x4_t lds_read_b128(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "DS offset field is 16 bits");
    u32x4_t r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
    return r;
}

// Wait until at most N LDS operations are outstanding (LDS returns in order);
// the fragment passes through the asm so its consumer stays after the wait.
template <int N>
__device__ __forceinline__ void lds_wait(u32x4_t& v) {
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait(u32x2_t& a, u32x2_t& b) {
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait(u32x4_t& a, u32x4_t& b) {
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait(u32x4_t& a, u32x4_t& b, u32x2_t& c) {
    asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(a), "+v"(b), "+v"(c) : "n"(N));
}
template <int OFF>
__device__ __forceinline__ uint32_t lds_read_b32(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "DS offset field is 16 bits");
    uint32_t r;
    asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
    return r;
}

// LDS reads still in flight after those of MFMA i of a matrix phase, when
// the reads run LA MFMAs ahead: MFMAs [0, NPV) take two reads, the rest RS.
template <int NPV, int NM, int LA, int RS>
constexpr int reads_after(int i) {
    int n = 0;
    for (int m = i + 1; m <= i + LA - 1 && m < NM; ++m) n += (m < NPV) ? 2 : RS;
    return n;
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// S^T block from fp8 operands: 32 keys x 32 queries over 64 head dims, A = K
// rows (32 bytes per lane), B = Q^T columns, each lane's 32-element block
// scaled by 2^(byte - 127) of its own row (key) and column (query).
// The A fragment is used again after the instruction (an empty asm), so it
// stays live across it and the result registers cannot be allocated on top
// of it: the compiler otherwise lets this instruction's destination overlap
// its A source, which no other MFMA of the kernel is allowed to do.
__device__ inline f32x16_t mfma_f8s(u32x4_t a0, u32x4_t a1, u32x4_t b0, u32x4_t b1, f32x16_t c, int sa, int sb) {
    const i32x8_t a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    const i32x8_t b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    const f32x16_t d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
    asm volatile("" ::"v"(a), "v"(b));
    return d;
}

// fp8 K tiles sit in the first 8 KiB of a K buffer; the 64 keys' scale words
// (the 4-byte word holding each key's scale byte) follow at this offset
constexpr int kExpOff = 8192;

// fp8 K tiles: 128-byte rows; physical 16-byte chunk of logical chunk c in
// row r is c ^ swz8(r), so any 8 consecutive rows read at one logical chunk
// hit 8 different chunk slots, and so do the rows of equal parity among 16
// consecutive ones (the two 128-byte halves of a 256-byte bank line).
__device__ inline int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }

struct Params {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    int64_t ldq, ldk, ldv;
    const int32_t* cu;
    int num_seqs;
    int64_t total;
    int n_kv, group;
    float c;            // scale * log2(e)
    uint16_t* o;
    int64_t ldo;
    int ntg;            // workgroup ranks per (sequence, kv head) in the grid
    int pair;           // 1: a workgroup takes a heavy and a light task group of its unit
    int units;          // num_seqs * n_kv
    int bt_cap;         // paged: block-table entries the LDS row holds (keys past bt_cap * 16 are not read)
    int persist;        // 1: one workgroup per CU walks its XCD's compact list (see the kernel)
    int tab_off;        // LDS byte offset of that list's counts and the slot -> sequence table
    // paged K/V (chunk over a cached prefix): k, v are the page pools
    // [page][slot][n_kv][hd]; key c of sequence b sits in page bt[b][c / 16],
    // slot c % 16; the sequence has ctx[b] keys, the last cu[b+1] - cu[b] of
    // them being the chunk's own
    const int32_t* bt;
    int mp;             // block-table row length
    const int32_t* ctx;
    uint32_t pool_bytes;
    int num_pages;      // paged: block-table entries outside [0, num_pages) read as zeros
    int window;         // > 0: sliding window, row r sees keys r - window < c <= r
    const float* k_scale;   // fp8 pages: per-(slot, kv head) scales [page][16][n_kv]
    const float* v_scale;
    // fp8 score operands: K codes (token rows, stride ldk8 bytes) and their
    // power-of-two scale bytes (token rows of n_kv, stride ldke)
    const uint8_t* k8;
    int64_t ldk8;
    const uint8_t* kex;
    int64_t ldke;
    // split key ranges (shallow grids, its own entry point): a task group with
    // more than split_t kv tiles runs as two chunks, tiles [0, nt / 2) and
    // [nt / 2, nt), on different workgroups; each chunk stores its partial
    // result in ws and the chunk that arrives second merges the two
    int split_t;
    float* ws;              // [slot][chunk][wave][DB * 4][lane][4] accumulators, then [slot][chunk][wave][lane][2]
    uint32_t* ws_cnt;       // [slot] chunks arrived; zero between calls
    int ws_slots;           // units * ntg
};

constexpr uint32_t kOob = 0x80000000u;  // a buffer offset past every pool: loads return 0
constexpr int kBtPerThread = 4;         // block-table entries per thread loaded ahead of the Q tile

// DMA of one K or V tile (keys [kbase, kbase + BK) of one sequence) into the
// LDS buffer `dst`: the buffer view starts at the tile, so keys at or past the
// sequence end read 0.  With NW waves issuing, issuing wave w fills the 1 KiB
// blocks w, w + NW, ...
template <int HD, int NW = kWaves>
__device__ __forceinline__ void dma_tile(const uint16_t* src, int64_t ld, int64_t s0, int Lb, int wave, int kbase,
                                         lds_char_t* dst, const uint32_t* off) {
    using C = Cfg<HD>;
    // the tile's base and extent are workgroup-uniform; readfirstlane keeps
    // them in scalar registers (a resource in vector registers would need a
    // per-lane loop around every DMA)
    const uint64_t base = (uint64_t)(src + (s0 + kbase) * ld);
    const uint64_t ubase = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(base >> 32)) << 32) |
                           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    const uint32_t bytes = (uint32_t)__builtin_amdgcn_readfirstlane((int)((int64_t)(Lb - kbase) * ld * 2));
    const __amdgpu_buffer_rsrc_t r = make_rsrc((const void*)ubase, bytes);
#pragma unroll
    for (int i = 0; i < (C::NBLK + NW - 1) / NW; ++i) {
        const int blk = wave + i * NW;
        if (C::NBLK % NW == 0 || blk < C::NBLK)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst + blk * 1024), 16, off[i], 0, 0, 0);
    }
}

// DMA of one fp8 K tile (keys [kbase, kbase + 64), 128 code bytes each) into
// the first 8 KiB of a K buffer: wave w fills the 1 KiB block of rows
// 8w .. 8w + 7; keys at or past the sequence end read 0.  `off` is the lane's
// byte offset (row, swizzled chunk, kv head) inside the tile.
// Wave 0 also moves the tile's scale words: lane l the 4-byte word holding
// key kbase + l's scale byte (ex_off = l * lde + the word of kv head g; the
// row stride lde is a multiple of 4, so the byte sits at bit 8 (g % 4) of
// every word), to kExpOff + 4 l.
__device__ __forceinline__ void dma_tile_k8(const uint8_t* src, int64_t ld, const uint8_t* ex, int64_t lde, int64_t s0,
                                            int Lb, int wave, int kbase, lds_char_t* dst, uint32_t off,
                                            uint32_t ex_off) {
    const uint64_t base = (uint64_t)(src + (s0 + kbase) * ld);
    const uint64_t ubase = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(base >> 32)) << 32) |
                           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    const uint32_t bytes = (uint32_t)__builtin_amdgcn_readfirstlane((int)((int64_t)(Lb - kbase) * ld));
    const __amdgpu_buffer_rsrc_t r = make_rsrc((const void*)ubase, bytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst + wave * 1024), 16, off, 0, 0, 0);
    if (wave == 0) {
        const uint64_t eb = (uint64_t)(ex + (s0 + kbase) * lde);
        const uint64_t ueb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(eb >> 32)) << 32) |
                             (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)eb);
        const uint32_t ebytes = (uint32_t)__builtin_amdgcn_readfirstlane((int)((int64_t)(Lb - kbase) * lde));
        const __amdgpu_buffer_rsrc_t re = make_rsrc((const void*)ueb, ebytes);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void_t*)(dst + kExpOff), 4, ex_off, 0, 0, 0);
    }
}

// DMA of one K or V tile from a page pool: key c = kbase + row of the tile
// comes from page bt[c / 16] (the sequence's block-table row, staged in LDS),
// slot c % 16, kv head g; keys at or past Lk read 0 through an out-of-range
// offset.  Same lane -> (row, swizzled chunk) map as dma_tile.
template <int HD>
__device__ __forceinline__ void dma_tile_paged(__amdgpu_buffer_rsrc_t r, int wave, int lane, int kbase, int Lk,
                                               int n_kv, int g, int num_pages, lds_char_t* dst,
                                               const __attribute__((address_space(3))) int32_t* lbt) {
    using C = Cfg<HD>;
#pragma unroll
    for (int i = 0; i < C::DMA_ITERS; ++i) {
        const int blk = wave + i * kWaves;
        if (C::NBLK % kWaves == 0 || blk < C::NBLK) {
            const int row = blk * C::RPI + lane / C::NC;
            const int lch = (lane % C::NC) ^ swz<HD>(row);
            const int c = kbase + row;
            uint32_t off = kOob;
            const int page = c < Lk ? lbt[c >> 4] : -1;
            if ((uint32_t)page < (uint32_t)num_pages) {   // a table entry outside the pool reads 0
                const int64_t slot = (int64_t)page * 16 + (c & 15);
                off = (uint32_t)(((slot * n_kv + g) * HD + lch * 8) * 2);
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst + blk * 1024), 16, off, 0, 0, 0);
        }
    }
}

// The pages of the lane's DMA rows of the tile at kbase (-1 past Lk), read
// from the LDS copy of the block table ahead of their dma_tile_paged_pg.
template <int HD>
__device__ __forceinline__ void paged_lookup(int wave, int lane, int kbase, int Lk,
                                             const __attribute__((address_space(3))) int32_t* lbt,
                                             int (&pg)[Cfg<HD>::DMA_ITERS]) {
    using C = Cfg<HD>;
#pragma unroll
    for (int i = 0; i < C::DMA_ITERS; ++i) {
        const int c = kbase + (wave + i * kWaves) * C::RPI + lane / C::NC;
        pg[i] = c < Lk ? lbt[c >> 4] : -1;
    }
}

// dma_tile_paged with the pages looked up beforehand (paged_lookup of the
// same tile), so no LDS read sits in front of the requests.
template <int HD>
__device__ __forceinline__ void dma_tile_paged_pg(__amdgpu_buffer_rsrc_t r, int wave, int lane, int kbase, int n_kv,
                                                  int g, int num_pages, lds_char_t* dst,
                                                  const int (&pg)[Cfg<HD>::DMA_ITERS]) {
    using C = Cfg<HD>;
#pragma unroll
    for (int i = 0; i < C::DMA_ITERS; ++i) {
        const int blk = wave + i * kWaves;
        if (C::NBLK % kWaves == 0 || blk < C::NBLK) {
            const int row = blk * C::RPI + lane / C::NC;
            const int lch = (lane % C::NC) ^ swz<HD>(row);
            const int c = kbase + row;
            uint32_t off = kOob;
            if ((uint32_t)pg[i] < (uint32_t)num_pages) {   // -1 past Lk, or a table entry outside the pool: reads 0
                const int64_t slot = (int64_t)pg[i] * 16 + (c & 15);
                off = (uint32_t)(((slot * n_kv + g) * HD + lch * 8) * 2);
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst + blk * 1024), 16, off, 0, 0, 0);
        }
    }
}

// DMA of one fp8 tile (E4M3 codes) from a page pool into the staging buffer
// `dst8`: wave w < NB8 loads block w, lane l the 16 codes of row
// w * RPI8 + l / (HD/16), column chunk l % (HD/16); it also loads that row's
// scale through the scale pool's own buffer resource `rs` (0 for keys at or
// past Lk and for block-table entries outside the pool).  Returns the scale.
template <int HD>
__device__ __forceinline__ float dma_tile_fp8(__amdgpu_buffer_rsrc_t r, __amdgpu_buffer_rsrc_t rs, int wave, int lane,
                                              int kbase, int Lk, int n_kv, int g, int num_pages, lds_char_t* dst8,
                                              const __attribute__((address_space(3))) int32_t* lbt) {
    using C = Cfg<HD>;
    float sc = 0.0f;
    if (wave < C::NB8) {
        const int row = wave * C::RPI8 + lane / (HD / 16);
        const int c = kbase + row;
        uint32_t off = kOob, soff = kOob;
        const int page = c < Lk ? lbt[c >> 4] : -1;
        if ((uint32_t)page < (uint32_t)num_pages) {
            const int64_t srow = ((int64_t)page * 16 + (c & 15)) * n_kv + g;
            off = (uint32_t)(srow * HD + (lane % (HD / 16)) * 16);
            soff = (uint32_t)(srow * 4);
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst8 + wave * 1024), 16, off, 0, 0, 0);
        sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soff, 0, 0));
    }
    return sc;
}

// The page of the lane's row of the fp8 tile at kbase (-1 past Lk or for
// waves that load no block), read ahead of its dma_tile_fp8_pg.
template <int HD>
__device__ __forceinline__ int paged_lookup8(int wave, int lane, int kbase, int Lk,
                                             const __attribute__((address_space(3))) int32_t* lbt) {
    using C = Cfg<HD>;
    const int c = kbase + wave * C::RPI8 + lane / (HD / 16);
    return wave < C::NB8 && c < Lk ? lbt[c >> 4] : -1;
}

// dma_tile_fp8 with the page looked up beforehand (paged_lookup8 of the same
// tile).  Returns the row's scale.
template <int HD>
__device__ __forceinline__ float dma_tile_fp8_pg(__amdgpu_buffer_rsrc_t r, __amdgpu_buffer_rsrc_t rs, int wave,
                                                 int lane, int kbase, int n_kv, int g, int num_pages, lds_char_t* dst8,
                                                 int page) {
    using C = Cfg<HD>;
    float sc = 0.0f;
    if (wave < C::NB8) {
        const int row = wave * C::RPI8 + lane / (HD / 16);
        const int c = kbase + row;
        uint32_t off = kOob, soff = kOob;
        if ((uint32_t)page < (uint32_t)num_pages) {
            const int64_t srow = ((int64_t)page * 16 + (c & 15)) * n_kv + g;
            off = (uint32_t)(srow * HD + (lane % (HD / 16)) * 16);
            soff = (uint32_t)(srow * 4);
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst8 + wave * 1024), 16, off, 0, 0, 0);
        sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soff, 0, 0));
    }
    return sc;
}

// After the wave's own fp8 DMA has landed (vmcnt 0): decode its 16 codes
// (OCP E4M3, exact in fp32), multiply by the row's scale, round to bf16 and
// store them as two 16-byte chunks of the bf16 tile, with the K/V swizzle.
template <int HD>
__device__ __forceinline__ void convert_fp8(int wave, int lane, const lds_char_t* src8, lds_char_t* dst, float sc) {
    using C = Cfg<HD>;
    if (wave >= C::NB8) return;
    const int row = wave * C::RPI8 + lane / (HD / 16);
    const int ch = lane % (HD / 16);
    const u32x4_t codes = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(src8 + wave * 1024 + lane * 16);
    u32x4_t out[2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[t], false);
        const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[t], true);
        out[t >> 1][(t & 1) * 2 + 0] = pack_bf16x2(a[0] * sc, a[1] * sc);
        out[t >> 1][(t & 1) * 2 + 1] = pack_bf16x2(b[0] * sc, b[1] * sc);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int lc = ch * 2 + h;
        *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(dst + row * C::ROWB + ((lc ^ swz<HD>(row)) * 16)) = out[h];
    }
}

// PAGED: 0 = K/V token-major rows of the chunk itself, 1 = bf16 page pools,
// 2 = fp8 (E4M3 + per-row scale) page pools, 3 = token-major rows with fp8
// score operands (K as E4M3 codes with power-of-two row scales, Q quantised
// here; V bf16).
template <int HD, int PAGED, bool WIN, bool SPLIT = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(Params p) {
    using C = Cfg<HD>;
    constexpr bool kPaged = PAGED == 1 || PAGED == 2;
    constexpr bool kF8S = PAGED == 3;
    static_assert(!kF8S || HD == 128, "fp8 score operands: two 64-wide head_dim slices");
    static_assert(!SPLIT || (PAGED == 0 && !WIN), "split key ranges: plain causal kernels");
    extern __shared__ __align__(16) uint16_t smem[];
    lds_char_t* lds = (lds_char_t*)smem;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool lead = wave < kWaves / 2;                       // group A: matrix phase first
    const int r32 = lane & 31, half = lane >> 5;

    // ---- batch slot -> sequence: slot b takes the b-th longest sequence (ties
    // by index), so batches run as if packed longest first, which measured up
    // to 1.2x faster than arbitrary orders of the same lengths.  Lane i ranks
    // sequence i against all others, once per workgroup (every wave alike).
    const bool ranked = p.cu != nullptr && p.num_seqs > 1 && p.num_seqs <= 64;
    auto seq_len = [&](int i) __attribute__((always_inline)) {
        const int64_t a0 = min<int64_t>(max<int64_t>(p.cu[i], 0), p.total);
        return min<int64_t>(max<int64_t>(p.cu[i + 1], a0), p.total) - a0;
    };
    int rank_i = 64;
    if (ranked && lane < p.num_seqs) {
        const int64_t li = seq_len(lane);
        rank_i = 0;
        for (int j = 0; j < p.num_seqs; ++j) {
            const int64_t lj = seq_len(j);
            rank_i += (lj > li || (lj == li && j < lane)) ? 1 : 0;
        }
    }

    // ---- persistent walk (p.persist; one workgroup per CU, a multiple of 8 of
    // them).  The non-empty virtual workgroups of the units an XCD owns (units
    // x, x + 8, ... for XCD x, heaviest first) form one compact list; the
    // workgroups of the XCD take its entries in snake order (pass m: entry
    // m * per + lp, or m * per + per - 1 - lp on odd passes).  No workgroup is
    // dispatched after the first, so none waits behind the in-order dispatch of
    // another XCD's workgroup.  tab[k] counts the non-empty virtual workgroups
    // of the XCD's units before its k-th (tab[per_xcd]: all of them); a unit's
    // non-empty ranks are its last ones.
    __attribute__((address_space(3))) int32_t* tab = (__attribute__((address_space(3))) int32_t*)(lds + p.tab_off);
    // (split: tab[0 .. 63] is the XCD's sorted entry list, tab[64] its length,
    // then the slot -> sequence table and one broadcast word)
    __attribute__((address_space(3))) int32_t* slot_to_seq = tab + (SPLIT ? 65 : p.units / kNumXcd + 1);
    [[maybe_unused]] __attribute__((address_space(3))) int32_t* bcast = tab + 129;
    const int xcd = blockIdx.x % kNumXcd, lp = blockIdx.x / kNumXcd, per = gridDim.x / kNumXcd;
    const int per_xcd = p.units / kNumXcd;
    int ncomp = 0;
    if constexpr (SPLIT) {
        // The XCD's entries: every task group of its units once, a split one
        // as its two chunks (weight = kv tiles), sorted heaviest first and
        // taken in snake order.  Lane i is task group i % ntg of the XCD's unit
        // i / ntg (the host keeps per_xcd * ntg <= 64).  Key: weight << 23 |
        // unit index << 16 | task group << 2 | chunk (0 whole, 1 first, 2 second).
        if (ranked && lane < p.num_seqs && wave == 0) slot_to_seq[rank_i] = lane;
        __syncthreads();
        if (wave == 0) {
            const int k = lane / p.ntg, t = lane % p.ntg;
            int key0 = 0, key1 = 0, cnt = 0;
            if (k < per_xcd) {
                const int slot = (k * kNumXcd + xcd) / p.n_kv;
                const int seq = ranked ? slot_to_seq[slot] : slot;
                const int64_t len = p.cu != nullptr ? seq_len(seq) : p.total;
                const int ntasks_u = (int)(p.group * ((len + BQ - 1) / BQ));
                if (t * kWaves < ntasks_u) {
                    const int last = min(t * kWaves + kWaves - 1, ntasks_u - 1);
                    const int nt = (int)((min<int64_t>(len, (int64_t)(last / p.group + 1) * BQ) + BK - 1) / BK);
                    if (nt > p.split_t) {
                        const int h = nt / 2;
                        key0 = ((nt - h) << 23) | (k << 16) | (t << 2) | 2;
                        key1 = (h << 23) | (k << 16) | (t << 2) | 1;
                        cnt = 2;
                    } else {
                        key0 = (nt << 23) | (k << 16) | (t << 2);
                        cnt = 1;
                    }
                }
            }
            int inc = cnt;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int up = __shfl_up(inc, d, 64);
                if (lane >= d) inc += up;
            }
            const int total = __shfl(inc, 63, 64);
            // (the host keeps the entries of an XCD within 64)
            if (cnt >= 1) tab[inc - cnt] = key0;
            if (cnt == 2) tab[inc - 1] = key1;
            int v = lane < total ? tab[lane] : 0;
            // bitonic sort, descending, one key per lane
#pragma unroll
            for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
                for (int stride = size / 2; stride > 0; stride >>= 1) {
                    const int o = __shfl_xor(v, stride, 64);
                    const bool keep_max = ((lane & size) == 0) == ((lane & stride) == 0);
                    v = keep_max ? max(v, o) : min(v, o);
                }
            tab[lane] = v;
            if (lane == 0) tab[64] = total;
        }
        __syncthreads();
        ncomp = __builtin_amdgcn_readfirstlane(tab[64]);
    } else if (p.persist) {
        if (ranked && lane < p.num_seqs && wave == 0) slot_to_seq[rank_i] = lane;
        __syncthreads();
        if (wave == 0) {
            int carry = 0;
            for (int k0 = 0; k0 < per_xcd; k0 += 64) {
                const int k = k0 + lane;
                int ne = 0;
                if (k < per_xcd) {
                    const int slot = (k * kNumXcd + xcd) / p.n_kv;
                    const int seq = ranked ? slot_to_seq[slot] : slot;
                    const int64_t len = p.cu != nullptr ? seq_len(seq) : p.total;
                    const int nt = (int)((p.group * ((len + BQ - 1) / BQ) + kWaves - 1) / kWaves);
                    ne = min(p.pair ? (nt + 1) / 2 : nt, p.ntg);
                }
                // inclusive scan over the wave
                int inc = ne;
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const int up = __shfl_up(inc, d, 64);
                    if (lane >= d) inc += up;
                }
                if (k < per_xcd) tab[k] = carry + inc - ne;
                carry += __shfl(inc, 63, 64);
            }
            if (lane == 0) tab[per_xcd] = carry;
        }
        __syncthreads();
        ncomp = __builtin_amdgcn_readfirstlane(tab[per_xcd]);
    }

    for (int pass = 0;; ++pass) {
    // ---- workgroup -> (unit = (sequence, kv head), task group), heaviest first
    int unit, rank;
    [[maybe_unused]] int chunk = 0;                              // split: 0 whole, 1 first, 2 second
    if constexpr (SPLIT) {
        const int c = pass * per + ((pass & 1) ? per - 1 - lp : lp);
        if (c >= ncomp) break;                                   // uniform per workgroup
        const int key = __builtin_amdgcn_readfirstlane(tab[c]);
        unit = ((key >> 16) & 127) * kNumXcd + xcd;
        rank = p.ntg - 1 - ((key >> 2) & 16383);
        chunk = key & 3;
    } else if (p.persist) {
        const int c = pass * per + ((pass & 1) ? per - 1 - lp : lp);
        if (c >= ncomp) break;                                   // uniform per workgroup
        // the unit holding entry c: the largest k with tab[k] <= c
        int lo = 0, hi = per_xcd - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tab[mid] <= c) lo = mid; else hi = mid - 1;
        }
        lo = __builtin_amdgcn_readfirstlane(lo);
        const int t0 = __builtin_amdgcn_readfirstlane(tab[lo]), t1 = __builtin_amdgcn_readfirstlane(tab[lo + 1]);
        unit = lo * kNumXcd + xcd;
        rank = p.ntg - (t1 - t0) + (c - t0);
    } else {
        if (pass > 0) break;
        const int L = blockIdx.x;
        if (p.units % kNumXcd == 0) {
            // XCD x runs units x, x + 8, x + 16, ...: with n_kv a multiple of 8 that is
            // one kv head of every sequence, so the XCDs get equal shares of work
            const int local = L / kNumXcd;
            if (p.pair) {
                // paired workgroups of one unit carry about equal work (its
                // task-group count plus one), so heaviest first is unit-major:
                // batch slot 0, the longest sequence, goes out first
                unit = (local / p.ntg) * kNumXcd + xcd;
                rank = local % p.ntg;
            } else {
                unit = (local % per_xcd) * kNumXcd + xcd;
                rank = local / per_xcd;
            }
        } else {
            unit = L % p.units;
            rank = L / p.units;
        }
    }
    const int g = unit % p.n_kv;
    int b = unit / p.n_kv;
    if (ranked) b = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(rank_i == b));
    int64_t s0 = 0, s1 = p.total;
    if (p.cu != nullptr) {
        s0 = min<int64_t>(max<int64_t>(p.cu[b], 0), p.total);
        s1 = min<int64_t>(max<int64_t>(p.cu[b + 1], s0), p.total);
    }
    // sequence bounds are workgroup-uniform: keep them in scalar registers so
    // the buffer resources built from them need no per-lane handling
    s0 = ((int64_t)__builtin_amdgcn_readfirstlane((int)(s0 >> 32)) << 32) |
         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)s0);
    const int Lb = __builtin_amdgcn_readfirstlane((int)(s1 - s0));   // query rows (the chunk)
    // keys: the chunk itself, or the cached prefix followed by the chunk; the
    // chunk's row r sits at key position pos0 + r
    int Lk = Lb;
    if constexpr (kPaged) Lk = __builtin_amdgcn_readfirstlane(min(min(max(p.ctx[b], Lb), p.mp * 16), p.bt_cap * 16));
    const int pos0 = Lk - Lb;
    const int G = p.group;
    const int nqb = (Lb + BQ - 1) / BQ;
    const int ntasks = G * nqb;
    const int ntg_b = (ntasks + kWaves - 1) / kWaves;
    // the workgroup's task groups (8 tasks = (query block, head) pairs each):
    // task group ntg - 1 - rank, or, paired, task groups ntg_b - 1 - i and i of
    // its own (sequence, kv head) with i = ntg - 1 - rank -- a heavy and a
    // light one, so every pair does about the same work and the per-workgroup
    // start-up is paid half as often; heaviest first either way
    int items[2], nitems;
    if (p.pair) {
        const int i = p.ntg - 1 - rank;
        const int hi = ntg_b - 1 - i;
        if (i > hi) continue;                                  // uniform per workgroup
        items[0] = hi;
        items[1] = i;
        nitems = i < hi ? 2 : 1;
    } else {
        items[0] = p.ntg - 1 - rank;
        if (items[0] >= ntg_b) continue;                       // uniform per workgroup
        nitems = 1;
    }

    // paged: first part of the sequence's block-table row (staged in LDS below)
    [[maybe_unused]] const int npg = (Lk + 15) >> 4;
    [[maybe_unused]] int32_t btv[kBtPerThread];
    if constexpr (kPaged) {
#pragma unroll
        for (int u = 0; u < kBtPerThread; ++u)
            btv[u] = u * kThreads + tid < npg ? p.bt[(int64_t)b * p.mp + u * kThreads + tid] : 0;
    }

    bf16x8_t qreg[C::DCH];   // the Q tile (loaded in the prologue)
    // fp8 score operands: the Q tile as codes (slice s of 64 head dims, two
    // 16-byte halves) and the row's scale byte; DMA offsets of the fp8 K tile
    // and of its scale words; LDS address of key r32's scale word
    [[maybe_unused]] u32x4_t q8[2][2];
    [[maybe_unused]] int qexp = 127;
    [[maybe_unused]] uint32_t dma_k8 = 0, dma_ex = 0, exaddr = 0;
    [[maybe_unused]] const int ex_shift = (g & 3) * 8;
    if constexpr (kF8S) {
        const int row = wave * 8 + lane / 8;
        dma_k8 = (uint32_t)(row * p.ldk8 + g * HD + (((lane & 7) ^ swz8(row)) * 16));
        dma_ex = (uint32_t)(lane * p.ldke + (g & ~3));
        exaddr = lds_addr(lds) + r32 * 4;              // + buffer + kExpOff as the immediate
    }

    // ---- DMA lane offsets: lane l writes bytes [16 l, 16 l + 16) of a 1 KiB block,
    // i.e. row l / NC, physical chunk l % NC, so it fetches the logical chunk the
    // swizzle puts there.  Plain kernels: only group B's four waves request
    // K/V tiles (a wave waits at its DMA instructions until the CU accepts
    // them, at about 64 bytes per clock; group A's waves request theirs right
    // before their matrix phase, so that wait delayed their MFMAs; group B
    // requests at the start of its softmax; +1-2.5%).  The other kernels: all
    // eight waves.
    constexpr int kDmaWaves = PAGED == 0 ? kWaves / 2 : kWaves;
    constexpr int kDmaIters = (C::NBLK + kDmaWaves - 1) / kDmaWaves;
    const int dwave = wave % kDmaWaves;                     // index among the requesting waves
    uint32_t dma_k[kDmaIters], dma_v[kDmaIters];
#pragma unroll
    for (int i = 0; i < kDmaIters; ++i) {
        const int row = (dwave + i * kDmaWaves) * C::RPI + lane / C::NC;
        const int lch = (lane % C::NC) ^ swz<HD>(row);
        dma_k[i] = (uint32_t)(((int64_t)row * p.ldk + g * HD + lch * 8) * 2);
        dma_v[i] = (uint32_t)(((int64_t)row * p.ldv + g * HD + lch * 8) * 2);
    }
    // paged: the sequence's block-table row, staged in LDS behind the K/V
    // buffers (and, for fp8 pages, behind the fp8 staging buffers)
    constexpr int kBtOff = PAGED == 2 ? C::LDS_FP8 : C::LDS_BYTES;
    const __attribute__((address_space(3))) int32_t* lbt =
        (const __attribute__((address_space(3))) int32_t*)(lds + kBtOff);
    [[maybe_unused]] __amdgpu_buffer_rsrc_t rk, rv, rks, rvs;
    if constexpr (kPaged) {
        rk = make_rsrc(p.k, p.pool_bytes);
        rv = make_rsrc(p.v, p.pool_bytes);
        if constexpr (PAGED == 2) {
            // the scale pools hold one fp32 per (slot, kv head): pool_bytes / HD * 4 bytes
            rks = make_rsrc(p.k_scale, p.pool_bytes / HD * 4);
            rvs = make_rsrc(p.v_scale, p.pool_bytes / HD * 4);
        }
        // the row was loaded into registers before the Q tile (both latencies overlap)
        __attribute__((address_space(3))) int32_t* wbt = (__attribute__((address_space(3))) int32_t*)(lds + kBtOff);
#pragma unroll
        for (int u = 0; u < kBtPerThread; ++u)
            if (u * kThreads + tid < npg) wbt[u * kThreads + tid] = btv[u];
        for (int i = kBtPerThread * kThreads + tid; i < npg; i += kThreads) wbt[i] = p.bt[(int64_t)b * p.mp + i];
        __syncthreads();
    }
    // fp8 pages: the tiles this wave loaded last and still has to convert
    // (fp8 staging buffer = bf16 buffer + the fixed distance below)
    [[maybe_unused]] float pend_ks = 0.0f, pend_vs = 0.0f;
    [[maybe_unused]] int pend_k = -1, pend_v = -1;   // bf16 buffer offsets, -1: nothing pending
    auto f8_of = [](int buf) __attribute__((always_inline)) {
        return buf == C::KBUF0 ? C::F8K0 : buf == C::KBUF1 ? C::F8K1 : buf == C::VBUF0 ? C::F8V0 : C::F8V1;
    };
    auto issue_k = [&](int tile, int buf) __attribute__((always_inline)) {
        if constexpr (kF8S) {
            dma_tile_k8(p.k8, p.ldk8, p.kex, p.ldke, s0, Lb, wave, tile * BK, lds + buf, dma_k8, dma_ex);
        } else if constexpr (PAGED == 2) {
            pend_ks = dma_tile_fp8<HD>(rk, rks, wave, lane, tile * BK, Lk, p.n_kv, g, p.num_pages, lds + f8_of(buf), lbt);
            pend_k = buf;
        } else if constexpr (PAGED == 1) {
            dma_tile_paged<HD>(rk, wave, lane, tile * BK, Lk, p.n_kv, g, p.num_pages, lds + buf, lbt);
        } else {
            if (!lead) dma_tile<HD, kDmaWaves>(p.k, p.ldk, s0, Lb, dwave, tile * BK, lds + buf, dma_k);
        }
    };
    auto issue_v = [&](int tile, int buf) __attribute__((always_inline)) {
        if constexpr (kF8S) {
            dma_tile<HD>(p.v, p.ldv, s0, Lb, wave, tile * BK, lds + buf, dma_v);
        } else if constexpr (PAGED == 2) {
            pend_vs = dma_tile_fp8<HD>(rv, rvs, wave, lane, tile * BK, Lk, p.n_kv, g, p.num_pages, lds + f8_of(buf), lbt);
            pend_v = buf;
        } else if constexpr (PAGED == 1) {
            dma_tile_paged<HD>(rv, wave, lane, tile * BK, Lk, p.n_kv, g, p.num_pages, lds + buf, lbt);
        } else {
            if (!lead) dma_tile<HD, kDmaWaves>(p.v, p.ldv, s0, Lb, dwave, tile * BK, lds + buf, dma_v);
        }
    };
    // wait for this wave's loads; for fp8 pages also convert what it loaded
    auto retire = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
        if constexpr (PAGED == 2) {
            if (pend_k >= 0) convert_fp8<HD>(wave, lane, lds + f8_of(pend_k), lds + pend_k, pend_ks);
            if (pend_v >= 0) convert_fp8<HD>(wave, lane, lds + f8_of(pend_v), lds + pend_v, pend_vs);
            pend_k = pend_v = -1;
        }
    };

    // ---- per-lane LDS read offsets
    // K operand (A of S^T): row = kb*32 + r32, logical chunk dc*2 + half
    uint32_t kaddr[C::DCH];
#pragma unroll
    for (int dc = 0; dc < C::DCH; ++dc)
        kaddr[dc] = lds_addr(lds) + r32 * C::ROWB + (((dc * 2 + half) ^ swz<HD>(r32)) * 16);
    // fp8 K operand: row kb*32 + r32, bytes [64 s + 32 half, +32) = logical
    // chunks 4 s + 2 half + c2
    [[maybe_unused]] uint32_t k8addr[2][2];
    if constexpr (kF8S) {
#pragma unroll
        for (int sl = 0; sl < 2; ++sl)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2)
                k8addr[sl][c2] = lds_addr(lds) + r32 * HD + (((4 * sl + 2 * half + c2) ^ swz8(r32)) * 16);
    }
    // V operand (A of O^T) through the transpose read: 16-lane group (u, dh), lane i = 4 kk + qq
    // reads key row 4u + 8jb + kk (+ kb*32 + h*16), d = db*32 + 16dh + 4qq .. +3.
    uint32_t vaddr[C::DB][2];
    {
        const int grp = lane >> 4, i = lane & 15;
        const int u = grp >> 1, dh = grp & 1, kk = i >> 2, qq = i & 3;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const int row = u * 4 + jb * 8 + kk;
                const int lch = (db * 32 + dh * 16 + qq * 4) / 8;
                vaddr[db][jb] = lds_addr(lds) + row * C::ROWB + ((lch ^ swz<HD>(row)) * 16) + (qq & 1) * 8;
            }
    }

    // The LDS buffers are free between items: each item ends with a barrier
    // that follows every wave's last LDS read.
    for (int it = 0; it < nitems; ++it) {
        const int tg = items[it];
        const int task = tg * kWaves + wave;
        const bool active = task < ntasks;
        const int qblk = active ? task / G : 0;
        const int head = g * G + (active ? task % G : 0);
        const int q0 = qblk * BQ;                                  // first query row (in sequence)
        const int last_task = min(tg * kWaves + kWaves - 1, ntasks - 1);
        const int kv_end = pos0 + min(Lb, (last_task / G + 1) * BQ);
        int ntiles = (kv_end + BK - 1) / BK;                       // tiles the workgroup visits
        const int wave_last_q = pos0 + min(q0 + BQ, Lb) - 1;       // key position of the wave's last query
        int wave_ntiles = active ? wave_last_q / BK + 1 : 0;       // tiles this wave computes
        // sliding window: the first tile holding a key that the wave's (the
        // workgroup's) first row sees; tiles before it are skipped
        int wave_first = 0, j0 = 0;
        if constexpr (WIN) {
            wave_first = max(0, pos0 + q0 - p.window + 1) / BK;
            j0 = __builtin_amdgcn_readfirstlane(max(0, pos0 + (tg * kWaves / G) * BQ - p.window + 1) / BK);
        }
        // split: the chunk's tiles (a wave may have none in the second chunk)
        if constexpr (SPLIT) {
            const int hsplit = ntiles / 2;
            if (chunk == 1) {
                ntiles = hsplit;
                wave_ntiles = min(wave_ntiles, hsplit);
            } else if (chunk == 2) {
                j0 = hsplit;
                wave_first = hsplit;
            }
        }

        f32x16_t oacc[C::DB];
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[db][e] = 0.0f;
        // Per row (lane): reference R in log2 units; every score chain starts from
        // the accumulator sinit = -R, so the MFMA hands over s * c - R directly.
        float R = 0.0f, l_run = 0.0f;
        f32x16_t sinit = {};
        f32x16_t s[2];          // scores of the tile whose softmax is next
        bf16x8_t pb[2][2];      // P of the tile whose P V product is next
        // zero until the wave's first softmax: the matrix phase before it (which
        // computes that tile's scores) then adds nothing to O
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int h = 0; h < 2; ++h) pb[kb][h] = as_bf16x8(u32x4_t{0u, 0u, 0u, 0u});
        bool rset = false;      // the row has a reference R (set at its first tile with a visible key)

        // Matrix phase of tile j: O^T += V^T P^T for tile j (V buffer VC), then
        // S^T = K Q^T for tile j + 1 (K buffer KN), as one sequence of NM MFMAs
        // whose LDS operands are read LA MFMAs ahead; scheduling barriers pin the
        // order, so every read has LA MFMAs (~LA * 32 cycles) to land.  P_j is
        // dead before the score accumulators come alive.  On the wave's last tile
        // the scores computed here are never used.
        // (fp8 score operands: NS = 4 MFMAs (sl, kb) of 64 head dims, two K reads
        // each; their scale bytes are the key's and the query's.)
        constexpr int LA = 4;
        constexpr int NPV = 4 * C::DB;         // (db, kb, h): V^T block x 16-key group
        constexpr int NS = kF8S ? 4 : 2 * C::DCH;   // (dc, kb): head_dim step x 32-key block
        constexpr int RS = kF8S ? 2 : 1;       // LDS reads per score MFMA
        constexpr int NM = NPV + NS;
        // scale byte of key kb * 32 + r32 from its word
        auto kexp = [&](const u32x2_t& w, int kb) __attribute__((always_inline)) {
            return (int)__builtin_amdgcn_ubfe(w[kb], (uint32_t)ex_shift, 8u);
        };
        auto matrix_phase = [&](int j, auto KNc, auto VCc) __attribute__((always_inline)) {
            if (j + 1 < wave_first || j >= wave_ntiles) return;
            constexpr int KB = decltype(KNc)::value, VB = decltype(VCc)::value;
            u32x2_t vlo[NPV], vhi[NPV];
            u32x4_t kf[NS * RS];
            // fp8: the two scale words of the next tile's keys go out first (older
            // than every operand read, so retired before the first score MFMA's)
            [[maybe_unused]] u32x2_t kw;
            if constexpr (kF8S) {
                kw[0] = lds_read_b32<KB + kExpOff>(exaddr);
                kw[1] = lds_read_b32<KB + kExpOff + 128>(exaddr);
            }
            auto issue = [&](auto Ic) __attribute__((always_inline)) {
                constexpr int i = decltype(Ic)::value;
                if constexpr (i < NPV) {
                    constexpr int db = i / 4, f = i % 4;
                    constexpr int off = VB + f * 16 * C::ROWB;      // key group f = (kb, h)
                    vlo[i] = lds_read_tr16<off>(vaddr[db][0]);      // key rows 0-3 of the group
                    vhi[i] = lds_read_tr16<off>(vaddr[db][1]);      // key rows 8-11
                } else if constexpr (kF8S) {
                    constexpr int m = i - NPV, sl = m / 2, kb = m % 2;
                    kf[2 * m] = lds_read_b128<KB + kb * 32 * HD>(k8addr[sl][0]);
                    kf[2 * m + 1] = lds_read_b128<KB + kb * 32 * HD>(k8addr[sl][1]);
                } else {
                    constexpr int m = i - NPV, dc = m / 2, kb = m % 2;
                    kf[m] = lds_read_b128<KB + kb * 32 * C::ROWB>(kaddr[dc]);
                }
            };
            __builtin_amdgcn_s_setprio(1);
            static_for<LA>([&](auto Ic) { issue(Ic); });
            static_for<NM>([&](auto Ic) {
                constexpr int i = decltype(Ic)::value;
                constexpr int n = reads_after<NPV, NM, LA, RS>(i);
                if constexpr (i < NPV) {
                    constexpr int db = i / 4, kb = (i % 4) / 2, h = i % 2;
                    lds_wait<n>(vlo[i], vhi[i]);
                    const u32x4_t w = {vlo[i][0], vlo[i][1], vhi[i][0], vhi[i][1]};
                    oacc[db] = mfma32x32x16(as_bf16x8(w), pb[kb][h], oacc[db]);
                } else if constexpr (kF8S) {
                    constexpr int m = i - NPV, sl = m / 2, kb = m % 2;
                    if constexpr (m == 0) lds_wait<n>(kf[0], kf[1], kw);
                    else lds_wait<n>(kf[2 * m], kf[2 * m + 1]);
                    s[kb] = mfma_f8s(kf[2 * m], kf[2 * m + 1], q8[sl][0], q8[sl][1], sl == 0 ? sinit : s[kb],
                                     kexp(kw, kb), qexp);
                } else {
                    constexpr int m = i - NPV, dc = m / 2, kb = m % 2;
                    lds_wait<n>(kf[m]);
                    // the first head_dim step starts from a zero accumulator
                    s[kb] = mfma32x32x16(as_bf16x8(kf[m]), qreg[dc], dc == 0 ? sinit : s[kb]);
                }
                if constexpr (i + LA < NM) issue(std::integral_constant<int, i + LA>{});
                __builtin_amdgcn_sched_barrier(0);
            });
            __builtin_amdgcn_s_setprio(0);
        };

        // S^T = K Q^T for the tile in K buffer KB (prologue only)
        // (all operand reads issued first, each MFMA waiting only for its own)
        auto scores = [&](auto KBc) __attribute__((always_inline)) {
            constexpr int KB = decltype(KBc)::value;
            if constexpr (kF8S) {
                u32x4_t kp[2 * NS];
                u32x2_t kw;
                kw[0] = lds_read_b32<KB + kExpOff>(exaddr);
                kw[1] = lds_read_b32<KB + kExpOff + 128>(exaddr);
                static_for<NS>([&](auto Mc) {
                    constexpr int m = decltype(Mc)::value, sl = m / 2, kb = m % 2;
                    kp[2 * m] = lds_read_b128<KB + kb * 32 * HD>(k8addr[sl][0]);
                    kp[2 * m + 1] = lds_read_b128<KB + kb * 32 * HD>(k8addr[sl][1]);
                });
                static_for<NS>([&](auto Mc) {
                    constexpr int m = decltype(Mc)::value, sl = m / 2, kb = m % 2;
                    if constexpr (m == 0) lds_wait<2 * (NS - 1 - m)>(kp[0], kp[1], kw);
                    else lds_wait<2 * (NS - 1 - m)>(kp[2 * m], kp[2 * m + 1]);
                    s[kb] = mfma_f8s(kp[2 * m], kp[2 * m + 1], q8[sl][0], q8[sl][1], sl == 0 ? sinit : s[kb],
                                     kexp(kw, kb), qexp);
                });
            } else {
                u32x4_t kp[NS];
                static_for<NS>([&](auto Mc) {
                    constexpr int m = decltype(Mc)::value, dc = m / 2, kb = m % 2;
                    kp[m] = lds_read_b128<KB + kb * 32 * C::ROWB>(kaddr[dc]);
                });
                static_for<NS>([&](auto Mc) {
                    constexpr int m = decltype(Mc)::value, dc = m / 2, kb = m % 2;
                    lds_wait<NS - 1 - m>(kp[m]);
                    s[kb] = mfma32x32x16(as_bf16x8(kp[m]), qreg[dc], dc == 0 ? sinit : s[kb]);
                });
            }
        };

        // Softmax phase of tile t (scores in s): P_t into pb, m and l updated.
        auto softmax_phase = [&](int t) __attribute__((always_inline)) {
            if (t < wave_first || t >= wave_ntiles) return;
            const int kbase = t * BK;
            // causal mask per element on tiles that reach past the first query;
            // window mask on tiles that start before the last query's window
            const bool upper = kbase + BK - 1 > pos0 + q0;
            const bool lower = WIN && kbase <= pos0 + q0 + BQ - 1 - p.window;
            if (upper || lower) {
                const int qry = pos0 + q0 + r32;
                // visible iff 0 <= qry - key < wlim: one unsigned compare per score
                const uint32_t wlim = WIN ? (uint32_t)p.window : 0x7FFFFFFFu;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int key = kbase + kb * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
                        if ((uint32_t)(qry - key) >= wlim) s[kb][e] = -__builtin_inff();
                    }
            }
            // Online softmax, one query per lane (its 64 keys split with lane ^ 32).
            // The scores already hold s * c - R, so the common case is one exp2 and
            // one add per score (p in fp32 for the row sum, rounded to bf16 for
            // the MFMA).  A row moves its reference R up to its tile max on the
            // wave's first tile and when its tile sum of p exceeds kSumLimit; the
            // fast path stays only while every lane's half-row sum is at most
            // kSumLimit / 2, which bounds every p by kSumLimit.  The result does
            // not depend on R (it cancels in O / l), and a row's arithmetic depends
            // on its own scores alone.
            float rs;
            auto exps = [&](float d) __attribute__((always_inline)) {
                rs = 0.0f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        u32x4_t w;
#pragma unroll
                        for (int t2 = 0; t2 < 4; ++t2) {
                            const float e0 = fast_exp2(s[kb][h * 8 + 2 * t2] - d);
                            const float e1 = fast_exp2(s[kb][h * 8 + 2 * t2 + 1] - d);
                            w[t2] = pack_bf16x2(e0, e1);
                            rs += e0;
                            rs += e1;
                        }
                        pb[kb][h] = as_bf16x8(w);
                    }
            };
            exps(0.0f);
            if (__builtin_amdgcn_ballot_w64(!rset || rs > 0.5f * kSumLimit) != 0) {
                float rlo, rhi;
                both_halves(rs, rlo, rhi);
                const bool move = !rset || rlo + rhi > kSumLimit;
                // rare: moving rows take their tile max as the new reference,
                // recompute p and rescale O and l (non-moving rows: d = 0, alpha = 1,
                // the same p as above)
                float mx = s[0][0];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) mx = __builtin_fmaxf(mx, s[kb][e]);
                float lo, hi;
                both_halves(mx, lo, hi);
                const float mrow = __builtin_fmaxf(lo, hi);
                // a row with no visible key in this tile (window) keeps no reference
                const bool ok = move && mrow > -__builtin_inff();
                const float d = ok ? mrow : 0.0f;
                rset = rset || ok;
                exps(d);
                // d > 0 for a row past the limit; on the first tile O and l are 0
                const float alpha = __builtin_fminf(fast_exp2(-d), 1.0f);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
                R += d;
#pragma unroll
                for (int e = 0; e < 16; ++e) sinit[e] = -R;
            }
            l_run += rs;
        };

        // The two groups run the same sequence of phases -- softmax of tile j,
        // then the matrix phase of tile j -- with group B one half-step behind
        // group A, so that in every half-step one wave of each SIMD is in its
        // matrix phase and the other in its softmax.  Half-steps end at workgroup
        // barriers; B starts with one extra barrier and A ends with one.
        //
        // DMA: in half-step 2m + 1 (A's matrix phase of tile m, B's softmax of
        // tile m) the requesting waves (group B for plain kernels, every wave
        // otherwise) issue their shares of K_{m+2} (into K_m's buffer) and
        // V_{m+1} (into V_{m-1}'s); both were last read in half-step 2m.  They are
        // waited for at the end of half-step 2m + 2 and first read in 2m + 3.
        // KC/KN: K buffers of tiles j and j + 1; VC/VN: V buffers of j and j + 1.
        // Paged: the pages of the tiles requested here were looked up one tile
        // earlier (kpg: K_{j+2}, vpg: V_{j+1}); then V_{j+2} takes K_{j+2}'s
        // pages and K_{j+3}'s are read, so no block-table read sits in front of
        // the requests (bf16 pages: it cost ~7% of the chunk attention)
        [[maybe_unused]] int kpg[C::DMA_ITERS], vpg[C::DMA_ITERS];
        [[maybe_unused]] int kpg8 = -1, vpg8 = -1;               // the same for fp8 pages
        auto issue_next = [&](int j, auto KCc, auto VNc) __attribute__((always_inline)) {
            if constexpr (PAGED == 2) {
                if (j + 2 < ntiles) {
                    pend_ks = dma_tile_fp8_pg<HD>(rk, rks, wave, lane, (j + 2) * BK, p.n_kv, g, p.num_pages,
                                                  lds + f8_of(decltype(KCc)::value), kpg8);
                    pend_k = decltype(KCc)::value;
                }
                if (j + 1 < ntiles) {
                    pend_vs = dma_tile_fp8_pg<HD>(rv, rvs, wave, lane, (j + 1) * BK, p.n_kv, g, p.num_pages,
                                                  lds + f8_of(decltype(VNc)::value), vpg8);
                    pend_v = decltype(VNc)::value;
                }
                vpg8 = kpg8;
                kpg8 = paged_lookup8<HD>(wave, lane, (j + 3) * BK, Lk, lbt);
            } else if constexpr (PAGED == 1) {
                if (j + 2 < ntiles)
                    dma_tile_paged_pg<HD>(rk, wave, lane, (j + 2) * BK, p.n_kv, g, p.num_pages,
                                          lds + decltype(KCc)::value, kpg);
                if (j + 1 < ntiles)
                    dma_tile_paged_pg<HD>(rv, wave, lane, (j + 1) * BK, p.n_kv, g, p.num_pages,
                                          lds + decltype(VNc)::value, vpg);
#pragma unroll
                for (int i = 0; i < C::DMA_ITERS; ++i) vpg[i] = kpg[i];
                paged_lookup<HD>(wave, lane, (j + 3) * BK, Lk, lbt, kpg);
            } else {
                if (j + 2 < ntiles) issue_k(j + 2, decltype(KCc)::value);
                if (j + 1 < ntiles) issue_v(j + 1, decltype(VNc)::value);
            }
        };
        auto tile = [&](int j, auto KCc, auto KNc, auto VCc, auto VNc) __attribute__((always_inline)) {
            if (!lead) issue_next(j, KCc, VNc);
            softmax_phase(j);
            if (lead) retire();
            wg_barrier();
            if (lead) issue_next(j, KCc, VNc);
            matrix_phase(j, KNc, VCc);
            if (!lead) retire();
            wg_barrier();
        };

        using K0 = std::integral_constant<int, C::KBUF0>;
        using K1 = std::integral_constant<int, C::KBUF1>;
        using V0 = std::integral_constant<int, C::VBUF0>;
        using V1 = std::integral_constant<int, C::VBUF1>;

        // prologue: K and V of the first tile j0 (0 unless a window skips the
        // start) and K of the next in flight, then every wave whose first tile it
        // is computes its scores; group B waits one half-step
        issue_k(j0, C::KBUF0);
        issue_v(j0, C::VBUF0);
        if constexpr (PAGED == 2) retire();   // fp8: K_j0 and V_j0 converted before K_j0+1 takes the pending slot
        if (j0 + 1 < ntiles) issue_k(j0 + 1, C::KBUF1);
        if constexpr (PAGED == 1) {
            paged_lookup<HD>(wave, lane, (j0 + 1) * BK, Lk, lbt, vpg);
            paged_lookup<HD>(wave, lane, (j0 + 2) * BK, Lk, lbt, kpg);
        } else if constexpr (PAGED == 2) {
            vpg8 = paged_lookup8<HD>(wave, lane, (j0 + 1) * BK, Lk, lbt);
            kpg8 = paged_lookup8<HD>(wave, lane, (j0 + 2) * BK, Lk, lbt);
        }

        // ---- Q tile in registers (its loads overlap the first tiles' DMA): B
        // operand of S^T = K Q^T (column = query r32)
        if constexpr (kF8S) {
            // lane (r32, half) holds head dims 64 s + 32 half .. +31 of its query:
            // y = q * c in binary32, the row's power-of-two scale from its amax
            // (the two halves exchange their maxima), codes of y * 2^-e
            const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + s0 * p.ldq, (uint32_t)((int64_t)Lb * p.ldq * 2));
            float y[2][32];
            float m = 0.0f;
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                    const uint32_t off =
                        (uint32_t)(((int64_t)(q0 + r32) * p.ldq + head * HD + sl * 64 + half * 32 + c4 * 8) * 2);
                    const u32x4_t raw = buf_load16(rq, off);
#pragma unroll
                    for (int t2 = 0; t2 < 4; ++t2) {
                        y[sl][c4 * 8 + 2 * t2] = bf16_lo(raw[t2]) * p.c;
                        y[sl][c4 * 8 + 2 * t2 + 1] = bf16_hi(raw[t2]) * p.c;
                        m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fabsf(y[sl][c4 * 8 + 2 * t2]),
                                                               __builtin_fabsf(y[sl][c4 * 8 + 2 * t2 + 1])));
                    }
                }
            float mlo, mhi;
            both_halves(m, mlo, mhi);
            const int e = pow2_exponent(__builtin_bit_cast(uint32_t, __builtin_fmaxf(mlo, mhi)));
            qexp = e + 127;
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const float* yy = &y[sl][c2 * 16 + w * 4];
                        q8[sl][c2][w] = e4m3x4(__builtin_ldexpf(yy[0], -e), __builtin_ldexpf(yy[1], -e),
                                               __builtin_ldexpf(yy[2], -e), __builtin_ldexpf(yy[3], -e));
                    }
        } else {
            const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + s0 * p.ldq, (uint32_t)((int64_t)Lb * p.ldq * 2));
#pragma unroll
            for (int dc = 0; dc < C::DCH; ++dc) {
                const uint32_t off = (uint32_t)(((int64_t)(q0 + r32) * p.ldq + head * HD + dc * 16 + half * 8) * 2);
                // scale * log2(e) folded into Q once (then rounded to bf16), so the
                // scores come out of the MFMA in log2 units
                const u32x4_t raw = buf_load16(rq, off);
                u32x4_t qs;
#pragma unroll
                for (int t2 = 0; t2 < 4; ++t2) qs[t2] = pack_bf16x2(bf16_lo(raw[t2]) * p.c, bf16_hi(raw[t2]) * p.c);
                qreg[dc] = as_bf16x8(qs);
            }
        }

        retire();
        __syncthreads();
        // group A's first scores go first (raised priority), so that group B's
        // run on the matrix cores while A does the first softmax
        if (lead) __builtin_amdgcn_s_setprio(1);
        if (wave_first == j0 && j0 < wave_ntiles) scores(K0{});
        if (lead) __builtin_amdgcn_s_setprio(0);
        if (!lead) wg_barrier();
        // two tiles per trip so every buffer offset is a compile-time constant
        for (int j = j0; j < ntiles; j += 2) {
            tile(j, K0{}, K1{}, V0{}, V1{});
            if (j + 1 >= ntiles) break;
            tile(j + 1, K1{}, K0{}, V1{}, V0{});
        }
        if (lead) wg_barrier();

        // ---- split chunk: the chunk stores its partial -- accumulators
        // relative to its reference R, R, and the lane's half-row sum -- and
        // counts its arrival.  The chunk that arrives second merges the two in
        // chunk order (so the result does not depend on which came first) and
        // goes on to the epilogue; the first skips the epilogue's stores.  A
        // row with no visible key in a chunk (sum 0) takes no weight from it.
        [[maybe_unused]] bool write_o = true;
        if constexpr (SPLIT) {
            if (chunk != 0) {
                // The partials go past the caches (sc0 sc1: written through to
                // memory, read from it), so the count needs only this wave's
                // stores to have completed, not a cache write-back: a fence
                // at device scope wrote back each XCD's whole L2 and cost more
                // than the split saved.
                constexpr int kCoherent = 1 | 16;
                const int slot = unit * p.ntg + tg;
                constexpr uint32_t kAccW = (uint32_t)C::DB * 4 * 64 * 4;    // floats per wave
                const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.ws, (uint32_t)p.ws_slots * 2u * kWaves * (kAccW + 128u) * 4u);
                auto acc_off = [&](int ci) __attribute__((always_inline)) {
                    return ((((uint32_t)slot * 2u + ci) * kWaves + wave) * kAccW + (uint32_t)lane * 4u) * 4u;
                };
                auto rl_off = [&](int ci) __attribute__((always_inline)) {
                    return ((uint32_t)p.ws_slots * 2u * kWaves * kAccW + (((uint32_t)slot * 2u + ci) * kWaves + wave) * 128u +
                            (uint32_t)lane * 2u) * 4u;
                };
                const uint32_t mine = acc_off(chunk - 1);
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        // (whole vectors are bit-cast: a bit-cast of one vector
                        // element read element 0)
                        const u32x4_t w4 = __builtin_bit_cast(
                            u32x4_t, f32x4_t{oacc[db][q4 * 4], oacc[db][q4 * 4 + 1], oacc[db][q4 * 4 + 2], oacc[db][q4 * 4 + 3]});
                        __builtin_amdgcn_raw_buffer_store_b128(w4, wr, mine + (uint32_t)((db * 4 + q4) * 64 * 16), 0, kCoherent);
                    }
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, f32x2_t{R, l_run}),
                                                      wr, rl_off(chunk - 1), 0, kCoherent);
                __builtin_amdgcn_s_waitcnt(kVmcnt0);   // this wave's partial is in memory
                __syncthreads();
                if (tid == 0) bcast[0] = (int)atomicAdd(&p.ws_cnt[slot], 1u);
                __syncthreads();
                write_o = __builtin_amdgcn_readfirstlane(bcast[0]) != 0;
                if (write_o) {
                    const uint32_t theirs = acc_off(2 - chunk);
                    const u32x2_t orl = __builtin_amdgcn_raw_buffer_load_b64(wr, rl_off(2 - chunk), 0, kCoherent);
                    // chunk 1's values first, then chunk 2's
                    const f32x2_t orf = __builtin_bit_cast(f32x2_t, orl);
                    const float oR = orf[0], oh = orf[1];
                    const float R1 = chunk == 1 ? R : oR, R2 = chunk == 1 ? oR : R;
                    const float h1 = chunk == 1 ? l_run : oh, h2 = chunk == 1 ? oh : l_run;
                    float a1, b1, a2, b2;
                    both_halves(h1, a1, b1);
                    both_halves(h2, a2, b2);
                    const bool v1 = a1 + b1 > 0.0f, v2 = a2 + b2 > 0.0f;
                    const float Rm = v1 && v2 ? __builtin_fmaxf(R1, R2) : (v1 ? R1 : R2);
                    const float w1 = v1 ? fast_exp2(R1 - Rm) : 0.0f, w2 = v2 ? fast_exp2(R2 - Rm) : 0.0f;
                    l_run = h1 * w1 + h2 * w2;
#pragma unroll
                    for (int db = 0; db < C::DB; ++db)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const u32x4_t ov = __builtin_amdgcn_raw_buffer_load_b128(wr, theirs + (uint32_t)((db * 4 + q4) * 64 * 16), 0, kCoherent);
                            const f32x4_t ovf = __builtin_bit_cast(f32x4_t, ov);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float m = oacc[db][q4 * 4 + e], o = ovf[e];
                                const float o1 = chunk == 1 ? m : o, o2 = chunk == 1 ? o : m;
                                oacc[db][q4 * 4 + e] = o1 * w1 + o2 * w2;
                            }
                        }
                    // both chunks have arrived: ready for the next call
                    if (tid == 0) __hip_atomic_store(&p.ws_cnt[slot], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }

        // ---- epilogue: O / l, bf16 RNE.  Each wave stages its 32 rows in its
        // eighth of the (now free) K/V buffers, 16-byte chunks XOR-swizzled by
        // row, and writes them back as whole head rows, 16 bytes per lane,
        // non-temporal (O is not read again here, and its lines then do not
        // push the shared K/V tiles out of L2).  No early return: every wave
        // runs every item's barriers.
        {
            lds_char_t* stg = lds + wave * (BQ * C::ROWB);
            // the lane's swizzle and row terms pass through an empty asm here, so
            // the addresses built from them are formed in the epilogue instead of
            // being hoisted out of the item loop and held in registers throughout
            int sw = r32 & (C::NC - 1), rl = lane / C::NC;
            asm volatile("" : "+v"(sw), "+v"(rl));
            if (active && write_o) {
                float l_lo, l_hi;
                both_halves(l_run, l_lo, l_hi);
                const float inv = 1.0f / (l_lo + l_hi);
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int pc = (db * 4 + gq) ^ sw;
                        const u32x2_t w2 = {pack_bf16x2(oacc[db][gq * 4 + 0] * inv, oacc[db][gq * 4 + 1] * inv),
                                            pack_bf16x2(oacc[db][gq * 4 + 2] * inv, oacc[db][gq * 4 + 3] * inv)};
                        *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>(stg + r32 * C::ROWB + pc * 16 + half * 8) = w2;
                    }
                constexpr int RPI = 64 / C::NC;          // rows per store instruction
                const int c = lane % C::NC;
#pragma unroll
                for (int k = 0; k < BQ / RPI; ++k) {
                    const int rr = k * RPI + rl;
                    const u32x4_t v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
                        stg + rr * C::ROWB + ((c ^ (rr & (C::NC - 1))) * 16));
                    const int row = q0 + rr;
                    if (row < Lb) __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p.o + (s0 + row) * p.ldo + head * HD + c * 8));
                }
            }
            // the staging areas are the next item's first K/V buffers
            wg_barrier();
        }
    }
    }   // pass
}

// largest dynamic LDS a workgroup may take (gfx950: 160 KiB per CU)
constexpr int kMaxLds = 160 * 1024;
// persistent walk: at most this many units per XCD (their counts live in LDS)
constexpr int kMaxPersistUnits = 4096;

// unpaired grids at least this large (4 workgroups per CU) use pairing
constexpr int64_t kPairMinWorkgroups = 1024;

template <int HD, int PAGED, bool WIN>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t s) {
    using C = Cfg<HD>;
    static const hipError_t attr = hipFuncSetAttribute((const void*)attn_fwd_kernel<HD, PAGED, WIN>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    if (attr != hipSuccess) return attr;
    Params p;
    p.q = a.q; p.k = a.k; p.v = a.v;
    p.ldq = a.ldq; p.ldk = a.ldk; p.ldv = a.ldv;
    p.cu = a.cu_seqlens;
    p.num_seqs = a.num_seqs;
    p.total = a.total_tokens;
    p.n_kv = a.n_kv_head;
    p.group = a.n_head / a.n_kv_head;
    p.c = a.scale * 1.4426950408889634f;
    p.o = a.o;
    p.ldo = a.ldo;
    const int nqb = (a.max_seqlen + BQ - 1) / BQ;
    const int ntg = (p.group * nqb + kWaves - 1) / kWaves;
    p.units = a.num_seqs * a.n_kv_head;
    // pair task groups only when the grid stays several workgroups per CU deep
    p.pair = (int64_t)ntg * p.units >= kPairMinWorkgroups ? 1 : 0;
    p.ntg = p.pair ? (ntg + 1) / 2 : ntg;
    p.bt = a.block_table;
    p.mp = a.max_pages_per_seq;
    p.ctx = a.ctx_lens;
    p.window = a.window;
    p.k_scale = a.k_scale;
    p.v_scale = a.v_scale;
    p.pool_bytes = (uint32_t)a.pool_bytes;
    p.num_pages = (int)a.num_pages;
    p.k8 = a.k8;
    p.ldk8 = a.ldk8;
    p.kex = a.kex;
    p.ldke = a.ldke;
    size_t lds = PAGED == 2 ? C::LDS_FP8 : C::LDS_BYTES;
    p.bt_cap = ((a.max_ctx + 15) / 16 + 3) / 4 * 4;
    if (PAGED == 1 || PAGED == 2) lds += (size_t)p.bt_cap * 4;   // the block-table row, int32
    if (lds > (size_t)kMaxLds) return hipErrorInvalidValue;
    int64_t grid = (int64_t)p.ntg * p.units;
    // deeper than one workgroup per CU, with the units spread evenly over the
    // XCDs: one workgroup per CU walks its XCD's list (the kernel's persistent walk)
    p.persist = 0;
    p.tab_off = 0;
    const int ncu = device_cus();
    const int nwg = ncu >= kNumXcd ? (ncu / kNumXcd) * kNumXcd : 0;
    const size_t lds_persist = ((lds + 15) & ~(size_t)15) + (size_t)(p.units / kNumXcd + 1 + 64) * 4;
    if (nwg > 0 && p.units % kNumXcd == 0 && grid > nwg && p.units / kNumXcd <= kMaxPersistUnits &&
        lds_persist <= (size_t)kMaxLds) {
        p.persist = 1;
        p.tab_off = (int)((lds + 15) & ~(size_t)15);
        lds = lds_persist;
        grid = nwg;
    }
    hipLaunchKernelGGL((attn_fwd_kernel<HD, PAGED, WIN>), dim3((uint32_t)grid), dim3(kThreads), lds, s, p);
    return hipGetLastError();
}

// Split key ranges (shallow grids): at most one task group per workgroup
// slot, the units spread evenly over the XCDs, at least 8 kv tiles.  Task
// groups with more than three quarters of the longest sequence's kv tiles
// run as two chunks.  Every item costs a fixed ~10 us here (first tiles in
// flight, pipeline fill and drain, epilogue) on top of its tiles, so only
// the heaviest task groups pay for being split: a quarter or a half split
// more of them and ran slower than no split.  Otherwise, and for deeper
// grids, the plain kernel runs.
static_assert(BQ == 32 && kWaves == 8, "the split workspace layout of pca_internal.hpp");

template <int HD>
hipError_t launch_split(const AttnArgs& a, hipStream_t s) {
    using C = Cfg<HD>;
    const int G = a.n_head / a.n_kv_head;
    const int ntg = (G * ((a.max_seqlen + BQ - 1) / BQ) + kWaves - 1) / kWaves;
    const int64_t units = (int64_t)a.num_seqs * a.n_kv_head;
    const int ncu = device_cus();
    const int nwg = ncu >= kNumXcd ? (ncu / kNumXcd) * kNumXcd : 0;
    const int max_nt = (a.max_seqlen + BK - 1) / BK;
    const bool use = nwg > 0 && units % kNumXcd == 0 && units * ntg <= nwg && units * ntg <= kSplitMaxSlots &&
                     (units / kNumXcd) * ntg <= 32 && max_nt >= 8;
    if (!use) return launch_cfg<HD, 0, false>(a, s);
    static const hipError_t attr = hipFuncSetAttribute((const void*)attn_fwd_kernel<HD, 0, false, true>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    if (attr != hipSuccess) return attr;
    Params p;
    memset(&p, 0, sizeof(p));
    p.q = a.q; p.k = a.k; p.v = a.v;
    p.ldq = a.ldq; p.ldk = a.ldk; p.ldv = a.ldv;
    p.cu = a.cu_seqlens;
    p.num_seqs = a.num_seqs;
    p.total = a.total_tokens;
    p.n_kv = a.n_kv_head;
    p.group = G;
    p.c = a.scale * 1.4426950408889634f;
    p.o = a.o;
    p.ldo = a.ldo;
    p.units = (int)units;
    p.pair = 0;
    p.ntg = ntg;
    p.split_t = max(4, max_nt * 3 / 4);
    p.ws_cnt = (uint32_t*)a.split_ws;
    p.ws = (float*)((char*)a.split_ws + kSplitCounterBytes);
    p.ws_slots = (int)(units * ntg);
    p.persist = 1;
    p.tab_off = (C::LDS_BYTES + 15) & ~15;
    const size_t lds = (size_t)p.tab_off + 130 * 4;     // entry list, its length, slot -> sequence, broadcast
    hipLaunchKernelGGL((attn_fwd_kernel<HD, 0, false, true>), dim3((uint32_t)nwg), dim3(kThreads), lds, s, p);
    return hipGetLastError();
}

template <int PAGED, bool WIN>
hipError_t launch_hd(const AttnArgs& a, hipStream_t s) {
    switch (a.head_dim) {
        case 32: return launch_cfg<32, PAGED, WIN>(a, s);
        case 64: return launch_cfg<64, PAGED, WIN>(a, s);
        case 128: return launch_cfg<128, PAGED, WIN>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
    if (a.split_ws != nullptr && a.k8 == nullptr && a.block_table == nullptr && a.window == 0) {
        switch (a.head_dim) {
            case 32: return launch_split<32>(a, s);
            case 64: return launch_split<64>(a, s);
            case 128: return launch_split<128>(a, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (a.k8 != nullptr) return a.head_dim == 128 ? launch_cfg<128, 3, false>(a, s) : hipErrorInvalidValue;
    if (a.block_table != nullptr) {
        if (a.window > 0) return a.k_scale != nullptr ? launch_hd<2, true>(a, s) : launch_hd<1, true>(a, s);
        return a.k_scale != nullptr ? launch_hd<2, false>(a, s) : launch_hd<1, false>(a, s);
    }
    return a.window > 0 ? launch_hd<0, true>(a, s) : launch_hd<0, false>(a, s);
}

}  // namespace pca
