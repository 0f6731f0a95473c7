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
//  * A wave owns 32 query rows of one head; a workgroup is 4 waves (one per
//    SIMD) that share one kv head and therefore the kv tiles in LDS: for
//    G >= 4 the 4 waves are 4 query heads at the same positions, for smaller
//    G consecutive query blocks.  Two workgroups per CU (2 waves per SIMD).
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the 32x32 accumulator then holds, in each
//    lane, 16 keys of ONE query (the lane's column).  Row max and row sum are
//    lane-local plus one exchange with lane ^ 32, and the accumulator is
//    already the B operand of the second product O^T = V^T P^T once
//    converted to bf16 -- no cross-lane shuffle of P.
//  * Software pipeline inside a wave: while the softmax of kv tile j runs on
//    the VALU, the scores of tile j + 1 are already on the matrix cores, so a
//    wave keeps its MFMA pipe busy through its own softmax; the other wave on
//    the SIMD fills the VALU while this one runs P V.  K therefore runs one
//    tile ahead of V: K and V have separate double buffers, and iteration j
//    reads K_{j+1} and V_j while K_{j+2} and V_{j+1} arrive.
//  * K and V tiles (64 keys) go from HBM/L2 straight into LDS with
//    buffer_load ... lds (no register staging).  Rows are stored key-major
//    with the 16-byte chunks of each row XOR-swizzled by the row index, so
//    that the K operand reads (ds_read_b128, 16 rows per 16 lanes) and the V
//    operand reads hit all 64 banks once.  V^T comes out of LDS with the
//    gfx950 transpose read ds_read_b64_tr_b16: each 16-lane group returns,
//    for 16 consecutive d, 4 keys per lane -- the A-operand layout of
//    O^T = V^T P^T, in the same key order the S^T accumulator hands to the B
//    operand (within 16 keys: 0-3, 8-11 | 4-7, 12-15).
//  * Q stays in registers (B operand of S^T) for the whole kv loop; the O^T
//    accumulator (fp32) likewise.
//  * exp is exp2 with scale*log2(e) folded into one FMA; m, l, P in fp32,
//    P rounded to bf16 only as the MFMA operand.  The reference max of a row
//    moves only when the row's scores exceed it by 2^8 (see below); the new
//    reference is a per-lane select, so the exponentials need no branch, and
//    only the rescale of O and l sits behind one -- taken on the first tile
//    and rarely after.  The common path is one straight block the scheduler
//    can interleave with the matrix-core work.
//  * The causal rule: a wave skips kv tiles that start after its last query,
//    and masks per element only on tiles that reach past its first query.
//    Workgroups are ordered heaviest-first and all workgroups of one
//    (sequence, kv head) are placed on one XCD (ids go round-robin over the
//    8 XCDs), so its K/V stays in that XCD's L2.
#include "pca_device.hpp"
#include "pca_internal.hpp"

#include <utility>

namespace pca {

namespace {

typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int BQ = 32;                  // query rows per wave
constexpr int BK = 64;                  // keys per kv tile
constexpr float kRescaleLog2 = 8.0f;    // lazy max update threshold (p stays <= 256)
constexpr int kVmcnt0 = 0x0F70;         // s_waitcnt vmcnt(0), other counters unconstrained

template <int HD>
struct Cfg {
    static constexpr int NC = HD / 8;                    // 16-byte chunks per key row
    static constexpr int ROWB = HD * 2;                  // bytes per key row
    static constexpr int TILE = BK * ROWB;               // bytes of one K (or V) tile
    static constexpr int KBUF0 = 0, KBUF1 = TILE;        // K double buffer
    static constexpr int VBUF0 = 2 * TILE, VBUF1 = 3 * TILE;   // V double buffer
    static constexpr int LDS_BYTES = 4 * TILE;
    static constexpr int RPI = 1024 / ROWB;              // rows per 1 KiB wave DMA instruction
    static constexpr int DMA_PER_WAVE = TILE / 1024 / kWaves;
    static constexpr int DCH = HD / 16;                  // k16 steps over head_dim
    static constexpr int DB = HD / 32;                   // 32-row blocks of O^T
    static_assert(DMA_PER_WAVE >= 1, "tile too small for the DMA split");
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

// ds_read_b64_tr_b16 as inline asm.  Issued through the builtin, the read
// carries no alias information, and the compiler then waits for every
// outstanding global->LDS DMA (the next kv tiles, which target the other
// buffers) before it; as asm its completion is tracked by lds_wait_block.
template <int OFF>
__device__ __forceinline__ u32x2_t lds_read_tr16(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "DS offset field is 16 bits");
    u32x2_t r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
    return r;
}

// The 8 V^T fragments of O^T block DB from the V buffer at byte offset VBUF:
// for each 16-key group f = (kb, h), the reads of key rows 0-3 and 8-11.
template <int HD, int VBUF, int DB>
__device__ __forceinline__ void read_v_block(const uint32_t (&vaddr)[Cfg<HD>::DB][2], u32x2_t (&out)[8]) {
    static_for<4>([&](auto F) {
        constexpr int f = decltype(F)::value;
        constexpr int off = VBUF + f * 16 * Cfg<HD>::ROWB;
        out[2 * f] = lds_read_tr16<off>(vaddr[DB][0]);
        out[2 * f + 1] = lds_read_tr16<off>(vaddr[DB][1]);
    });
}

// Wait until at most N LDS operations are outstanding (LDS returns in order);
// the fragments pass through the asm so their consumers stay after the wait.
template <int N>
__device__ __forceinline__ void lds_wait_block(u32x2_t (&v)[8]) {
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
                 : "n"(N));
}

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
    int ntg;            // task groups per (sequence, kv head) in the grid
    int units;          // num_seqs * n_kv
};

// DMA of one K or V tile (keys [kbase, kbase + BK) of one sequence) into the
// LDS buffer `dst`: the buffer view starts at the tile, so keys at or past the
// sequence end read 0.  Wave w fills the 1 KiB blocks [w*DMA_PER_WAVE, ...).
template <int HD>
__device__ __forceinline__ void dma_tile(const uint16_t* src, int64_t ld, int64_t s0, int Lb, int wave, int kbase,
                                         lds_char_t* dst, const uint32_t* off) {
    using C = Cfg<HD>;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src + (s0 + kbase) * ld, (uint32_t)((int64_t)(Lb - kbase) * ld * 2));
#pragma unroll
    for (int i = 0; i < C::DMA_PER_WAVE; ++i) {
        const int blk = wave * C::DMA_PER_WAVE + i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst + blk * 1024), 16, off[i], 0, 0, 0);
    }
}

template <int HD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(Params p) {
    using C = Cfg<HD>;
    extern __shared__ __align__(16) uint16_t smem[];
    lds_char_t* lds = (lds_char_t*)smem;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r32 = lane & 31, half = lane >> 5;

    // ---- workgroup -> (unit = (sequence, kv head), task group), heaviest first
    int unit, rank;
    {
        const int L = blockIdx.x;
        if (p.units % kNumXcd == 0) {
            // XCD x runs units x, x + 8, x + 16, ...: with n_kv a multiple of 8 that is
            // one kv head of every sequence, so the XCDs get equal shares of work
            const int per_xcd = p.units / kNumXcd;
            const int xcd = L % kNumXcd, local = L / kNumXcd;
            unit = (local % per_xcd) * kNumXcd + xcd;
            rank = local / per_xcd;
        } else {
            unit = L % p.units;
            rank = L / p.units;
        }
    }
    const int b = unit / p.n_kv;
    const int g = unit - b * p.n_kv;
    int64_t s0 = 0, s1 = p.total;
    if (p.cu != nullptr) {
        s0 = min<int64_t>(max<int64_t>(p.cu[b], 0), p.total);
        s1 = min<int64_t>(max<int64_t>(p.cu[b + 1], s0), p.total);
    }
    const int Lb = (int)(s1 - s0);
    const int G = p.group;
    const int nqb = (Lb + BQ - 1) / BQ;
    const int ntasks = G * nqb;
    const int ntg_b = (ntasks + kWaves - 1) / kWaves;
    const int tg = p.ntg - 1 - rank;
    if (tg >= ntg_b) return;                                   // uniform per workgroup

    const int task = tg * kWaves + wave;
    const bool active = task < ntasks;
    const int qblk = active ? task / G : 0;
    const int head = g * G + (active ? task % G : 0);
    const int q0 = qblk * BQ;                                  // first query row (in sequence)
    const int last_task = min(tg * kWaves + kWaves - 1, ntasks - 1);
    const int kv_end = min(Lb, (last_task / G + 1) * BQ);
    const int ntiles = (kv_end + BK - 1) / BK;                 // tiles the workgroup visits
    const int wave_last_q = min(q0 + BQ, Lb) - 1;
    const int wave_ntiles = active ? wave_last_q / BK + 1 : 0; // tiles this wave computes

    // ---- Q tile in registers: B operand of S^T = K Q^T (column = query r32)
    bf16x8_t qreg[C::DCH];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + s0 * p.ldq, (uint32_t)((int64_t)Lb * p.ldq * 2));
#pragma unroll
        for (int dc = 0; dc < C::DCH; ++dc) {
            const uint32_t off = (uint32_t)(((int64_t)(q0 + r32) * p.ldq + head * HD + dc * 16 + half * 8) * 2);
            qreg[dc] = as_bf16x8(buf_load16(rq, off));
        }
    }

    // ---- DMA lane offsets: lane l writes bytes [16 l, 16 l + 16) of a 1 KiB block,
    // i.e. row l / NC, physical chunk l % NC, so it fetches the logical chunk the
    // swizzle puts there.
    uint32_t dma_k[C::DMA_PER_WAVE], dma_v[C::DMA_PER_WAVE];
#pragma unroll
    for (int i = 0; i < C::DMA_PER_WAVE; ++i) {
        const int row = (wave * C::DMA_PER_WAVE + i) * C::RPI + lane / C::NC;
        const int lch = (lane % C::NC) ^ swz<HD>(row);
        dma_k[i] = (uint32_t)(((int64_t)row * p.ldk + g * HD + lch * 8) * 2);
        dma_v[i] = (uint32_t)(((int64_t)row * p.ldv + g * HD + lch * 8) * 2);
    }
    auto issue_k = [&](int tile, int buf) { dma_tile<HD>(p.k, p.ldk, s0, Lb, wave, tile * BK, lds + buf, dma_k); };
    auto issue_v = [&](int tile, int buf) { dma_tile<HD>(p.v, p.ldv, s0, Lb, wave, tile * BK, lds + buf, dma_v); };

    // ---- per-lane LDS read offsets
    // K operand (A of S^T): row = kb*32 + r32, logical chunk dc*2 + half
    uint32_t koff[C::DCH];
#pragma unroll
    for (int dc = 0; dc < C::DCH; ++dc)
        koff[dc] = r32 * C::ROWB + (((dc * 2 + half) ^ swz<HD>(r32)) * 16);
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

    f32x16_t oacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.0f;
    float m_run = -1.0e30f, l_run = 0.0f;
    const float c = p.c;

    // S^T = K Q^T for the tile in K buffer KB: 2 blocks of 32 keys
    auto scores = [&](auto KBc, f32x16_t (&s)[2]) {
        constexpr int KB = decltype(KBc)::value;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) s[kb][e] = 0.0f;
#pragma unroll
        for (int dc = 0; dc < C::DCH; ++dc)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8_t ka = as_bf16x8(*(const lds_u32x4_t*)(lds + KB + kb * 32 * C::ROWB + koff[dc]));
                s[kb] = mfma32x32x16(ka, qreg[dc], s[kb]);
            }
    };

    // p = exp2(s*c - mc) in place, row sum, bf16 packing as the B operand of O^T
    auto exponentiate = [&](f32x16_t (&s)[2], float mc, bf16x8_t (&pb)[2][2]) -> float {
        float rs = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float pe = fast_exp2(__builtin_fmaf(s[kb][e], c, -mc));
                s[kb][e] = pe;
                rs += pe;
            }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4_t w;
#pragma unroll
                for (int t = 0; t < 4; ++t) w[t] = pack_bf16x2(s[kb][h * 8 + 2 * t], s[kb][h * 8 + 2 * t + 1]);
                pb[kb][h] = as_bf16x8(w);
            }
        return rs;
    };

    // O^T += V^T P^T from V buffer VB.  The V^T fragments of block db + 1 are in
    // flight while block db is on the matrix cores (lgkmcnt(8) retires block db).
    auto pv = [&](auto VBc, const bf16x8_t (&pb)[2][2]) {
        constexpr int VB = decltype(VBc)::value;
        u32x2_t vf[2][8];
        read_v_block<HD, VB, 0>(vaddr, vf[0]);
        static_for<C::DB>([&](auto DBc) {
            constexpr int db = decltype(DBc)::value;
            if constexpr (db + 1 < C::DB) {
                read_v_block<HD, VB, db + 1>(vaddr, vf[(db + 1) & 1]);
                lds_wait_block<8>(vf[db & 1]);
            } else {
                lds_wait_block<0>(vf[db & 1]);
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int f = (kb * 2 + h) * 2;
                    const u32x4_t w = {vf[db & 1][f][0], vf[db & 1][f][1], vf[db & 1][f + 1][0], vf[db & 1][f + 1][1]};
                    oacc[db] = mfma32x32x16(as_bf16x8(w), pb[kb][h], oacc[db]);
                }
        });
    };

    // score accumulators: tile j in one, tile j + 1 in the other, roles swapping each tile
    f32x16_t s_a[2], s_b[2];

    // One kv tile j: softmax of S_j (in s_cur) while S_{j+1} goes to the matrix
    // cores (into s_next), then O += P_j V_j.  KN: K buffer of tile j + 1, VC: V
    // buffer of tile j.  On a wave's last tile the scores of "tile j + 1" are
    // computed from whatever the K buffer holds and never used.
    auto step = [&](int j, auto KNc, auto VCc, f32x16_t (&s_cur)[2], f32x16_t (&s_next)[2]) {
        const int kbase = j * BK;
        // causal mask per element on tiles that reach past the first query
        if (kbase + BK - 1 > q0) {
            const int qry = q0 + r32;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = kbase + kb * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
                    if (key > qry) s_cur[kb][e] = -__builtin_inff();
                }
        }
        scores(KNc, s_next);
        // Online softmax, one query per lane (its 64 keys split with lane ^ 32).
        // A row's reference max only moves when the row's tile max exceeds it by
        // more than kRescaleLog2 (log2 units): the result does not depend on the
        // reference (it cancels in O / l) and p stays <= 2^kRescaleLog2.  Only
        // rows past the threshold move, so a row's arithmetic depends on its own
        // scores alone.
        float mx = s_cur[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = __builtin_fmaxf(mx, s_cur[kb][e]);
        mx = __builtin_fmaxf(mx, swap_halves(mx));
        const bool move = (mx - m_run) * c > kRescaleLog2;
        const float m_ref = move ? mx : m_run;
        bf16x8_t pb[2][2];
        const float rs = exponentiate(s_cur, m_ref * c, pb);
        // keep the exponentials in this block, next to the score MFMAs, instead
        // of letting them sink past the rare branch
        asm volatile("" : : "v"(pb[0][0]), "v"(pb[0][1]), "v"(pb[1][0]), "v"(pb[1][1]), "v"(rs));
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
            // rare: rows past the threshold move their reference; rescale their O and l
            const float alpha = fast_exp2((m_run - m_ref) * c);
            m_run = m_ref;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
        }
        l_run += rs;
        pv(VCc, pb);
    };

    // One loop iteration: DMA of K_{j+2} (into K_j's buffer) and V_{j+1}, then
    // tile j.  Tile j's K buffer is (j & 1), its V buffer (j & 1).
    auto iteration = [&](int j, auto KCc, auto KNc, auto VCc, auto VNc, f32x16_t (&s_cur)[2], f32x16_t (&s_next)[2]) {
        constexpr int KC = decltype(KCc)::value, VN = decltype(VNc)::value;
        if (j + 2 < ntiles) issue_k(j + 2, KC);
        if (j + 1 < ntiles) issue_v(j + 1, VN);
        if (j < wave_ntiles) step(j, KNc, VCc, s_cur, s_next);
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
        __syncthreads();
    };

    using K0 = std::integral_constant<int, C::KBUF0>;
    using K1 = std::integral_constant<int, C::KBUF1>;
    using V0 = std::integral_constant<int, C::VBUF0>;
    using V1 = std::integral_constant<int, C::VBUF1>;

    // prologue: K_0, V_0 and K_1 in flight, scores of tile 0, and a barrier so
    // that K_0's buffer is free before K_2 lands in it
    issue_k(0, C::KBUF0);
    issue_v(0, C::VBUF0);
    if (1 < ntiles) issue_k(1, C::KBUF1);
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    if (0 < wave_ntiles) scores(K0{}, s_a);
    __syncthreads();
    // two tiles per trip so every buffer offset is a compile-time constant
    for (int j = 0; j < ntiles; j += 2) {
        iteration(j, K0{}, K1{}, V0{}, V1{}, s_a, s_b);
        if (j + 1 >= ntiles) break;
        iteration(j + 1, K1{}, K0{}, V1{}, V0{}, s_b, s_a);
    }

    if (!active) return;
    // ---- epilogue: O / l, bf16 RNE, 4 consecutive d per store
    const float l_tot = l_run + swap_halves(l_run);
    const float inv = 1.0f / l_tot;
    const int row = q0 + r32;
    if (row >= Lb) return;
    uint16_t* dst = p.o + (s0 + row) * p.ldo + head * HD;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int d = db * 32 + gq * 8 + half * 4;
            u32x2_t w2 = {pack_bf16x2(oacc[db][gq * 4 + 0] * inv, oacc[db][gq * 4 + 1] * inv),
                          pack_bf16x2(oacc[db][gq * 4 + 2] * inv, oacc[db][gq * 4 + 3] * inv)};
            *reinterpret_cast<u32x2_t*>(dst + d) = w2;
        }
}

template <int HD>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t s) {
    using C = Cfg<HD>;
    static const hipError_t attr = hipFuncSetAttribute((const void*)attn_fwd_kernel<HD>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       C::LDS_BYTES);
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
    p.ntg = (p.group * nqb + kWaves - 1) / kWaves;
    p.units = a.num_seqs * a.n_kv_head;
    const int64_t grid = (int64_t)p.ntg * p.units;
    hipLaunchKernelGGL((attn_fwd_kernel<HD>), dim3((uint32_t)grid), dim3(kThreads), C::LDS_BYTES, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
    switch (a.head_dim) {
        case 32: return launch_cfg<32>(a, s);
        case 64: return launch_cfg<64>(a, s);
        case 128: return launch_cfg<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pca
