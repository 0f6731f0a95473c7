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
//  * A wave owns 32*NQB query rows of one head (NQB = 1 for every head_dim); a workgroup is 4 waves that
//    share one kv head and the same kv tiles, loaded once into LDS per
//    workgroup: for G >= 4 the 4 waves are 4 query heads at the same
//    positions, for smaller G consecutive query blocks.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the 32x32 accumulator then holds, in each
//    lane, 16 keys of ONE query (the lane's column).  Row max and row sum are
//    lane-local plus one exchange with lane ^ 32, and the accumulator is
//    already the B operand of the second product O^T = V^T P^T once
//    converted to bf16 -- no cross-lane shuffle of P.  The contraction index
//    of that product pairs (lane half, element) in both operands, so V^T is
//    laid out in LDS with the same key order the accumulator has (within
//    each 16 keys: 0-3, 8-11 | 4-7, 12-15).
//  * Q stays in registers (B operand of S^T) for the whole kv loop; the O^T
//    accumulator (fp32) likewise; K tiles are stored row-major in LDS and V
//    tiles transposed, both double-buffered: tile j+1 is fetched into
//    registers while tile j is on the matrix cores.
//  * exp is exp2 with scale*log2(e) folded into one FMA; m, l, P in fp32,
//    P rounded to bf16 only as the MFMA operand.  The reference max of a row
//    moves only when the row's scores exceed it by 2^8 (see below), so the
//    rescale of the O accumulators is nearly always skipped.
//  * One wave per 32 query rows and two waves per SIMD (221 VGPRs): the
//    softmax of one wave overlaps the matrix-core work of the other.
//  * The causal rule: a wave skips kv tiles that start after its last query,
//    and masks per element only on tiles that reach past its first query.
//    Workgroups are ordered heaviest-first and all workgroups of one
//    (sequence, kv head) are placed on one XCD (ids go round-robin over the
//    8 XCDs), so its K/V stays in that XCD's L2.
#include "pca_device.hpp"
#include "pca_internal.hpp"

namespace pca {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int BK = 64;   // keys per kv tile
constexpr float kRescaleLog2 = 8.0f;   // lazy max update threshold (p stays <= 256)

template <int HD, int NQB>
struct Cfg {
    static constexpr int BQW = 32 * NQB;          // query rows per wave
    static constexpr int KROW = HD + 8;           // K tile row stride (elements), 16-byte pad
    static constexpr int VROW = BK + 8;           // V^T tile row stride (elements), 16-byte pad
    static constexpr int K_ELEMS = BK * KROW;
    static constexpr int V_ELEMS = HD * VROW;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static constexpr int LDS_BYTES = 2 * STAGE * 2;
    static constexpr int DCH = HD / 16;            // k16 steps over head_dim
    static constexpr int DB = HD / 32;             // 32-row blocks of O^T
    static constexpr int K_LOADS = BK * HD / 8 / kThreads;     // 16-byte chunks per thread
    static constexpr int V_BLOCKS = (BK / 8) * (HD / 4);       // 8-key x 4-d blocks per tile
};

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

template <int HD, int NQB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3 - NQB, 3 - NQB)))
void attn_fwd_kernel(Params p) {
    using C = Cfg<HD, NQB>;
    extern __shared__ __align__(16) uint16_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r32 = lane & 31, half = lane >> 5;

    // ---- workgroup -> (unit = (sequence, kv head), task group), heaviest first
    int unit, rank;
    {
        const int L = blockIdx.x;
        if (p.units % kNumXcd == 0) {
            const int per_xcd = p.units / kNumXcd;
            const int xcd = L % kNumXcd, local = L / kNumXcd;
            unit = xcd * per_xcd + local % per_xcd;
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
    const int nqb = (Lb + C::BQW - 1) / C::BQW;
    const int ntasks = G * nqb;
    const int ntg_b = (ntasks + kWaves - 1) / kWaves;
    const int tg = p.ntg - 1 - rank;
    if (tg >= ntg_b) return;                                   // uniform per workgroup

    const int task = tg * kWaves + wave;
    const bool active = task < ntasks;
    const int qblk = active ? task / G : 0;
    const int head = g * G + (active ? task % G : 0);
    const int q0 = qblk * C::BQW;                              // first query row (in sequence)
    const int last_task = min(tg * kWaves + kWaves - 1, ntasks - 1);
    const int kv_end = min(Lb, (last_task / G + 1) * C::BQW);
    const int ntiles = (kv_end + BK - 1) / BK;
    const int wave_last_q = min(q0 + C::BQW, Lb) - 1;
    const int wave_ntiles = active ? wave_last_q / BK + 1 : 0;

    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + s0 * p.ldq, (uint32_t)((int64_t)Lb * p.ldq * 2));
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + s0 * p.ldk, (uint32_t)((int64_t)Lb * p.ldk * 2));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + s0 * p.ldv, (uint32_t)((int64_t)Lb * p.ldv * 2));

    // ---- Q tile in registers: B operand of S^T = K Q^T (column = query r32)
    bf16x8_t qreg[NQB][C::DCH];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int dc = 0; dc < C::DCH; ++dc) {
            const uint32_t off = (uint32_t)(((int64_t)(q0 + qb * 32 + r32) * p.ldq + head * HD + dc * 16 + half * 8) * 2);
            qreg[qb][dc] = as_bf16x8(buf_load16(rq, off));
        }

    // ---- K/V tile staging (all 256 threads)
    u32x4_t kst[C::K_LOADS];
    u32x2_t vst[8];
    const int v_kg = tid / (HD / 4), v_dq = tid % (HD / 4);   // V block: 8 keys x 4 d
    const int v_key0 = (v_kg >> 1) * 16 + (v_kg & 1) * 4;
    const bool v_loader = tid < C::V_BLOCKS;
    auto global_load = [&](int kbase) {
#pragma unroll
        for (int i = 0; i < C::K_LOADS; ++i) {
            const int id = i * kThreads + tid;
            const int key = id / (HD / 8), ch = id % (HD / 8);
            const uint32_t off = (uint32_t)(((int64_t)(kbase + key) * p.ldk + g * HD + ch * 8) * 2);
            kst[i] = buf_load16(rk, off);
        }
        if (v_loader) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int key = kbase + v_key0 + (j & 3) + (j >> 2) * 8;
                const uint32_t off = (uint32_t)(((int64_t)key * p.ldv + g * HD + v_dq * 4) * 2);
                vst[j] = buf_load8(rv, off);
            }
        }
    };
    auto lds_store = [&](int st) {
        uint16_t* ks = smem + st * C::STAGE;
        uint16_t* vt = ks + C::K_ELEMS;
#pragma unroll
        for (int i = 0; i < C::K_LOADS; ++i) {
            const int id = i * kThreads + tid;
            const int key = id / (HD / 8), ch = id % (HD / 8);
            *reinterpret_cast<u32x4_t*>(ks + key * C::KROW + ch * 8) = kst[i];
        }
        if (v_loader) {
            // transpose 8 keys x 4 d into 4 rows (d) of 8 keys each
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) {
                u32x4_t w;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t a0 = vst[2 * j][dd >> 1], a1 = vst[2 * j + 1][dd >> 1];
                    w[j] = (dd & 1) ? ((a0 >> 16) | (a1 & 0xFFFF0000u)) : ((a0 & 0xFFFFu) | (a1 << 16));
                }
                *reinterpret_cast<u32x4_t*>(vt + (v_dq * 4 + dd) * C::VROW + (v_kg >> 1) * 16 + (v_kg & 1) * 8) = w;
            }
        }
    };

    f32x16_t oacc[NQB][C::DB];
    float m_run[NQB], l_run[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        m_run[qb] = -1.0e30f;
        l_run[qb] = 0.0f;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[qb][db][e] = 0.0f;
    }
    const float c = p.c;

    global_load(0);
    lds_store(0);
    __syncthreads();

    for (int j = 0; j < ntiles; ++j) {
        const int st = j & 1;
        const int kbase = j * BK;
        if (j + 1 < ntiles) global_load(kbase + BK);

        if (j < wave_ntiles) {
            const uint16_t* ks = smem + st * C::STAGE;
            const uint16_t* vt = ks + C::K_ELEMS;
            // S^T = K Q^T: 2 blocks of 32 keys x NQB blocks of 32 queries
            f32x16_t s[2][NQB];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) s[kb][qb][e] = 0.0f;
#pragma unroll
            for (int dc = 0; dc < C::DCH; ++dc) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8_t ka = as_bf16x8(*reinterpret_cast<const u32x4_t*>(
                        ks + (kb * 32 + r32) * C::KROW + dc * 16 + half * 8));
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) s[kb][qb] = mfma32x32x16(ka, qreg[qb][dc], s[kb][qb]);
                }
            }
            // causal mask per element on tiles that reach past the first query
            if (kbase + BK - 1 > q0) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int key = kbase + kb * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
                            const int qry = q0 + qb * 32 + r32;
                            if (key > qry) s[kb][qb][e] = -__builtin_inff();
                        }
            }
            // online softmax (one query per lane; its 32 keys split with lane ^ 32).
            // The running max is only moved when a row's tile max exceeds it by
            // more than kRescaleLog2 (in log2 units): the result is the same for
            // any reference value (it cancels in O / l), and the skipped moves keep
            // p <= 2^kRescaleLog2.  So the rescale of O -- the only VALU work on
            // the accumulators -- runs on the first tile and then only rarely.
            bf16x8_t pb[NQB][2][2];
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                float mx = s[0][qb][0];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) mx = __builtin_fmaxf(mx, s[kb][qb][e]);
                mx = __builtin_fmaxf(mx, swap_halves(mx));
                const bool move = (mx - m_run[qb]) * c > kRescaleLog2;
                if (__builtin_amdgcn_ballot_w64(move) != 0) {
                    // only rows past the threshold move, so every row's arithmetic
                    // depends on its own scores alone (alpha = 1 is exact elsewhere)
                    const float m_new = move ? mx : m_run[qb];
                    const float alpha = move ? fast_exp2((m_run[qb] - m_new) * c) : 1.0f;
                    m_run[qb] = m_new;
                    l_run[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < C::DB; ++db)
#pragma unroll
                        for (int e = 0; e < 16; ++e) oacc[qb][db][e] *= alpha;
                }
                const float mc = m_run[qb] * c;
                float rs = 0.0f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const float pe = fast_exp2(__builtin_fmaf(s[kb][qb][e], c, -mc));
                        s[kb][qb][e] = pe;
                        rs += pe;
                    }
                l_run[qb] += rs;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        u32x4_t w;
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            w[t] = pack_bf16x2(s[kb][qb][h * 8 + 2 * t], s[kb][qb][h * 8 + 2 * t + 1]);
                        pb[qb][kb][h] = as_bf16x8(w);
                    }
            }
            // O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const bf16x8_t va = as_bf16x8(*reinterpret_cast<const u32x4_t*>(
                            vt + (db * 32 + r32) * C::VROW + (kb * 2 + h) * 16 + half * 8));
#pragma unroll
                        for (int qb = 0; qb < NQB; ++qb) oacc[qb][db] = mfma32x32x16(va, pb[qb][kb][h], oacc[qb][db]);
                    }
        }
        if (j + 1 < ntiles) lds_store(st ^ 1);
        __syncthreads();
    }

    if (!active) return;
    // ---- epilogue: O / l, bf16 RNE, 4 consecutive d per store
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const float l_tot = l_run[qb] + swap_halves(l_run[qb]);
        const float inv = 1.0f / l_tot;
        const int row = q0 + qb * 32 + r32;
        if (row >= Lb) continue;
        uint16_t* dst = p.o + (s0 + row) * p.ldo + head * HD;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d = db * 32 + gq * 8 + half * 4;
                u32x2_t w2 = {pack_bf16x2(oacc[qb][db][gq * 4 + 0] * inv, oacc[qb][db][gq * 4 + 1] * inv),
                              pack_bf16x2(oacc[qb][db][gq * 4 + 2] * inv, oacc[qb][db][gq * 4 + 3] * inv)};
                *reinterpret_cast<u32x2_t*>(dst + d) = w2;
            }
    }
}

template <int HD, int NQB>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t s) {
    using C = Cfg<HD, NQB>;
    static const hipError_t attr = hipFuncSetAttribute((const void*)attn_fwd_kernel<HD, NQB>,
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
    const int nqb = (a.max_seqlen + C::BQW - 1) / C::BQW;
    p.ntg = (p.group * nqb + kWaves - 1) / kWaves;
    p.units = a.num_seqs * a.n_kv_head;
    const int64_t grid = (int64_t)p.ntg * p.units;
    hipLaunchKernelGGL((attn_fwd_kernel<HD, NQB>), dim3((uint32_t)grid), dim3(kThreads), C::LDS_BYTES, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
    switch (a.head_dim) {
        case 32: return launch_cfg<32, 1>(a, s);
        case 64: return launch_cfg<64, 1>(a, s);
        case 128: return launch_cfg<128, 1>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pca
