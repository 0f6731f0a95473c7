// FP8 (OCP E4M3) operands for the projection GEMM, fp32 accumulation.
//
// The tuning notes (hncyxsy.com/news/227904) §2.3 list FP8 inputs with wider
// accumulation among the prefill levers (the softmax stays in higher
// precision).  Here both operands of y = x w^T are quantised row-wise with
// the same absmax rule as the fp8 KV cache: for each row r of x (tokens) and
// of w^T (output features), scale[r] = amax / 448 and
// code = E4M3_RNE_saturate(v * (448 / amax)); then
//   y[m, n] = RNE_bf16(sx[m] * sw[n] * sum_k dec(xq[m, k]) * dec(wq[n, k])).
//
// gfx950 design: the bf16 GEMM's tiling, DMA and LDS layout byte for byte
// (a K step is 128 fp8 = 128 bytes per row, two 64-wide slices), with
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales): 2x the bf16 MFMA
// rate per cycle, half the LDS bytes per flop.  Eight waves, two per SIMD,
// each 64 (m) x 128 (n) as 2 x 4 blocks with its 128 fp32 accumulators in
// AGPRs and its operands in VGPRs.  A slice is two 16-byte parts per lane
// and block (lane half h takes bytes 32h .. 32h+31 of the slice in both
// operands, so the products pair up), read as one 8-register tuple.  The next
// slice's x blocks are read at a slice's start, and its W block i right
// after block i's two MFMAs into the same registers, so 64 operand registers
// keep two slices in flight.  The row scales multiply the fp32 accumulators
// in the staged epilogue, before the single rounding.
#include "gemm_common.hpp"
#include "kv_common.hpp"
#include "pca_internal.hpp"

namespace pca {

namespace {

using namespace gemm;

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int BK8 = 128;                      // fp8 elements per K step (ROWB bytes)

// Eight waves, two per SIMD, each BMT / 4 (m) x 128 (n) as FM8 x 4 blocks
// (BMT = 256 or 128 rows of x per tile): the bf16 GEMM's tiling, DMA and LDS
// layout, with a K step of 128 fp8 bytes = two 64-wide MFMA slices.  Only
// waves 0-3 request tiles; the other wave of each SIMD issues MFMAs through
// their wait at the DMA.
constexpr int kWavesF8 = 8;
constexpr int kThreadsF8 = kWavesF8 * 64;
constexpr int FN8 = 4;                         // blocks per wave along n
constexpr int kLdsF8 = LDS_BYTES + (BN + BM) * 4;   // operand stages, then the tile's scales

// Wait until at most N LDS reads are outstanding (LDS returns in order); the
// operand tuples pass through the asm so the MFMAs stay after it.
template <int N>
__device__ __forceinline__ void lds_wait_ops8(i32x8_t (&w)[4], i32x8_t (&x)[2], i32x8_t (&xn)[2]) {
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(x[0]), "+v"(x[1]), "+v"(xn[0]), "+v"(xn[1])
                 : "n"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait_ops8(i32x8_t (&w)[4], i32x8_t (&x)[1], i32x8_t (&xn)[1]) {
    asm volatile("s_waitcnt lgkmcnt(%6)"
                 : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(x[0]), "+v"(xn[0])
                 : "n"(N));
}

// One workgroup computes output tile (tm, tn) of BMT rows.
template <int BMT>
__device__ __forceinline__ void gemm_fp8_tile(const Fp8GemmArgs& a, int tm, int tn) {
    constexpr int FM8 = BMT / 128;                 // blocks per wave along m
    constexpr int WMR = 32 * FM8;                  // x rows per wave
    constexpr int DMA_X = BMT / 32;                // 1 KiB DMA blocks of the x tile per requesting wave
    extern __shared__ __align__(16) uint16_t smem[];
    lds_char_t* lds = (lds_char_t*)smem;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;       // 4 (m) x 2 (n)
    const int r32 = lane & 31, half = lane >> 5;

    const int m0 = tm * BMT, n0 = tn * BN;
    const int rows_x = min(BMT, a.M - m0), rows_w = min(BN, a.N - n0);
    const int nk = (a.K + BK8 - 1) / BK8;

    // DMA (waves 0-3: 8 blocks of the W tile, DMA_X of the x tile each):
    // block i of wave w covers rows (nb w + i) * 8 .. + 7 of its operand (nb
    // its blocks per wave); lane l fetches logical chunk (l % 8) ^ swz(row) of
    // row (nb w + i) * 8 + l / 8.  swz of that row depends on i only through
    // i & 1 (nb w * 8 is a multiple of 32), so two lane chunk values serve all
    // blocks, and block i adds the uniform 8 i rows.
    const int dw = wave & 3;
    const int row0w = dw * 64 + lane / 8, row0x = dw * DMA_X * 8 + lane / 8;
    int lch[2];
    lch[0] = (lane % 8) ^ swz(row0w);
    lch[1] = (lane % 8) ^ swz(row0w + 8);
    const uint32_t basew = (uint32_t)((int64_t)row0w * a.ldw), basex = (uint32_t)((int64_t)row0x * a.ldx);
    auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
        if (wave >= 4) return;                        // uniform per wave
        const int k0 = kt * BK8;
        const bool tail = k0 + BK8 > a.K;
        const __amdgpu_buffer_rsrc_t rw = uniform_rsrc(a.w + (int64_t)n0 * a.ldw + k0, (int64_t)rows_w * a.ldw - k0);
        const __amdgpu_buffer_rsrc_t rx = uniform_rsrc(a.x + (int64_t)m0 * a.ldx + k0, (int64_t)rows_x * a.ldx - k0);
        lds_char_t* dst = lds + stage * STAGE_B;
        // (the whole offset in the VGPR: the range check covers it, not soffset)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool oob = tail && (k0 + lch[i & 1] * 16 >= a.K);
            const uint32_t ow = basew + (uint32_t)(i * 8 * a.ldw) + (uint32_t)(lch[i & 1] * 16);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)(dst + (dw * 8 + i) * 1024), 16, oob ? kOob : ow,
                                                     0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < DMA_X; ++i) {
            const bool oob = tail && (k0 + lch[i & 1] * 16 >= a.K);
            const uint32_t ox = basex + (uint32_t)(i * 8 * a.ldx) + (uint32_t)(lch[i & 1] * 16);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(dst + TILE_B + (dw * DMA_X + i) * 1024), 16,
                                                     oob ? kOob : ox, 0, 0, 0);
        }
    };

    // operand reads of slice s (bytes 64 s .. 64 s + 63 of the K step), part
    // q: logical chunk 4 s + 2 half + q of row block * 32 + r32
    uint32_t rdaddr[2][2];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
        for (int q = 0; q < 2; ++q)
            rdaddr[sl][q] = (uint32_t)(uintptr_t)lds + r32 * ROWB + (((sl * 4 + half * 2 + q) ^ swz(r32)) * 16);
    const uint32_t woff = wn * 128 * ROWB, xoff = TILE_B + wm * WMR * ROWB;

    f32x16_t acc[FN8][FM8];
#pragma unroll
    for (int i = 0; i < FN8; ++i)
#pragma unroll
        for (int j = 0; j < FM8; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Operands of the slice on the matrix cores: wf[2i + q] = W block i part
    // q, xf[2j + q] = X block j part q.  The next slice's X parts are read
    // into xn at the slice's start; its W block i is read into wf[2i..2i+1]
    // right after block i's two MFMAs, so 64 operand registers serve two
    // slices in flight.  LDS returns in order, so each block's wait counts
    // the reads issued after it.
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    // one 8-register tuple per block (both 16-byte parts), as the MFMA takes it
    i32x8_t wf[4], xf[FM8], xn[FM8];
    auto pair = [](u32x4_t lo, u32x4_t hi) __attribute__((always_inline)) {
        return __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto read_w = [&](uint32_t soff, auto Sc, auto Ic) __attribute__((always_inline)) {
        constexpr int sl = decltype(Sc)::value, i = decltype(Ic)::value;
        wf[i] = pair(lds_read_b128<i * 32 * ROWB>(rdaddr[sl][0] + soff + woff),
                     lds_read_b128<i * 32 * ROWB>(rdaddr[sl][1] + soff + woff));
    };
    auto read_x = [&](uint32_t soff, auto Sc, i32x8_t (&x)[FM8]) __attribute__((always_inline)) {
        constexpr int sl = decltype(Sc)::value;
        static_for<FM8>([&](auto Jc) {
            constexpr int j = decltype(Jc)::value;
            x[j] = pair(lds_read_b128<j * 32 * ROWB>(rdaddr[sl][0] + soff + xoff),
                        lds_read_b128<j * 32 * ROWB>(rdaddr[sl][1] + soff + xoff));
        });
    };
    auto wait_ops = [&](auto Nc) __attribute__((always_inline)) { lds_wait_ops8<decltype(Nc)::value>(wf, xf, xn); };
    // the slice's 8 MFMAs, block by block, with the next slice's W block read
    // in behind each (into stage soff_next, slice SN)
    auto run_slice = [&](uint32_t soff_next, auto SNc) __attribute__((always_inline)) {
        static_for<FN8>([&](auto Ic) {
            constexpr int i = decltype(Ic)::value;
            // outstanding before block i's wait: this slice's W blocks i+1..3
            // (2 reads each, issued in the previous slice), then xn (2 FM8),
            // then the next slice's W blocks 0..i-1 (2 each)
            wait_ops(std::integral_constant<int, 2 * (FN8 - 1 - i) + 2 * FM8 + 2 * i>{});
            static_for<FM8>([&](auto Jc) {
                constexpr int j = decltype(Jc)::value;
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[i], xf[j], acc[i][j], 0, 0, 0, 127, 0,
                                                                            127);
                // keep the accumulators in AGPRs (the VGPRs hold the operands)
                asm volatile("" : "+a"(acc[i][j]));
            });
            __builtin_amdgcn_sched_barrier(0);
            read_w(soff_next, SNc, Ic);
            __builtin_amdgcn_sched_barrier(0);
        });
#pragma unroll
        for (int j = 0; j < FM8; ++j) xf[j] = xn[j];
    };

    // the tile's row and column scales, one per thread, into an LDS area past
    // the operand stages: requested ahead of the first tiles, so their
    // latency hides behind that wait (read from memory in the epilogue, 32
    // per lane in batches of four, each batch waited for, they cost 5-7%)
    // [0, 256): sw of the tile's columns, [256, 512): sx of its rows
    __attribute__((address_space(3))) float* lsc = (__attribute__((address_space(3))) float*)(lds + LDS_BYTES);
    {
        float v = 0.0f;
        if (tid < BN) {
            if (n0 + tid < a.N) v = a.sw[n0 + tid];
        } else if (tid - BN < BMT && m0 + (tid - BN) < a.M) {
            v = a.sx[m0 + tid - BN];
        }
        issue(0, 0);
        if (1 < nk) issue(1, 1);
        lsc[tid] = v;
    }
    if (1 < nk) __builtin_amdgcn_s_waitcnt(vmcnt_imm(8 + DMA_X));   // step 0 only
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    wg_barrier();
    static_for<FN8>([&](auto Ic) { read_w(0u, S0{}, Ic); });
    read_x(0u, S0{}, xf);
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        const uint32_t soff = (uint32_t)(st * STAGE_B);
        // slice 0 of step kt; slice 1's operands (same stage) read behind it
        read_x(soff, S1{}, xn);
        run_slice(soff, S1{});
        wait_ops(std::integral_constant<int, 0>{});
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));    // this wave's loads of step kt + 1
        wg_barrier();
        // slice 1; the next step's slice 0 (other stage) read behind it, and
        // step kt + 2's tiles requested into this stage
        // (after the last step these reads fetch stale LDS bytes that are
        // never used: unconditional, so no branch splits the MFMA sequence)
        read_x(soff ^ (uint32_t)STAGE_B, S0{}, xn);
        if (kt + 2 < nk) issue(kt + 2, st);
        run_slice(soff ^ (uint32_t)STAGE_B, S0{});
    }

    // epilogue: y = sx[m] * sw[n] * acc, rounded once, staged through LDS and
    // written as full rows
    wg_barrier();
    lds_char_t* stg = lds + wave * (WMR * 256);
    const int m_lo = m0 + wm * WMR;
#pragma unroll
    for (int j = 0; j < FM8; ++j) {
        const float sxm = lsc[BN + wm * WMR + j * 32 + r32];         // 0 past M
#pragma unroll
        for (int i = 0; i < FN8; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int nl = wn * 128 + i * 32 + g * 8 + half * 4;      // column within the tile
                const f32x4_t sw4 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4_t*>(lsc + nl);   // 0 past N
                float t[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] = acc[i][j][g * 4 + e] * sxm * sw4[e];
                const int ml = j * 32 + r32, ci = i * 4 + g;
                *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>(
                    stg + ml * 256 + ((ci ^ (ml & 15)) * 16) + half * 8) = u32x2_t{pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3])};
            }
    }
    const int c = lane & 15;
    const int n = n0 + wn * 128 + c * 8;
#pragma unroll 4
    for (int r = 0; r < WMR / 4; ++r) {
        const int ml = r * 4 + (lane >> 4);
        const u32x4_t v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
            stg + ml * 256 + ((c ^ (ml & 15)) * 16));
        const int m = m_lo + ml;
        if (m >= a.M) continue;
        uint16_t* dst = a.y + (int64_t)m * a.ldy + n;
        if (n + 7 < a.N) {
            *reinterpret_cast<u32x4_t*>(dst) = v;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < a.N) dst[e] = (uint16_t)((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        }
    }
}

// The grid (the bf16 GEMM's plan_tiles): BMT 256 or 128, tiles of that
// height; BMT 0, the first split_n column strips in 256-row tiles, then the
// rest of N in 128-row tiles.
template <int BMT>
__global__ __launch_bounds__(kThreadsF8) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_fp8_kernel(Fp8GemmArgs a, int split_n) {
    const int tiles_n = (a.N + BN - 1) / BN;
    int tm, tn;
    if constexpr (BMT != 0) {
        tile_coords_id((int)blockIdx.x, (a.M + BMT - 1) / BMT, tiles_n, tm, tn);
        gemm_fp8_tile<BMT>(a, tm, tn);
    } else {
        const int tm256 = (a.M + 255) / 256, big = tm256 * split_n;
        if ((int)blockIdx.x < big) {
            tile_coords_id((int)blockIdx.x, tm256, split_n, tm, tn);
            gemm_fp8_tile<256>(a, tm, tn);
        } else {
            tile_coords_id((int)blockIdx.x - big, (a.M + 127) / 128, tiles_n - split_n, tm, tn);
            gemm_fp8_tile<128>(a, tm, tn + split_n);
        }
    }
}

template <int BMT>
hipError_t launch_fp8_tiles(const Fp8GemmArgs& a, int tiles, int split_n, hipStream_t s) {
    static const hipError_t attr = hipFuncSetAttribute((const void*)gemm_fp8_kernel<BMT>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsF8);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((gemm_fp8_kernel<BMT>), dim3(tiles), dim3(kThreadsF8), kLdsF8, s, a, split_n);
    return hipGetLastError();
}

// Row-wise E4M3 quantisation: one wave per row, amax over the row (16-byte
// loads, cross-lane max), then the codes with the KV cache's encoder.
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t* x, int64_t ldx, int M, int K,
                                                            uint8_t* q, int64_t ldq, float* scales) {
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;                                   // uniform per wave
    const uint16_t* row = x + (int64_t)m * ldx;
    float amax = 0.0f;
    for (int k = lane * 8; k < K; k += 64 * 8) {          // K is a multiple of 16
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(row + k);
#pragma unroll
        for (int t = 0; t < 4; ++t)
            amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(bf16_lo(v[t])), __builtin_fabsf(bf16_hi(v[t]))));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off));
    // binary32 round-to-nearest division (no fast-math): scale = amax / 448, inv = 448 / amax
    const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
    for (int k = lane * 8; k < K; k += 64 * 8) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(row + k);
        const uint32_t lo = e4m3x4(bf16_lo(v[0]) * inv, bf16_hi(v[0]) * inv, bf16_lo(v[1]) * inv, bf16_hi(v[1]) * inv);
        const uint32_t hi = e4m3x4(bf16_lo(v[2]) * inv, bf16_hi(v[2]) * inv, bf16_lo(v[3]) * inv, bf16_hi(v[3]) * inv);
        *reinterpret_cast<u32x2_t*>(q + (int64_t)m * ldq + k) = u32x2_t{lo, hi};
    }
    if (lane == 0) scales[m] = amax / 448.0f;
}

// The same for rows of at most NI * 512 elements, held in registers between
// the amax and the encoding, so x is read once (the loop above reads each row
// twice; the second pass mostly hits the caches but still costs the loads).
template <int NI>
__global__ __launch_bounds__(256) void quantize_rows_reg_kernel(const uint16_t* x, int64_t ldx, int M, int K,
                                                                uint8_t* q, int64_t ldq, float* scales) {
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;                                   // uniform per wave
    const uint16_t* row = x + (int64_t)m * ldx;
    u32x4_t v[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int k = lane * 8 + i * 512;                 // K is a multiple of 16
        v[i] = k < K ? *reinterpret_cast<const u32x4_t*>(row + k) : u32x4_t{0u, 0u, 0u, 0u};
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t)
            amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(bf16_lo(v[i][t])), __builtin_fabsf(bf16_hi(v[i][t]))));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off));
    // binary32 round-to-nearest division (no fast-math): scale = amax / 448, inv = 448 / amax
    const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int k = lane * 8 + i * 512;
        if (k < K) {
            const uint32_t lo = e4m3x4(bf16_lo(v[i][0]) * inv, bf16_hi(v[i][0]) * inv, bf16_lo(v[i][1]) * inv,
                                       bf16_hi(v[i][1]) * inv);
            const uint32_t hi = e4m3x4(bf16_lo(v[i][2]) * inv, bf16_hi(v[i][2]) * inv, bf16_lo(v[i][3]) * inv,
                                       bf16_hi(v[i][3]) * inv);
            *reinterpret_cast<u32x2_t*>(q + (int64_t)m * ldq + k) = u32x2_t{lo, hi};
        }
    }
    if (lane == 0) scales[m] = amax / 448.0f;
}

// Per-(token, head) E4M3 rows with power-of-two scales (the fp8 operands of
// the attention scores): R = head_dim / 8 lanes hold one row, 16 bytes each;
// y = x * prescale in binary32, the row's amax by DPP (unsigned max of the
// bit patterns), e = pow2_exponent(amax), codes of y * 2^-e (exact scaling)
// and the scale byte e + 127 from the row's first lane.  Rows are R-aligned
// groups of consecutive ids and the grid stride is a multiple of 256, so a
// row's lanes run every loop trip together.
template <int R>
__global__ __launch_bounds__(256) void quantize_heads_kernel(const uint16_t* x, int64_t ldx, int64_t T, int H,
                                                             float prescale, uint8_t* q, int64_t ldq, uint8_t* ex,
                                                             int64_t lde) {
    const int64_t total = T * H * R;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x; id < total; id += stride) {
        const int64_t row = id / R;
        const int ch = (int)(id - row * R);
        const int64_t t = row / H;
        const int h = (int)(row - t * H);
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(x + t * ldx + (int64_t)h * R * 8 + ch * 8);
        float y[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            y[2 * j] = bf16_lo(v[j]) * prescale;
            y[2 * j + 1] = bf16_hi(v[j]) * prescale;
        }
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(y[j]));
        const int e = pow2_exponent(group_umax<R>(__builtin_bit_cast(uint32_t, m)));
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = __builtin_ldexpf(y[j], -e);
        const uint32_t lo = e4m3x4(y[0], y[1], y[2], y[3]);
        const uint32_t hi = e4m3x4(y[4], y[5], y[6], y[7]);
        *reinterpret_cast<u32x2_t*>(q + t * ldq + (int64_t)h * R * 8 + ch * 8) = u32x2_t{lo, hi};
        if (ch == 0) ex[t * lde + h] = (uint8_t)(e + 127);
    }
}

}  // namespace

hipError_t launch_quantize_heads(const uint16_t* x, int64_t ldx, int64_t T, int H, int hd, float prescale, uint8_t* q,
                                 int64_t ldq, uint8_t* ex, int64_t lde, hipStream_t s) {
    const int64_t blocks = (T * H * (hd / 8) + 255) / 256;
    const dim3 grid((uint32_t)(blocks > 16384 ? 16384 : (blocks < 1 ? 1 : blocks)));
    switch (hd) {
        case 32: hipLaunchKernelGGL(quantize_heads_kernel<4>, grid, dim3(256), 0, s, x, ldx, T, H, prescale, q, ldq, ex, lde); break;
        case 64: hipLaunchKernelGGL(quantize_heads_kernel<8>, grid, dim3(256), 0, s, x, ldx, T, H, prescale, q, ldq, ex, lde); break;
        case 128: hipLaunchKernelGGL(quantize_heads_kernel<16>, grid, dim3(256), 0, s, x, ldx, T, H, prescale, q, ldq, ex, lde); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemm_fp8(const Fp8GemmArgs& a, hipStream_t s) {
    const TilePlan t = plan_tiles(a.M, a.N, device_cus());
    if (t.bmt == 128) return launch_fp8_tiles<128>(a, t.tiles, 0, s);
    if (t.bmt == 0) return launch_fp8_tiles<0>(a, t.tiles, t.split_n, s);
    return launch_fp8_tiles<256>(a, t.tiles, 0, s);
}

hipError_t launch_quantize_rows(const uint16_t* x, int64_t ldx, int M, int K, uint8_t* q, int64_t ldq, float* scales,
                                hipStream_t s) {
    const dim3 grid((uint32_t)((M + 3) / 4));
    if (K <= 8 * 512)
        hipLaunchKernelGGL(quantize_rows_reg_kernel<8>, grid, dim3(256), 0, s, x, ldx, M, K, q, ldq, scales);
    else if (K <= 16 * 512)
        hipLaunchKernelGGL(quantize_rows_reg_kernel<16>, grid, dim3(256), 0, s, x, ldx, M, K, q, ldq, scales);
    else
        hipLaunchKernelGGL(quantize_rows_kernel, grid, dim3(256), 0, s, x, ldx, M, K, q, ldq, scales);
    return hipGetLastError();
}

}  // namespace pca
