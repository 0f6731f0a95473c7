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
// gfx950 design: the bf16 GEMM's tiles, DMA and LDS layout unchanged in bytes
// (a K step is 128 fp8 = 128 bytes per row), with
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales): 2x the bf16 MFMA rate
// per cycle, half the LDS bytes per flop.  A 64-wide MFMA K slice is two
// 16-byte chunks per lane (lane half h takes bytes 32h .. 32h+31 of the
// slice in both operands, so the products pair up), 16 reads per slice for
// the 4 x 4 blocks, which exceeds the 15 LDS operations a wave can track: the
// next slice's reads go out in two groups of 8 between the current slice's
// two groups of 8 MFMAs.  The row scales multiply the fp32 accumulators in
// the staged epilogue, before the single rounding.
#include "gemm_common.hpp"
#include "kv_common.hpp"
#include "pca_internal.hpp"

namespace pca {

namespace {

using namespace gemm;

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int BK8 = 128;                      // fp8 elements per K step (ROWB bytes)

template <int N>
__device__ __forceinline__ void lds_wait16(u32x4_t (&f)[16]) {
    asm volatile("s_waitcnt lgkmcnt(%16)"
                 : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]), "+v"(f[5]), "+v"(f[6]), "+v"(f[7]),
                   "+v"(f[8]), "+v"(f[9]), "+v"(f[10]), "+v"(f[11]), "+v"(f[12]), "+v"(f[13]), "+v"(f[14]),
                   "+v"(f[15])
                 : "n"(N));
}

__device__ inline f32x16_t mfma_f8(u32x4_t a0, u32x4_t a1, u32x4_t b0, u32x4_t b1, f32x16_t c) {
    const i32x8_t a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    const i32x8_t b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    // formats 0/0: E4M3 for A and B; block scales 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_fp8_kernel(Fp8GemmArgs a) {
    extern __shared__ __align__(16) uint16_t smem[];
    lds_char_t* lds = (lds_char_t*)smem;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int r32 = lane & 31, half = lane >> 5;

    const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int rows_x = min(BM, a.M - m0), rows_w = min(BN, a.N - n0);
    const int nk = (a.K + BK8 - 1) / BK8;

    // DMA: block b of a wave covers rows 8b .. 8b + 7 (128 bytes each); lane l
    // fetches logical chunk (l % 8) ^ swz(row) of row 8b + l / 8
    uint32_t offx[DMA_PER_WAVE], offw[DMA_PER_WAVE];
    int lchunk[DMA_PER_WAVE];
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
        const int row = (wave * DMA_PER_WAVE + i) * 8 + lane / 8;
        lchunk[i] = (lane % 8) ^ swz(row);
        offx[i] = (uint32_t)((int64_t)row * a.ldx + lchunk[i] * 16);
        offw[i] = (uint32_t)((int64_t)row * a.ldw + lchunk[i] * 16);
    }
    auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
        const int k0 = kt * BK8;
        const bool tail = k0 + BK8 > a.K;
        const __amdgpu_buffer_rsrc_t rw = uniform_rsrc(a.w + (int64_t)n0 * a.ldw + k0, (int64_t)rows_w * a.ldw - k0);
        const __amdgpu_buffer_rsrc_t rx = uniform_rsrc(a.x + (int64_t)m0 * a.ldx + k0, (int64_t)rows_x * a.ldx - k0);
        lds_char_t* dst = lds + stage * STAGE_B;
#pragma unroll
        for (int i = 0; i < DMA_PER_WAVE; ++i) {
            const int blk = wave * DMA_PER_WAVE + i;
            const bool oob = tail && (k0 + lchunk[i] * 16 >= a.K);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)(dst + blk * 1024), 16,
                                                     oob ? kOob : offw[i], 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(dst + TILE_B + blk * 1024), 16,
                                                     oob ? kOob : offx[i], 0, 0, 0);
        }
    };

    // operand addresses: slice ks (bytes 64 ks .. 64 ks + 63 of the K step),
    // part q: logical chunk 4 ks + 2 half + q of row block*32 + r32
    uint32_t waddr[2][2], xaddr[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t base = (uint32_t)(uintptr_t)lds + r32 * ROWB + (((ks * 4 + half * 2 + q) ^ swz(r32)) * 16);
            waddr[ks][q] = base + wn * 128 * ROWB;
            xaddr[ks][q] = base + wm * 128 * ROWB;
        }

    f32x16_t acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // reads of slice ks: W blocks (f[0..7] = block i, part q at 2i + q), then
    // X blocks (f[8..15])
    auto read_w = [&](uint32_t soff, auto KSc, u32x4_t (&f)[16]) __attribute__((always_inline)) {
        constexpr int ks = decltype(KSc)::value;
        static_for<FN>([&](auto Ic) {
            constexpr int i = decltype(Ic)::value;
            f[2 * i] = lds_read_b128<i * 32 * ROWB>(waddr[ks][0] + soff);
            f[2 * i + 1] = lds_read_b128<i * 32 * ROWB>(waddr[ks][1] + soff);
        });
    };
    auto read_x = [&](uint32_t soff, auto KSc, u32x4_t (&f)[16]) __attribute__((always_inline)) {
        constexpr int ks = decltype(KSc)::value;
        static_for<FM>([&](auto Jc) {
            constexpr int j = decltype(Jc)::value;
            f[8 + 2 * j] = lds_read_b128<TILE_B + j * 32 * ROWB>(xaddr[ks][0] + soff);
            f[8 + 2 * j + 1] = lds_read_b128<TILE_B + j * 32 * ROWB>(xaddr[ks][1] + soff);
        });
    };
    // the 16 MFMAs of a slice in two halves (W blocks 0-1, then 2-3)
    auto mfmas = [&](auto Hc, const u32x4_t (&f)[16]) __attribute__((always_inline)) {
        constexpr int h = decltype(Hc)::value;
        static_for<8>([&](auto Ic) {
            constexpr int i = h * 2 + decltype(Ic)::value / FM, j = decltype(Ic)::value % FM;
            acc[i][j] = mfma_f8(f[2 * i], f[2 * i + 1], f[8 + 2 * j], f[8 + 2 * j + 1], acc[i][j]);
        });
        // the products' next use is past the barrier and the loop's branches;
        // an asm that reads them keeps the compiler from sinking these MFMAs
        // down to it (they would then no longer overlap the operand reads)
#pragma unroll
        for (int q = 0; q < 8; ++q) asm volatile("" ::"a"(acc[h * 2 + q / FM][q % FM]));
        __builtin_amdgcn_sched_barrier(0);
    };
    using KS0 = std::integral_constant<int, 0>;
    using KS1 = std::integral_constant<int, 1>;
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;

    issue(0, 0);
    if (1 < nk) issue(1, 1);
    if (1 < nk) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * DMA_PER_WAVE));   // step 0 only
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    wg_barrier();
    u32x4_t f0[16], f1[16];
    read_w(0u, KS0{}, f0);
    read_x(0u, KS0{}, f0);
    lds_wait16<0>(f0);
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        const uint32_t soff = (uint32_t)(st * STAGE_B);
        // slice 0 on the matrix cores, slice 1's operands read in between
        mfmas(H0{}, f0);
        read_w(soff, KS1{}, f1);
        mfmas(H1{}, f0);
        read_x(soff, KS1{}, f1);
        lds_wait16<0>(f1);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // this wave's loads of step kt + 1
        wg_barrier();
        // slice 1 on the matrix cores, the next step's slice 0 read in between
        mfmas(H0{}, f1);
        if (kt + 1 < nk) read_w(soff ^ (uint32_t)STAGE_B, KS0{}, f0);
        if (kt + 2 < nk) issue(kt + 2, st);
        mfmas(H1{}, f1);
        if (kt + 1 < nk) read_x(soff ^ (uint32_t)STAGE_B, KS0{}, f0);
        lds_wait16<0>(f0);
    }

    // epilogue: y = sx[m] * sw[n] * acc, rounded once, staged through LDS and
    // written as full rows (as in the bf16 GEMM)
    wg_barrier();
    lds_char_t* stg = lds + wave * (128 * 256);
    const int m_lo = m0 + wm * 128;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int m = m_lo + j * 32 + r32;
        const float sxm = m < a.M ? a.sx[m] : 0.0f;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int nn = n0 + wn * 128 + i * 32 + g * 8 + half * 4;
                float t[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] = acc[i][j][g * 4 + e] * sxm * (nn + e < a.N ? a.sw[nn + e] : 0.0f);
                const int ml = j * 32 + r32, ci = i * 4 + g;
                *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>(
                    stg + ml * 256 + ((ci ^ (ml & 15)) * 16) + half * 8) = u32x2_t{pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3])};
            }
    }
    const int c = lane & 15;
    const int n = n0 + wn * 128 + c * 8;
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
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
    static const hipError_t attr = hipFuncSetAttribute((const void*)gemm_fp8_kernel,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (attr != hipSuccess) return attr;
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    hipLaunchKernelGGL(gemm_fp8_kernel, dim3(tiles), dim3(kThreads), LDS_BYTES, s, a);
    return hipGetLastError();
}

hipError_t launch_quantize_rows(const uint16_t* x, int64_t ldx, int M, int K, uint8_t* q, int64_t ldq, float* scales,
                                hipStream_t s) {
    hipLaunchKernelGGL(quantize_rows_kernel, dim3((uint32_t)((M + 3) / 4)), dim3(256), 0, s, x, ldx, M, K, q, ldq,
                       scales);
    return hipGetLastError();
}

}  // namespace pca
