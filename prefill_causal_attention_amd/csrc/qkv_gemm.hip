// Fused QKV projection: y[M, N] = x[M, K] * w[N, K]^T (bf16 in, fp32 accumulate,
// bf16 RNE out).
//
// One GEMM with the Q, K and V weights concatenated, so the activation is read
// from HBM once (prefill data-flow article (hncyxsy.com/news/270449) §2.1 and
// §4.1); the weight arrives pre-transposed to (N, K) so both operands are read
// along K (§5.1).
//
// gfx950 design.  Workgroup tile 256 x 256 (M x N), K step 64, four waves in a
// 2 x 2 grid, each wave a 128 x 128 sub-tile of 4 x 4 v_mfma_f32_32x32x16_bf16
// blocks (256 fp32 accumulators per lane).  The wave computes the transposed
// product (rows = n, columns = m), so each lane's accumulator holds 4
// consecutive n of one m: the epilogue writes 8-byte runs of a y row.  Tiles
// are staged in LDS with a 16-byte row pad (rows 144 B apart: 16 consecutive
// rows start on 16 distinct 4-bank groups, so the 16-byte operand reads do not
// conflict), double-buffered: the next K step's global loads are in flight in
// registers while the current step runs on the matrix cores.  Ragged M, N and
// K tails read zeros through buffer-resource range checks.
//
// Tile order: consecutive workgroup ids go round-robin to the 8 XCDs, so the
// id is first remapped so that each XCD owns one contiguous range of tiles,
// which is then walked in groups of 8 M-tiles: the tiles resident on one XCD
// at a time share A rows and B columns in that XCD's L2.
#include "pca_device.hpp"
#include "pca_internal.hpp"

namespace pca {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int WTM = 128, WTN = 128;           // wave tile (m, n)
constexpr int FM = WTM / 32, FN = WTN / 32;   // 32x32 blocks per wave
constexpr int ROW = BK + 8;                   // LDS row stride in elements (144 B)
constexpr int A_ELEMS = BM * ROW;
constexpr int B_ELEMS = BN * ROW;
constexpr int STAGE = A_ELEMS + B_ELEMS;
constexpr int CHUNKS_PER_ROW = BK / 8;        // 16-byte chunks per tile row
constexpr int A_LOADS = BM * CHUNKS_PER_ROW / kThreads;   // 8
constexpr int B_LOADS = BN * CHUNKS_PER_ROW / kThreads;   // 8
constexpr int kGroupM = 8;
constexpr uint32_t kOob = 0x80000000u;        // an offset past every buffer: loads return 0

__device__ inline void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
    int total = tiles_m * tiles_n;
    int id = blockIdx.x;
    if (total % kNumXcd == 0) id = (id % kNumXcd) * (total / kNumXcd) + id / kNumXcd;
    int per_group = kGroupM * tiles_n;
    int group = id / per_group;
    int first_m = group * kGroupM;
    int gsize = min(tiles_m - first_m, kGroupM);
    int in_group = id - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void qkv_gemm_kernel(GemmArgs a) {
    extern __shared__ __align__(16) uint16_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;     // wave position in the 2 x 2 grid

    int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // buffer views start at the tile's first row; rows past M (N) read 0
    const int rows_a = min(BM, a.M - m0), rows_b = min(BN, a.N - n0);
    __amdgpu_buffer_rsrc_t ra = make_rsrc(a.x + (int64_t)m0 * a.ldx, (uint32_t)((int64_t)(rows_a - 1) * a.ldx * 2 + (int64_t)a.K * 2));
    __amdgpu_buffer_rsrc_t rb = make_rsrc(a.w + (int64_t)n0 * a.ldw, (uint32_t)((int64_t)(rows_b - 1) * a.ldw * 2 + (int64_t)a.K * 2));

    // per-thread load coordinates: chunk id = i*256 + tid -> (row, chunk)
    int ld_row[A_LOADS], ld_col[A_LOADS];
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
        int id = i * kThreads + tid;
        ld_row[i] = id / CHUNKS_PER_ROW;
        ld_col[i] = (id % CHUNKS_PER_ROW) * 8;
    }

    u32x4_t stage_a[A_LOADS], stage_b[B_LOADS];
    auto global_load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            int kk = k0 + ld_col[i];
            uint32_t off = (ld_row[i] < rows_a && kk < a.K) ? (uint32_t)(((int64_t)ld_row[i] * a.ldx + kk) * 2) : kOob;
            stage_a[i] = buf_load16(ra, off);
        }
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) {
            int kk = k0 + ld_col[i];
            uint32_t off = (ld_row[i] < rows_b && kk < a.K) ? (uint32_t)(((int64_t)ld_row[i] * a.ldw + kk) * 2) : kOob;
            stage_b[i] = buf_load16(rb, off);
        }
    };
    auto lds_store = [&](int st) {
        uint16_t* sa = smem + st * STAGE;
        uint16_t* sb = sa + A_ELEMS;
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i)
            *reinterpret_cast<u32x4_t*>(sa + ld_row[i] * ROW + ld_col[i]) = stage_a[i];
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i)
            *reinterpret_cast<u32x4_t*>(sb + ld_row[i] * ROW + ld_col[i]) = stage_b[i];
    };

    f32x16_t acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int nk = (a.K + BK - 1) / BK;
    global_load(0);
    lds_store(0);
    __syncthreads();

    const int r32 = lane & 31, half = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < nk) global_load((kt + 1) * BK);
        const uint16_t* sa = smem + st * STAGE;
        const uint16_t* sb = sa + A_ELEMS;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8_t fa[FM], fb[FN];
#pragma unroll
            for (int j = 0; j < FM; ++j)
                fa[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(sa + (wm * WTM + j * 32 + r32) * ROW + ks * 16 + half * 8));
#pragma unroll
            for (int i = 0; i < FN; ++i)
                fb[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(sb + (wn * WTN + i * 32 + r32) * ROW + ks * 16 + half * 8));
            // transposed product: MFMA rows come from w (n), columns from x (m)
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) acc[i][j] = mfma32x32x16(fb[i], fa[j], acc[i][j]);
        }
        if (kt + 1 < nk) lds_store(st ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds, per block, column m = r32 and rows n = g*8 + half*4 + 0..3
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int m = m0 + wm * WTM + j * 32 + r32;
            if (m >= a.M) continue;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WTN + i * 32 + g * 8 + half * 4;
                uint16_t* dst = a.y + (int64_t)m * a.ldy + n;
                if (n + 3 < a.N) {
                    u32x2_t w2 = {pack_bf16x2(acc[i][j][g * 4 + 0], acc[i][j][g * 4 + 1]),
                                  pack_bf16x2(acc[i][j][g * 4 + 2], acc[i][j][g * 4 + 3])};
                    *reinterpret_cast<u32x2_t*>(dst) = w2;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < a.N) dst[e] = (uint16_t)(pack_bf16x2(acc[i][j][g * 4 + e], 0.0f) & 0xFFFFu);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_qkv_gemm(const GemmArgs& a, hipStream_t s) {
    static bool configured = false;
    const size_t lds = 2 * STAGE * sizeof(uint16_t);
    if (!configured) {
        hipError_t e = hipFuncSetAttribute((const void*)qkv_gemm_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        configured = true;
    }
    int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    hipLaunchKernelGGL(qkv_gemm_kernel, dim3(tiles), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace pca
