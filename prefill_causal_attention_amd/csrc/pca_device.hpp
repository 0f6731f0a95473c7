// Device-side helpers shared by the gfx950 kernels of libpca.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pca {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;   // MI355X: 8 XCDs, workgroups dispatched round-robin over them

// Raw buffer resource over [base, base + bytes): loads past the end return 0,
// which gives ragged tiles zero fill without branches.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ inline u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

__device__ inline u32x2_t buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t v = {lo, hi};
    bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ inline float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

__device__ inline bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ inline f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// OCP E4M3 codes of four binary32 values packed into a word (byte j holds the
// code of the j-th argument): round to nearest even, finite overflow
// saturating to +-448, the sign copied (so -0 gives 0x80).  gfx950's
// conversion instruction rounds to nearest even but turns magnitudes above 464
// into NaN, so each value is first clamped to [-448, 448]; values in
// (448, 464] round to 448 either way, which makes the pair saturating over
// every finite input.  NaN inputs are outside the contract.
__device__ inline uint32_t e4m3x4(float a, float b, float c, float d) {
    const auto cl = [](float x) { return __builtin_amdgcn_fmed3f(x, -448.0f, 448.0f); };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
    return (uint32_t)w;
}

// Power-of-two scale of an fp8 operand row: the smallest e in [-127, 127]
// with amax * 2^-e <= 448 = 1.75 * 2^8, from amax's bit pattern (a
// non-negative finite binary32).  amax = 1.m * 2^E fits 448 * 2^(E-8) when
// 1.m <= 1.75, else needs 2^(E-7); a zero or subnormal amax takes -127.
__device__ inline int pow2_exponent(uint32_t amax_bits) {
    if (amax_bits < 0x00800000u) return -127;
    const int E = (int)(amax_bits >> 23) - 127;
    const int e = (amax_bits & 0x7FFFFFu) <= 0x600000u ? E - 8 : E - 7;
    return e < -127 ? -127 : e;
}

// For every lane l: lo = v of lane l % 32, hi = v of lane l % 32 + 32.
// v_permlane32_swap exchanges the upper 32 lanes of one register with the
// lower 32 lanes of another in the VALU, so this needs no LDS round trip
// (a ds_bpermute would queue behind other waves' LDS traffic).  The nops
// cover the VALU-write -> permlane-read and permlane -> VALU-read hazards.
__device__ inline void both_halves(float v, float& lo, float& hi) {
    float a = v, b = v;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    lo = a;   // [v_lo | v_lo]
    hi = b;   // [v_hi | v_hi]
}

}  // namespace pca
