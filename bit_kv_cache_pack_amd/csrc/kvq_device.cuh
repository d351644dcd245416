// Device-side types and helpers shared by the libkvq kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
// kvq_jensen values the kernels branch on
enum : int { JENSEN_ISO = 2, JENSEN_EXACT = 3 };

constexpr int kWave = 64;

// ---- scalar conversions (round to nearest even, hardware converts on gfx950) ----
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
    return (float)v;
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}
// two floats -> packed pair {lo, hi}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 r;
    r.x = (__bf16)lo;
    r.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f16x2 r;
    r.x = (_Float16)lo;
    r.y = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, r);
}
// packed bf16 pair -> packed fp16 pair, exact for values inside fp16's normal range
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t p) {
    float lo = __uint_as_float(p << 16), hi = __uint_as_float(p & 0xffff0000u);
    return pack_f16x2(lo, hi);
}

// Load one element of a tensor of runtime dtype as float (exact).
__device__ __forceinline__ float load_elem(const void *base, int dtype, size_t idx) {
    if (dtype == DT_F32) return reinterpret_cast<const float *>(base)[idx];
    uint32_t b = reinterpret_cast<const uint16_t *>(base)[idx];
    return dtype == DT_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

// ---- MFMA wrappers (wave64) ----
// 32x32x16: A lane L holds A[L%32][8*(L/32)+0..7], B lane L holds B[8*(L/32)+0..7][L%32],
// C lane L holds C[8*(j/4) + 4*(L/32) + j%4][L%32] for j = 0..15.
__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f16(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// 16x16x32: A lane L holds A[L%16][8*(L/16)+0..7], B lane L holds B[8*(L/16)+0..7][L%16],
// C lane L holds C[4*(L/16) + j][L%16] for j = 0..3.
__device__ __forceinline__ f32x4 mfma16_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_f16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace kvq
