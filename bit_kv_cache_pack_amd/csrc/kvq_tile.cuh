// Dequantization of one (token, 16-channel block) unit of a packed cache row, and the
// small lane helpers both attention kernels use (gfx950).
//
// Dequantized value of code c with the fp16 {step, zero} of its group:
//   x = E(fl32(c * step + zero)),  E = round to the element dtype (bf16 or fp16),
// c * step is exact in fp32 (c <= 15, step has 11 significant bits), so one fused
// multiply-add rounds once, as the plain mul-then-add would.
//
// Inside a 16-channel block, values are emitted in "position" order: position 4j + k
// holds channel 4k + j (a 4x4 transpose, an involution). That is the order in which
// INT2 codes fall out of a word when it is shifted by 2j and masked per byte, and the
// order the attention kernels keep in LDS and in their MFMA operands; Q is loaded in the
// same order and O is written back in channel order.
#pragma once

#include "kvq_device.cuh"

namespace kvq {

// position <-> channel inside a 16-channel block: p = 4j + k  <->  c = 4k + j
__device__ __forceinline__ int swap_pos(int c) { return (c & ~15) | ((c & 3) << 2) | ((c >> 2) & 3); }

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}
// a * (fp16 in the low half of m) + (fp16 in the high half of m), one rounding in fp32
__device__ __forceinline__ float fma_mix(float a, uint32_t m) {
    const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)(m & 0xffffu));
    const _Float16 z = __builtin_bit_cast(_Float16, (uint16_t)(m >> 16));
    return __builtin_fmaf(a, (float)s, (float)z);
}
// a * (fp16 in the low half of m)
__device__ __forceinline__ float mul_step(float a, uint32_t m) {
    return a * (float)__builtin_bit_cast(_Float16, (uint16_t)(m & 0xffffu));
}
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// Entry g of a K-group table, read through a global-address-space pointer. Through a
// generic pointer the read could be private memory, which makes its value (and every
// walker decision taken from it) per-lane; as a global read of a uniform address it is
// uniform, and with no global store before the kernels' epilogues it can be a scalar load.
__device__ __forceinline__ int group_start(const int32_t *tab, int g) {
    typedef const __attribute__((address_space(1))) int32_t *gptr;
    return ((gptr)tab)[g];
}
// log2(sinh(a) / a) for a >= 0: the all-orders Jensen term of one key channel whose
// logit noise is uniform on [-a, a] (E[exp(x)] = sinh(a) / a). Below a = 1 from the Taylor
// series of ln(sinh a / a) in u = a^2 (six terms, the seventh below 1.6e-8); from 1 on as
// a - ln(2a) + ln(1 - e^{-2a}), where nothing cancels. The second form is only evaluated
// when some lane of the wave needs it.
__device__ __forceinline__ float log2_sinhc(float a) {
    constexpr float kLog2e = 1.4426950408889634f;
    const float u = a * a;
    float f = __builtin_fmaf(u, -1.80366e-7f, 2.1377799e-6f);   // -2^12 B12 / (12 * 12!), 1/467775
    f = __builtin_fmaf(u, f, -2.6455026e-5f);                  // -1/37800
    f = __builtin_fmaf(u, f, 3.5273369e-4f);                   // 1/2835
    f = __builtin_fmaf(u, f, -5.5555556e-3f);                  // -1/180
    f = __builtin_fmaf(u, f, 0.16666667f);                     // 1/6
    f = f * u * kLog2e;
    const bool big = a >= 1.0f;
    if (__builtin_expect(__any(big), 0)) {
        const float x = a * kLog2e;
        const float t = __builtin_amdgcn_exp2f(-2.0f * x);     // e^{-2a}
        const float g = x - 1.0f - __builtin_amdgcn_logf(a) + __builtin_amdgcn_logf(1.0f - t);
        f = big ? g : f;
    }
    return f;
}

// value of lane L ^ 32
__device__ __forceinline__ float other_half(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

template <bool BF16> struct Elem;
template <> struct Elem<true> {
    typedef bf16x8 vec;
    static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_bf16x2(a, b); }
    // element-dtype rounding of two values, returned as the fp16 pair the PV product uses
    static __device__ __forceinline__ uint32_t pack_v(float a, float b) { return bf16x2_to_f16x2(pack_bf16x2(a, b)); }
    static __device__ __forceinline__ uint32_t raw_to_f16(uint32_t p) { return bf16x2_to_f16x2(p); }
    static __device__ __forceinline__ f32x16 mma(vec a, vec b, f32x16 c) { return mfma32_bf16(a, b, c); }
    static __device__ __forceinline__ f32x4 mma16(vec a, vec b, f32x4 c) { return mfma16_bf16(a, b, c); }
    static __device__ __forceinline__ float val(uint32_t bits16) { return bf16_bits_to_f32(bits16); }
};
template <> struct Elem<false> {
    typedef f16x8 vec;
    static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_f16x2(a, b); }
    static __device__ __forceinline__ uint32_t pack_v(float a, float b) { return pack_f16x2(a, b); }
    static __device__ __forceinline__ uint32_t raw_to_f16(uint32_t p) { return p; }
    static __device__ __forceinline__ f32x16 mma(vec a, vec b, f32x16 c) { return mfma32_f16(a, b, c); }
    static __device__ __forceinline__ f32x4 mma16(vec a, vec b, f32x4 c) { return mfma16_f16(a, b, c); }
    static __device__ __forceinline__ float val(uint32_t bits16) { return f16_bits_to_f32(bits16); }
};

// 16 raw 16-bit values of one block in channel order (dword m = channels 2m, 2m+1) to
// position order.
__device__ __forceinline__ void to_positions(const uint32_t (&d)[8], uint32_t (&o)[8]) {
    // positions (4j, 4j+1) = channels (j, 4+j); (4j+2, 4j+3) = channels (8+j, 12+j)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        o[2 * j] = perm(d[2 + j / 2], d[j / 2], sel);
        o[2 * j + 1] = perm(d[6 + j / 2], d[4 + j / 2], sel);
    }
}

// Two codes (bytes 0,1 or, with HI, bytes 2,3 of x; each 0..15) as exact floats: bytes
// 0..15 read as OCP e4m3 are c * 2^-9 (subnormals up to 7, then 1.mmm * 2^-6), and the
// conversion scales them back by 2^9.
template <bool HI>
__device__ __forceinline__ float2 codes2(uint32_t x) {
    const auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x, 512.0f, HI);
    return float2{r[0], r[1]};
}

// Keys, INT2: word w holds the block's 16 codes (channel c at bits 2c); km[c] is the
// {step, zero} of channel c. Step j (0..3) emits position pairs 2j, 2j+1 (channels j,
// 4+j and 8+j, 12+j) of the 8 element-dtype pairs, position order.
template <bool BF16>
__device__ __forceinline__ void k2_step(uint32_t w, const uint32_t *km, int j, uint32_t (&ko)[8]) {
    typedef Elem<BF16> E;
    const uint32_t x = (w >> (2 * j)) & 0x03030303u;   // bytes: channels j, 4+j, 8+j, 12+j
    const float2 a = codes2<false>(x), b = codes2<true>(x);
    ko[2 * j] = E::pack(fma_mix(a.x, km[j]), fma_mix(a.y, km[4 + j]));
    ko[2 * j + 1] = E::pack(fma_mix(b.x, km[8 + j]), fma_mix(b.y, km[12 + j]));
}
template <bool BF16>
__device__ __forceinline__ void k2_block(uint32_t w, const uint32_t *km, uint32_t (&ko)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) k2_step<BF16>(w, km, j, ko);
}
// Keys, INT4: w0 holds channels 0..7, w1 channels 8..15 (channel c at bits 4 (c mod 8)).
// Step jj (0..1) emits pairs 2jj, 2jj+1, 2jj+4, 2jj+5.
template <bool BF16>
__device__ __forceinline__ void k4_step(uint32_t w0, uint32_t w1, const uint32_t *km, int jj, uint32_t (&ko)[8]) {
    typedef Elem<BF16> E;
    // bytes of x0: channels jj, 2+jj, 4+jj, 6+jj; of x1: the same plus 8
    const uint32_t x0 = (w0 >> (4 * jj)) & 0x0f0f0f0fu, x1 = (w1 >> (4 * jj)) & 0x0f0f0f0fu;
    const float2 a0 = codes2<false>(x0), b0 = codes2<true>(x0);
    const float2 a1 = codes2<false>(x1), b1 = codes2<true>(x1);
    ko[2 * jj] = E::pack(fma_mix(a0.x, km[jj]), fma_mix(b0.x, km[4 + jj]));
    ko[2 * jj + 1] = E::pack(fma_mix(a1.x, km[8 + jj]), fma_mix(b1.x, km[12 + jj]));
    ko[2 * jj + 4] = E::pack(fma_mix(a0.y, km[2 + jj]), fma_mix(b0.y, km[6 + jj]));
    ko[2 * jj + 5] = E::pack(fma_mix(a1.y, km[10 + jj]), fma_mix(b1.y, km[14 + jj]));
}
template <bool BF16>
__device__ __forceinline__ void k4_block(uint32_t w0, uint32_t w1, const uint32_t *km, uint32_t (&ko)[8]) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) k4_step<BF16>(w0, w1, km, jj, ko);
}

// Values, INT2: the 4 possible dequantized values of a (token, V group) as fp16 (after
// rounding to the element dtype), split into a table of low bytes and one of high bytes.
template <bool BF16>
__device__ __forceinline__ void v_int2_table(uint32_t vmeta, uint32_t &tlo, uint32_t &thi) {
    typedef Elem<BF16> E;
    const uint32_t p01 = E::pack_v(fma_mix(0.0f, vmeta), fma_mix(1.0f, vmeta));
    const uint32_t p23 = E::pack_v(fma_mix(2.0f, vmeta), fma_mix(3.0f, vmeta));
    tlo = perm(p23, p01, 0x06040200u);
    thi = perm(p23, p01, 0x07050301u);
}
// Values, INT2: one word of 16 codes through the table; code c selects byte c of the
// low table and byte c of the high table (selector c + 4). Step j emits fp16 pairs 2j,
// 2j+1, position order.
__device__ __forceinline__ void v_int2_step(uint32_t w, uint32_t tlo, uint32_t thi, int j, uint32_t (&vo)[8]) {
    const uint32_t x = (w >> (2 * j)) & 0x03030303u;
    const uint32_t x4 = x | 0x04040404u;
    vo[2 * j] = perm(thi, tlo, perm(x4, x, 0x05010400u));
    vo[2 * j + 1] = perm(thi, tlo, perm(x4, x, 0x07030602u));
}
__device__ __forceinline__ void v_int2_block(uint32_t w, uint32_t tlo, uint32_t thi, uint32_t (&vo)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v_int2_step(w, tlo, thi, j, vo);
}
// Values, INT4, one block with one {step, zero}: fp16 pairs in position order; step jj
// emits pairs 2jj, 2jj+1, 2jj+4, 2jj+5.
template <bool BF16>
__device__ __forceinline__ void v4_step(uint32_t w0, uint32_t w1, uint32_t vm, int jj, uint32_t (&vo)[8]) {
    typedef Elem<BF16> E;
    const uint32_t x0 = (w0 >> (4 * jj)) & 0x0f0f0f0fu, x1 = (w1 >> (4 * jj)) & 0x0f0f0f0fu;
    const float2 a0 = codes2<false>(x0), b0 = codes2<true>(x0);
    const float2 a1 = codes2<false>(x1), b1 = codes2<true>(x1);
    vo[2 * jj] = E::pack_v(fma_mix(a0.x, vm), fma_mix(b0.x, vm));
    vo[2 * jj + 1] = E::pack_v(fma_mix(a1.x, vm), fma_mix(b1.x, vm));
    vo[2 * jj + 4] = E::pack_v(fma_mix(a0.y, vm), fma_mix(b0.y, vm));
    vo[2 * jj + 5] = E::pack_v(fma_mix(a1.y, vm), fma_mix(b1.y, vm));
}
template <bool BF16>
__device__ __forceinline__ void v4_block(uint32_t w0, uint32_t w1, uint32_t vm, uint32_t (&vo)[8]) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) v4_step<BF16>(w0, w1, vm, jj, vo);
}

}  // namespace kvq
