// Quantize-append of one K-group, as a device function: the arithmetic of
// kvq_quantize_append, shared by its own kernel (quant.hip) and by the attention kernel,
// whose launch can quantize the current chunk into the cache on CUs the attention leaves
// idle (attention.hip).
//
// Method: "Quantized Keys Steal Attention: Bias Correction for KV-Cache Compression in
// Video Diffusion" (abstract: a KV cache of earlier chunks, quantized to low bit-widths,
// read through the cached keys' quantization step sizes) and the WindowQuant notes
// ("技術的に面白い点": windows of one bit-width stored together, here via gather lists).
// The pages give no quantizer formula; the one used is plain min/max asymmetric
// quantization:
//   step = fp16(fl32(max - min) / L), zero = fp16(min),
//   code = clamp(rint(fl32(x - zero) / step), 0, L), 0 when step == 0,
// with IEEE fp32 division and no contraction (every file that includes this one is built
// with -ffp-contract=off), so codes are reproducible bit for bit.
//
// A workgroup quantizes one K-group (<= k_group_tokens tokens) of one (batch, head):
// the K statistics run down the group's tokens per channel, the V statistics across
// each token's 32-channel runs (quant_group); the append kernel gives the keys and the
// values of a K-group to two workgroups (quant_group_part).
#pragma once

#include <type_traits>

#include "kvq_device.cuh"
#include "kvq_internal.h"

namespace kvq {
namespace qz {

constexpr int kBatch1 = 8;   // rows per thread in flight while the K extremes are taken
constexpr int kBatch2 = 4;   // rows per thread in flight while codes are made

// 8 consecutive source elements starting at p (16-byte aligned): load() fetches them as
// stored, unpack() widens them to fp32.
template <typename T> struct Src;
template <> struct Src<float> {
    struct Raw { f32x4 a, b; };
    static __device__ __forceinline__ Raw load(const float *p) {
        return Raw{*reinterpret_cast<const f32x4 *>(p), *reinterpret_cast<const f32x4 *>(p + 4)};
    }
    static __device__ __forceinline__ void unpack(const Raw &r, float (&x)[8]) {
        x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
        x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
    }
};
template <> struct Src<__bf16> {
    typedef u32x4 Raw;
    static __device__ __forceinline__ Raw load(const __bf16 *p) { return *reinterpret_cast<const u32x4 *>(p); }
    static __device__ __forceinline__ void unpack(const Raw &w, float (&x)[8]) {
        const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(a[i] << 16);
            x[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
        }
    }
};
template <> struct Src<_Float16> {
    typedef u32x4 Raw;
    static __device__ __forceinline__ Raw load(const _Float16 *p) { return *reinterpret_cast<const u32x4 *>(p); }
    static __device__ __forceinline__ void unpack(const Raw &w, float (&x)[8]) {
        const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = f16_bits_to_f32(a[i] & 0xffffu);
            x[2 * i + 1] = f16_bits_to_f32(a[i] >> 16);
        }
    }
};

// step/zero of a group from its extremes, and the code of one element.
struct Quant {
    float step, zero;
    uint32_t meta;  // fp16 step in the low half, fp16 zero in the high half
    __device__ __forceinline__ void set(float mn, float mx, int L) {
        mn = mn + 0.0f;  // -0 -> +0: the extremes of a group are taken as signless zeros
        mx = mx + 0.0f;
        float range = mx - mn;
        float step32 = range / (float)L;
        uint16_t sh = f32_to_f16_bits(step32);
        uint16_t zh = f32_to_f16_bits(mn);
        step = f16_bits_to_f32(sh);
        zero = f16_bits_to_f32(zh);
        meta = (uint32_t)sh | ((uint32_t)zh << 16);
    }
    __device__ __forceinline__ uint32_t code(float x, int L) const {
        if (step == 0.0f) return 0u;
        float t = (x - zero) / step;
        float r = __builtin_rintf(t);
        r = fminf(fmaxf(r, 0.0f), (float)L);
        return (uint32_t)r;
    }
    // 1 / step within 1 ulp (the hardware reciprocal; step is a normal fp32 number), 0 for
    // a zero step (whose codes are all 0)
    __device__ __forceinline__ float inv() const { return step == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(step); }
};

// The same code through the reciprocal, without a division per element. With r within
// 1 ulp (2^-23 relative) of 1/step, t' = fl32(fl32(x - zero) r) is within 2^-22 |t| of
// the IEEE quotient t = fl32(fl32(x - zero) / step) (r's error plus one rounding of the
// product and one of t, 2^-24 each), i.e. within 2^-18 for |t| < 16, so
// rint(t') == rint(t) unless t' lies within 2^-17 of a half-integer; such elements raise
// `near` and the caller recomputes with the division. For |t| >= 16 both clamp to the same
// end of [0, L] (L <= 15).
// A zero step gives r = 0, t' = 0, code 0, as the division path does. The code comes
// back as a float (an integer 0..L).
__device__ __forceinline__ float fast_code(float x, float zero, float r, int L, bool &near) {
    const float t = (x - zero) * r;
    const float c = __builtin_rintf(t);
    near |= __builtin_fabsf(t - c) > 0.5f - 0x1p-17f;
    return __builtin_amdgcn_fmed3f(c, 0.0f, (float)L);
}

// Packs 8 codes at BITS bits each (code i at bit BITS i). The codes are summed as exact
// floats, c_i 2^(BITS i) over at most 16 bits per sum, and converted once.
template <int BITS>
__device__ __forceinline__ uint32_t pack_codes(const float (&c)[8]) {
    constexpr int PER = 16 / BITS;   // codes per 16-bit sum
    uint32_t w = 0;
#pragma unroll
    for (int h = 0; h < 8 / PER; ++h) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < PER; ++i) acc = __builtin_fmaf(c[h * PER + i], (float)(1u << (BITS * i)), acc);
        w |= (uint32_t)acc << (16 * h);
    }
    return w;
}

// value of the lane whose index differs in bit 0 (XOR1) or bit 1 (XOR2), within a quad
__device__ __forceinline__ float quad_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false));
}
__device__ __forceinline__ float quad_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xf, 0xf, false));
}
__device__ __forceinline__ uint32_t quad_xor1(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, false);
}

// Source span and destination offset of appended group g. Contiguous appends cut
// the source into k_group_tokens-long groups; gather appends take the listed spans in
// order (entries clamped so every access stays inside the buffers). Uniform per block.
template <int NT>
__device__ __forceinline__ void group_span(const QuantAppendParams &p, int g, int &src0, int &len,
                                           int &dst0) {
    if (p.src_groups == nullptr) {
        src0 = g * p.k_group_tokens;
        len = min(p.k_group_tokens, p.n_new - src0);
        dst0 = src0;
        return;
    }
    __shared__ int s_red[NT / kWave];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    int part = 0;
    for (int i = tid; i < g; i += NT)
        part += min(max(p.src_groups[2 * i + 1], 0), p.k_group_tokens);
    for (int o = kWave / 2; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if (lane == 0) s_red[wave] = part;
    __syncthreads();
    dst0 = 0;
    for (int w = 0; w < NT / kWave; ++w) dst0 += s_red[w];
    src0 = min(max(p.src_groups[2 * g], 0), (int)max(p.src_tokens - 1, (int64_t)0));
    len = min(max(p.src_groups[2 * g + 1], 0), p.k_group_tokens);
    len = (int)min((int64_t)len, p.src_tokens - src0);
    len = min(len, p.n_new - dst0);
}

// Codes of one row's 8 channels of V (a quad holds one 32-channel group) and their
// store. Rows past the group end (r >= len) are clamped copies: computed, not stored.
// Called by whole quads in uniform control flow.
template <int HD, int BITS>
__device__ __forceinline__ void v_row(const float (&y)[8], int r, int len, int cc, uint32_t *vcodes,
                                      uint32_t *vm_base) {
    constexpr int L = (1 << BITS) - 1;
    constexpr int WPR = HD * BITS / 32;
    constexpr int VG = 32;
    float a = y[0], z = y[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) { a = fminf(a, y[i]); z = fmaxf(z, y[i]); }
    a = fminf(a, quad_xor1(a)); z = fmaxf(z, quad_xor1(z));
    a = fminf(a, quad_xor2(a)); z = fmaxf(z, quad_xor2(z));
    Quant vq;
    vq.set(a, z, L);
    const float vinv = vq.inv();
    bool near = false;
    float vc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) vc[i] = fast_code(y[i], vq.zero, vinv, L, near);
    uint32_t vbits = pack_codes<BITS>(vc);
    if (__builtin_expect(__any(near), 0)) {
        vbits = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) vbits |= vq.code(y[i], L) << (BITS * i);
    }
    // 16 channels per INT2 word: the even chunk takes its odd neighbour's half
    const uint32_t vn = quad_xor1(vbits);
    if (r < len) {
        if ((cc & 3) == 0) vm_base[(size_t)r * (HD / VG) + cc / 4] = vq.meta;
        if (BITS == 4) vcodes[(size_t)r * WPR + cc] = vbits;
        else if ((cc & 1) == 0) vcodes[(size_t)r * WPR + cc / 2] = vbits | (vn << 16);
    }
}

// value of the lane whose index differs in bit 2 or bit 3 (the 8-channel chunks of a row
// are consecutive lanes)
__device__ __forceinline__ float lane_xor(float v, int m) { return __shfl_xor(v, m); }

// Codes of one row's 8 channels of K with per-token groups of GW channels (GW / 8 lanes of
// the row share a group), their step/zero, and the store. As v_row, for any group width.
template <int HD, int BITS, int GW>
__device__ __forceinline__ void k_token_row(const float (&x)[8], int r, int len, int cc, uint32_t *kcodes,
                                            uint32_t *km_base) {
    constexpr int L = (1 << BITS) - 1;
    constexpr int WPR = HD * BITS / 32;
    constexpr int LPG = GW / 8;   // lanes per group
    float a = x[0], z = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) { a = fminf(a, x[i]); z = fmaxf(z, x[i]); }
    a = fminf(a, quad_xor1(a)); z = fmaxf(z, quad_xor1(z));
    a = fminf(a, quad_xor2(a)); z = fmaxf(z, quad_xor2(z));
    if (LPG >= 8) { a = fminf(a, lane_xor(a, 4)); z = fmaxf(z, lane_xor(z, 4)); }
    if (LPG >= 16) { a = fminf(a, lane_xor(a, 8)); z = fmaxf(z, lane_xor(z, 8)); }
    Quant kq;
    kq.set(a, z, L);
    const float kinv = kq.inv();
    bool near = false;
    float kc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) kc[i] = fast_code(x[i], kq.zero, kinv, L, near);
    uint32_t kbits = pack_codes<BITS>(kc);
    if (__builtin_expect(__any(near), 0)) {
        kbits = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) kbits |= kq.code(x[i], L) << (BITS * i);
    }
    const uint32_t kn = quad_xor1(kbits);
    if (r < len) {
        if (cc % LPG == 0) km_base[(size_t)r * (HD / GW) + cc / LPG] = kq.meta;
        if (BITS == 4) kcodes[(size_t)r * WPR + cc] = kbits;
        else if ((cc & 1) == 0) kcodes[(size_t)r * WPR + cc / 2] = kbits | (kn << 16);
    }
}

// The compensation of one row: c_j = sum over the row's channels of U[c][j] (x_c - khat_c),
// khat the dequantized key (the element dtype's rounding of code * step + zero), each of
// the row's lanes taking its 8 channels, the sum completed across the row's CC lanes in
// fp32, then one rounding to bf16. U is staged in LDS as [j][channel]. The row's first lane
// stores the 8 bf16 entries (zeros past the rank).
template <int HD, int BITS, bool BF16>
__device__ __forceinline__ void comp_row(const float (&x)[8], const uint32_t kbits, int r, int len, int cc,
                                         const Quant (&kq)[8], const float *u_lds, int rank, uint16_t *comp) {
    constexpr int CC = HD / 8;
    constexpr uint32_t M = (1u << BITS) - 1;
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float y = __builtin_fmaf((float)((kbits >> (BITS * i)) & M), kq[i].step, kq[i].zero);
        const float yh = BF16 ? (float)(__bf16)y : (float)(_Float16)y;
        e[i] = x[i] - yh;
    }
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
    for (int j = 0; j < rank; ++j) {
        const f32x4 u0 = *reinterpret_cast<const f32x4 *>(u_lds + j * HD + cc * 8);
        const f32x4 u1 = *reinterpret_cast<const f32x4 *>(u_lds + j * HD + cc * 8 + 4);
        float acc = u0.x * e[0];
        acc = __builtin_fmaf(u0.y, e[1], acc);
        acc = __builtin_fmaf(u0.z, e[2], acc);
        acc = __builtin_fmaf(u0.w, e[3], acc);
        acc = __builtin_fmaf(u1.x, e[4], acc);
        acc = __builtin_fmaf(u1.y, e[5], acc);
        acc = __builtin_fmaf(u1.z, e[6], acc);
        acc = __builtin_fmaf(u1.w, e[7], acc);
#pragma unroll
        for (int o = 1; o < CC; o <<= 1) acc += __shfl_xor(acc, o);
        const uint32_t hb = f32_to_bf16_bits(acc);
        packed[j / 2] |= hb << (16 * (j % 2));
    }
    if (r < len && cc == 0)
        *reinterpret_cast<u32x4 *>(comp + (size_t)r * 8) = u32x4{packed[0], packed[1], packed[2], packed[3]};
}

// Codes of one row's 8 channels of K against the group's per-channel step/zero, and
// their store (as v_row).
template <int HD, int BITS>
__device__ __forceinline__ uint32_t k_row(const float (&x)[8], int r, int len, int cc, const Quant (&kq)[8],
                                          const float (&kinv)[8], uint32_t *kcodes) {
    constexpr int L = (1 << BITS) - 1;
    constexpr int WPR = HD * BITS / 32;
    bool near = false;
    float kc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) kc[i] = fast_code(x[i], kq[i].zero, kinv[i], L, near);
    uint32_t kbits = pack_codes<BITS>(kc);
    if (__builtin_expect(__any(near), 0)) {
        kbits = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) kbits |= kq[i].code(x[i], L) << (BITS * i);
    }
    const uint32_t kn = quad_xor1(kbits);
    if (r < len) {
        if (BITS == 4) kcodes[(size_t)r * WPR + cc] = kbits;
        else if ((cc & 1) == 0) kcodes[(size_t)r * WPR + cc / 2] = kbits | (kn << 16);
    }
    return kbits;
}

// The K-group's per-channel step/zero from each thread's running extremes (mn, mx over
// its rows of the thread's 8 channels): the extremes are combined across the lanes and
// waves that hold the same channels, the meta is stored by the first row pass, and the
// reciprocals of the steps are returned for fast_code. Called by every thread of the
// workgroup in uniform control flow; holds a barrier.
template <int HD, int BITS, int NT>
__device__ __forceinline__ void k_group_quant(const QuantAppendParams &p, float (&mn)[8], float (&mx)[8], int g,
                                              size_t bh, Quant (&kq)[8], float (&kinv)[8]) {
    constexpr int L = (1 << BITS) - 1;
    constexpr int CC = HD / 8;
    const int tid = threadIdx.x;
    const int cc = tid % CC, rp = tid / CC;
    const int lane = tid % kWave, wave = tid / kWave;
    // lanes holding the same channels differ in the bits above log2(CC)
#pragma unroll
    for (int o = CC; o < kWave; o <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            mn[i] = fminf(mn[i], __shfl_xor(mn[i], o));
            mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], o));
        }
    }
    __shared__ float s_mn[NT / kWave][HD], s_mx[NT / kWave][HD];
    if (lane < CC) {
#pragma unroll
        for (int i = 0; i < 8; ++i) { s_mn[wave][cc * 8 + i] = mn[i]; s_mx[wave][cc * 8 + i] = mx[i]; }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float a = s_mn[0][cc * 8 + i], z = s_mx[0][cc * 8 + i];
#pragma unroll
        for (int w = 1; w < NT / kWave; ++w) {
            a = fminf(a, s_mn[w][cc * 8 + i]);
            z = fmaxf(z, s_mx[w][cc * 8 + i]);
        }
        kq[i].set(a, z, L);
    }
    if (rp == 0) {
        uint32_t *km = reinterpret_cast<uint32_t *>(p.k_meta) +
                       (bh * p.kgroup_capacity + p.n_kgroups + g) * HD + cc * 8;
        *reinterpret_cast<u32x4 *>(km) = u32x4{kq[0].meta, kq[1].meta, kq[2].meta, kq[3].meta};
        *reinterpret_cast<u32x4 *>(km + 4) = u32x4{kq[4].meta, kq[5].meta, kq[6].meta, kq[7].meta};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) kinv[i] = kq[i].inv();
}

// Per-token K groups: no K-group statistics; rows are coded one after another, keys as
// values are, with the group width of the segment.
template <typename T, int HD, int BITS, int NT, int GW>
__device__ __forceinline__ void token_group_rows(const T *ks, const T *vs, int len, uint32_t *kcodes,
                                                 uint32_t *vcodes, uint32_t *km_base, uint32_t *vm_base) {
    constexpr int CC = HD / 8;
    constexpr int RP = NT / CC;
    typedef typename Src<T>::Raw Raw;
    const int tid = threadIdx.x, cc = tid % CC, rp = tid / CC;
    for (int b0 = 0; b0 < len; b0 += kBatch2 * RP) {
        Raw kraw[kBatch2], vraw[kBatch2];
#pragma unroll
        for (int u = 0; u < kBatch2; ++u) {
            const int rr = min(b0 + u * RP + rp, len - 1);
            kraw[u] = Src<T>::load(ks + (size_t)rr * HD);
            vraw[u] = Src<T>::load(vs + (size_t)rr * HD);
        }
#pragma unroll
        for (int u = 0; u < kBatch2; ++u) {
            float x[8], y[8];
            Src<T>::unpack(kraw[u], x);
            Src<T>::unpack(vraw[u], y);
            v_row<HD, BITS>(y, b0 + u * RP + rp, len, cc, vcodes, vm_base);
            k_token_row<HD, BITS, GW>(x, b0 + u * RP + rp, len, cc, kcodes, km_base);
        }
    }
}

// One K-group g (of n_groups appended) of one (batch b, KV head h) by a workgroup of NT
// threads: K and V codes, step/zero, and (by the (0, 0) pair) the group-table entries.
// Every thread of the workgroup calls it, in uniform control flow; it holds barriers, and
// a caller that runs it again must pass a barrier in between (the LDS statistics are
// reused).
// EXT: also the per-token K groups and the compensation (off where only the plain layout
// can occur, so that those paths take no code or registers there).
template <typename T, int HD, int BITS, int NT, bool EXT = true>
__device__ __forceinline__ void quant_group(const QuantAppendParams &p, int g, int h, int b, int n_groups) {
    constexpr int CC = HD / 8;            // 8-channel chunks per token row
    constexpr int RP = NT / CC;           // rows processed per pass
    constexpr int WPR = HD * BITS / 32;   // packed words per token row
    constexpr int VG = 32;                // V-group width
    typedef typename Src<T>::Raw Raw;
    const int tid = threadIdx.x;
    const int cc = tid % CC, rp = tid / CC;

    // ---- which source tokens, and where they land ----
    int src0, len, dst0;
    group_span<NT>(p, g, src0, len, dst0);
    if (b == 0 && h == 0 && tid == 0) {
        p.kgroup_start[p.n_kgroups + g] = p.n_tokens + min(dst0, p.n_new);
        if (g == n_groups - 1) p.kgroup_start[p.n_kgroups + g + 1] = p.n_tokens + p.n_new;
    }
    if (len <= 0) return;  // only reachable with a malformed gather list

    const size_t bh = (size_t)b * p.n_kv_heads + h;
    const T *ks = reinterpret_cast<const T *>(p.k_src) + (bh * p.src_tokens + src0) * HD + cc * 8;
    const T *vs = reinterpret_cast<const T *>(p.v_src) + (bh * p.src_tokens + src0) * HD + cc * 8;
    uint32_t *kcodes = reinterpret_cast<uint32_t *>(p.k_dst) + (bh * p.capacity + p.n_tokens + dst0) * WPR;
    uint32_t *vcodes = reinterpret_cast<uint32_t *>(p.v_dst) + (bh * p.capacity + p.n_tokens + dst0) * WPR;
    uint32_t *vm_base = reinterpret_cast<uint32_t *>(p.v_meta) + (bh * p.capacity + p.n_tokens + dst0) * (HD / VG);

    if (EXT && p.k_group_channels > 0) {
        uint32_t *km_base = reinterpret_cast<uint32_t *>(p.k_meta) +
                            (bh * p.capacity + p.n_tokens + dst0) * (HD / p.k_group_channels);
        if (p.k_group_channels == 32)
            token_group_rows<T, HD, BITS, NT, 32>(ks, vs, len, kcodes, vcodes, km_base, vm_base);
        else if (p.k_group_channels == 64)
            token_group_rows<T, HD, BITS, NT, 64>(ks, vs, len, kcodes, vcodes, km_base, vm_base);
        else
            token_group_rows<T, HD, BITS, NT, HD>(ks, vs, len, kcodes, vcodes, km_base, vm_base);
        return;
    }
    // the compensation basis of head h, as [j][channel], for comp_row
    __shared__ float u_lds[EXT ? 8 * HD : 1];
    const int rank = EXT ? p.comp_rank : 0;
    if (rank > 0) {
        const float *U = p.comp_basis + (size_t)h * HD * rank;
        for (int i = tid; i < HD * rank; i += NT) u_lds[(i % rank) * HD + i / rank] = U[i];
    }
    uint16_t *comp = rank > 0 ? reinterpret_cast<uint16_t *>(p.k_comp) + (bh * p.capacity + p.n_tokens + dst0) * 8
                              : nullptr;
    constexpr bool kBf16Elem = std::is_same<T, __bf16>::value;

    // ---- K: per-channel extremes over the group's tokens ----
    // Rows are read in batches whose loads are all in flight together; a thread's rows
    // past the group end read the group's last row again (a repeat leaves the extremes
    // unchanged, and its codes are not stored), so every load is unconditional. With
    // 16-bit sources and a group of at most kBatch1 rows per thread, the K rows stay in
    // registers until their codes are made, and the first V rows (which do not depend on
    // the K statistics) are coded while the K loads land.
    const bool resident = sizeof(Raw) == 16 && len <= kBatch1 * RP;
    float mn[8], mx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) { mn[i] = __builtin_inff(); mx[i] = -__builtin_inff(); }
    Raw kres[kBatch1];
    if (resident) {
#pragma unroll
        for (int u = 0; u < kBatch1; ++u)
            if (u * RP < len) kres[u] = Src<T>::load(ks + (size_t)min(u * RP + rp, len - 1) * HD);
        Raw vraw[kBatch2];
#pragma unroll
        for (int u = 0; u < kBatch2; ++u)
            if (u * RP < len) vraw[u] = Src<T>::load(vs + (size_t)min(u * RP + rp, len - 1) * HD);
#pragma unroll
        for (int u = 0; u < kBatch2; ++u) {
            if (u * RP < len) {
                float y[8];
                Src<T>::unpack(vraw[u], y);
                v_row<HD, BITS>(y, u * RP + rp, len, cc, vcodes, vm_base);
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch1; ++u) {
            if (u * RP < len) {
                float x[8];
                Src<T>::unpack(kres[u], x);
#pragma unroll
                for (int i = 0; i < 8; ++i) { mn[i] = fminf(mn[i], x[i]); mx[i] = fmaxf(mx[i], x[i]); }
            }
        }
    } else {
        for (int b0 = 0; b0 < len; b0 += kBatch1 * RP) {
            Raw raw[kBatch1];
#pragma unroll
            for (int u = 0; u < kBatch1; ++u)
                raw[u] = Src<T>::load(ks + (size_t)min(b0 + u * RP + rp, len - 1) * HD);
#pragma unroll
            for (int u = 0; u < kBatch1; ++u) {
                float x[8];
                Src<T>::unpack(raw[u], x);
#pragma unroll
                for (int i = 0; i < 8; ++i) { mn[i] = fminf(mn[i], x[i]); mx[i] = fmaxf(mx[i], x[i]); }
            }
        }
    }
    Quant kq[8];
    float kinv[8];
    k_group_quant<HD, BITS, NT>(p, mn, mx, g, bh, kq, kinv);

    // ---- codes: the remaining V rows, then K ----
    // Batches of rows as above. The four lanes of a quad hold one row (CC is a multiple of
    // 4), so the quad exchanges in the row helpers see one row's lanes.
    if (resident) {
        for (int b0 = kBatch2 * RP; b0 < len; b0 += kBatch2 * RP) {
            Raw vraw[kBatch2];
#pragma unroll
            for (int u = 0; u < kBatch2; ++u) vraw[u] = Src<T>::load(vs + (size_t)min(b0 + u * RP + rp, len - 1) * HD);
#pragma unroll
            for (int u = 0; u < kBatch2; ++u) {
                float y[8];
                Src<T>::unpack(vraw[u], y);
                v_row<HD, BITS>(y, b0 + u * RP + rp, len, cc, vcodes, vm_base);
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch1; ++u) {
            if (u * RP < len) {
                float x[8];
                Src<T>::unpack(kres[u], x);
                const uint32_t kb = k_row<HD, BITS>(x, u * RP + rp, len, cc, kq, kinv, kcodes);
                if (rank > 0) comp_row<HD, BITS, kBf16Elem>(x, kb, u * RP + rp, len, cc, kq, u_lds, rank, comp);
            }
        }
    } else {
        for (int b0 = 0; b0 < len; b0 += kBatch2 * RP) {
            Raw kraw[kBatch2], vraw[kBatch2];
#pragma unroll
            for (int u = 0; u < kBatch2; ++u) {
                const int rr = min(b0 + u * RP + rp, len - 1);
                kraw[u] = Src<T>::load(ks + (size_t)rr * HD);
                vraw[u] = Src<T>::load(vs + (size_t)rr * HD);
            }
#pragma unroll
            for (int u = 0; u < kBatch2; ++u) {
                float x[8], y[8];
                Src<T>::unpack(kraw[u], x);
                Src<T>::unpack(vraw[u], y);
                v_row<HD, BITS>(y, b0 + u * RP + rp, len, cc, vcodes, vm_base);
                const uint32_t kb = k_row<HD, BITS>(x, b0 + u * RP + rp, len, cc, kq, kinv, kcodes);
                if (rank > 0)
                    comp_row<HD, BITS, kBf16Elem>(x, kb, b0 + u * RP + rp, len, cc, kq, u_lds, rank, comp);
            }
        }
    }
}


// The same K-group's work in two halves for two workgroups, so that the append launch has
// twice as many, half as long: PART 1 takes the keys (statistics, step/zero, codes, the
// group-table entries and the compensation), PART 2 the values (a group per token and 32
// channels). The arithmetic is quant_group's, element for element; only the split differs.
// Plain per-channel K groups only (per-token K groups take quant_group). Every thread of
// the workgroup calls it, in uniform control flow.
template <typename T, int HD, int BITS, int NT, int PART>
__device__ __forceinline__ void quant_group_part(const QuantAppendParams &p, int g, int h, int b, int n_groups) {
    constexpr int CC = HD / 8;
    constexpr int RP = NT / CC;
    constexpr int WPR = HD * BITS / 32;
    constexpr int VG = 32;
    typedef typename Src<T>::Raw Raw;
    const int tid = threadIdx.x;
    const int cc = tid % CC, rp = tid / CC;
    int src0, len, dst0;
    group_span<NT>(p, g, src0, len, dst0);
    if (PART == 1 && b == 0 && h == 0 && tid == 0) {
        p.kgroup_start[p.n_kgroups + g] = p.n_tokens + min(dst0, p.n_new);
        if (g == n_groups - 1) p.kgroup_start[p.n_kgroups + g + 1] = p.n_tokens + p.n_new;
    }
    if (len <= 0) return;  // only reachable with a malformed gather list
    const size_t bh = (size_t)b * p.n_kv_heads + h;

    if constexpr (PART == 2) {
        // values: rows in batches whose loads are all in flight together (rows past the
        // group end repeat its last row and are not stored)
        const T *vs = reinterpret_cast<const T *>(p.v_src) + (bh * p.src_tokens + src0) * HD + cc * 8;
        uint32_t *vcodes = reinterpret_cast<uint32_t *>(p.v_dst) + (bh * p.capacity + p.n_tokens + dst0) * WPR;
        uint32_t *vm_base =
            reinterpret_cast<uint32_t *>(p.v_meta) + (bh * p.capacity + p.n_tokens + dst0) * (HD / VG);
        for (int b0 = 0; b0 < len; b0 += kBatch1 * RP) {
            Raw vraw[kBatch1];
#pragma unroll
            for (int u = 0; u < kBatch1; ++u) vraw[u] = Src<T>::load(vs + (size_t)min(b0 + u * RP + rp, len - 1) * HD);
#pragma unroll
            for (int u = 0; u < kBatch1; ++u) {
                float y[8];
                Src<T>::unpack(vraw[u], y);
                v_row<HD, BITS>(y, b0 + u * RP + rp, len, cc, vcodes, vm_base);
            }
        }
    } else {
        // keys: extremes, step/zero, codes, as quant_group without its value rows
        const T *ks = reinterpret_cast<const T *>(p.k_src) + (bh * p.src_tokens + src0) * HD + cc * 8;
        uint32_t *kcodes = reinterpret_cast<uint32_t *>(p.k_dst) + (bh * p.capacity + p.n_tokens + dst0) * WPR;
        __shared__ float u_lds[8 * HD];
        const int rank = p.comp_rank;
        if (rank > 0) {
            const float *U = p.comp_basis + (size_t)h * HD * rank;
            for (int i = tid; i < HD * rank; i += NT) u_lds[(i % rank) * HD + i / rank] = U[i];
        }
        uint16_t *comp = rank > 0 ? reinterpret_cast<uint16_t *>(p.k_comp) + (bh * p.capacity + p.n_tokens + dst0) * 8
                                  : nullptr;
        constexpr bool kBf16Elem = std::is_same<T, __bf16>::value;
        const bool resident = sizeof(Raw) == 16 && len <= kBatch1 * RP;
        float mn[8], mx[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) { mn[i] = __builtin_inff(); mx[i] = -__builtin_inff(); }
        Raw kres[kBatch1];
        if (resident) {
#pragma unroll
            for (int u = 0; u < kBatch1; ++u)
                if (u * RP < len) kres[u] = Src<T>::load(ks + (size_t)min(u * RP + rp, len - 1) * HD);
#pragma unroll
            for (int u = 0; u < kBatch1; ++u) {
                if (u * RP < len) {
                    float x[8];
                    Src<T>::unpack(kres[u], x);
#pragma unroll
                    for (int i = 0; i < 8; ++i) { mn[i] = fminf(mn[i], x[i]); mx[i] = fmaxf(mx[i], x[i]); }
                }
            }
        } else {
            for (int b0 = 0; b0 < len; b0 += kBatch1 * RP) {
                Raw raw[kBatch1];
#pragma unroll
                for (int u = 0; u < kBatch1; ++u)
                    raw[u] = Src<T>::load(ks + (size_t)min(b0 + u * RP + rp, len - 1) * HD);
#pragma unroll
                for (int u = 0; u < kBatch1; ++u) {
                    float x[8];
                    Src<T>::unpack(raw[u], x);
#pragma unroll
                    for (int i = 0; i < 8; ++i) { mn[i] = fminf(mn[i], x[i]); mx[i] = fmaxf(mx[i], x[i]); }
                }
            }
        }
        Quant kq[8];
        float kinv[8];
        k_group_quant<HD, BITS, NT>(p, mn, mx, g, bh, kq, kinv);
        if (resident) {
#pragma unroll
            for (int u = 0; u < kBatch1; ++u) {
                if (u * RP < len) {
                    float x[8];
                    Src<T>::unpack(kres[u], x);
                    const uint32_t kb = k_row<HD, BITS>(x, u * RP + rp, len, cc, kq, kinv, kcodes);
                    if (rank > 0) comp_row<HD, BITS, kBf16Elem>(x, kb, u * RP + rp, len, cc, kq, u_lds, rank, comp);
                }
            }
        } else {
            for (int b0 = 0; b0 < len; b0 += kBatch2 * RP) {
                Raw kraw[kBatch2];
#pragma unroll
                for (int u = 0; u < kBatch2; ++u)
                    kraw[u] = Src<T>::load(ks + (size_t)min(b0 + u * RP + rp, len - 1) * HD);
#pragma unroll
                for (int u = 0; u < kBatch2; ++u) {
                    float x[8];
                    Src<T>::unpack(kraw[u], x);
                    const uint32_t kb = k_row<HD, BITS>(x, b0 + u * RP + rp, len, cc, kq, kinv, kcodes);
                    if (rank > 0)
                        comp_row<HD, BITS, kBf16Elem>(x, kb, b0 + u * RP + rp, len, cc, kq, u_lds, rank, comp);
                }
            }
        }
    }
}

}  // namespace qz
}  // namespace kvq
