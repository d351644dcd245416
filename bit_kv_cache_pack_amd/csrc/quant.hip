// Quantize-append: asymmetric INT2/INT4 group quantization of a finished chunk's keys
// (one group per K-group of tokens and channel) and values (one group per token and
// run of 32 channels), fp16 step/zero, dense packing, appended to a cache segment.
//
// Method: "Quantized Keys Steal Attention: Bias Correction for KV-Cache Compression in
// Video Diffusion" (abstract: a KV cache of earlier chunks, quantized to low bit-widths,
// read through the cached keys' quantization step sizes) and the WindowQuant notes
// ("技術的に面白い点": windows of one bit-width stored together, here via gather lists).
// The pages give no quantizer formula; the one used is plain min/max asymmetric
// quantization:
//   step = fp16(fl32(max - min) / L), zero = fp16(min),
//   code = clamp(rint(fl32(x - zero) / step), 0, L), 0 when step == 0,
// with IEEE fp32 division and no contraction (this file is built with
// -ffp-contract=off), so codes are reproducible bit for bit.
//
// One workgroup quantizes one K-group (<= k_group_tokens tokens) of one (batch, head):
// the K statistics run down the group's tokens per channel, the V statistics across
// each token's 32-channel runs, so the gather mapping (window -> destination) is known
// per workgroup and a single launch appends K and V.
#include "kvq_device.cuh"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;

template <typename T> struct Src;
template <> struct Src<float> {
    // 8 consecutive elements starting at p (16-byte aligned for 8 floats = 32 bytes)
    static __device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
        f32x4 a = *reinterpret_cast<const f32x4 *>(p);
        f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
};
template <> struct Src<__bf16> {
    static __device__ __forceinline__ void load8(const __bf16 *p, float (&x)[8]) {
        u32x4 w = *reinterpret_cast<const u32x4 *>(p);
        uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(a[i] << 16);
            x[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
        }
    }
};
template <> struct Src<_Float16> {
    static __device__ __forceinline__ void load8(const _Float16 *p, float (&x)[8]) {
        u32x4 w = *reinterpret_cast<const u32x4 *>(p);
        uint32_t a[4] = {w.x, w.y, w.z, w.w};
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
};

// Source span and destination offset of appended group g. Contiguous appends cut
// the source into k_group_tokens-long groups; gather appends take the listed spans in
// order (entries clamped so every access stays inside the buffers). Uniform per block.
__device__ __forceinline__ void group_span(const QuantAppendParams &p, int g, int &src0, int &len,
                                           int &dst0) {
    if (p.src_groups == nullptr) {
        src0 = g * p.k_group_tokens;
        len = min(p.k_group_tokens, p.n_new - src0);
        dst0 = src0;
        return;
    }
    __shared__ int s_red[kThreads / kWave];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    int part = 0;
    for (int i = tid; i < g; i += kThreads)
        part += min(max(p.src_groups[2 * i + 1], 0), p.k_group_tokens);
    for (int o = kWave / 2; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if (lane == 0) s_red[wave] = part;
    __syncthreads();
    dst0 = 0;
    for (int w = 0; w < kThreads / kWave; ++w) dst0 += s_red[w];
    src0 = min(max(p.src_groups[2 * g], 0), (int)max(p.src_tokens - 1, (int64_t)0));
    len = min(max(p.src_groups[2 * g + 1], 0), p.k_group_tokens);
    len = (int)min((int64_t)len, p.src_tokens - src0);
    len = min(len, p.n_new - dst0);
}

template <typename T, int HD, int BITS>
__global__ __launch_bounds__(kThreads) void quant_append_kernel(QuantAppendParams p) {
    constexpr int L = (1 << BITS) - 1;
    constexpr int CC = HD / 8;            // 8-channel chunks per token row
    constexpr int RP = kThreads / CC;     // rows processed per pass
    constexpr int WPR = HD * BITS / 32;   // packed words per token row
    constexpr int VG = 32;                // V-group width
    const int g = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int cc = tid % CC, rp = tid / CC;
    const int lane = tid % kWave, wave = tid / kWave;

    // ---- which source tokens, and where they land ----
    int src0, len, dst0;
    group_span(p, g, src0, len, dst0);
    if (b == 0 && h == 0 && tid == 0) {
        p.kgroup_start[p.n_kgroups + g] = p.n_tokens + min(dst0, p.n_new);
        if (g == gridDim.x - 1) p.kgroup_start[p.n_kgroups + g + 1] = p.n_tokens + p.n_new;
    }
    if (len <= 0) return;  // only reachable with a malformed gather list

    const size_t bh = (size_t)b * gridDim.y + h;
    const T *ks = reinterpret_cast<const T *>(p.k_src) + (bh * p.src_tokens + src0) * HD + cc * 8;
    const T *vs = reinterpret_cast<const T *>(p.v_src) + (bh * p.src_tokens + src0) * HD + cc * 8;
    uint32_t *kcodes = reinterpret_cast<uint32_t *>(p.k_dst) + (bh * p.capacity + p.n_tokens + dst0) * WPR;
    uint32_t *vcodes = reinterpret_cast<uint32_t *>(p.v_dst) + (bh * p.capacity + p.n_tokens + dst0) * WPR;

    // ---- K: per-channel extremes over the group's tokens ----
    float mn[8], mx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) { mn[i] = __builtin_inff(); mx[i] = -__builtin_inff(); }
    for (int r = rp; r < len; r += RP) {
        float x[8];
        Src<T>::load8(ks + (size_t)r * HD, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) { mn[i] = fminf(mn[i], x[i]); mx[i] = fmaxf(mx[i], x[i]); }
    }
    // lanes holding the same channels differ in the bits above log2(CC)
#pragma unroll
    for (int o = CC; o < kWave; o <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            mn[i] = fminf(mn[i], __shfl_xor(mn[i], o));
            mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], o));
        }
    }
    __shared__ float s_mn[kThreads / kWave][HD], s_mx[kThreads / kWave][HD];
    if (lane < CC) {
#pragma unroll
        for (int i = 0; i < 8; ++i) { s_mn[wave][cc * 8 + i] = mn[i]; s_mx[wave][cc * 8 + i] = mx[i]; }
    }
    __syncthreads();
    Quant kq[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float a = s_mn[0][cc * 8 + i], z = s_mx[0][cc * 8 + i];
#pragma unroll
        for (int w = 1; w < kThreads / kWave; ++w) {
            a = fminf(a, s_mn[w][cc * 8 + i]);
            z = fmaxf(z, s_mx[w][cc * 8 + i]);
        }
        kq[i].set(a, z, L);
    }
    if (rp == 0) {
        uint32_t *km = reinterpret_cast<uint32_t *>(p.k_meta) +
                       (bh * p.kgroup_capacity + p.n_kgroups + g) * HD + cc * 8;
        u32x4 m0 = {kq[0].meta, kq[1].meta, kq[2].meta, kq[3].meta};
        u32x4 m1 = {kq[4].meta, kq[5].meta, kq[6].meta, kq[7].meta};
        *reinterpret_cast<u32x4 *>(km) = m0;
        *reinterpret_cast<u32x4 *>(km + 4) = m1;
    }

    // ---- K codes and V (per token, per 32-channel run) ----
    uint32_t *vm_base = reinterpret_cast<uint32_t *>(p.v_meta) + (bh * p.capacity + p.n_tokens + dst0) * (HD / VG);
    for (int r = rp; r < len; r += RP) {
        float x[8];
        Src<T>::load8(ks + (size_t)r * HD, x);
        uint32_t kbits = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) kbits |= kq[i].code(x[i], L) << (BITS * i);

        float y[8];
        Src<T>::load8(vs + (size_t)r * HD, y);
        float a = y[0], z = y[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) { a = fminf(a, y[i]); z = fmaxf(z, y[i]); }
        // the 4 lanes of one 32-channel run are tid^1, tid^2 neighbours (CC % 4 == 0)
        a = fminf(a, __shfl_xor(a, 1)); z = fmaxf(z, __shfl_xor(z, 1));
        a = fminf(a, __shfl_xor(a, 2)); z = fmaxf(z, __shfl_xor(z, 2));
        Quant vq;
        vq.set(a, z, L);
        uint32_t vbits = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) vbits |= vq.code(y[i], L) << (BITS * i);
        if ((cc & 3) == 0) vm_base[(size_t)r * (HD / VG) + cc / 4] = vq.meta;

        if (BITS == 4) {
            kcodes[(size_t)r * WPR + cc] = kbits;
            vcodes[(size_t)r * WPR + cc] = vbits;
        } else {
            // 16 channels per word: the even chunk takes its odd neighbour's half
            uint32_t kn = __shfl_xor(kbits, 1), vn = __shfl_xor(vbits, 1);
            if ((cc & 1) == 0) {
                kcodes[(size_t)r * WPR + cc / 2] = kbits | (kn << 16);
                vcodes[(size_t)r * WPR + cc / 2] = vbits | (vn << 16);
            }
        }
    }
}

// bits == 16: copy tokens into a raw segment, rounding to the element dtype.
template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void raw_append_kernel(QuantAppendParams p) {
    constexpr int CC = HD / 8;
    constexpr int RP = kThreads / CC;
    const int g = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, cc = tid % CC, rp = tid / CC;
    int src0, len, dst0;
    group_span(p, g, src0, len, dst0);
    if (len <= 0) return;
    const size_t bh = (size_t)b * gridDim.y + h;
    const T *ks = reinterpret_cast<const T *>(p.k_src) + (bh * p.src_tokens + src0) * HD + cc * 8;
    const T *vs = reinterpret_cast<const T *>(p.v_src) + (bh * p.src_tokens + src0) * HD + cc * 8;
    uint16_t *kd = reinterpret_cast<uint16_t *>(p.k_dst) + (bh * p.capacity + p.n_tokens + dst0) * HD + cc * 8;
    uint16_t *vd = reinterpret_cast<uint16_t *>(p.v_dst) + (bh * p.capacity + p.n_tokens + dst0) * HD + cc * 8;
    for (int r = rp; r < len; r += RP) {
        float x[8], y[8];
        Src<T>::load8(ks + (size_t)r * HD, x);
        Src<T>::load8(vs + (size_t)r * HD, y);
        u32x4 ko, vo;
        uint32_t kw[4], vw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kw[i] = p.elem_dtype == DT_BF16 ? pack_bf16x2(x[2 * i], x[2 * i + 1]) : pack_f16x2(x[2 * i], x[2 * i + 1]);
            vw[i] = p.elem_dtype == DT_BF16 ? pack_bf16x2(y[2 * i], y[2 * i + 1]) : pack_f16x2(y[2 * i], y[2 * i + 1]);
        }
        ko = {kw[0], kw[1], kw[2], kw[3]};
        vo = {vw[0], vw[1], vw[2], vw[3]};
        *reinterpret_cast<u32x4 *>(kd + (size_t)r * HD) = ko;
        *reinterpret_cast<u32x4 *>(vd + (size_t)r * HD) = vo;
    }
}

template <typename T, int HD>
hipError_t launch_t(const QuantAppendParams &p, int bits, int n_groups, hipStream_t s) {
    dim3 grid(n_groups, p.n_kv_heads, p.batch);
    if (bits == 2)
        hipLaunchKernelGGL((quant_append_kernel<T, HD, 2>), grid, dim3(kThreads), 0, s, p);
    else if (bits == 4)
        hipLaunchKernelGGL((quant_append_kernel<T, HD, 4>), grid, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((raw_append_kernel<T, HD>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_hd(const QuantAppendParams &p, int bits, int n_groups, hipStream_t s) {
    return p.head_dim == 64 ? launch_t<T, 64>(p, bits, n_groups, s) : launch_t<T, 128>(p, bits, n_groups, s);
}

}  // namespace

hipError_t launch_quant_append(const QuantAppendParams &p, int bits, int n_groups, hipStream_t s) {
    if (p.src_dtype == DT_F32) return launch_hd<float>(p, bits, n_groups, s);
    if (p.src_dtype == DT_BF16) return launch_hd<__bf16>(p, bits, n_groups, s);
    return launch_hd<_Float16>(p, bits, n_groups, s);
}

}  // namespace kvq
