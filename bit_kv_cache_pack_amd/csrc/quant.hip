// Quantize-append kernels: per (K-group, KV head, batch), two workgroups (keys, values)
// or, for per-token K groups, one, run the quantizer of kvq_quant.cuh (asymmetric
// INT2/INT4 group quantization of a finished chunk's keys, one group per K-group of tokens
// and channel, and values, one group per token and run of 32 channels; fp16 step/zero;
// dense packing), or copies the tokens of a raw (bits 16) segment.
#include "kvq_quant.cuh"

namespace kvq {
namespace {

using namespace qz;

constexpr int kThreads = 256;

// Per-token K groups, and K-groups of fewer than 64 tokens: one workgroup per (K-group,
// KV head, batch) takes keys and values.
template <typename T, int HD, int BITS>
__global__ __launch_bounds__(kThreads) void quant_append_kernel(QuantAppendParams p) {
    quant_group<T, HD, BITS, kThreads>(p, blockIdx.x, blockIdx.y, blockIdx.z, gridDim.x);
}

// Per-channel K groups of 64 tokens or more: blockIdx.x < n_groups takes the keys of
// K-group blockIdx.x, the rest the values of K-group blockIdx.x - n_groups. Twice the
// workgroups of half the work each: measured on the long-rollout chunk (40 heads x 4,680
// tokens) 30.4 against 36.5 us, on the video chunk (12 heads) 12.5 against 16.1 us. For
// 32-token groups (WindowQuant windows, gathered) the halves are too small to pay for
// the extra workgroups: 40.8 against 34.4 us for the three gathered appends of a step.
template <typename T, int HD, int BITS>
__global__ __launch_bounds__(kThreads) void quant_split_kernel(QuantAppendParams p) {
    const int ng = gridDim.x / 2;
    if ((int)blockIdx.x < ng) quant_group_part<T, HD, BITS, kThreads, 1>(p, blockIdx.x, blockIdx.y, blockIdx.z, ng);
    else quant_group_part<T, HD, BITS, kThreads, 2>(p, blockIdx.x - ng, blockIdx.y, blockIdx.z, ng);
}

// bits == 16: copy tokens into a raw segment, rounding to the element dtype.
template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void raw_append_kernel(QuantAppendParams p) {
    constexpr int CC = HD / 8;
    constexpr int RP = kThreads / CC;
    const int g = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, cc = tid % CC, rp = tid / CC;
    int src0, len, dst0;
    group_span<kThreads>(p, g, src0, len, dst0);
    if (len <= 0) return;
    const size_t bh = (size_t)b * gridDim.y + h;
    const T *ks = reinterpret_cast<const T *>(p.k_src) + (bh * p.src_tokens + src0) * HD + cc * 8;
    const T *vs = reinterpret_cast<const T *>(p.v_src) + (bh * p.src_tokens + src0) * HD + cc * 8;
    uint16_t *kd = reinterpret_cast<uint16_t *>(p.k_dst) + (bh * p.capacity + p.n_tokens + dst0) * HD + cc * 8;
    uint16_t *vd = reinterpret_cast<uint16_t *>(p.v_dst) + (bh * p.capacity + p.n_tokens + dst0) * HD + cc * 8;
    for (int r = rp; r < len; r += RP) {
        float x[8], y[8];
        Src<T>::unpack(Src<T>::load(ks + (size_t)r * HD), x);
        Src<T>::unpack(Src<T>::load(vs + (size_t)r * HD), y);
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
    if (bits != 16 && p.k_group_channels == 0 && p.k_group_tokens >= 64) {
        const dim3 split(2 * n_groups, p.n_kv_heads, p.batch);
        if (bits == 2)
            hipLaunchKernelGGL((quant_split_kernel<T, HD, 2>), split, dim3(kThreads), 0, s, p);
        else
            hipLaunchKernelGGL((quant_split_kernel<T, HD, 4>), split, dim3(kThreads), 0, s, p);
        return hipGetLastError();
    }
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
