// Streaming-read probe: reads a device buffer once with 16-byte loads, to measure the HBM
// read bandwidth a plain stream reaches on this device (the attention and quantize-append
// kernels are rated against it as well as against the published 8 TB/s). Not part of the
// method.
//
// Every workgroup walks its own contiguous slice of the buffer (so each wave's loads are
// consecutive 1 KiB lines), four 16-byte loads in flight per lane; the loaded words are
// folded into an XOR that reaches memory only if it equals a fixed constant, which keeps
// the loads live without writing anything in practice.
#include "kvq_device.cuh"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;
constexpr uint32_t kProbeMagic = 0x9e3779b9u;

__global__ __launch_bounds__(kProbeThreads) void hbm_read_kernel(const u32x4 *__restrict__ p, size_t n16,
                                                                 size_t per_block, uint32_t *sink) {
    const size_t b0 = (size_t)blockIdx.x * per_block;
    const size_t b1 = b0 + per_block < n16 ? b0 + per_block : n16;
    uint32_t acc = 0;
    constexpr size_t step = (size_t)kProbeThreads * kProbeUnroll;
    size_t i = b0 + threadIdx.x;
    for (; i + (kProbeUnroll - 1) * kProbeThreads < b1; i += step) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + (size_t)u * kProbeThreads);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < b1; i += kProbeThreads) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == kProbeMagic) atomicXor(sink, acc);
}

}  // namespace

hipError_t launch_hbm_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s) {
    const size_t n16 = bytes / 16;
    // about 8 workgroups per compute unit of a 256-CU part, each a contiguous slice
    const size_t blocks = n16 < (size_t)kProbeThreads * 2048 ? (n16 + kProbeThreads - 1) / kProbeThreads : 2048;
    const size_t per_block = (n16 + blocks - 1) / blocks;
    hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s,
                       reinterpret_cast<const u32x4 *>(buf), n16, per_block, sink);
    return hipGetLastError();
}

}  // namespace kvq
