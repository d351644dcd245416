// WindowQuant window scoring and bit-width assignment.
//
// WindowQuant notes ("論文メモ：動画VLMのKV Cacheを軽量化するWindowQuant"): visual tokens are
// split into 32-token windows (section "実装者視点で気になった点"); each window is compared
// with the text query by cosine similarity ("何が新しいのか"); high / middle / low relevance
// is kept in FP16 / INT4 / INT2; the first window stays FP16 whatever its score, and
// windows of one bit-width are laid out together ("技術的に面白い点").
//
// Score of a window: for each KV head the window's mean key, cosine with the text vector,
// averaged over heads. Everything in double, summed in index order (this file is built
// with -ffp-contract=off), so the scores and therefore the ranking are reproducible.
#include "kvq_device.cuh"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kSelectThreads = 1024;
constexpr int kMaxWindows = 16384;

constexpr int kScoreThreads = 256;
constexpr int kScoreMeans = 2048;   // (head, channel) means held in LDS at once

// One workgroup per window. All (head, channel) means of a chunk of heads are taken in
// parallel (tokens in order, loads issued four at a time), then thread h takes head h's dot
// product and norms (channels in order), and thread 0 averages the heads' cosines in head
// order: the same fp64 operations in the same order as a one-thread loop.
__global__ __launch_bounds__(kScoreThreads) void window_score_kernel(WindowParams p) {
    __shared__ double mean[kScoreMeans];
    __shared__ double cs[kScoreThreads];
    const int w = blockIdx.x, tid = threadIdx.x;
    const int d = p.head_dim, H = p.n_kv_heads;
    const int t0 = w * p.window, t1 = min(p.n_tokens, t0 + p.window);
    const int hc = min(kScoreMeans / d, kScoreThreads);   // heads per chunk
    double acc = 0.0;
    for (int h0 = 0; h0 < H; h0 += hc) {
        const int nh = min(hc, H - h0);
        __syncthreads();
        for (int idx = tid; idx < nh * d; idx += kScoreThreads) {
            const int h = h0 + idx / d, c = idx % d;
            const size_t base = (size_t)h * p.n_tokens * d + c;
            double sum = 0.0;
            int t = t0;
            for (; t + 4 <= t1; t += 4) {
                const double a0 = (double)load_elem(p.k, p.k_dtype, base + (size_t)t * d);
                const double a1 = (double)load_elem(p.k, p.k_dtype, base + (size_t)(t + 1) * d);
                const double a2 = (double)load_elem(p.k, p.k_dtype, base + (size_t)(t + 2) * d);
                const double a3 = (double)load_elem(p.k, p.k_dtype, base + (size_t)(t + 3) * d);
                sum += a0;
                sum += a1;
                sum += a2;
                sum += a3;
            }
            for (; t < t1; ++t) sum += (double)load_elem(p.k, p.k_dtype, base + (size_t)t * d);
            mean[idx] = sum / (double)(t1 - t0);
        }
        __syncthreads();
        if (tid < nh) {
            const double *mh = mean + tid * d;
            double dot = 0.0, nm = 0.0, nt = 0.0;
            for (int i = 0; i < d; ++i) {
                const double tv = (double)p.text[i];
                dot += mh[i] * tv;
                nm += mh[i] * mh[i];
                nt += tv * tv;
            }
            cs[tid] = (nm * nt == 0.0) ? 0.0 : dot / (__builtin_sqrt(nm) * __builtin_sqrt(nt));
        }
        __syncthreads();
        if (tid == 0)
            for (int k = 0; k < nh; ++k) acc += cs[k];
    }
    if (tid == 0) p.score[w] = acc / (double)H;
}

// one workgroup: rank windows 1..W-1 (score descending, ties to the lower index), cut
// into FP16 / INT4 / INT2 by the budget, then list each class ascending.
__global__ __launch_bounds__(kSelectThreads) void window_select_kernel(WindowParams p) {
    __shared__ int8_t cls[kMaxWindows];
    __shared__ double sc[kMaxWindows];   // the scores, read W times each by the ranking
    const int W = p.n_windows;
    for (int w = threadIdx.x; w < W; w += kSelectThreads) sc[w] = p.score[w];
    __syncthreads();
    for (int w = threadIdx.x; w < W; w += kSelectThreads) {
        int8_t bits = 16;
        if (w > 0) {
            const double s = sc[w];
            int rank = 0;
            for (int v = 1; v < W; ++v) {
                const double t = sc[v];
                rank += (t > s || (t == s && v < w)) ? 1 : 0;
            }
            bits = rank < p.n_fp16 - 1 ? 16 : (rank < p.n_fp16 - 1 + p.n_int4 ? 4 : 2);
        }
        cls[w] = bits;
        p.bits_out[w] = bits;
    }
    __syncthreads();
    const int n16 = p.n_fp16, n4 = p.n_int4;
    for (int w = threadIdx.x; w < W; w += kSelectThreads) {
        const int8_t b = cls[w];
        int before = 0;
        for (int v = 0; v < w; ++v) before += cls[v] == b ? 1 : 0;
        const int base = b == 16 ? 0 : (b == 4 ? n16 : n16 + n4);
        // ranks form a permutation unless scores are NaN; never write outside the list
        if (base + before < W) p.order_out[base + before] = w;
    }
}

}  // namespace

hipError_t launch_windows(const WindowParams &p, hipStream_t s) {
    hipLaunchKernelGGL(window_score_kernel, dim3(p.n_windows), dim3(kScoreThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(window_select_kernel, dim3(1), dim3(kSelectThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace kvq
