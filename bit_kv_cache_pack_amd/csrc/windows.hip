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

constexpr int kSortMax = 8192;   // windows ranked by a sort in LDS; more are ranked by counting

// window a comes before window b: higher score, ties to the lower index
__device__ __forceinline__ bool before(double sa, int ia, double sb, int ib) {
    return sa > sb || (sa == sb && ia < ib);
}

// One workgroup: rank windows 1..W-1 (score descending, ties to the lower index), cut
// into FP16 / INT4 / INT2 by the budget (window 0 is FP16), then list each class in
// ascending window order. The ranking is a bitonic sort of (score, index) in LDS; the
// lists come from a block prefix sum, over the windows in index order, of three class
// counters packed in one 64-bit word.
__global__ __launch_bounds__(kSelectThreads) void window_select_kernel(WindowParams p) {
    __shared__ int8_t cls[kMaxWindows];
    __shared__ double key[kSortMax];
    __shared__ int idx[kSortMax];
    __shared__ unsigned long long wsum[kSelectThreads / kWave];
    const int W = p.n_windows, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int n16 = p.n_fp16, n4 = p.n_int4;
    const int M = W - 1;
    auto class_of = [&](int rank) -> int8_t { return rank < n16 - 1 ? 16 : (rank < n16 - 1 + n4 ? 4 : 2); };
    if (M <= kSortMax) {
        int N = 1;
        while (N < M) N <<= 1;
        for (int i = tid; i < N; i += kSelectThreads) {
            key[i] = i < M ? p.score[i + 1] : -__builtin_inf();
            idx[i] = i < M ? i + 1 : 0x7fffffff;   // pads sort last
        }
        __syncthreads();
        for (int k = 2; k <= N; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int i = tid; i < N; i += kSelectThreads) {
                    const int l = i ^ j;
                    if (l > i) {
                        const double si = key[i], sl = key[l];
                        const int ii = idx[i], il = idx[l];
                        // blocks with bit k clear end in "before" order, the others in reverse
                        const bool swap = (i & k) == 0 ? before(sl, il, si, ii) : before(si, ii, sl, il);
                        if (swap) {
                            key[i] = sl; key[l] = si;
                            idx[i] = il; idx[l] = ii;
                        }
                    }
                }
                __syncthreads();
            }
        }
        // position r holds the window of rank r
        for (int r = tid; r < M; r += kSelectThreads) cls[idx[r]] = class_of(r);
    } else {
        for (int w = threadIdx.x; w < W; w += kSelectThreads) {
            if (w == 0) continue;
            const double s = p.score[w];
            int rank = 0;
            for (int v = 1; v < W; ++v) {
                const double t = p.score[v];
                rank += before(t, v, s, w) ? 1 : 0;
            }
            cls[w] = class_of(rank);
        }
    }
    if (tid == 0) cls[0] = 16;
    __syncthreads();
    // class lists, each in ascending window order: FP16 at 0, INT4 at n16, INT2 at n16 + n4
    unsigned long long carry = 0;   // counts of the windows before this chunk, 21 bits per class
    for (int w0 = 0; w0 < W; w0 += kSelectThreads) {
        const int w = w0 + tid;
        const int8_t b = w < W ? cls[w] : 0;
        if (w < W) p.bits_out[w] = b;
        const int sh = b == 16 ? 0 : (b == 4 ? 21 : 42);
        const unsigned long long v = w < W ? 1ull << sh : 0ull;
        unsigned long long x = v;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const unsigned long long y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        if (lane == kWave - 1) wsum[wave] = x;
        __syncthreads();
        unsigned long long pre = carry + x - v, tot = carry;
        for (int k = 0; k < kSelectThreads / kWave; ++k) {
            if (k < wave) pre += wsum[k];
            tot += wsum[k];
        }
        if (w < W) {
            const int before_w = (int)((pre >> sh) & 0x1fffff);
            const int base = b == 16 ? 0 : (b == 4 ? n16 : n16 + n4);
            // ranks form a permutation, so this stays inside the list; never write outside it
            if (base + before_w < W) p.order_out[base + before_w] = w;
        }
        carry = tot;
        __syncthreads();
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
