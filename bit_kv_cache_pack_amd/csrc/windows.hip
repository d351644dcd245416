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
// Several independent caches (layers) are scored and assigned by the same three launches:
// blockIdx.y is the layer. The selection also writes the grouped layout's gather lists
// ({first token, length} of every window, FP16 windows first, then INT4, then INT2, each
// ascending) and each class's token count, so that the appends can take them as they are.
#include "kvq_device.cuh"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kSelectThreads = 1024;

constexpr int kScoreThreads = 256;
constexpr int kScoreMeans = 2048;   // (head, channel) means held in LDS at once

// One workgroup per window. All (head, channel) means of a chunk of heads are taken in
// parallel (tokens in order, loads issued four at a time), then thread h takes head h's dot
// product and norms (channels in order), and thread 0 averages the heads' cosines in head
// order: the same fp64 operations in the same order as a one-thread loop.
__global__ __launch_bounds__(kScoreThreads) void window_score_kernel(WindowParams p) {
    __shared__ double mean[kScoreMeans];
    __shared__ double cs[kScoreThreads];
    const int w = blockIdx.x, tid = threadIdx.x, layer = blockIdx.y;
    const int d = p.head_dim, H = p.n_kv_heads;
    const size_t kbase = (size_t)layer * H * p.n_tokens * d;
    const float *text = p.text + (size_t)layer * d;
    const int t0 = w * p.window, t1 = min(p.n_tokens, t0 + p.window);
    const int hc = min(kScoreMeans / d, kScoreThreads);   // heads per chunk
    double acc = 0.0;
    for (int h0 = 0; h0 < H; h0 += hc) {
        const int nh = min(hc, H - h0);
        __syncthreads();
        for (int idx = tid; idx < nh * d; idx += kScoreThreads) {
            const int h = h0 + idx / d, c = idx % d;
            const size_t base = kbase + (size_t)h * p.n_tokens * d + c;
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
                const double tv = (double)text[i];
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
    if (tid == 0) p.score[(size_t)layer * p.n_windows + w] = acc / (double)H;
}

// window a comes before window b: higher score, ties to the lower index
__device__ __forceinline__ bool before(double sa, int ia, double sb, int ib) {
    return sa > sb || (sa == sb && ia < ib);
}
__device__ __forceinline__ int8_t class_of(int rank, int n16, int n4) {
    return rank < n16 - 1 ? 16 : (rank < n16 - 1 + n4 ? 4 : 2);
}

constexpr int kRankWaves = 4;

// Rank of windows 1..W-1 among themselves (score descending, ties to the lower index),
// counted: the rank of a window is the number of windows before it. Lane L of workgroup x
// ranks window 1 + 64 x + L; wave q counts over the q-th quarter of the windows, and the
// quarters' counts are summed through LDS. "before" is a strict total order on (score,
// index), so the counts are exactly the positions a sort by it gives. The class follows
// from the rank and the budget (the first n16 - 1 FP16, the next n4 INT4, the rest INT2);
// window 0 is FP16 whatever its score.
__global__ __launch_bounds__(kRankWaves * kWave) void window_rank_kernel(WindowParams p) {
    __shared__ int part[kRankWaves][kWave];
    const int W = p.n_windows, lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const size_t lw = (size_t)blockIdx.y * W;
    const double *score = p.score + lw;
    const int w = 1 + blockIdx.x * kWave + lane;
    const double s = w < W ? score[w] : 0.0;
    const int per = (W - 1 + kRankWaves - 1) / kRankWaves;
    const int v0 = 1 + wave * per, v1 = min(W, v0 + per);
    int rank = 0;
    int v = v0;
    // every lane reads the same score: one request per wave; eight in flight at a time
    for (; v + 8 <= v1; v += 8) {
        double t[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) t[k] = score[v + k];
#pragma unroll
        for (int k = 0; k < 8; ++k) rank += before(t[k], v + k, s, w) ? 1 : 0;
    }
    for (; v < v1; ++v) rank += before(score[v], v, s, w) ? 1 : 0;
    part[wave][lane] = rank;
    __syncthreads();
    if (wave == 0 && w < W) {
        int r = 0;
#pragma unroll
        for (int q = 0; q < kRankWaves; ++q) r += part[q][lane];
        p.bits_out[lw + w] = class_of(r, p.n_fp16, p.n_int4);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) p.bits_out[lw] = 16;
}

// One workgroup per layer, after window_rank_kernel: each class listed in ascending window
// order (FP16 at 0, INT4 at n16, INT2 at n16 + n4) through a block prefix sum, over the
// windows in index order, of three class counters packed in one 64-bit word; the gather
// lists and each class's token count alongside.
__global__ __launch_bounds__(kSelectThreads) void window_select_kernel(WindowParams p) {
    __shared__ int8_t cls[kMaxWindowsPerLayer];
    __shared__ unsigned long long wsum[kSelectThreads / kWave];
    const int W = p.n_windows, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int n16 = p.n_fp16, n4 = p.n_int4;
    const size_t lw = (size_t)blockIdx.y * W;   // this layer's windows
    const int8_t *bits_in = p.bits_out + lw;
    int32_t *order_out = p.order_out + lw;
    int32_t *groups_out = p.groups_out != nullptr ? p.groups_out + 2 * lw : nullptr;
    for (int w = tid; w < W; w += kSelectThreads) cls[w] = bits_in[w];
    __syncthreads();
    // class lists, each in ascending window order: FP16 at 0, INT4 at n16, INT2 at n16 + n4
    unsigned long long carry = 0;   // counts of the windows before this chunk, 21 bits per class
    for (int w0 = 0; w0 < W; w0 += kSelectThreads) {
        const int w = w0 + tid;
        const int8_t b = w < W ? cls[w] : 0;
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
            const int pos = base + before_w;
            if (pos < W) {
                order_out[pos] = w;
                if (groups_out != nullptr) {
                    const int t0 = w * p.window;
                    groups_out[2 * pos] = t0;
                    groups_out[2 * pos + 1] = min(p.window, p.n_tokens - t0);
                }
            }
        }
        carry = tot;
        __syncthreads();
    }
    // tokens per class: whole windows, less what the last window lacks in its own class
    if (tid == 0 && p.class_tokens_out != nullptr) {
        const int last = cls[W - 1];
        const int short_by = W * p.window - p.n_tokens;
        const int counts[3] = {n16, n4, W - n16 - n4};
        const int which[3] = {16, 4, 2};
        int32_t *ct = p.class_tokens_out + 3 * (size_t)blockIdx.y;
        for (int k = 0; k < 3; ++k) ct[k] = counts[k] * p.window - (which[k] == last ? short_by : 0);
    }
}

}  // namespace

hipError_t launch_windows(const WindowParams &p, hipStream_t s) {
    hipLaunchKernelGGL(window_score_kernel, dim3(p.n_windows, p.n_layers), dim3(kScoreThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int rank_wg = p.n_windows > 1 ? (p.n_windows - 1 + kWave - 1) / kWave : 1;
    hipLaunchKernelGGL(window_rank_kernel, dim3(rank_wg, p.n_layers), dim3(kRankWaves * kWave), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(window_select_kernel, dim3(1, p.n_layers), dim3(kSelectThreads), 0, s, p);
    return hipGetLastError();
}

void window_budget(int n_windows, int pct_fp16, int pct_int4, int *n_fp16, int *n_int4) {
    // floor over all windows in integer arithmetic; window 0 counts inside the FP16 share,
    // which keeps at least one window
    const long long W = n_windows;
    long long n16 = W * pct_fp16 / 100;
    long long n4 = W * (pct_fp16 + pct_int4) / 100 - n16;
    if (n16 < 1) n16 = 1;
    if (n4 > W - n16) n4 = W - n16;
    if (n4 < 0) n4 = 0;
    *n_fp16 = (int)n16;
    *n_int4 = (int)n4;
}

}  // namespace kvq
