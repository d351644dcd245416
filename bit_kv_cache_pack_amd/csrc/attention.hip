// Fused chunk attention over a packed low-bit KV cache plus an unquantized current chunk,
// with the per-score Jensen-bias correction.
//
// Method: "Quantized Keys Steal Attention: Bias Correction for KV-Cache Compression in
// Video Diffusion", abstract: queries of the current chunk attend a quantized cache of
// earlier chunks and their own unquantized chunk; rounding noise on cached keys raises
// their softmax weight on average (exp is convex), which a per-score term computed from
// the keys' step sizes and the query removes to second order. Here that term is
//   beta(i, g) = tau^2/24 * sum_c q_ic^2 step_gc^2
// (half the variance of tau * q . e for e_c uniform on [-step_c/2, step_c/2]),
// subtracted from every logit of a token in K-group g. "KV Cache Quantization for
// Self-Forcing Video Generation", abstract: rebuilding full-precision K/V buffers
// during attention forfeits the memory saved, so dequantized tiles live only in LDS.
// WindowQuant notes ("技術的に面白い点"): windows of one bit-width are stored together;
// each such segment is walked with its own bit-width.
//
// Workgroup: 4 waves, 128 query rows (32 per wave; rows of a KV head's query heads
// are packed, so GQA decode fills the rows), one (batch, KV head), one token split.
// Per 64-token tile (never straddling a K-group):
//   1. all threads dequantize K into LDS as [token][channel] (element dtype) and V
//      into LDS as [channel][token] in fp16, token order permuted inside each
//      16-token block so a PV operand is one 16-byte read;
//   2. each wave computes S^T = K Q^T (MFMA 32x32x16, lanes own queries), applies
//      scale, Jensen term, ragged-tile mask and the online softmax (per-lane max/sum,
//      one cross-lane exchange), and accumulates O^T += V^T P^T (MFMA 32x32x16 f16,
//      P in fp16).
// With several splits, unnormalized partials go to the workspace and a combine
// kernel merges them by log-sum-exp.
#include "kvq_device.cuh"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 128;   // query rows per workgroup
constexpr int TT = 64;    // tokens per tile
constexpr int PAD = 8;    // LDS row padding, elements
constexpr float kLn2 = 0.69314718055994530942f;

template <int HD> struct alignas(16) Smem {
    uint16_t k[TT][HD + PAD];      // dequantized keys, element dtype
    uint16_t vt[HD][TT + PAD];     // dequantized values, fp16, transposed + permuted
    float step[2][HD];             // K step of the current group (double-buffered)
    float zero[2][HD];
};

// Position of token t (0..63) inside a V^T row: bits 2 and 3 of t swapped.
__device__ __forceinline__ int vpos(int t) {
    return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1);
}

template <bool BF16> struct Elem;
template <> struct Elem<true> {
    typedef bf16x8 vec;
    static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_bf16x2(a, b); }
    // spec rounding of a value, returned as the fp16 pair used by the PV product
    static __device__ __forceinline__ uint32_t pack_v(float a, float b) {
        return bf16x2_to_f16x2(pack_bf16x2(a, b));
    }
    static __device__ __forceinline__ uint32_t raw_to_f16(uint32_t p) { return bf16x2_to_f16x2(p); }
    static __device__ __forceinline__ f32x16 mma(vec a, vec b, f32x16 c) { return mfma32_bf16(a, b, c); }
    static __device__ __forceinline__ float to_f32(uint32_t bits) { return bf16_bits_to_f32(bits); }
};
template <> struct Elem<false> {
    typedef f16x8 vec;
    static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_f16x2(a, b); }
    static __device__ __forceinline__ uint32_t pack_v(float a, float b) { return pack_f16x2(a, b); }
    static __device__ __forceinline__ uint32_t raw_to_f16(uint32_t p) { return p; }
    static __device__ __forceinline__ f32x16 mma(vec a, vec b, f32x16 c) { return mfma32_f16(a, b, c); }
    static __device__ __forceinline__ float to_f32(uint32_t bits) { return f16_bits_to_f32(bits); }
};

template <int HD, bool BF16> struct Ctx {
    typedef Elem<BF16> E;
    typedef typename E::vec vec;
    static constexpr int KS = HD / 16;   // k-steps of the QK product
    static constexpr int DB = HD / 32;   // 32-channel blocks of the output

    vec q[KS];          // this lane's query row, B-operand layout
    f32x16 o[DB];       // O^T accumulators
    float m, l;         // running max (log2 domain) and this lane's partial sum
    float beta;         // Jensen term of the current group, log2 domain
};

// ---------------------------------------------------------------- tile loaders
template <int HD, bool BF16, int BITS>
__device__ __forceinline__ void load_packed_tile(Smem<HD> &sm, int slot, const SegmentView &sg,
                                                 size_t row0, int t0, int len) {
    typedef Elem<BF16> E;
    constexpr int CPW = 32 / BITS;           // channels per word
    constexpr int WPR = HD * BITS / 32;      // words per token row
    constexpr uint32_t LM = (1u << BITS) - 1u;
    const int tid = threadIdx.x;
    const uint32_t *kc = reinterpret_cast<const uint32_t *>(sg.k) + (row0 + t0) * WPR;
    const uint32_t *vc = reinterpret_cast<const uint32_t *>(sg.v) + (row0 + t0) * WPR;

    // K: one word (CPW channels of one token) per unit
    for (int u = tid; u < TT * WPR; u += kThreads) {
        const int r = u / WPR, wc = u % WPR;
        uint32_t w = r < len ? kc[(size_t)r * WPR + wc] : 0u;
        uint32_t out[CPW / 2];
#pragma unroll
        for (int i = 0; i < CPW; i += 2) {
            const int c = wc * CPW + i;
            float a = fmaf((float)((w >> (BITS * i)) & LM), sm.step[slot][c], sm.zero[slot][c]);
            float b = fmaf((float)((w >> (BITS * (i + 1))) & LM), sm.step[slot][c + 1], sm.zero[slot][c + 1]);
            out[i / 2] = r < len ? E::pack(a, b) : 0u;
        }
        uint32_t *dst = reinterpret_cast<uint32_t *>(&sm.k[r][wc * CPW]);
#pragma unroll
        for (int i = 0; i < CPW / 2; i += 4) {
            u32x4 v4 = {out[i], out[i + 1], out[i + 2], out[i + 3]};
            *reinterpret_cast<u32x4 *>(dst + i) = v4;
        }
    }
    // V: a pair of tokens x one word per unit; V groups are 32 channels per token
    const uint32_t *vm = sg.v_meta + (row0 + t0) * (HD / 32);
    for (int u = tid; u < (TT / 2) * WPR; u += kThreads) {
        const int pr = u % (TT / 2), wc = u / (TT / 2);
        const int r0 = 2 * pr, r1 = r0 + 1;
        const int gv = (wc * CPW) / 32;
        uint32_t w0 = r0 < len ? vc[(size_t)r0 * WPR + wc] : 0u;
        uint32_t w1 = r1 < len ? vc[(size_t)r1 * WPR + wc] : 0u;
        uint32_t m0 = r0 < len ? vm[(size_t)r0 * (HD / 32) + gv] : 0u;
        uint32_t m1 = r1 < len ? vm[(size_t)r1 * (HD / 32) + gv] : 0u;
        const float s0 = f16_bits_to_f32(m0 & 0xffffu), z0 = f16_bits_to_f32(m0 >> 16);
        const float s1 = f16_bits_to_f32(m1 & 0xffffu), z1 = f16_bits_to_f32(m1 >> 16);
        const int pos = vpos(r0);
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            float a = fmaf((float)((w0 >> (BITS * i)) & LM), s0, z0);
            float b = fmaf((float)((w1 >> (BITS * i)) & LM), s1, z1);
            uint32_t pk = E::pack_v(a, b);
            if (r0 >= len) pk = 0u;
            else if (r1 >= len) pk &= 0xffffu;
            *reinterpret_cast<uint32_t *>(&sm.vt[wc * CPW + i][pos]) = pk;
        }
    }
}

// raw tokens (bits-16 segment or the current chunk): [token][channel] element dtype
template <int HD, bool BF16>
__device__ __forceinline__ void load_raw_tile(Smem<HD> &sm, const uint16_t *kbase, const uint16_t *vbase,
                                              int len) {
    typedef Elem<BF16> E;
    constexpr int CH = HD / 8;  // 16-byte chunks per row
    const int tid = threadIdx.x;
    for (int u = tid; u < TT * CH; u += kThreads) {
        const int r = u / CH, c8 = u % CH;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < len) v = *reinterpret_cast<const u32x4 *>(kbase + (size_t)r * HD + c8 * 8);
        *reinterpret_cast<u32x4 *>(&sm.k[r][c8 * 8]) = v;
    }
    for (int u = tid; u < (TT / 2) * CH; u += kThreads) {
        const int pr = u % (TT / 2), c8 = u / (TT / 2);
        const int r0 = 2 * pr, r1 = r0 + 1;
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (r0 < len) a = *reinterpret_cast<const u32x4 *>(vbase + (size_t)r0 * HD + c8 * 8);
        if (r1 < len) b = *reinterpret_cast<const u32x4 *>(vbase + (size_t)r1 * HD + c8 * 8);
        uint32_t aw[4] = {E::raw_to_f16(a.x), E::raw_to_f16(a.y), E::raw_to_f16(a.z), E::raw_to_f16(a.w)};
        uint32_t bw[4] = {E::raw_to_f16(b.x), E::raw_to_f16(b.y), E::raw_to_f16(b.z), E::raw_to_f16(b.w)};
        const int pos = vpos(r0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // channel 2i: low halves of a and b; channel 2i+1: high halves
            *reinterpret_cast<uint32_t *>(&sm.vt[c8 * 8 + 2 * i][pos]) = (aw[i] & 0xffffu) | (bw[i] << 16);
            *reinterpret_cast<uint32_t *>(&sm.vt[c8 * 8 + 2 * i + 1][pos]) = (aw[i] >> 16) | (bw[i] & 0xffff0000u);
        }
    }
}

// ---------------------------------------------------------------- per-wave compute
template <int HD, bool BF16>
__device__ __forceinline__ void compute_tile(Ctx<HD, BF16> &cx, const Smem<HD> &sm, int len, float scale_log2,
                                             float beta_log2) {
    typedef Ctx<HD, BF16> C;
    typedef typename C::vec vec;
    const int lane = threadIdx.x % kWave;
    const int r32 = lane % 32, hh = lane / 32;

    // S^T (tokens x queries): two 32-token row blocks
    f32x16 s[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        s[rb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            vec a = *reinterpret_cast<const vec *>(&sm.k[32 * rb + r32][16 * ks + 8 * hh]);
            s[rb] = C::E::mma(a, cx.q[ks], s[rb]);
        }
    }
    // online softmax, log2 domain; token of s[rb][j] = 32 rb + 8 (j/4) + 4 hh + j%4
    float mt = -__builtin_inff();
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int tok = 32 * rb + 8 * (j / 4) + 4 * hh + (j % 4);
            float x = fmaf(s[rb][j], scale_log2, -beta_log2);
            x = tok < len ? x : -__builtin_inff();
            s[rb][j] = x;
            mt = fmaxf(mt, x);
        }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mnew = fmaxf(cx.m, mt);
    const float alpha = exp2f(cx.m - mnew);
    cx.m = mnew;
    float ps = 0.f;
    f16x8 pf[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float p = exp2f(s[st / 2][8 * (st % 2) + i] - mnew);
            ps += p;
            pf[st][i] = (_Float16)p;
        }
    }
    cx.l = cx.l * alpha + ps;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) cx.o[db] *= alpha;
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            f16x8 a = *reinterpret_cast<const f16x8 *>(&sm.vt[32 * db + r32][16 * st + 8 * hh]);
            cx.o[db] = mfma32_f16(a, pf[st], cx.o[db]);
        }
}

// Jensen term of one K-group for this lane's query (log2 domain).
template <int HD, bool BF16>
__device__ __forceinline__ float group_beta(const Ctx<HD, BF16> &cx, const Smem<HD> &sm, int slot,
                                            float beta_log2) {
    const int hh = (threadIdx.x % kWave) / 32;
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < Ctx<HD, BF16>::KS; ++ks) {
        const u32x4 qw = __builtin_bit_cast(u32x4, cx.q[ks]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t bits = (qw[i / 2] >> (16 * (i % 2))) & 0xffffu;
            const float qv = Elem<BF16>::to_f32(bits);
            const float t = qv * sm.step[slot][16 * ks + 8 * hh + i];
            acc = fmaf(t, t, acc);
        }
    }
    acc += __shfl_xor(acc, 32);
    return acc * beta_log2;
}

template <int HD, bool BF16>
__global__ __launch_bounds__(kThreads) void attention_kernel(AttnParams p) {
    typedef Ctx<HD, BF16> C;
    typedef typename C::vec vec;
    __shared__ Smem<HD> sm;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int r32 = lane % 32, hh = lane / 32;
    const int b = blockIdx.y / p.n_kv_heads, h = blockIdx.y % p.n_kv_heads;
    const int gqa = p.n_q_heads / p.n_kv_heads;
    const int rows = gqa * p.n_q;
    const int row = blockIdx.x * BM + wave * 32 + r32;
    const bool row_ok = row < rows;
    const bool wave_ok = blockIdx.x * BM + wave * 32 < rows;
    const int hq = h * gqa + (row_ok ? row / p.n_q : 0);
    const int qi = row_ok ? row % p.n_q : 0;
    const size_t qrow = ((size_t)b * p.n_q_heads + hq) * p.n_q + qi;

    C cx;
    {
        const uint16_t *qp = reinterpret_cast<const uint16_t *>(p.q) + qrow * HD + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row_ok) v = *reinterpret_cast<const u32x4 *>(qp + 16 * ks);
            cx.q[ks] = __builtin_bit_cast(vec, v);
        }
    }
#pragma unroll
    for (int db = 0; db < C::DB; ++db) cx.o[db] = f32x16{};
    cx.m = -__builtin_inff();
    cx.l = 0.f;

    const int tb = blockIdx.z * p.split_tokens;
    const int te = min(p.n_total, tb + p.split_tokens);
    const size_t bh = (size_t)b * p.n_kv_heads + h;
    int gcount = 0;  // groups visited, selects the meta slot

    for (int si = 0; si < p.n_segs; ++si) {
        const SegmentView &sg = p.segs[si];
        const int a = max(tb, sg.token_begin) - sg.token_begin;
        const int e = min(te, sg.token_begin + sg.n_tokens) - sg.token_begin;
        if (a >= e) continue;
        const size_t row0 = bh * (size_t)sg.capacity;
        if (sg.bits == 16) {
            for (int t = a; t < e; t += TT) {
                const int len = min(TT, e - t);
                __syncthreads();
                load_raw_tile<HD, BF16>(sm, reinterpret_cast<const uint16_t *>(sg.k) + (row0 + t) * HD,
                                        reinterpret_cast<const uint16_t *>(sg.v) + (row0 + t) * HD, len);
                __syncthreads();
                if (wave_ok) compute_tile<HD, BF16>(cx, sm, len, p.scale_log2, 0.f);
            }
            continue;
        }
        // first K-group ending after token a
        int lo = 0, hi = sg.n_kgroups - 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (sg.kgroup_start[mid + 1] <= a) lo = mid + 1; else hi = mid;
        }
        for (int g = lo; g < sg.n_kgroups; ++g) {
            // clamped: a corrupt table must not send reads outside the segment
            const int gs = min(max(sg.kgroup_start[g], 0), sg.n_tokens);
            const int ge = min(max(sg.kgroup_start[g + 1], gs), sg.n_tokens);
            if (gs >= e) break;
            const int t0 = max(gs, a), t1 = min(ge, e);
            if (t0 >= t1) continue;
            const int slot = gcount & 1;
            ++gcount;
            const uint32_t *km = sg.k_meta + (bh * sg.kgroup_capacity + g) * HD;
            for (int c = tid; c < HD; c += kThreads) {
                const uint32_t mv = km[c];
                sm.step[slot][c] = f16_bits_to_f32(mv & 0xffffu);
                sm.zero[slot][c] = f16_bits_to_f32(mv >> 16);
            }
            bool first = true;
            for (int t = t0; t < t1; t += TT) {
                const int len = min(TT, t1 - t);
                __syncthreads();
                if (sg.bits == 2) load_packed_tile<HD, BF16, 2>(sm, slot, sg, row0, t, len);
                else load_packed_tile<HD, BF16, 4>(sm, slot, sg, row0, t, len);
                __syncthreads();
                if (wave_ok) {
                    if (first) cx.beta = group_beta<HD, BF16>(cx, sm, slot, p.beta_log2);
                    compute_tile<HD, BF16>(cx, sm, len, p.scale_log2, cx.beta);
                }
                first = false;
            }
        }
    }
    // current chunk
    {
        const int cb = p.n_total - p.n_cur;
        const int a = max(tb, cb) - cb, e = min(te, p.n_total) - cb;
        const size_t row0 = bh * (size_t)p.n_cur;
        for (int t = a; t < e; t += TT) {
            const int len = min(TT, e - t);
            __syncthreads();
            load_raw_tile<HD, BF16>(sm, reinterpret_cast<const uint16_t *>(p.k_cur) + (row0 + t) * HD,
                                    reinterpret_cast<const uint16_t *>(p.v_cur) + (row0 + t) * HD, len);
            __syncthreads();
            if (wave_ok) compute_tile<HD, BF16>(cx, sm, len, p.scale_log2, 0.f);
        }
    }

    // epilogue: lane (query r32, half hh) holds O^T[32 db + 8 (j/4) + 4 hh + j%4][query]
    const float lt = cx.l + __shfl_xor(cx.l, 32);
    if (!row_ok) return;
    if (p.n_split == 1) {
        const float inv = 1.0f / lt;
        if (p.out_dtype == DT_F32) {
            float *op = reinterpret_cast<float *>(p.out) + qrow * HD;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    f32x4 v = {cx.o[db][4 * jj] * inv, cx.o[db][4 * jj + 1] * inv, cx.o[db][4 * jj + 2] * inv,
                               cx.o[db][4 * jj + 3] * inv};
                    *reinterpret_cast<f32x4 *>(op + 32 * db + 8 * jj + 4 * hh) = v;
                }
        } else {
            uint16_t *op = reinterpret_cast<uint16_t *>(p.out) + qrow * HD;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float v0 = cx.o[db][4 * jj] * inv, v1 = cx.o[db][4 * jj + 1] * inv;
                    const float v2 = cx.o[db][4 * jj + 2] * inv, v3 = cx.o[db][4 * jj + 3] * inv;
                    u32x2 w;
                    if (p.out_dtype == DT_BF16) {
                        w.x = pack_bf16x2(v0, v1);
                        w.y = pack_bf16x2(v2, v3);
                    } else {
                        w.x = pack_f16x2(v0, v1);
                        w.y = pack_f16x2(v2, v3);
                    }
                    *reinterpret_cast<u32x2 *>(op + 32 * db + 8 * jj + 4 * hh) = w;
                }
        }
        if (p.lse != nullptr && hh == 0) p.lse[qrow] = (cx.m + __log2f(lt)) * kLn2;
    } else {
        const size_t n_rows_total = (size_t)p.batch * p.n_q_heads * p.n_q;
        float *pp = p.partial + ((size_t)blockIdx.z * n_rows_total + qrow) * (HD + 2);
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                // partial rows are HD+2 floats: not 16-byte aligned in general
#pragma unroll
                for (int k = 0; k < 4; ++k) pp[32 * db + 8 * jj + 4 * hh + k] = cx.o[db][4 * jj + k];
            }
        if (hh == 0) {
            pp[HD] = cx.m;
            pp[HD + 1] = lt;
        }
    }
}

// Merge token splits: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <int HD>
__global__ __launch_bounds__(HD) void combine_kernel(AttnParams p) {
    const size_t row = blockIdx.x;
    const size_t n_rows_total = (size_t)p.batch * p.n_q_heads * p.n_q;
    const int c = threadIdx.x;
    float M = -__builtin_inff();
    for (int s = 0; s < p.n_split; ++s) M = fmaxf(M, p.partial[((size_t)s * n_rows_total + row) * (HD + 2) + HD]);
    float L = 0.f, acc = 0.f;
    for (int s = 0; s < p.n_split; ++s) {
        const float *pp = p.partial + ((size_t)s * n_rows_total + row) * (HD + 2);
        const float w = exp2f(pp[HD] - M);
        L = fmaf(w, pp[HD + 1], L);
        acc = fmaf(w, pp[c], acc);
    }
    const float v = acc / L;
    if (p.out_dtype == DT_F32) reinterpret_cast<float *>(p.out)[row * HD + c] = v;
    else if (p.out_dtype == DT_BF16) reinterpret_cast<uint16_t *>(p.out)[row * HD + c] = f32_to_bf16_bits(v);
    else reinterpret_cast<uint16_t *>(p.out)[row * HD + c] = f32_to_f16_bits(v);
    if (c == 0 && p.lse != nullptr) p.lse[row] = (M + __log2f(L)) * kLn2;
}

template <int HD, bool BF16>
hipError_t launch_t(const AttnParams &p, hipStream_t s) {
    const int rows = (p.n_q_heads / p.n_kv_heads) * p.n_q;
    dim3 grid((rows + BM - 1) / BM, p.batch * p.n_kv_heads, p.n_split);
    hipLaunchKernelGGL((attention_kernel<HD, BF16>), grid, dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_split == 1) return e;
    const unsigned n_rows_total = (unsigned)p.batch * p.n_q_heads * p.n_q;
    hipLaunchKernelGGL((combine_kernel<HD>), dim3(n_rows_total), dim3(HD), 0, s, p);
    return hipGetLastError();
}

}  // namespace

void attention_plan(int batch, int n_q_heads, int n_kv_heads, int head_dim, int n_q, int n_total,
                    int *n_split, int *split_tokens, size_t *workspace_bytes) {
    const long rows = (long)(n_q_heads / n_kv_heads) * n_q;
    const long base = (rows + BM - 1) / BM * (long)batch * n_kv_heads;
    long ns = 1;
    if (base < 256) {
        const long want = (512 + base - 1) / base;
        const long cap = (n_total + 255) / 256;  // at least 256 tokens per split
        ns = want < cap ? want : cap;
        if (ns < 1) ns = 1;
    }
    long st = (n_total + ns - 1) / ns;
    st = (st + TT - 1) / TT * TT;
    if (st < TT) st = TT;
    ns = (n_total + st - 1) / st;
    if (ns < 1) ns = 1;
    *n_split = (int)ns;
    *split_tokens = (int)st;
    *workspace_bytes = ns > 1 ? (size_t)ns * batch * n_q_heads * n_q * (head_dim + 2) * sizeof(float) : 0;
}

hipError_t launch_attention(const AttnParams &p, hipStream_t s) {
    const bool bf = p.dtype == DT_BF16;
    if (p.head_dim == 64) return bf ? launch_t<64, true>(p, s) : launch_t<64, false>(p, s);
    return bf ? launch_t<128, true>(p, s) : launch_t<128, false>(p, s);
}

}  // namespace kvq
