// Decode-shaped attention over a packed low-bit KV cache: at most 16 query rows per
// (batch, KV head) -- in GQA decode, one token of each query head that shares the KV
// head -- against a long quantized history (plus, optionally, an unquantized current
// chunk). Built for bf16 elements, INT2 at head_dim 64 or 128 and INT4 at head_dim 128,
// one packed segment; other calls take the chunk kernel (decode_eligible).
//
// Method: as the chunk kernel ("Quantized Keys Steal Attention: Bias Correction for
// KV-Cache Compression in Video Diffusion", abstract): logits over packed tokens are
// corrected by beta = tau^2/24 * sum_c q_c^2 step_c^2 of their K-group; no mask; the
// dequantized keys and values exist only in registers and LDS ("KV Cache Quantization
// for Self-Forcing Video Generation", abstract).
//
// With so few rows the work is streaming the packed cache and expanding it, so the
// layout is built for memory-level parallelism and for few vector instructions per
// code rather than for MFMA reuse:
//   - every wave walks its own contiguous token range (no barriers until the end) in
//     steps of 64 INT2 / 32 INT4 tokens (16 for current-chunk tokens); the codes of the next step
//     are loaded into one 20-register set as soon as this step's copy has been expanded
//     (keys after the QK product, values after their LDS write), so each load has about
//     a whole step to land;
//   - keys are dequantized straight into 16x16x32 MFMA operands in registers: lane
//     (token t = L % 16, quarter j = L / 16) expands the codes of its token's quarter
//     row, S^T (tokens x rows) = K^ Q^T; codes become floats two at a time through the
//     fp8 conversion (bytes 0..15 read as OCP e4m3 are c * 2^-9, scaled back by 2^9);
//     the lane keeps the {step, zero} of its quarter's channels for the current K-group;
//   - values are expanded into a wave-private LDS tile (INT2 through a 4-entry table per
//     (token, V group)) and read back transposed into the A operand of
//     O^T += V^T P^T (P in fp16);
//   - online softmax in the log2 domain with a lazily moved running maximum;
//   - the four waves of a workgroup merge their (m, l, O) in LDS at the end; with more
//     than one workgroup per (batch, KV head), the merged partials go to the workspace
//     and the split-combine kernel finishes them.
// Channel order inside 16-channel blocks is the position order of kvq_tile.cuh for K
// operands, Q and V rows; O is written back in channel order.
#include "decode_walk.cuh"
#include "kvq_internal.h"
#include "kvq_tile.cuh"

namespace kvq {
namespace {

using dwalk::DGeo;
using dwalk::kDWaves;
using dwalk::ST_CUR;
using dwalk::ST_END;
using dwalk::ST_PACKED;
using dwalk::Step;
using dwalk::TP;
constexpr int kDThreads = kDWaves * kWave;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kDRescale = 8.0f;  // log2 headroom before the running max is moved

__device__ __forceinline__ Step uniform(Step s) {
    s.kind = __builtin_amdgcn_readfirstlane(s.kind);
    s.seg = __builtin_amdgcn_readfirstlane(s.seg);
    s.g = __builtin_amdgcn_readfirstlane(s.g);
    s.t = __builtin_amdgcn_readfirstlane(s.t);
    s.len = __builtin_amdgcn_readfirstlane(s.len);
    s.new_group = __builtin_amdgcn_readfirstlane(s.new_group);
    s.bits = __builtin_amdgcn_readfirstlane(s.bits);
    return s;
}

// K-group tables read as uniform scalar loads (group_start)
struct DevTab {
    static __device__ __forceinline__ int start(const int32_t *tab, int g) { return group_start(tab, g); }
};
typedef dwalk::Walker<DevTab> Walker;

// Registers of one packed step, loaded a step ahead (8 + 8 + 4 words per lane):
//   INT2: k words 2 b .. (b = 0..3) = token 16 b + L%16, quarter L/16 (HD/64 words each);
//         v = the whole code row of token L; vm = its V {step, zero}s.
//   INT4: k words 4 b .. (b = 0..1) = token 16 b + L%16, quarter L/16 (HD/32 words each);
//         v = half L%2 of the code row of token L/2; vm = the {step, zero}s of that half.
struct DSet {
    u32x4 k[2];
    u32x4 v[2];
    u32x4 vm;
};

template <int N>
__device__ __forceinline__ uint32_t word_of(const u32x4 (&a)[N], int w) {
    const u32x4 x = a[w >> 2];
    return (w & 3) == 0 ? x.x : (w & 3) == 1 ? x.y : (w & 3) == 2 ? x.z : x.w;
}
template <int N>
__device__ __forceinline__ void set_word(u32x4 (&a)[N], int w, uint32_t v) {
    if ((w & 3) == 0) a[w >> 2].x = v;
    else if ((w & 3) == 1) a[w >> 2].y = v;
    else if ((w & 3) == 2) a[w >> 2].z = v;
    else a[w >> 2].w = v;
}

// The next step's loads are unconditional, from rows clamped into the step (a token past
// it repeats the last one: its keys' scores are masked and its values are zeroed in LDS):
// a load under a per-lane condition would have to land before its registers are merged
// with the old contents, which turns every prefetch into a wait for memory.
template <int HD, int PB>
__device__ __forceinline__ void load_k(DSet &d, const AttnParams &p, const Step &st, size_t bh) {
    const int lane = threadIdx.x % kWave;
    const SegmentView &sg = p.segs[st.seg];
    const size_t row0 = bh * (size_t)sg.capacity + st.t;
    const uint32_t *kc = reinterpret_cast<const uint32_t *>(sg.k);
    if (HD == 64 || PB == 2) {   // INT4 only at head_dim 128
        // dwalk::k_words: HD / 64 words per load
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t *src = kc + dwalk::k_word(HD, 2, row0, st.len, b, lane);
            if (HD == 128) {
                const u32x2 w = *reinterpret_cast<const u32x2 *>(src);
                set_word(d.k, 2 * b, w.x);
                set_word(d.k, 2 * b + 1, w.y);
            } else {
                set_word(d.k, b, *src);
            }
        }
    } else {
        // INT4, head_dim 128: 4 words per load
#pragma unroll
        for (int b = 0; b < 2; ++b) d.k[b] = *reinterpret_cast<const u32x4 *>(kc + dwalk::k_word(HD, 4, row0, st.len, b, lane));
    }
}

template <int HD, int PB>
__device__ __forceinline__ void load_v(DSet &d, const AttnParams &p, const Step &st, size_t bh) {
    const int lane = threadIdx.x % kWave;
    const SegmentView &sg = p.segs[st.seg];
    const size_t row0 = bh * (size_t)sg.capacity + st.t;
    const uint32_t *vc = reinterpret_cast<const uint32_t *>(sg.v);
    // dwalk::v_words = HD / 16 words (an INT2 row, an INT4 half row), in 16-byte loads
    if (HD == 64 || PB == 2) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(vc + dwalk::v_word(HD, 2, row0, st.len, lane));
#pragma unroll
        for (int i = 0; i < HD / 64; ++i) d.v[i] = src[i];
        const uint32_t *vm = sg.v_meta + dwalk::vm_word(HD, 2, row0, st.len, lane);   // HD / 32 words
        if (HD == 128) {
            d.vm = *reinterpret_cast<const u32x4 *>(vm);
        } else {
            const u32x2 m = *reinterpret_cast<const u32x2 *>(vm);
            d.vm.x = m.x;
            d.vm.y = m.y;
        }
    } else {   // INT4 at head_dim 128
        const u32x4 *src = reinterpret_cast<const u32x4 *>(vc + dwalk::v_word(HD, 4, row0, st.len, lane));
#pragma unroll
        for (int i = 0; i < HD / 64; ++i) d.v[i] = src[i];
        const u32x2 m = *reinterpret_cast<const u32x2 *>(sg.v_meta + dwalk::vm_word(HD, 4, row0, st.len, lane));
        d.vm.x = m.x;
        d.vm.y = m.y;
    }
}

template <int HD, bool BF16> struct DCtx {
    typedef typename Elem<BF16>::vec vec;
    vec qb[DGeo<HD>::KS];              // B operand: Q^T, quarter L/16 of row L%16, position order
    f32x4 o[DGeo<HD>::DB];             // O^T: positions 16 db + 4 (L/16) + i, row L%16
    u32x4 km[4 * DGeo<HD>::NBL];       // {step, zero} of the quarter's channels, channel order
                                       // (kept as the 16-byte words they are loaded in)
    float m, l, beta;
};

template <int HD>
__device__ __forceinline__ void load_kmeta(u32x4 (&km)[4 * DGeo<HD>::NBL], const AttnParams &p, const Step &st,
                                           size_t bh) {
    const SegmentView &sg = p.segs[st.seg];
    const u32x4 *src =
        reinterpret_cast<const u32x4 *>(sg.k_meta + dwalk::km_word(HD, bh, sg.kgroup_capacity, st.g, threadIdx.x % kWave));
#pragma unroll
    for (int i = 0; i < 4 * DGeo<HD>::NBL; ++i) km[i] = src[i];
}

// the {step, zero}s of 16-channel block bl of the quarter, channel order
template <int HD>
__device__ __forceinline__ void kmeta_block(const u32x4 (&km)[4 * DGeo<HD>::NBL], int bl, uint32_t (&o)[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[4 * i] = km[4 * bl + i].x;
        o[4 * i + 1] = km[4 * bl + i].y;
        o[4 * i + 2] = km[4 * bl + i].z;
        o[4 * i + 3] = km[4 * bl + i].w;
    }
}

// sum over the row's channels of (q_c step_c)^2, for the lane's row; in the isotropic
// form |q|^2 * mean_c step_c^2 instead
// The all-orders form: sum over the row's channels of log2(sinh(a) / a), a = (tau / 2)
// |q_c| step_c (log2 domain already).
template <int HD, bool BF16>
__device__ __forceinline__ float jensen_sum_exact(const DCtx<HD, BF16> &cx, float half_scale) {
    typedef DGeo<HD> G;
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
        const u32x4 qw = __builtin_bit_cast(u32x4, cx.qb[ks]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int pos = 8 * (ks & 1) + i;
            const int ch = 16 * (ks >> 1) + swap_pos(pos);
            const float qv = Elem<BF16>::val((qw[i / 2] >> (16 * (i % 2))) & 0xffffu);
            const float st = mul_step(1.0f, cx.km[ch / 4][ch % 4]);
            acc += log2_sinhc(half_scale * __builtin_fabsf(qv) * st);
        }
    }
    acc += __shfl_xor(acc, 16);
    acc += other_half(acc);
    return acc;
}

template <int HD, bool BF16>
__device__ __forceinline__ float jensen_sum(const DCtx<HD, BF16> &cx, bool iso) {
    typedef DGeo<HD> G;
    float acc = 0.f, qq = 0.f, ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
        const u32x4 qw = __builtin_bit_cast(u32x4, cx.qb[ks]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int pos = 8 * (ks & 1) + i;                // position inside block ks / 2
            const int ch = 16 * (ks >> 1) + swap_pos(pos);   // channel inside the quarter
            const uint32_t qbits = (qw[i / 2] >> (16 * (i % 2))) & 0xffffu;
            const float qv = Elem<BF16>::val(qbits);
            const float t = mul_step(qv, cx.km[ch / 4][ch % 4]);
            acc = __builtin_fmaf(t, t, acc);
            if (iso) {
                const float st = mul_step(1.0f, cx.km[ch / 4][ch % 4]);
                qq = __builtin_fmaf(qv, qv, qq);
                ss = __builtin_fmaf(st, st, ss);
            }
        }
    }
    if (iso) {
        qq += __shfl_xor(qq, 16);
        qq += other_half(qq);
        ss += __shfl_xor(ss, 16);
        ss += other_half(ss);
        return qq * ss * (1.0f / HD);
    }
    acc += __shfl_xor(acc, 16);
    acc += other_half(acc);
    return acc;
}

template <int HD, bool BF16, bool EXACT, int PB, bool CUR>
__device__ __forceinline__ void process_step(DCtx<HD, BF16> &cx, DSet &d, const Step &st, const Step &nx,
                                             uint16_t *vt, const AttnParams &p, size_t bh) {
    typedef DGeo<HD> G;
    typedef Elem<BF16> E;
    typedef typename DCtx<HD, BF16>::vec vec;
    typedef __attribute__((ext_vector_type(4))) short s16x4;
    const int lane = threadIdx.x % kWave, j = lane / 16;
    const bool packed = !CUR || st.kind == ST_PACKED;   // without CUR every step is packed
    const int bits = packed ? PB : 16;   // the launch's one packed segment has PB bits
    const int len = st.len;
    const bool nx_packed = nx.kind == ST_PACKED;

    if (packed && st.new_group) {
        if constexpr (EXACT)
            cx.beta = jensen_sum_exact<HD, BF16>(cx, p.half_scale);
        else
            cx.beta = p.jensen ? p.beta_log2 * jensen_sum<HD, BF16>(cx, p.jensen == JENSEN_ISO) : 0.f;
    }
    if (!packed) cx.beta = 0.f;

    // ---- S^T = K^ Q^T: s[b][i] = logit of token 16 b + 4 j + i for row r16
    // every block of the step, also past its end: those rows repeat the last token (the loads
    // are clamped) and their scores are masked; straight-line code schedules better than
    // blocks split by branches on the step length
    f32x4 s[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) s[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (bits == 2) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int bl = 0; bl < G::NBL; ++bl) {
                uint32_t ko[8], kmb[16];
                kmeta_block<HD>(cx.km, bl, kmb);
                k2_block<BF16>(word_of(d.k, G::NBL * b + bl), kmb, ko);
                s[b] = E::mma16(__builtin_bit_cast(vec, u32x4{ko[0], ko[1], ko[2], ko[3]}), cx.qb[2 * bl], s[b]);
                s[b] = E::mma16(__builtin_bit_cast(vec, u32x4{ko[4], ko[5], ko[6], ko[7]}), cx.qb[2 * bl + 1], s[b]);
            }
        }
    } else if (HD == 128 && bits == 4) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int bl = 0; bl < G::NBL; ++bl) {
                uint32_t ko[8], kmb[16];
                kmeta_block<HD>(cx.km, bl, kmb);
                k4_block<BF16>(word_of(d.k, 2 * G::NBL * b + 2 * bl), word_of(d.k, 2 * G::NBL * b + 2 * bl + 1),
                               kmb, ko);
                s[b] = E::mma16(__builtin_bit_cast(vec, u32x4{ko[0], ko[1], ko[2], ko[3]}), cx.qb[2 * bl], s[b]);
                s[b] = E::mma16(__builtin_bit_cast(vec, u32x4{ko[4], ko[5], ko[6], ko[7]}), cx.qb[2 * bl + 1], s[b]);
            }
        }
    } else {
        // current-chunk keys, read now (a few steps at the end of the walk): quarter j of token r16
        u32x4 kq[G::QV];
        const size_t row0 = bh * (size_t)p.n_cur + st.t;
        const uint16_t *kb = reinterpret_cast<const uint16_t *>(p.k_cur);
        const u32x4 *src = reinterpret_cast<const u32x4 *>(kb + dwalk::ck_elem(HD, row0, len, lane));
#pragma unroll
        for (int i = 0; i < G::QV; ++i) kq[i] = src[i];
#pragma unroll
        for (int bl = 0; bl < G::NBL; ++bl) {
            uint32_t dd[8], ko[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) dd[q] = word_of(kq, 8 * bl + q);
            to_positions(dd, ko);
            s[0] = E::mma16(__builtin_bit_cast(vec, u32x4{ko[0], ko[1], ko[2], ko[3]}), cx.qb[2 * bl], s[0]);
            s[0] = E::mma16(__builtin_bit_cast(vec, u32x4{ko[4], ko[5], ko[6], ko[7]}), cx.qb[2 * bl + 1], s[0]);
        }
    }
    // this step's keys are expanded: fetch the next step's keys and K-group {step, zero}
    if (nx_packed) {
        if (nx.new_group) load_kmeta<HD>(cx.km, p, nx, bh);
        load_k<HD, PB>(d, p, nx, bh);
    }

    // ---- values -> LDS (row = token, position order); rows past the step repeat its last
    // token (finite, and multiplied by p = 0)
    if (bits == 2) {
#pragma unroll
        for (int gv = 0; gv < HD / 32; ++gv) {
            uint32_t tlo, thi;
            v_int2_table<BF16>(d.vm[gv], tlo, thi);
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const int blk = 2 * gv + bb;
                uint32_t vo[8];
                v_int2_block(word_of(d.v, blk), tlo, thi, vo);
                *reinterpret_cast<u32x4 *>(vt + dwalk::vt_int2<HD>(lane, blk, 0)) = u32x4{vo[0], vo[1], vo[2], vo[3]};
                *reinterpret_cast<u32x4 *>(vt + dwalk::vt_int2<HD>(lane, blk, 1)) = u32x4{vo[4], vo[5], vo[6], vo[7]};
            }
        }
    } else if (HD == 128 && bits == 4) {
#pragma unroll
        for (int hb = 0; hb < HD / 32; ++hb) {
            uint32_t vo[8];
            v4_block<BF16>(word_of(d.v, 2 * hb), word_of(d.v, 2 * hb + 1), d.vm[hb / 2], vo);
            *reinterpret_cast<u32x4 *>(vt + dwalk::vt_int4<HD>(lane, hb, 0)) = u32x4{vo[0], vo[1], vo[2], vo[3]};
            *reinterpret_cast<u32x4 *>(vt + dwalk::vt_int4<HD>(lane, hb, 1)) = u32x4{vo[4], vo[5], vo[6], vo[7]};
        }
    } else {
        // current-chunk values, read now: quarter lane % 4 of token lane / 4
        const bool ok = lane / 4 < len;
        const size_t row0 = bh * (size_t)p.n_cur + st.t;
        const uint16_t *vb = reinterpret_cast<const uint16_t *>(p.v_cur);
        u32x4 vq[G::QV];
        const u32x4 *src = reinterpret_cast<const u32x4 *>(vb + dwalk::cv_elem(HD, row0, len, lane));
#pragma unroll
        for (int i = 0; i < G::QV; ++i) vq[i] = src[i];
#pragma unroll
        for (int bl = 0; bl < G::NBL; ++bl) {
            uint32_t dd[8], vo[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) dd[q] = word_of(vq, 8 * bl + q);
            to_positions(dd, vo);
#pragma unroll
            for (int q = 0; q < 8; ++q) vo[q] = ok ? E::raw_to_f16(vo[q]) : 0u;
            *reinterpret_cast<u32x4 *>(vt + dwalk::vt_cur<HD>(lane, bl, 0)) = u32x4{vo[0], vo[1], vo[2], vo[3]};
            *reinterpret_cast<u32x4 *>(vt + dwalk::vt_cur<HD>(lane, bl, 1)) = u32x4{vo[4], vo[5], vo[6], vo[7]};
        }
    }
    // this step's values are in LDS: fetch the next step's
    if (nx_packed) load_v<HD, PB>(d, p, nx, bh);

    // ---- online softmax (log2 domain); tokens past the step do not exist
    if (len < TP) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) s[b][i] = 16 * b + 4 * j + i < len ? s[b][i] : -__builtin_inff();
    }
    float sm = max3(s[0][0], s[0][1], s[0][2]);
    sm = max3(sm, s[0][3], s[1][0]);
    sm = max3(sm, s[1][1], s[1][2]);
    sm = max3(sm, s[1][3], s[2][0]);
    sm = max3(sm, s[2][1], s[2][2]);
    sm = max3(sm, s[2][3], s[3][0]);
    sm = max3(sm, s[3][1], s[3][2]);
    sm = fmaxf(sm, s[3][3]);
    float mt = __builtin_fmaf(sm, p.scale_log2, -cx.beta);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, other_half(mt));
    if (__any(mt > cx.m + kDRescale)) {
        const float mnew = fmaxf(cx.m, mt);
        const float alpha = exp2_fast(cx.m - mnew);
        cx.m = mnew;
        cx.l *= alpha;
#pragma unroll
        for (int db = 0; db < G::DB; ++db) cx.o[db] *= alpha;
    }
    const float off = -(cx.beta + cx.m);
    f16x8 pf[2];
    float ps = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            f16x2 pr;
            pr.x = (_Float16)exp2_fast(__builtin_fmaf(s[2 * h + i / 4][i % 4], p.scale_log2, off));
            pr.y = (_Float16)exp2_fast(__builtin_fmaf(s[2 * h + i / 4][i % 4 + 1], p.scale_log2, off));
            pf[h][i] = pr.x;
            pf[h][i + 1] = pr.y;
            ps = __builtin_amdgcn_fdot2(pr, f16x2{(_Float16)1.0f, (_Float16)1.0f}, ps, false);
        }
    }
    cx.l += ps;

    // ---- O^T += V^T P^T over 32-token slices. A operand, lane group j: positions
    // 16 db + L%16 at tokens 32 h + 4 j + 0..3 (k-slots 0..3) and 32 h + 16 + 4 j + 0..3
    // (k-slots 4..7), the same tokens P's k-slots hold. In each 16-lane group, source lane
    // 4 jj + aa addresses token T + jj at positions 16 db + 4 aa.
    // the wave's own LDS writes above are read below: one wave's LDS operations complete
    // in issue order, and the compiler keeps the reads after the stores they may alias
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int db = 0; db < G::DB; ++db) {
            const uint16_t *p0 = vt + dwalk::vt_read<HD>(lane, h, db);
            const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(p0));
            const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(p0 + 16 * G::VROW));
            const u32x2 lo2 = __builtin_bit_cast(u32x2, lo4), hi2 = __builtin_bit_cast(u32x2, hi4);
            const f16x8 a = __builtin_bit_cast(f16x8, u32x4{lo2.x, lo2.y, hi2.x, hi2.y});
            cx.o[db] = mfma16_f16(a, pf[h], cx.o[db]);
        }
    }
}

// EXACT: the all-orders Jensen form, in its own instance (as in the chunk kernel). PB: the
// bit-width of the launch's packed segment, one instance each. CUR: the launch has a
// current chunk (without it, INT2 instances hold no code for its steps).
template <int HD, bool BF16, bool EXACT, int PB, bool CUR>
__global__ __launch_bounds__(kDThreads, 2) void decode_kernel(AttnParams p) {
    typedef DGeo<HD> G;
    typedef typename DCtx<HD, BF16>::vec vec;
    __shared__ __attribute__((aligned(16))) uint16_t smem[kDWaves * G::VTILE];
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: the walk runs on scalars
    const int r16 = lane % 16, j = lane / 16;
    const int b = blockIdx.y / p.n_kv_heads, h = blockIdx.y % p.n_kv_heads;
    const int gqa = p.n_q_heads / p.n_kv_heads;
    const int rows = gqa * p.n_q;   // <= 16
    const size_t bh = (size_t)b * p.n_kv_heads + h;
    uint16_t *vt = smem + wave * G::VTILE;

    DCtx<HD, BF16> cx;
    {
        // Q^T operand: quarter j of row r16 in position order
        u32x4 qv[G::QV];
        if (r16 < rows) {
            const size_t qrow = dwalk::out_row(b, h, r16, p.n_q_heads, p.n_kv_heads, p.n_q);
            const u32x4 *src =
                reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(p.q) + dwalk::q_elem(HD, qrow, j));
#pragma unroll
            for (int i = 0; i < G::QV; ++i) qv[i] = src[i];
        } else {
#pragma unroll
            for (int i = 0; i < G::QV; ++i) qv[i] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int bl = 0; bl < G::NBL; ++bl) {
            uint32_t dd[8], o8[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) dd[q] = word_of(qv, 8 * bl + q);
            to_positions(dd, o8);
            cx.qb[2 * bl] = __builtin_bit_cast(vec, u32x4{o8[0], o8[1], o8[2], o8[3]});
            cx.qb[2 * bl + 1] = __builtin_bit_cast(vec, u32x4{o8[4], o8[5], o8[6], o8[7]});
        }
    }
#pragma unroll
    for (int db = 0; db < G::DB; ++db) cx.o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4 * G::NBL; ++i) cx.km[i] = u32x4{0u, 0u, 0u, 0u};
    cx.m = -__builtin_inff();
    cx.l = 0.f;
    cx.beta = 0.f;
    // the value tile starts finite: rows past a short step are multiplied by p = 0
    for (int i = lane; i < G::VTILE / 8; i += kWave) reinterpret_cast<u32x4 *>(vt)[i] = u32x4{0u, 0u, 0u, 0u};

    const int part = blockIdx.x * kDWaves + wave;
    const int tb = part * p.split_tokens;
    const int te = min(p.n_total, tb + p.split_tokens);
    Walker wk;
    wk.init();
    DSet d;
#pragma unroll
    for (int i = 0; i < 2; ++i) d.k[i] = d.v[i] = u32x4{0u, 0u, 0u, 0u};
    d.vm = u32x4{0u, 0u, 0u, 0u};
    Step s0 = uniform(wk.next(p, tb, te));
    Step s1 = uniform(wk.next(p, tb, te));
    if (s0.kind == ST_PACKED) {
        load_kmeta<HD>(cx.km, p, s0, bh);
        load_k<HD, PB>(d, p, s0, bh);
        load_v<HD, PB>(d, p, s0, bh);
    }
    while (s0.kind != ST_END) {
        process_step<HD, BF16, EXACT, PB, CUR>(cx, d, s0, s1, vt, p, bh);
        s0 = s1;
        s1 = uniform(wk.next(p, tb, te));
    }

    // ---- merge the four waves: (m, l, O) per row through LDS
    float lt = cx.l + __shfl_xor(cx.l, 16);
    lt += other_half(lt);
    float *sc = reinterpret_cast<float *>(vt);   // the wave's own value tile, no longer read
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[dwalk::epi_o<HD>(r16, swap_pos(16 * db + 4 * j + i))] = cx.o[db][i];
    if (j == 0) {
        sc[dwalk::epi_m<HD>(r16)] = cx.m;
        sc[dwalk::epi_l<HD>(r16)] = lt;
    }
    __syncthreads();
    const size_t n_rows_total = (size_t)p.batch * p.n_q_heads * p.n_q;
    for (int idx = tid; idx < rows * HD; idx += kDThreads) {
        const int r = idx / HD, c = idx % HD;
        float M = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < kDWaves; ++w)
            M = fmaxf(M, reinterpret_cast<const float *>(smem + w * G::VTILE)[dwalk::epi_m<HD>(r)]);
        float L = 0.f, acc = 0.f;
        if (M != -__builtin_inff()) {
#pragma unroll
            for (int w = 0; w < kDWaves; ++w) {
                const float *sw = reinterpret_cast<const float *>(smem + w * G::VTILE);
                const float wt = exp2_fast(sw[dwalk::epi_m<HD>(r)] - M);
                L = __builtin_fmaf(wt, sw[dwalk::epi_l<HD>(r)], L);
                acc = __builtin_fmaf(wt, sw[dwalk::epi_o<HD>(r, c)], acc);
            }
        }
        const size_t qrow = dwalk::out_row(b, h, r, p.n_q_heads, p.n_kv_heads, p.n_q);
        if (gridDim.x == 1) {
            const float v = acc / L;
            if (p.out_dtype == DT_F32) reinterpret_cast<float *>(p.out)[qrow * HD + c] = v;
            else if (p.out_dtype == DT_BF16) reinterpret_cast<uint16_t *>(p.out)[qrow * HD + c] = f32_to_bf16_bits(v);
            else reinterpret_cast<uint16_t *>(p.out)[qrow * HD + c] = f32_to_f16_bits(v);
            if (c == 0 && p.lse != nullptr) p.lse[qrow] = (M + __log2f(L)) * kLn2;
        } else {
            float *pp = p.partial + dwalk::ws_row(blockIdx.x, n_rows_total, qrow) * (HD + 2);
            pp[c] = acc;
            if (c == 0) {
                pp[HD] = M;
                pp[HD + 1] = L;
            }
        }
    }
}

template <int HD, int PB, bool CUR>
hipError_t launch_d(const AttnParams &p, hipStream_t s) {
    constexpr bool BF16 = true;
    dim3 grid(p.n_split, p.batch * p.n_kv_heads);
    if (p.jensen == JENSEN_EXACT)
        hipLaunchKernelGGL((decode_kernel<HD, BF16, true, PB, CUR>), grid, dim3(kDThreads), 0, s, p);
    else
        hipLaunchKernelGGL((decode_kernel<HD, BF16, false, PB, CUR>), grid, dim3(kDThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_split == 1) return e;
    return launch_combine(p, s);
}

}  // namespace

bool decode_eligible(int dtype, int batch, int n_q_heads, int n_kv_heads, int head_dim, int n_q,
                     const int *seg_bits, int n_segs, int n_cur, int n_total) {
    // built for bf16 only, one packed segment (the multi-segment walk is not covered by a
    // passing GPU run), no raw segments, INT4 only at head_dim 128
    if ((long)(n_q_heads / n_kv_heads) * n_q > kDecodeRows || dtype != DT_BF16) return false;
    if (n_segs > 1) return false;
    for (int i = 0; i < n_segs; ++i) {
        if (seg_bits[i] == 16) return false;
        if (seg_bits[i] == 4 && head_dim != 128) return false;
    }
    // the current chunk only when one workgroup walks a (batch, KV head) alone
    if (n_cur > 0) {
        int nw, wt;
        decode_plan(batch, n_kv_heads, n_total, &nw, &wt);
        if (nw != 1) return false;
    }
    return true;
}

void decode_plan(int batch, int n_kv_heads, int n_total, int *n_wg, int *wave_tokens) {
    const long bh = (long)batch * n_kv_heads;
    const long want = (512 + bh - 1) / bh;                       // two workgroups per CU
    const long cap = (n_total + kDWaves * 256 - 1) / (kDWaves * 256);  // >= 256 tokens per wave
    long nw = want < cap ? want : cap;
    if (nw < 1) nw = 1;
    long wt = (n_total + kDWaves * nw - 1) / (kDWaves * nw);
    wt = (wt + TP - 1) / TP * TP;
    nw = (n_total + kDWaves * wt - 1) / (kDWaves * wt);
    if (nw < 1) nw = 1;
    *n_wg = (int)nw;
    *wave_tokens = (int)wt;
}

hipError_t launch_decode(const AttnParams &p, hipStream_t s) {
    // only what decode_eligible admits is built
    if (p.dtype != DT_BF16) return hipErrorInvalidValue;
    // one packed segment at most (none: only current-chunk steps, which any instance walks)
    const int pb = p.n_segs > 0 ? p.segs[0].bits : 2;
    // INT2 without a current chunk in instances of their own (measured faster); INT4 keeps
    // one instance (its specialized one measured slower)
    if (p.head_dim == 64) {
        if (pb != 2) return hipErrorInvalidValue;
        return p.n_cur > 0 ? launch_d<64, 2, true>(p, s) : launch_d<64, 2, false>(p, s);
    }
    if (pb == 4) return launch_d<128, 4, true>(p, s);
    return p.n_cur > 0 ? launch_d<128, 2, true>(p, s) : launch_d<128, 2, false>(p, s);
}

}  // namespace kvq
