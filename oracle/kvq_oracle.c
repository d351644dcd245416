/*
 * kvq_oracle.c -- TEST INFRASTRUCTURE, not part of the product.
 *
 * A plain, slow, scalar CPU model of low-bit KV-cache quantize-pack and of
 * Jensen-corrected attention over such a cache. Only the test-suite, the smoke
 * check and the benchmark's CPU-baseline leg load it. It shares no code, header,
 * table or helper with the HIP library, and neither side includes the other.
 *
 * Sources (cited by page title and section):
 *  [JB]  "Quantized Keys Steal Attention: Bias Correction for KV-Cache Compression
 *        in Video Diffusion", abstract: chunk-wise cache of earlier chunks; the
 *        Jensen bias of quantized keys against the unquantized current chunk; a
 *        per-score correction from the cached keys' step sizes and the query,
 *        second-order Taylor form, no extra memory; INT2.
 *  [SF]  "KV Cache Quantization for Self-Forcing Video Generation: A 33-Method
 *        Empirical Study", abstract: INT4 KV caches; integrations that rebuild
 *        BF16 buffers during attention.
 *  [WQ]  WindowQuant notes ("論文メモ：動画VLMのKV Cacheを軽量化するWindowQuant"),
 *        sections "何が新しいのか", "技術的に面白い点", "実装者視点で気になった点":
 *        32-token windows, cosine similarity to the text query, FP16/INT4/INT2 by
 *        relevance, window 0 kept in FP16, equal-bit windows stored together.
 *  [QW]  "QuantWM Preserves Attention in 2-Bit KV Cache Quantization for Video
 *        World Models": 2-bit K/V caches; keys matter through the logits.
 *
 * The pages give no formula for the quantizer; the readings used here (asymmetric
 * min/max groups, fp16 step and zero, codes from the fp16-rounded step, ties to
 * even, per-channel K groups, per-token V groups of 32 channels, dense packing LSB
 * first) are the plainest ones consistent with "quantization step sizes" [JB] and
 * with INT2/INT4 caches [JB][SF][WQ].
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -shared -fPIC. With
 * -ffp-contract=off and SSE arithmetic every float expression below is rounded
 * once per operation, in the order written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2

/* ------------------------------------------------------------------------ */
/* Number formats. IEEE binary16 and bfloat16, round to nearest, ties to even. */

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* binary16 -> value: (-1)^s * 2^(e-15) * 1.m, subnormal 2^-14 * 0.m */
double orc_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

float orc_f16_to_f32(uint16_t h) { return (float)orc_f16_to_f64(h); }

/* value -> nearest binary16, ties to even (x must be exactly representable as a
 * double, which every float and every exact sum used here is). */
uint16_t orc_f64_to_f16(double x)
{
    if (isnan(x))
        return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a >= 65520.0) /* half-way between 65504 and 2^16 rounds to even = 2^16 */
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) { /* subnormal: units of 2^-24 */
        double q = nearbyint(ldexp(a, 24));           /* ties to even */
        return sign | (uint16_t)q;                     /* q == 1024 is the min normal */
    }
    int E;
    frexp(a, &E);                                      /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1;                                     /* a in [2^e, 2^(e+1)) */
    double q = nearbyint(ldexp(a, 10 - e));            /* in [1024, 2048] */
    uint32_t bits = (uint32_t)((e + 15) << 10) + (uint32_t)q - 1024u; /* carry bumps e */
    return sign | (uint16_t)bits;
}

uint16_t orc_f32_to_f16(float x) { return orc_f64_to_f16((double)x); }

float orc_bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

/* float -> nearest bfloat16 (8 significant bits, float's exponent range) */
uint16_t orc_f32_to_bf16(float x)
{
    uint32_t u = f32_bits(x);
    if (isnan(x))
        return (uint16_t)((u >> 16) | 0x40);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb; /* below half: truncates; above: carries; exactly half: to even */
    return (uint16_t)(u >> 16);
}

/* value -> nearest bfloat16, ties to even (x exactly representable as a double): 8
 * significant bits, float's exponent range; below 2^-126 in units of 2^-133. */
uint16_t orc_f64_to_bf16(double x)
{
    if (isnan(x))
        return 0x7fc0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a >= ldexp(255.0 / 128.0 + 1.0 / 256.0, 127)) /* half-way past the largest bf16: to infinity */
        return sign | 0x7f80;
    if (a < ldexp(1.0, -126)) {
        double q = nearbyint(ldexp(a, 133));
        return sign | (uint16_t)q;
    }
    int E;
    frexp(a, &E);
    int e = E - 1;                                     /* a in [2^e, 2^(e+1)) */
    double q = nearbyint(ldexp(a, 7 - e));             /* in [128, 256] */
    uint32_t bits = (uint32_t)((e + 127) << 7) + (uint32_t)q - 128u;
    return sign | (uint16_t)bits;
}

/* Round a float to an element dtype and return the rounded value as a double. */
static double round_elem(float y, int elem_dtype)
{
    if (elem_dtype == ORC_F16)
        return orc_f16_to_f64(orc_f32_to_f16(y));
    if (elem_dtype == ORC_BF16)
        return (double)orc_bf16_to_f32(orc_f32_to_bf16(y));
    return (double)y;
}

/* ------------------------------------------------------------------------ */
/* Q1: asymmetric min/max quantization of one group of n values.
 *   mn, mx       extremes of the group
 *   step         = fp16(fl32(fl32(mx - mn) / (2^b - 1)))
 *   zero         = fp16(mn)
 *   code_i       = clamp(rint(fl32(fl32(x_i - zero) / step)), 0, 2^b - 1), 0 if step == 0
 * Codes are taken against the fp16-rounded step and zero, the values a reader of
 * the cache has. x is read with a stride so one routine serves K (a channel over
 * the tokens of a group) and V (a run of channels of one token). */
void orc_quantize_group(const float *x, int64_t n, int64_t stride, int bits,
                        uint16_t *step_h, uint16_t *zero_h, uint8_t *codes, int64_t code_stride)
{
    const int L = (1 << bits) - 1;
    float mn = x[0], mx = x[0];
    for (int64_t i = 1; i < n; ++i) {
        float v = x[i * stride];
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    mn = mn + 0.0f; /* a zero extreme is taken as +0, whichever signed zero came first */
    mx = mx + 0.0f;
    float range = mx - mn;
    float step32 = range / (float)L;
    uint16_t sh = orc_f32_to_f16(step32);
    uint16_t zh = orc_f32_to_f16(mn);
    float step = orc_f16_to_f32(sh), zero = orc_f16_to_f32(zh);
    for (int64_t i = 0; i < n; ++i) {
        int c = 0;
        if (step != 0.0f) {
            float diff = x[i * stride] - zero;
            float t = diff / step;
            float r = rintf(t); /* current rounding mode: nearest, ties to even */
            if (r < 0.0f) r = 0.0f;
            if (r > (float)L) r = (float)L;
            c = (int)r;
        }
        codes[i * code_stride] = (uint8_t)c;
    }
    *step_h = sh;
    *zero_h = zh;
}

/* A1: the dequantized element as the cache's reader sees it:
 *   exact == 0: E(fl32(code * step + zero)), E = rounding to the element dtype
 *   exact != 0: code * step + zero in real arithmetic (exact in double)          */
double orc_dequant(int code, uint16_t step_h, uint16_t zero_h, int elem_dtype, int exact)
{
    if (exact)
        return (double)code * orc_f16_to_f64(step_h) + orc_f16_to_f64(zero_h);
    float prod = (float)code * orc_f16_to_f32(step_h); /* exact: <= 4 x 11 significant bits */
    float y = prod + orc_f16_to_f32(zero_h);
    return round_elem(y, elem_dtype);
}

/* ------------------------------------------------------------------------ */
/* Q2: dense packing of one token row of d codes into d*bits/32 words: word w holds
 * channels [w*32/bits, (w+1)*32/bits); channel c sits at bit bits*(c mod 32/bits),
 * least significant first. */
void orc_pack_row(const uint8_t *codes, int d, int bits, uint32_t *words)
{
    const int per = 32 / bits;
    for (int w = 0; w < d * bits / 32; ++w)
        words[w] = 0;
    for (int c = 0; c < d; ++c)
        words[c / per] |= (uint32_t)codes[c] << (bits * (c % per));
}

void orc_unpack_row(const uint32_t *words, int d, int bits, uint8_t *codes)
{
    const int per = 32 / bits;
    const uint32_t mask = (1u << bits) - 1u;
    for (int c = 0; c < d; ++c)
        codes[c] = (uint8_t)((words[c / per] >> (bits * (c % per))) & mask);
}

/* ------------------------------------------------------------------------ */
/* Q3: append n_new tokens to a segment (all arrays host, library layout):
 *   codes   uint32 [B][H][cap][d*bits/32]
 *   k_meta  uint16 [B][H][kgroup_cap][d][2]   {step, zero} per (K-group, channel)
 *   v_meta  uint16 [B][H][cap][d/Gv][2]       {step, zero} per (token, V-group)
 *   kgroup_start int32 [kgroup_cap + 1]       group g = tokens [start[g], start[g+1])
 *   raw     uint16 [B][H][cap][d]             bits == 16: elements of elem_dtype
 * Source: float [B][H][src_tokens][d]. Contiguous mode (groups == NULL) takes source
 * tokens [0, n_new) in K-groups of Gk from token 0, the last one possibly short.
 * Gather mode takes groups[g] = {start, len} in list order; each becomes one K-group.
 * Destination tokens are [n_tokens, n_tokens + n_new). Returns the number of new
 * K-groups, or -1 on a malformed request (nothing written). */
int orc_append(int bits, int elem_dtype, int B, int H, int d, int cap, int n_tokens,
               int Gk, int Gv, int kgroup_cap, int n_kgroups,
               uint32_t *k_codes, uint32_t *v_codes, uint16_t *k_meta, uint16_t *v_meta,
               int32_t *kgroup_start, uint16_t *k_raw, uint16_t *v_raw,
               const float *k_src, const float *v_src, int64_t src_tokens, int n_new,
               const int32_t *groups, int n_groups_in,
               int kgc, int comp_rank, const float *comp_basis, uint16_t *k_comp)
{
    int n_groups;
    if (groups) {
        n_groups = n_groups_in;
        int64_t total = 0;
        for (int g = 0; g < n_groups; ++g) {
            if (groups[2 * g + 1] < 1 || groups[2 * g] < 0 ||
                (int64_t)groups[2 * g] + groups[2 * g + 1] > src_tokens)
                return -1;
            total += groups[2 * g + 1];
        }
        if (total != n_new)
            return -1;
    } else {
        if (n_new > src_tokens)
            return -1;
        n_groups = (n_new + Gk - 1) / Gk;
    }
    if (n_tokens + n_new > cap)
        return -1;
    if (bits != 16 && kgc == 0 && n_kgroups + n_groups > kgroup_cap)
        return -1;
    if (kgc < 0 || (kgc > 0 && d % kgc != 0) || (kgc > 0 && comp_rank > 0) || comp_rank < 0 || comp_rank > 8)
        return -1;

    /* source token of the i-th appended token, and its K-group */
    int32_t *src_of = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_new > 0 ? n_new : 1));
    int32_t *gstart = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_groups + 1));
    int32_t *glen = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_groups + 1));
    int pos = 0;
    for (int g = 0; g < n_groups; ++g) {
        int s = groups ? groups[2 * g] : g * Gk;
        int len = groups ? groups[2 * g + 1] : (n_new - g * Gk < Gk ? n_new - g * Gk : Gk);
        gstart[g] = pos;
        glen[g] = len;
        for (int t = 0; t < len; ++t)
            src_of[pos + t] = s + t;
        pos += len;
    }

    const int wpr = d * bits / 32; /* words per token row (packed) */
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const size_t bh = (size_t)b * H + h;
            const float *ks = k_src + bh * (size_t)src_tokens * d;
            const float *vs = v_src + bh * (size_t)src_tokens * d;
            if (bits == 16) {
                for (int i = 0; i < n_new; ++i)
                    for (int c = 0; c < d; ++c) {
                        size_t o = (bh * cap + (size_t)(n_tokens + i)) * d + c;
                        float kx = ks[(size_t)src_of[i] * d + c], vx = vs[(size_t)src_of[i] * d + c];
                        k_raw[o] = elem_dtype == ORC_F16 ? orc_f32_to_f16(kx) : orc_f32_to_bf16(kx);
                        v_raw[o] = elem_dtype == ORC_F16 ? orc_f32_to_f16(vx) : orc_f32_to_bf16(vx);
                    }
                continue;
            }
            uint8_t *codes = (uint8_t *)malloc((size_t)(n_new > 0 ? n_new : 1) * d);
            if (kgc > 0) {
                /* K: per (token, run of kgc channels), as V */
                for (int i = 0; i < n_new; ++i)
                    for (int gk = 0; gk < d / kgc; ++gk) {
                        uint16_t *m = k_meta + ((bh * cap + (size_t)(n_tokens + i)) * (d / kgc) + gk) * 2;
                        orc_quantize_group(ks + (size_t)src_of[i] * d + (size_t)gk * kgc, kgc, 1, bits,
                                           &m[0], &m[1], codes + (size_t)i * d + (size_t)gk * kgc, 1);
                    }
            } else {
                /* K: per (K-group, channel) over the group's tokens */
                for (int g = 0; g < n_groups; ++g) {
                    float *col = (float *)malloc(sizeof(float) * (size_t)glen[g]);
                    for (int c = 0; c < d; ++c) {
                        for (int t = 0; t < glen[g]; ++t)
                            col[t] = ks[(size_t)src_of[gstart[g] + t] * d + c];
                        uint16_t *m = k_meta + ((bh * kgroup_cap + (size_t)(n_kgroups + g)) * d + c) * 2;
                        orc_quantize_group(col, glen[g], 1, bits, &m[0], &m[1],
                                           codes + (size_t)gstart[g] * d + c, d);
                    }
                    free(col);
                }
            }
            for (int i = 0; i < n_new; ++i)
                orc_pack_row(codes + (size_t)i * d, d, bits,
                             k_codes + (bh * cap + (size_t)(n_tokens + i)) * wpr);
            /* compensation: the key's rounding error (source minus dequantized key, exact)
             * projected on the basis of head h, rounded once to bf16 */
            if (comp_rank > 0) {
                const float *U = comp_basis + (size_t)h * d * comp_rank;
                for (int i = 0; i < n_new; ++i) {
                    int gi = 0; /* K-group of appended token i */
                    while (gi + 1 < n_groups && gstart[gi + 1] <= i)
                        ++gi;
                    for (int j = 0; j < comp_rank; ++j) {
                        double acc = 0.0;
                        for (int c = 0; c < d; ++c) {
                            const uint16_t *m = k_meta + ((bh * kgroup_cap + (size_t)(n_kgroups + gi)) * d + c) * 2;
                            const double x = ks[(size_t)src_of[i] * d + c];
                            const double xh = orc_dequant(codes[(size_t)i * d + c], m[0], m[1], elem_dtype, 0);
                            acc += (double)U[(size_t)c * comp_rank + j] * (x - xh);
                        }
                        k_comp[(bh * cap + (size_t)(n_tokens + i)) * 8 + j] = orc_f64_to_bf16(acc);
                    }
                    for (int j = comp_rank; j < 8; ++j)
                        k_comp[(bh * cap + (size_t)(n_tokens + i)) * 8 + j] = 0;
                }
            }
            /* V: per (token, run of Gv channels) */
            for (int i = 0; i < n_new; ++i) {
                for (int gv = 0; gv < d / Gv; ++gv) {
                    uint16_t *m = v_meta + ((bh * cap + (size_t)(n_tokens + i)) * (d / Gv) + gv) * 2;
                    orc_quantize_group(vs + (size_t)src_of[i] * d + (size_t)gv * Gv, Gv, 1, bits,
                                       &m[0], &m[1], codes + (size_t)i * d + (size_t)gv * Gv, 1);
                }
                orc_pack_row(codes + (size_t)i * d, d, bits,
                             v_codes + (bh * cap + (size_t)(n_tokens + i)) * wpr);
            }
            free(codes);
        }
    if (bits != 16 && kgc == 0 && kgroup_start) {
        for (int g = 0; g < n_groups; ++g)
            kgroup_start[n_kgroups + g] = n_tokens + gstart[g];
        kgroup_start[n_kgroups + n_groups] = n_tokens + n_new;
    }
    free(src_of);
    free(gstart);
    free(glen);
    return kgc > 0 ? 0 : n_groups;
}

/* ------------------------------------------------------------------------ */
/* Attention of one query row over a dense key/value list (A2, A3).
 *   s_j = scale * (q . k_j + add_j) - beta(q, group(j))   token j in a quantized K-group
 *   s_j = scale * (q . k_j + add_j)                      raw token (group < 0)
 * (add_j = logit_add[j], 0 when logit_add is NULL: the compensation term of a segment
 * that stores one)
 *   beta(q, g) = scale^2 / 24 * sum_c q_c^2 * step_{g,c}^2    (jensen == 1)
 *   beta(q, g) = scale^2 / 24 * |q|^2 * mean_c step_{g,c}^2   (jensen == 2)
 *   beta(q, g) = sum_c log(sinh(a_c) / a_c), a_c = scale |q_c| step_{g,c} / 2  (jensen == 3)
 * beta is half the variance of the logit noise scale * q . e when each key
 * channel's rounding error e_c is uniform on [-step/2, step/2] (variance step^2/12)
 * and independent: the second-order term of log E[exp(scale * q . e)], which is what
 * quantization noise adds to a cached key's logit on average [JB]. The second form
 * is the one [JB] states through the query's norm: each channel's step^2 replaced by
 * its mean over the group's channels (the two agree when the steps are equal across
 * channels). The third is the same model taken to all orders: log E[exp(scale q . e)]
 * itself, since E[exp(x)] = sinh(a)/a for x uniform on [-a, a] and the channels are
 * independent; its second-order term is the first form.
 * out_c = sum_j softmax(s)_j v_jc; lse = log sum_j exp(s_j); mass = softmax mass
 * on tokens with group >= 0 (the quantized history). Everything in double. */
/* log(sinh(a) / a) for a >= 0: the log of E[exp(x)] for x uniform on [-a, a]. Near 0
 * it is taken from its Taylor series (u/6 - u^2/180 + u^3/2835, u = a^2), for large a
 * from sinh(a) = e^a (1 - e^{-2a}) / 2, which keeps it finite. */
double orc_log_sinhc(double a)
{
    if (a < 0.01) { /* sinh(a)/a - 1 would cancel: its series, next term a^8/37800 < 3e-21 */
        const double u = a * a;
        return u / 6.0 - u * u / 180.0 + u * u * u / 2835.0;
    }
    if (a > 20.0)
        return a - log(2.0 * a) + log1p(-exp(-2.0 * a));
    return log(sinh(a) / a);
}

void orc_attend_row(const double *q, int d, const double *K, const double *V,
                    const int32_t *tok_group, int64_t N, const double *step_sq, int n_groups,
                    double scale, int jensen, const double *logit_add, double *out, double *lse,
                    double *mass)
{
    double *s = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double *beta = (double *)malloc(sizeof(double) * (size_t)(n_groups > 0 ? n_groups : 1));
    for (int g = 0; g < n_groups; ++g) {
        double acc = 0.0, qq = 0.0, ss = 0.0, lg = 0.0;
        for (int c = 0; c < d; ++c) {
            acc += q[c] * q[c] * step_sq[(size_t)g * d + c];
            qq += q[c] * q[c];
            ss += step_sq[(size_t)g * d + c];
            if (jensen == 3) /* a_c = scale |q_c| step_c / 2: half-width of scale q_c e_c */
                lg += orc_log_sinhc(scale * fabs(q[c]) * sqrt(step_sq[(size_t)g * d + c]) / 2.0);
        }
        if (jensen == 1)
            beta[g] = scale * scale / 24.0 * acc;
        else if (jensen == 2)
            beta[g] = scale * scale / 24.0 * qq * (ss / d);
        else if (jensen == 3)
            beta[g] = lg;
        else
            beta[g] = 0.0;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < N; ++j) {
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
            dot += q[c] * K[(size_t)j * d + c];
        if (logit_add)
            dot += logit_add[j];
        s[j] = scale * dot - (tok_group[j] >= 0 ? beta[tok_group[j]] : 0.0);
        if (s[j] > m) m = s[j];
    }
    double l = 0.0, lq = 0.0;
    for (int c = 0; c < d; ++c)
        out[c] = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        double p = exp(s[j] - m);
        l += p;
        if (tok_group[j] >= 0) lq += p;
        for (int c = 0; c < d; ++c)
            out[c] += p * V[(size_t)j * d + c];
    }
    for (int c = 0; c < d; ++c)
        out[c] /= l;
    if (lse) *lse = m + log(l);
    if (mass) *mass = lq / l;
    free(s);
    free(beta);
}

/* A segment of the cache as the attention oracle reads it (host arrays, layout as
 * in orc_append). */
typedef struct orc_segment {
    int32_t bits, elem_dtype, capacity, n_tokens, n_kgroups, kgroup_capacity, v_group_channels;
    const uint32_t *k_codes, *v_codes;
    const uint16_t *k_meta, *v_meta;
    const int32_t *kgroup_start;
    const uint16_t *k_raw, *v_raw;
    int32_t k_group_channels, comp_rank;
    const float *comp_basis;    /* [H][d][comp_rank] */
    const uint16_t *k_comp;     /* bf16 bits [B][H][cap][8], the first comp_rank used */
} orc_segment;

/* Chunk attention: queries q [B][Hq][nq][d] (float values of the query dtype), the
 * history as segments, the unquantized current chunk k_cur/v_cur [B][Hkv][n_cur][d].
 * Query head hq reads KV head hq * Hkv / Hq. There is no mask: every query sees the
 * whole history and the whole current chunk. Only the query rows listed in rows[]
 * (NULL: all nq) are computed; out is [B][Hq][n_rows][d], lse [B][Hq][n_rows].
 * Returns 0, or -1 on a malformed request. */
int orc_attention(const float *q, int B, int Hq, int Hkv, int d, int nq,
                  const orc_segment *segs, int n_segs,
                  const float *k_cur, const float *v_cur, int n_cur,
                  double scale, int jensen, int exact,
                  const int32_t *rows, int n_rows, double *out, double *lse, double *mass)
{
    if (Hkv <= 0 || Hq % Hkv != 0 || d < 1 || d > 256)
        return -1;
    if (!rows)
        n_rows = nq;
    int64_t N = n_cur;
    int G = 0, any_comp = 0;
    for (int s = 0; s < n_segs; ++s) {
        N += segs[s].n_tokens;
        if (segs[s].bits != 16)
            G += segs[s].k_group_channels > 0 ? segs[s].n_tokens : segs[s].n_kgroups;
        if (segs[s].bits != 16 && segs[s].comp_rank > 0)
            any_comp = 1;
    }
    const int gqa = Hq / Hkv;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hkv; ++h) {
            const size_t bh = (size_t)b * Hkv + h;
            double *K = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * d);
            double *V = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * d);
            int32_t *tg = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
            double *ssq = (double *)malloc(sizeof(double) * (size_t)(G > 0 ? G : 1) * d);
            int64_t j = 0;
            int gbase = 0;
            for (int s = 0; s < n_segs; ++s) {
                const orc_segment *sg = &segs[s];
                const size_t row0 = bh * (size_t)sg->capacity;
                if (sg->bits == 16) {
                    for (int t = 0; t < sg->n_tokens; ++t, ++j) {
                        for (int c = 0; c < d; ++c) {
                            uint16_t kb = sg->k_raw[(row0 + t) * d + c], vb = sg->v_raw[(row0 + t) * d + c];
                            K[j * d + c] = sg->elem_dtype == ORC_F16 ? orc_f16_to_f64(kb) : orc_bf16_to_f32(kb);
                            V[j * d + c] = sg->elem_dtype == ORC_F16 ? orc_f16_to_f64(vb) : orc_bf16_to_f32(vb);
                        }
                        tg[j] = -1;
                    }
                    continue;
                }
                const int wpr = d * sg->bits / 32, Gv = sg->v_group_channels;
                uint8_t *kc = (uint8_t *)malloc((size_t)d), *vc = (uint8_t *)malloc((size_t)d);
                if (sg->k_group_channels > 0) {
                    /* per-token K groups: every token is its own group of step sizes */
                    const int kgc = sg->k_group_channels;
                    for (int t = 0; t < sg->n_tokens; ++t, ++j) {
                        orc_unpack_row(sg->k_codes + (row0 + t) * wpr, d, sg->bits, kc);
                        orc_unpack_row(sg->v_codes + (row0 + t) * wpr, d, sg->bits, vc);
                        for (int c = 0; c < d; ++c) {
                            const uint16_t *km = sg->k_meta + ((row0 + t) * (d / kgc) + c / kgc) * 2;
                            const uint16_t *vm = sg->v_meta + ((row0 + t) * (d / Gv) + c / Gv) * 2;
                            double st = orc_f16_to_f64(km[0]);
                            ssq[(size_t)(gbase + t) * d + c] = st * st;
                            K[j * d + c] = orc_dequant(kc[c], km[0], km[1], sg->elem_dtype, exact);
                            V[j * d + c] = orc_dequant(vc[c], vm[0], vm[1], sg->elem_dtype, exact);
                        }
                        tg[j] = gbase + t;
                    }
                    free(kc);
                    free(vc);
                    gbase += sg->n_tokens;
                    continue;
                }
                for (int g = 0; g < sg->n_kgroups; ++g) {
                    const uint16_t *km = sg->k_meta + (bh * sg->kgroup_capacity + (size_t)g) * d * 2;
                    for (int c = 0; c < d; ++c) {
                        double st = orc_f16_to_f64(km[2 * c]);
                        ssq[(size_t)(gbase + g) * d + c] = st * st;
                    }
                    for (int t = sg->kgroup_start[g]; t < sg->kgroup_start[g + 1]; ++t, ++j) {
                        orc_unpack_row(sg->k_codes + (row0 + t) * wpr, d, sg->bits, kc);
                        orc_unpack_row(sg->v_codes + (row0 + t) * wpr, d, sg->bits, vc);
                        for (int c = 0; c < d; ++c) {
                            const uint16_t *vm = sg->v_meta + ((row0 + t) * (d / Gv) + c / Gv) * 2;
                            K[j * d + c] = orc_dequant(kc[c], km[2 * c], km[2 * c + 1], sg->elem_dtype, exact);
                            V[j * d + c] = orc_dequant(vc[c], vm[0], vm[1], sg->elem_dtype, exact);
                        }
                        tg[j] = gbase + g;
                    }
                }
                free(kc);
                free(vc);
                gbase += sg->n_kgroups;
            }
            for (int t = 0; t < n_cur; ++t, ++j) {
                for (int c = 0; c < d; ++c) {
                    K[j * d + c] = k_cur[(bh * n_cur + t) * d + c];
                    V[j * d + c] = v_cur[(bh * n_cur + t) * d + c];
                }
                tg[j] = -1;
            }
#pragma omp parallel for collapse(2) schedule(dynamic)
            for (int r = 0; r < gqa; ++r)
                for (int ri = 0; ri < n_rows; ++ri) {
                    const int hq = h * gqa + r;
                    const int i = rows ? rows[ri] : ri;
                    double qd[256];
                    const float *qr = q + (((size_t)b * Hq + hq) * nq + i) * d;
                    for (int c = 0; c < d; ++c)
                        qd[c] = qr[c];
                    /* compensation: (U_h^T q) . c_t for the tokens of segments that store c */
                    double *add = NULL;
                    if (any_comp) {
                        add = (double *)calloc((size_t)(j > 0 ? j : 1), sizeof(double));
                        int64_t t0 = 0;
                        for (int s = 0; s < n_segs; ++s) {
                            const orc_segment *sg = &segs[s];
                            if (sg->bits != 16 && sg->comp_rank > 0) {
                                const int r_ = sg->comp_rank;
                                const float *U = sg->comp_basis + (size_t)h * d * r_;
                                double uq[8];
                                for (int jj = 0; jj < r_; ++jj) {
                                    uq[jj] = 0.0;
                                    for (int c = 0; c < d; ++c)
                                        uq[jj] += (double)U[(size_t)c * r_ + jj] * qd[c];
                                }
                                for (int t = 0; t < sg->n_tokens; ++t) {
                                    const uint16_t *ct = sg->k_comp + (bh * (size_t)sg->capacity + t) * 8;
                                    double acc = 0.0;
                                    for (int jj = 0; jj < r_; ++jj)
                                        acc += uq[jj] * (double)orc_bf16_to_f32(ct[jj]);
                                    add[t0 + t] = acc;
                                }
                            }
                            t0 += sg->n_tokens;
                        }
                    }
                    const size_t o = ((size_t)b * Hq + hq) * n_rows + ri;
                    orc_attend_row(qd, d, K, V, tg, j, ssq, gbase, scale, jensen, add, out + o * d,
                                   lse ? lse + o : NULL, mass ? mass + o : NULL);
                    free(add);
                }
            free(K);
            free(V);
            free(tg);
            free(ssq);
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* W1: window scores. Keys k [H][N][d] (float values). Windows are
 * [window*w, min(window*w + window, N)). For each KV head, in double and in this
 * order: the mean key of the window (tokens summed in index order, then divided by
 * the token count), dot = sum_c mean_c t_c, nm = sum_c mean_c^2, nt = sum_c t_c^2
 * (channels ascending), cos = dot / (sqrt(nm) * sqrt(nt)), 0 when nm * nt == 0. The
 * score is the mean of the heads' cosines (summed heads ascending) [WQ]. */
void orc_window_scores(const float *k, int H, int N, int d, int window, const float *text,
                       double *score)
{
    const int W = (N + window - 1) / window;
    if (d > 256)
        return;
#pragma omp parallel for schedule(static)
    for (int w = 0; w < W; ++w) {
        const int t0 = w * window, t1 = (t0 + window < N) ? t0 + window : N;
        double acc = 0.0;
        for (int h = 0; h < H; ++h) {
            double mean[256];
            for (int c = 0; c < d; ++c) {
                double sum = 0.0;
                for (int t = t0; t < t1; ++t)
                    sum += (double)k[((size_t)h * N + t) * d + c];
                mean[c] = sum / (double)(t1 - t0);
            }
            double dot = 0.0, nm = 0.0, nt = 0.0;
            for (int c = 0; c < d; ++c) {
                dot += mean[c] * (double)text[c];
                nm += mean[c] * mean[c];
                nt += (double)text[c] * (double)text[c];
            }
            double cs = (nm * nt == 0.0) ? 0.0 : dot / (sqrt(nm) * sqrt(nt));
            acc += cs;
        }
        score[w] = acc / (double)H;
    }
}

/* W2: bit-width of each window and the grouped order [WQ]. Window 0 is FP16 whatever
 * its score. Windows 1..W-1 are ranked by score, highest first, ties to the lower
 * index; the first n_fp16 - 1 of them are FP16, the next n_int4 INT4, the rest INT2.
 * order lists the FP16 windows ascending, then the INT4 ones, then the INT2 ones.
 * A plain O(W^2) rank count. Returns -1 on a bad budget. */
int orc_assign_windows(const double *score, int W, int n_fp16, int n_int4, int8_t *bits,
                       int32_t *order)
{
    if (W < 1 || n_fp16 < 1 || n_int4 < 0 || n_fp16 + n_int4 > W)
        return -1;
    bits[0] = 16;
    for (int w = 1; w < W; ++w) {
        int rank = 0; /* windows (other than 0) that come before w */
        for (int v = 1; v < W; ++v)
            if (score[v] > score[w] || (score[v] == score[w] && v < w))
                ++rank;
        bits[w] = rank < n_fp16 - 1 ? 16 : (rank < n_fp16 - 1 + n_int4 ? 4 : 2);
    }
    int pos = 0;
    const int cls[3] = {16, 4, 2};
    for (int k = 0; k < 3; ++k)
        for (int w = 0; w < W; ++w)
            if (bits[w] == cls[k])
                order[pos++] = w;
    return 0;
}

/* A6: the grouped layout's gather lists [WQ "技術的に面白い点": windows of one bit-width
 * are stored together]. Row i of groups is {first token, length} of window order[i], so
 * the FP16, INT4 and INT2 lists follow one another in the order assign_windows makes;
 * class_tokens holds the tokens of the FP16, INT4 and INT2 windows (the last window may
 * be short). */
void orc_window_groups(const int8_t *bits, const int32_t *order, int W, int N, int window,
                       int32_t *groups, int32_t *class_tokens)
{
    class_tokens[0] = class_tokens[1] = class_tokens[2] = 0;
    for (int i = 0; i < W; ++i) {
        const int w = order[i];
        const int start = w * window;
        const int len = (start + window <= N) ? window : N - start;
        groups[2 * i] = start;
        groups[2 * i + 1] = len;
        const int k = bits[w] == 16 ? 0 : (bits[w] == 4 ? 1 : 2);
        class_tokens[k] += len;
    }
}

/* FP16 and INT4 window counts from percentages: floor over all W in integer
 * arithmetic, window 0 counted within the FP16 share, at least one FP16 window. */
void orc_window_budget(int W, int pct_fp16, int pct_int4, int *n_fp16, int *n_int4)
{
    int n16 = (W * pct_fp16) / 100;
    int n_le4 = (W * (pct_fp16 + pct_int4)) / 100;
    int n4 = n_le4 - n16;
    if (n16 < 1) n16 = 1;
    if (n4 > W - n16) n4 = W - n16;
    if (n4 < 0) n4 = 0;
    *n_fp16 = n16;
    *n_int4 = n4;
}

/* Array forms of the format conversions (for the tests' exhaustive checks). */
void orc_f32_to_f16_n(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f32_to_f16(x[i]);
}

void orc_f32_to_bf16_n(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f32_to_bf16(x[i]);
}

void orc_f16_to_f64_n(const uint16_t *h, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f16_to_f64(h[i]);
}
