// Host-side launch interface between the C ABI layer (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace kvq {

// One quantize-append launch (all pointers device, validated by the caller).
struct QuantAppendParams {
    const void *k_src, *v_src;
    int32_t src_dtype;
    int64_t src_tokens;
    int32_t n_new;
    const int32_t *src_groups;   // nullptr: contiguous
    int32_t k_group_tokens;
    int32_t batch, n_kv_heads, head_dim;
    int32_t capacity, kgroup_capacity;
    int32_t n_tokens, n_kgroups;  // destination state before the append
    int32_t elem_dtype;          // bits 16: element dtype written
    void *k_dst, *v_dst;
    void *k_meta, *v_meta;
    int32_t *kgroup_start;
};
hipError_t launch_quant_append(const QuantAppendParams &p, int bits, int n_groups, hipStream_t s);

struct WindowParams {
    const void *k;
    int32_t k_dtype;
    int32_t n_kv_heads, head_dim, n_tokens, window, n_windows;
    const float *text;
    int32_t n_fp16, n_int4;
    int8_t *bits_out;
    int32_t *order_out;
    double *score;
};
hipError_t launch_windows(const WindowParams &p, hipStream_t s);

constexpr int kMaxSegments = 8;

struct SegmentView {
    int32_t bits, n_tokens, n_kgroups, capacity, kgroup_capacity, v_group_channels, token_begin, pad_;
    const void *k, *v;
    const uint32_t *k_meta, *v_meta;
    const int32_t *kgroup_start;
};

struct AttnParams {
    const void *q;
    int32_t dtype;                 // 1 = fp16, 2 = bf16 (q, current chunk, cache elements)
    int32_t batch, n_q_heads, n_kv_heads, head_dim, n_q;
    int32_t n_segs;
    SegmentView segs[kMaxSegments];
    const void *k_cur, *v_cur;
    int32_t n_cur;
    int32_t n_total;               // history + current tokens
    float scale_log2;              // softmax scale * log2(e)
    float beta_log2;               // scale^2 / 24 * log2(e) when Jensen is on, else 0
    int32_t jensen;                // kvq_jensen
    void *out;
    int32_t out_dtype;
    float *lse;
    // decode kernel
    int32_t n_split;               // workgroups per (batch, KV head); > 1 writes partials
    int32_t split_tokens;          // tokens per wave, multiple of 64
    // chunk kernel: row block rb (of n_rb per (batch, KV head)) owns work positions
    // [rb tok_pad, (rb + 1) tok_pad); workgroup w takes [w quota, (w + 1) quota) of the
    // work positions
    int32_t n_rb, tok_pad;
    int64_t quota, work;
    float *partial;                // decode: [n_split][rows][head_dim + 2];
                                   // chunk: [workgroup][2][row in block][head_dim + 4]
    int32_t decode;                // run the decode-shaped kernel (decided by decode_eligible)
};
struct AttnPlan {
    int32_t n_split, split_tokens;   // decode kernel
    int32_t n_rb, tok_pad;           // chunk kernel
    int64_t quota, work;
    size_t workspace_bytes;
};
// How either kernel divides the work (decode selects the decode-shaped one), and the
// workspace its partials need.
void attention_plan(int batch, int n_q_heads, int n_kv_heads, int head_dim, int n_q, int n_total, bool decode,
                    AttnPlan *plan);
hipError_t launch_attention(const AttnParams &p, hipStream_t s);
// Log-sum-exp merge of n_split partials into the output.
hipError_t launch_combine(const AttnParams &p, hipStream_t s);

// Decode-shaped attention: at most kDecodeRows query rows per (batch, KV head), bf16, and
// packed segments only (INT2; INT4 at head_dim 128). Raw segments, fp16 and INT4 at
// head_dim 64 run on the chunk kernel.
constexpr int kDecodeRows = 16;
bool decode_eligible(int dtype, int n_q_heads, int n_kv_heads, int head_dim, int n_q, const int *seg_bits,
                     int n_segs);
// Workgroups per (batch, KV head) and tokens per wave.
void decode_plan(int batch, int n_kv_heads, int n_total, int *n_wg, int *wave_tokens);
hipError_t launch_decode(const AttnParams &p, hipStream_t s);

}  // namespace kvq
