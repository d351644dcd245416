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
    int32_t k_group_channels;    // > 0: per-token K groups of that many channels
    int32_t comp_rank;           // > 0: write the compensation c_t (rank <= 8)
    const float *comp_basis;     // [n_kv_heads][head_dim][comp_rank]
    void *k_comp;                // bf16 [batch][n_kv_heads][capacity][8]
};
hipError_t launch_quant_append(const QuantAppendParams &p, int bits, int n_groups, hipStream_t s);

struct WindowParams {
    const void *k;                 // [n_layers][n_kv_heads][n_tokens][head_dim]
    int32_t k_dtype;
    int32_t n_layers, n_kv_heads, head_dim, n_tokens, window, n_windows;
    const float *text;             // [n_layers][head_dim]
    int32_t n_fp16, n_int4;        // windows per class (the same for every layer)
    int8_t *bits_out;              // [n_layers][n_windows]
    int32_t *order_out;            // [n_layers][n_windows]
    double *score;                 // [n_layers][n_windows]
    int32_t *groups_out;           // [n_layers][n_windows][2] or nullptr
    int32_t *class_tokens_out;     // [n_layers][3] or nullptr
};
constexpr int kMaxWindowsPerLayer = 16384;
constexpr int kMaxWindowLayers = 65535;
hipError_t launch_windows(const WindowParams &p, hipStream_t s);
// FP16 and INT4 window counts from percentages of n_windows.
void window_budget(int n_windows, int pct_fp16, int pct_int4, int *n_fp16, int *n_int4);

constexpr int kMaxSegments = 8;

struct SegmentView {
    int32_t bits, n_tokens, n_kgroups, capacity, kgroup_capacity, v_group_channels, token_begin;
    int32_t k_group_channels;      // > 0: per-token K groups (k_meta [cap][head_dim / k_group_channels])
    const void *k, *v;
    const uint32_t *k_meta, *v_meta;
    const int32_t *kgroup_start;
    const uint16_t *k_comp;        // compensation c_t, bf16 [cap][8] per (b, h); nullptr: none
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
    float beta_log2;               // scale^2 / 24 * log2(e) for the second-order forms, 1 for
                                   // the all-orders one (computed in log2 units), else 0
    float half_scale;              // scale / 2: a_c = half_scale |q_c| step_c (all-orders form)
    int32_t jensen;                // kvq_jensen
    // per-token K columns: 0 none, 1 per-token K groups of aug_kgc channels, 2 the low-rank
    // compensation of rank aug_rank with basis aug_basis [n_kv_heads][head_dim][aug_rank]
    int32_t aug, aug_kgc, aug_rank;
    const float *aug_basis;
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
                                   // chunk: [workgroup][2][row in block] rows of 2 head_dim + 16
                                   // bytes (int16 mantissas; m, l, exponent, pad)
    int32_t decode;                // run the decode-shaped kernel (decided by decode_eligible)
    // quantize-append of the current chunk in the same call (app_bits 0: none). The chunk
    // kernel runs it in workgroups after its own (blocks past n_attn_wg, app_per_wg units
    // of (K-group, KV head, batch) each, on the CUs the attention leaves idle in its last
    // round); other paths launch the quantize-append kernel after the attention.
    QuantAppendParams app;
    int32_t app_bits, app_groups, n_attn_wg, app_per_wg;
};
struct AttnPlan {
    int32_t n_split, split_tokens;   // decode kernel
    int32_t n_rb, tok_pad;           // chunk kernel
    int64_t quota, work;
    size_t workspace_bytes;
};
// Compute units of the current device (256 when there is none to ask).
int device_cus();
// How either kernel divides the work (decode selects the decode-shaped one), and the
// workspace its partials need.
void attention_plan(int batch, int n_q_heads, int n_kv_heads, int head_dim, int n_q, int n_total, bool decode,
                    AttnPlan *plan);
hipError_t launch_attention(const AttnParams &p, hipStream_t s);
// Log-sum-exp merge of n_split partials into the output.
hipError_t launch_combine(const AttnParams &p, hipStream_t s);

// Decode-shaped attention: at most kDecodeRows query rows per (batch, KV head), bf16, at
// most one packed segment (INT2; INT4 at head_dim 128), and a current chunk only when one
// workgroup takes each (batch, KV head). Every other call runs on the chunk kernel: raw
// segments, fp16, INT4 at head_dim 64 and several segments faulted in decode_kernel on
// the one run that took them there, with the cause not found.
constexpr int kDecodeRows = 16;
bool decode_eligible(int dtype, int batch, int n_q_heads, int n_kv_heads, int head_dim, int n_q,
                     const int *seg_bits, int n_segs, int n_cur, int n_total);
// Workgroups per (batch, KV head) and tokens per wave.
void decode_plan(int batch, int n_kv_heads, int n_total, int *n_wg, int *wave_tokens);
hipError_t launch_decode(const AttnParams &p, hipStream_t s);

// Streaming read of a device buffer (bandwidth probe).
hipError_t launch_hbm_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s);

}  // namespace kvq
