/*
 * kvq.h -- C ABI of libkvq: low-bit KV-cache quantize-pack and fused attention over
 * the packed cache, for AMD Instinct MI355X (gfx950).
 *
 * The method comes from four web pages, cited by title and section:
 *  [JB] "Quantized Keys Steal Attention: Bias Correction for KV-Cache Compression in
 *       Video Diffusion", abstract -- chunk-wise autoregressive video diffusion keeps a
 *       KV cache of earlier chunks; INT2 keys inflate their softmax weight (the
 *       "Jensen bias") against the unquantized current chunk; a per-score correction
 *       from the cached keys' step sizes and the query, second-order Taylor form, no
 *       memory beyond the cache.
 *  [SF] "KV Cache Quantization for Self-Forcing Video Generation: A 33-Method
 *       Empirical Study", abstract -- INT4 caches; integrations that rebuild BF16
 *       buffers during attention lose the memory they saved.
 *  [WQ] WindowQuant notes (zenn.dev, "論文メモ：動画VLMのKV Cacheを軽量化するWindowQuant"),
 *       sections "何が新しいのか", "技術的に面白い点", "実装者視点で気になった点" --
 *       32-token windows scored by cosine similarity to the text query, FP16 / INT4 /
 *       INT2 by relevance, window 0 always FP16, windows of one bit-width stored
 *       together.
 *  [QW] "QuantWM Preserves Attention in 2-Bit KV Cache Quantization for Video World
 *       Models" -- 2-bit KV caches; keys act through the attention logits.
 *
 * Conventions for every call:
 *  - Device pointers are plain HIP device addresses on the current device; host
 *    pointers are marked "host". The caller owns every buffer. The library never
 *    allocates, frees or synchronizes; each call only enqueues kernels on `stream`
 *    (a hipStream_t; NULL = the null stream) and returns.
 *  - Pointers must stay valid until the stream has run the work. Device buffers must
 *    be 16-byte aligned.
 *  - Every argument is checked on the host before anything is enqueued. On any error
 *    nothing is enqueued and no output, buffer or descriptor is changed.
 *    KVQ_ERR_HIP reports a launch failure (hipGetLastError after the launch); device
 *    faults surface at the caller's next synchronization.
 *  - No global mutable state (except the static scratch of kvq_chunk_attention_noalloc,
 *    see there): calls are reentrant and may run on several streams at once if they
 *    touch disjoint buffers. No C++ exception crosses this ABI.
 *  - Elements of fp16 / bf16 inputs must lie within fp16's finite range
 *    (|x| <= 65504); step and zero are stored in fp16.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 3
#define KVQ_MAX_SEGMENTS 8

typedef enum kvq_status {
    KVQ_OK = 0,
    KVQ_ERR_ARG = -1,          /* null pointer, bad size, inconsistent shapes */
    KVQ_ERR_UNSUPPORTED = -2,  /* bits, head_dim, group size or dtype outside the table */
    KVQ_ERR_CAPACITY = -3,     /* an append would overflow a segment */
    KVQ_ERR_WORKSPACE = -4,    /* workspace null or smaller than kvq_attention_workspace_size */
    KVQ_ERR_HIP = -5           /* a kernel launch failed */
} kvq_status;

typedef enum kvq_dtype { KVQ_F32 = 0, KVQ_F16 = 1, KVQ_BF16 = 2 } kvq_dtype;

/* Jensen-bias correction applied to logits of quantized cached keys [JB]. */
typedef enum kvq_jensen {
    KVQ_JENSEN_OFF = 0,
    /* beta(i, g) = tau^2 / 24 * sum_c q_ic^2 * step_gc^2, subtracted from every logit of a
     * token of K-group g: half the variance of the logit noise tau * q . e when each key
     * channel's rounding error e_c is uniform on [-step/2, step/2], i.e. the second-order
     * term of log E[exp(tau q . e)]. step is the stored fp16 step; no extra memory. */
    KVQ_JENSEN_TAYLOR2 = 1,
    /* beta(i, g) = tau^2 / 24 * |q_i|^2 * mean_c step_gc^2: the form [JB] states through
     * the query's norm, i.e. TAYLOR2 with every channel's step^2 replaced by its mean over
     * the group's channels (equal to TAYLOR2 when a group's steps are equal across
     * channels; the mean of TAYLOR2 over cyclic shifts of the step vector otherwise). */
    KVQ_JENSEN_ISO = 2,
    /* beta(i, g) = sum_c log(sinh(a_c) / a_c), a_c = tau * |q_ic| * step_gc / 2: the same
     * uniform-noise model taken to all orders, log E[exp(tau q . e)] exactly (E[exp(x)] =
     * sinh(a)/a for x uniform on [-a, a], channels independent); TAYLOR2 is its
     * second-order term. */
    KVQ_JENSEN_EXACT = 3
} kvq_jensen;

/*
 * One segment of the cache: every token in it has the same bit-width [WQ]. A plain
 * chunk-wise cache is one packed segment [JB]; the WindowQuant layout is three (FP16,
 * INT4, INT2), each holding its windows contiguously [WQ].
 *
 * Quantization (bits 2 or 4, L = 2^bits - 1), asymmetric min/max per group:
 *   step = fp16(fl32(fl32(max - min) / L)), zero = fp16(min),
 *   code = clamp(rint(fl32(fl32(x - zero) / step)), 0, L)   (0 when step == 0),
 *   codes taken against the fp16-rounded step and zero, ties to even, IEEE fp32
 *   division. K groups: one per (K-group of tokens, channel). V groups: one per (token,
 *   run of v_group_channels channels).
 * Dequantized element (what attention reads): E(fl32(code * step + zero)), E = rounding
 *   to elem_dtype (bf16 or fp16), nearest-even.
 *
 * Layout per (batch b, KV head h), token-major, capacity slots each:
 *   k, v     bits 2|4: uint32 [batch][n_kv_heads][capacity][head_dim*bits/32]; word w of a
 *            token row holds channels [w*32/bits, (w+1)*32/bits), channel c at bit
 *            bits*(c mod 32/bits), least significant first.
 *            bits 16: elem_dtype [batch][n_kv_heads][capacity][head_dim], raw elements.
 *   k_meta   bits 2|4: {fp16 step, fp16 zero} [batch][n_kv_heads][kgroup_capacity][head_dim]
 *   v_meta   bits 2|4: {fp16 step, fp16 zero} [batch][n_kv_heads][capacity][head_dim/v_group_channels]
 *   kgroup_start  bits 2|4: int32 [kgroup_capacity + 1]; K-group g holds tokens
 *            [kgroup_start[g], kgroup_start[g+1]), the same for every (b, h).
 *   For bits 16 k_meta, v_meta and kgroup_start are unused and may be NULL.
 *
 * Per-token K groups (k_group_channels > 0; 0 is the per-channel layout above): keys are
 * grouped like values, one group per (token, run of k_group_channels channels), the
 * geometry in which the Jensen term's query-norm form is exact [JB: "computed ... from the
 * quantization step sizes of the cached keys and the query norm"]: with k_group_channels
 * == head_dim every channel of a token has the same step, and the channel-weighted term
 * is tau^2/24 * |q|^2 * step_t^2.
 *   k_meta   {fp16 step, fp16 zero} [batch][n_kv_heads][capacity][head_dim/k_group_channels];
 *            kgroup_start, kgroup_capacity and n_kgroups are unused (kgroup_start may be
 *            NULL; n_kgroups stays 0), and k_group_tokens only sets how many tokens one
 *            append workgroup takes.
 *
 * Low-rank logit compensation (comp_rank r > 0, PSAC-style ["QuantWM Preserves Attention
 * in 2-Bit KV Cache Quantization for Video World Models": compensating key error along
 * the dominant query subspace]): each appended token stores the projection of its key's
 * rounding error onto an r-dimensional query subspace, and attention adds it back for the
 * part of the query inside that subspace. For queries in the subspace the logits are those
 * of the unquantized keys (up to the bf16 rounding of the stored projection); the part of
 * the query orthogonal to it sees the quantized keys alone.
 *   comp_basis  device float32 [n_kv_heads][head_dim][r]: U_h, orthonormal columns (the
 *            caller's estimate of the dominant subspace of the queries that read KV head h).
 *   k_comp   device bf16 [batch][n_kv_heads][capacity][8]: c_t = bf16(U_h^T (k_t - khat_t))
 *            in the first r entries of token t's row, zeros after, khat_t the dequantized
 *            key (written by kvq_quantize_append; the difference is exact, the projection
 *            summed in fp32).
 *   Attention adds tau * (U_h^T q) . c_t to the logit of token t. 1 <= r <= 8.
 * A segment uses per-token K groups or the compensation, not both.
 */
typedef struct kvq_segment {
    int32_t bits;              /* 2, 4 (packed codes) or 16 (raw elements) */
    int32_t elem_dtype;        /* KVQ_BF16 or KVQ_F16: raw dtype / dequantization rounding */
    int32_t batch, n_kv_heads, head_dim;   /* head_dim: 64 or 128 */
    int32_t capacity;          /* token slots per (b, h) */
    int32_t n_tokens;          /* valid tokens, [0, capacity] */
    int32_t k_group_tokens;    /* K-group length of contiguous appends; max length of a gathered group; 1..1024 */
    int32_t v_group_channels;  /* V-group width: 32 */
    int32_t kgroup_capacity;   /* entries of k_meta per (b, h) */
    int32_t n_kgroups;         /* valid K-groups */
    void *k, *v;               /* device */
    void *k_meta, *v_meta;     /* device */
    int32_t *kgroup_start;     /* device */
    int32_t k_group_channels;  /* 0: per-channel K groups; 32, 64 or 128 (<= head_dim): per-token */
    int32_t comp_rank;         /* 0: no compensation; 1..8: rank r */
    const float *comp_basis;   /* device, comp_rank > 0 */
    void *k_comp;              /* device, comp_rank > 0 */
} kvq_segment;

/*
 * kvq_quantize_append -- quantize a finished chunk and append it to a segment [JB: the
 * cache holds previously generated chunks; WQ: each window is stored at its bit-width].
 *   dst         host descriptor; on KVQ_OK its n_tokens grows by n_new and n_kgroups by
 *               the number of new K-groups.
 *   k_src, v_src  device [batch][n_kv_heads][src_tokens][head_dim] of src_dtype (F32, F16
 *               or BF16), the dst segment's batch / heads / head_dim.
 *   src_tokens  token stride of the source per (b, h).
 *   n_new       tokens to append. Contiguous mode (src_groups == NULL): source tokens
 *               [0, n_new), cut into K-groups of k_group_tokens from the first appended
 *               token, the last one possibly shorter. Gather mode: src_groups is a
 *               DEVICE int32 array [n_src_groups][2] of {first source token, length};
 *               each entry becomes one K-group, appended in list order. The caller
 *               guarantees every entry lies in [0, src_tokens), lengths are in
 *               [1, k_group_tokens] and sum to n_new; entries outside are clamped on the
 *               device (no out-of-bounds access) and leave the segment's contents
 *               unspecified.
 *   Destination: tokens [n_tokens, n_tokens + n_new) of every (b, h).
 *   bits 16 segments copy the tokens, rounding to elem_dtype (nearest-even).
 * Errors: KVQ_ERR_ARG (null pointers, n_new < 0, shape mismatch), KVQ_ERR_UNSUPPORTED
 * (bits, head_dim, group sizes, dtypes), KVQ_ERR_CAPACITY (n_tokens + n_new > capacity
 * or the new K-groups exceed kgroup_capacity). n_new == 0 is a no-op returning KVQ_OK.
 */
typedef struct kvq_append_args {
    kvq_segment *dst;          /* host */
    const void *k_src, *v_src; /* device */
    int32_t src_dtype;
    int64_t src_tokens;
    int32_t n_new;
    const int32_t *src_groups; /* device, optional */
    int32_t n_src_groups;
} kvq_append_args;

kvq_status kvq_quantize_append(const kvq_append_args *args, void *stream);

/*
 * kvq_window_budget -- how many windows each bit-width class gets [WQ: high / middle / low
 * relevance kept in FP16 / INT4 / INT2]. Host only, no device work.
 *   n_fp16 = floor(n_windows * pct_fp16 / 100), at least 1 (window 0 is FP16 and counts
 *   inside this share); n_int4 = floor(n_windows * (pct_fp16 + pct_int4) / 100) - the
 *   unraised n_fp16, capped so the two fit in n_windows; the rest are INT2. Integer
 *   arithmetic throughout. 613 windows at 10 % / 30 % give 61 FP16, 184 INT4, 368 INT2.
 * Errors: KVQ_ERR_ARG (null outputs, n_windows < 1, a percentage outside [0, 100], or
 * pct_fp16 + pct_int4 > 100).
 */
kvq_status kvq_window_budget(int32_t n_windows, int32_t pct_fp16, int32_t pct_int4, int32_t *n_fp16,
                             int32_t *n_int4);

/*
 * kvq_assign_windows -- WindowQuant bit-widths and grouped layout for n_layers independent
 * caches (e.g. the layers of a model) in one pair of launches [WQ].
 *   k            device [n_layers][n_kv_heads][n_tokens][head_dim] of k_dtype (F16, BF16
 *                or F32), head_dim 1..256.
 *   text_query   device float32 [n_layers][head_dim]: each layer's text-query vector.
 *   Windows are [window*w, min(window*w + window, n_tokens)), w < n_windows =
 *   ceil(n_tokens / window) <= 16384.
 *   Score: per KV head, the window's mean key (tokens summed in index order, in
 *   double, divided by the token count); cosine with the layer's text query as
 *   dot / (sqrt(|mean|^2) * sqrt(|t|^2)), sums over channels in index order, 0 if either
 *   norm is zero; score = mean over KV heads (summed in order).
 *   Assignment (per layer): window 0 is FP16 whatever its score; windows 1.. are ranked
 *   by score, highest first, ties to the lower index; with n_fp16 / n_int4 from
 *   kvq_window_budget(n_windows, pct_fp16, pct_int4), the first n_fp16 - 1 get FP16, the
 *   next n_int4 INT4, the rest INT2.
 *   bits_out     device int8 [n_layers][n_windows]: 16, 4 or 2.
 *   order_out    device int32 [n_layers][n_windows]: the FP16 windows ascending, then
 *                INT4 ascending, then INT2 ascending (the grouped storage order).
 *   score_out    device double [n_layers][n_windows] (required: also the ranking's input).
 *   groups_out   device int32 [n_layers][n_windows][2], optional (NULL: not written):
 *                {first token, length} of the windows in order_out's order. Rows
 *                [0, n_fp16), [n_fp16, n_fp16 + n_int4) and [n_fp16 + n_int4, n_windows)
 *                are the gather lists kvq_quantize_append takes for the FP16, INT4 and
 *                INT2 segments.
 *   class_tokens_out  device int32 [n_layers][3], optional: tokens of the FP16, INT4 and
 *                INT2 classes (each class's n_new for those appends).
 * Errors: KVQ_ERR_ARG (nulls, n_layers < 1, n_tokens < 1, window < 1, a bad budget as in
 * kvq_window_budget), KVQ_ERR_UNSUPPORTED (k_dtype, head_dim outside 1..256, n_windows >
 * 16384, n_layers > 65535).
 */
typedef struct kvq_window_args {
    const void *k;
    int32_t k_dtype;
    int32_t n_layers;
    int32_t n_kv_heads, head_dim, n_tokens, window;
    const float *text_query;
    int32_t pct_fp16, pct_int4;
    int8_t *bits_out;
    int32_t *order_out;
    double *score_out;
    int32_t *groups_out;
    int32_t *class_tokens_out;
} kvq_window_args;

kvq_status kvq_assign_windows(const kvq_window_args *args, void *stream);

/*
 * kvq_chunk_attention -- one chunk of queries over the quantized history plus the
 * unquantized current chunk [JB], reading the packed cache directly (no dequantized
 * copy of the cache is ever written to memory [SF]).
 *   q        device [batch][n_q_heads][n_q][head_dim] of dtype (BF16 or F16).
 *   segs     host array of n_segs (0..KVQ_MAX_SEGMENTS) segment descriptors: the
 *            history, in any order (softmax does not depend on token order). All share
 *            batch, n_kv_heads and head_dim with q, and elem_dtype == dtype.
 *   k_cur, v_cur  device [batch][n_kv_heads][n_cur][head_dim] of dtype, may be NULL
 *            when n_cur == 0.
 *   Query head hq reads KV head hq * n_kv_heads / n_q_heads. No mask: every query sees
 *   all history and the whole current chunk.
 *   Logits: s = tau * q . k - beta, tau = softmax_scale (0 means 1/sqrt(head_dim));
 *   beta as kvq_jensen for tokens of packed segments, 0 for bits-16 segments and for
 *   the current chunk.
 *   out      device [batch][n_q_heads][n_q][head_dim] of out_dtype (F32, F16 or BF16):
 *            softmax(s) . V.
 *   lse      device float32 [batch][n_q_heads][n_q], optional: log sum_j exp(s_j).
 *   workspace  device scratch of at least kvq_attention_workspace_size bytes (may be
 *            NULL when that size is 0). Contents on entry do not matter.
 *   append_dst  optional host descriptor (NULL: none): the current chunk is also
 *            quantized and appended to this segment in the same call, as
 *            kvq_quantize_append with k_src = k_cur, v_src = v_cur, src_tokens = n_new =
 *            n_cur would do it [JB: the finished chunk joins the cache of earlier chunks],
 *            and the descriptor is advanced on KVQ_OK. The attention reads every segment
 *            as it was before the call, so append_dst may be one of segs (the new tokens
 *            land past its n_tokens). For packed segments on the chunk-shaped path the
 *            append runs in extra workgroups of the attention's own launch, placed after
 *            the attention's so that they fill the CUs its last round leaves idle; the
 *            decode-shaped path and raw segments launch the quantize-append kernel right
 *            after the attention. Capacity and shape errors are those of
 *            kvq_quantize_append, reported before anything is enqueued.
 * Errors: KVQ_ERR_ARG (nulls, shape mismatch, no tokens at all, n_q_heads not a
 * multiple of n_kv_heads), KVQ_ERR_UNSUPPORTED (dtypes, head_dim, bits, too many
 * segments, jensen not a kvq_jensen value, KVQ_JENSEN_EXACT with a segment that holds
 * per-token K groups or a compensation basis, segments whose per-token K groups or
 * compensation differ in kind, width or basis), KVQ_ERR_WORKSPACE.
 */
typedef struct kvq_attn_args {
    const void *q;
    int32_t dtype;
    int32_t batch, n_q_heads, n_kv_heads, head_dim, n_q;
    const kvq_segment *segs;   /* host */
    int32_t n_segs;
    const void *k_cur, *v_cur;
    int32_t n_cur;
    float softmax_scale;
    int32_t jensen;
    void *out;
    int32_t out_dtype;
    float *lse;
    void *workspace;
    size_t workspace_bytes;
    kvq_segment *append_dst;   /* host, optional (see above) */
} kvq_attn_args;

/*
 * kvq_chunk_attention_noalloc -- kvq_chunk_attention for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same checks, kernels and results, but the partial results go to a
 * static device array of the library (KVQ_NOALLOC_SCRATCH_BYTES per GPU, held from the
 * first use on that GPU until the process ends) instead of a caller workspace;
 * workspace and workspace_bytes are ignored. The call allocates and frees nothing. Its
 * first call on a device looks up the array's address there (with that device current).
 * All calls on one GPU share that GPU's array: calls that overlap in time on one GPU (two
 * streams, or two host threads) race on it and must be serialized by the caller. The
 * array needs no clearing: every partial a call reads was written earlier in the same
 * call.
 * Errors: as kvq_chunk_attention; KVQ_ERR_WORKSPACE when the call needs more scratch than
 * the array holds (kvq_attention_workspace_size > KVQ_NOALLOC_SCRATCH_BYTES; on MI355X the
 * largest plan needs 35.7 MB, so no valid call is refused there); KVQ_ERR_HIP when the
 * array's address cannot be looked up.
 */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)36 << 20)
kvq_status kvq_chunk_attention_noalloc(const kvq_attn_args *args, void *stream);

/* Bytes of workspace kvq_chunk_attention needs for these arguments (pointers are not
 * read). Host only; returns KVQ_ERR_ARG / KVQ_ERR_UNSUPPORTED for arguments that
 * kvq_chunk_attention would reject on shape grounds. The size does not grow with the
 * cache: it is 0 when the work divides into whole row blocks of 256 query rows, at most
 * 2 x CUs x 256 rows x (2 head_dim + 16) bytes when the chunk-shaped path splits row
 * blocks between workgroups (35.7 MB at head_dim 128 on 256 CUs; partial rows are kept
 * as 16-bit mantissas with a per-row power-of-two scale), and at most
 * 1023 x 16 rows x (head_dim + 2) x 4 bytes on the decode-shaped path. */
kvq_status kvq_attention_workspace_size(const kvq_attn_args *args, size_t *bytes);

kvq_status kvq_chunk_attention(const kvq_attn_args *args, void *stream);

/*
 * kvq_probe_hbm_read -- a measurement aid, not a step of the method: reads the `bytes`
 * bytes at device address `buf` once, as a plain coalesced stream of 16-byte loads, so
 * that timing it on `stream` gives the HBM read bandwidth the device reaches (the
 * attention and quantize-append kernels are rated against that as well as against the
 * published peak). Use a buffer well above the last-level cache (256 MB on MI355X).
 * `sink` (device uint32) is written only if an XOR of everything read equals a fixed
 * constant; its contents do not matter.
 * Errors: KVQ_ERR_ARG (null or misaligned buf, bytes 0 or not a multiple of 16, null sink).
 */
kvq_status kvq_probe_hbm_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* Static, never-NULL description of a status code. */
const char *kvq_status_string(kvq_status status);

/* KVQ_ABI_VERSION of the loaded library. */
int32_t kvq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
