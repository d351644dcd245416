// C ABI of libkvq (declared and documented in include/kvq.h): argument checks on the host,
// then kernel launches on the caller's stream. Nothing here allocates, frees or waits.
#include <math.h>

#include "kvq.h"
#include "kvq_internal.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool half_dtype(int32_t d) { return d == KVQ_F16 || d == KVQ_BF16; }
bool any_dtype(int32_t d) { return d == KVQ_F32 || d == KVQ_F16 || d == KVQ_BF16; }
// the kernels compare the jensen field with this value (JENSEN_ISO)
static_assert(KVQ_JENSEN_ISO == 2, "isotropic Jensen form value");

kvq_status check_segment_shape(const kvq_segment &s) {
    if (s.bits != 2 && s.bits != 4 && s.bits != 16) return KVQ_ERR_UNSUPPORTED;
    if (!half_dtype(s.elem_dtype)) return KVQ_ERR_UNSUPPORTED;
    if (s.head_dim != 64 && s.head_dim != 128) return KVQ_ERR_UNSUPPORTED;
    if (s.batch < 1 || s.n_kv_heads < 1 || s.capacity < 0 || s.n_tokens < 0 || s.n_tokens > s.capacity)
        return KVQ_ERR_ARG;
    if (s.k_group_tokens < 1 || s.k_group_tokens > 1024) return KVQ_ERR_UNSUPPORTED;
    if (s.bits != 16) {
        if (s.v_group_channels != 32) return KVQ_ERR_UNSUPPORTED;
        if (s.kgroup_capacity < 0 || s.n_kgroups < 0 || s.n_kgroups > s.kgroup_capacity) return KVQ_ERR_ARG;
    }
    return KVQ_OK;
}

kvq_status check_segment_ptrs(const kvq_segment &s) {
    if (!s.k || !s.v || !aligned16(s.k) || !aligned16(s.v)) return KVQ_ERR_ARG;
    if (s.bits != 16) {
        if (!s.k_meta || !s.v_meta || !s.kgroup_start) return KVQ_ERR_ARG;
        if (!aligned16(s.k_meta) || !aligned16(s.v_meta)) return KVQ_ERR_ARG;
    }
    return KVQ_OK;
}

// Shape checks shared by kvq_chunk_attention and kvq_attention_workspace_size.
kvq_status check_attention_shape(const kvq_attn_args *a, long long *n_total) {
    if (!a) return KVQ_ERR_ARG;
    if (!half_dtype(a->dtype)) return KVQ_ERR_UNSUPPORTED;
    if (a->head_dim != 64 && a->head_dim != 128) return KVQ_ERR_UNSUPPORTED;
    if (a->batch < 1 || a->n_q_heads < 1 || a->n_kv_heads < 1 || a->n_q < 1 || a->n_cur < 0)
        return KVQ_ERR_ARG;
    if (a->n_q_heads % a->n_kv_heads != 0) return KVQ_ERR_ARG;
    if (a->n_segs < 0) return KVQ_ERR_ARG;
    if (a->n_segs > KVQ_MAX_SEGMENTS) return KVQ_ERR_UNSUPPORTED;
    if (a->n_segs > 0 && !a->segs) return KVQ_ERR_ARG;
    if (a->jensen != KVQ_JENSEN_OFF && a->jensen != KVQ_JENSEN_TAYLOR2 && a->jensen != KVQ_JENSEN_ISO)
        return KVQ_ERR_UNSUPPORTED;
    if (!any_dtype(a->out_dtype)) return KVQ_ERR_UNSUPPORTED;
    if (!(a->softmax_scale >= 0.0f) || isinf(a->softmax_scale)) return KVQ_ERR_ARG;
    long long n = a->n_cur;
    for (int i = 0; i < a->n_segs; ++i) {
        const kvq_segment &s = a->segs[i];
        kvq_status st = check_segment_shape(s);
        if (st != KVQ_OK) return st;
        if (s.elem_dtype != a->dtype) return KVQ_ERR_UNSUPPORTED;
        if (s.batch != a->batch || s.n_kv_heads != a->n_kv_heads || s.head_dim != a->head_dim)
            return KVQ_ERR_ARG;
        n += s.n_tokens;
    }
    if (n < 1 || n > (1ll << 30)) return KVQ_ERR_ARG;
    const long long rows = (long long)a->batch * a->n_q_heads * a->n_q;
    if (rows > (1ll << 31) / a->head_dim) return KVQ_ERR_ARG;
    *n_total = n;
    return KVQ_OK;
}

// Which attention kernel a call runs (the workspace size depends on it).
bool use_decode(const kvq_attn_args *a) {
    int bits[KVQ_MAX_SEGMENTS];
    int n = 0;
    for (int i = 0; i < a->n_segs; ++i)
        if (a->segs[i].n_tokens > 0) bits[n++] = a->segs[i].bits;
    return kvq::decode_eligible(a->dtype, a->n_q_heads, a->n_kv_heads, a->head_dim, a->n_q, bits, n);
}

}  // namespace

extern "C" {

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char *kvq_status_string(kvq_status status) {
    switch (status) {
        case KVQ_OK: return "ok";
        case KVQ_ERR_ARG: return "invalid argument";
        case KVQ_ERR_UNSUPPORTED: return "unsupported bit-width, head_dim, group size or dtype";
        case KVQ_ERR_CAPACITY: return "segment capacity exceeded";
        case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
        case KVQ_ERR_HIP: return "HIP launch failure";
    }
    return "unknown status";
}

kvq_status kvq_quantize_append(const kvq_append_args *a, void *stream) {
    if (!a || !a->dst) return KVQ_ERR_ARG;
    kvq_segment &s = *a->dst;
    kvq_status st = check_segment_shape(s);
    if (st != KVQ_OK) return st;
    if (!any_dtype(a->src_dtype)) return KVQ_ERR_UNSUPPORTED;
    if (a->n_new < 0) return KVQ_ERR_ARG;
    if (a->n_new == 0) return KVQ_OK;
    if ((st = check_segment_ptrs(s)) != KVQ_OK) return st;
    if (!a->k_src || !a->v_src || !aligned16(a->k_src) || !aligned16(a->v_src)) return KVQ_ERR_ARG;
    int n_groups;
    if (a->src_groups) {
        if (a->n_src_groups < 1 || a->n_src_groups > a->n_new || a->src_tokens < 1) return KVQ_ERR_ARG;
        if ((long long)a->n_src_groups * s.k_group_tokens < a->n_new) return KVQ_ERR_ARG;
        n_groups = a->n_src_groups;
    } else {
        if (a->src_tokens < a->n_new) return KVQ_ERR_ARG;
        n_groups = (a->n_new + s.k_group_tokens - 1) / s.k_group_tokens;
    }
    if ((long long)s.n_tokens + a->n_new > s.capacity) return KVQ_ERR_CAPACITY;
    if (s.bits != 16 && (long long)s.n_kgroups + n_groups > s.kgroup_capacity) return KVQ_ERR_CAPACITY;

    kvq::QuantAppendParams p;
    p.k_src = a->k_src;
    p.v_src = a->v_src;
    p.src_dtype = a->src_dtype;
    p.src_tokens = a->src_tokens;
    p.n_new = a->n_new;
    p.src_groups = a->src_groups;
    p.k_group_tokens = s.k_group_tokens;
    p.batch = s.batch;
    p.n_kv_heads = s.n_kv_heads;
    p.head_dim = s.head_dim;
    p.capacity = s.capacity;
    p.kgroup_capacity = s.kgroup_capacity;
    p.n_tokens = s.n_tokens;
    p.n_kgroups = s.n_kgroups;
    p.elem_dtype = s.elem_dtype;
    p.k_dst = s.k;
    p.v_dst = s.v;
    p.k_meta = s.k_meta;
    p.v_meta = s.v_meta;
    p.kgroup_start = s.kgroup_start;
    if (kvq::launch_quant_append(p, s.bits, n_groups, (hipStream_t)stream) != hipSuccess) return KVQ_ERR_HIP;
    s.n_tokens += a->n_new;
    if (s.bits != 16) s.n_kgroups += n_groups;
    return KVQ_OK;
}

kvq_status kvq_assign_windows(const kvq_window_args *a, void *stream) {
    if (!a) return KVQ_ERR_ARG;
    if (!any_dtype(a->k_dtype)) return KVQ_ERR_UNSUPPORTED;
    if (a->head_dim < 1 || a->head_dim > 256) return KVQ_ERR_UNSUPPORTED;
    if (a->n_kv_heads < 1 || a->n_tokens < 1 || a->window < 1) return KVQ_ERR_ARG;
    if (!a->k || !a->text_query || !a->bits_out || !a->order_out || !a->score_out) return KVQ_ERR_ARG;
    const long long W = ((long long)a->n_tokens + a->window - 1) / a->window;
    if (W > 16384) return KVQ_ERR_UNSUPPORTED;
    if (a->n_fp16 < 1 || a->n_int4 < 0 || (long long)a->n_fp16 + a->n_int4 > W) return KVQ_ERR_ARG;
    kvq::WindowParams p;
    p.k = a->k;
    p.k_dtype = a->k_dtype;
    p.n_kv_heads = a->n_kv_heads;
    p.head_dim = a->head_dim;
    p.n_tokens = a->n_tokens;
    p.window = a->window;
    p.n_windows = (int32_t)W;
    p.text = a->text_query;
    p.n_fp16 = a->n_fp16;
    p.n_int4 = a->n_int4;
    p.bits_out = a->bits_out;
    p.order_out = a->order_out;
    p.score = a->score_out;
    return kvq::launch_windows(p, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

kvq_status kvq_attention_workspace_size(const kvq_attn_args *a, size_t *bytes) {
    if (!bytes) return KVQ_ERR_ARG;
    long long n_total = 0;
    kvq_status st = check_attention_shape(a, &n_total);
    if (st != KVQ_OK) return st;
    kvq::AttnPlan plan;
    kvq::attention_plan(a->batch, a->n_q_heads, a->n_kv_heads, a->head_dim, a->n_q, (int)n_total, use_decode(a),
                        &plan);
    *bytes = plan.workspace_bytes;
    return KVQ_OK;
}

kvq_status kvq_chunk_attention(const kvq_attn_args *a, void *stream) {
    long long n_total = 0;
    kvq_status st = check_attention_shape(a, &n_total);
    if (st != KVQ_OK) return st;
    if (!a->q || !aligned16(a->q) || !a->out || !aligned16(a->out)) return KVQ_ERR_ARG;
    if (a->n_cur > 0 && (!a->k_cur || !a->v_cur || !aligned16(a->k_cur) || !aligned16(a->v_cur)))
        return KVQ_ERR_ARG;
    for (int i = 0; i < a->n_segs; ++i)
        if (a->segs[i].n_tokens > 0 && (st = check_segment_ptrs(a->segs[i])) != KVQ_OK) return st;
    const bool decode = use_decode(a);
    kvq::AttnPlan plan;
    kvq::attention_plan(a->batch, a->n_q_heads, a->n_kv_heads, a->head_dim, a->n_q, (int)n_total, decode, &plan);
    const size_t need = plan.workspace_bytes;
    if (need > 0 && (!a->workspace || a->workspace_bytes < need || !aligned16(a->workspace)))
        return KVQ_ERR_WORKSPACE;

    kvq::AttnParams p;
    p.q = a->q;
    p.dtype = a->dtype;
    p.batch = a->batch;
    p.n_q_heads = a->n_q_heads;
    p.n_kv_heads = a->n_kv_heads;
    p.head_dim = a->head_dim;
    p.n_q = a->n_q;
    p.n_segs = 0;
    int begin = 0;
    for (int i = 0; i < a->n_segs; ++i) {
        const kvq_segment &s = a->segs[i];
        if (s.n_tokens == 0) continue;
        kvq::SegmentView &v = p.segs[p.n_segs++];
        v.bits = s.bits;
        v.n_tokens = s.n_tokens;
        v.n_kgroups = s.bits == 16 ? 0 : s.n_kgroups;
        v.capacity = s.capacity;
        v.kgroup_capacity = s.kgroup_capacity;
        v.v_group_channels = s.v_group_channels;
        v.token_begin = begin;
        v.pad_ = 0;
        v.k = s.k;
        v.v = s.v;
        v.k_meta = reinterpret_cast<const uint32_t *>(s.k_meta);
        v.v_meta = reinterpret_cast<const uint32_t *>(s.v_meta);
        v.kgroup_start = s.kgroup_start;
        begin += s.n_tokens;
    }
    p.k_cur = a->k_cur;
    p.v_cur = a->v_cur;
    p.n_cur = a->n_cur;
    p.n_total = (int32_t)n_total;
    const double scale = a->softmax_scale > 0.0f ? (double)a->softmax_scale : 1.0 / sqrt((double)a->head_dim);
    const double log2e = 1.4426950408889634074;
    p.scale_log2 = (float)(scale * log2e);
    p.beta_log2 = a->jensen != KVQ_JENSEN_OFF ? (float)(scale * scale / 24.0 * log2e) : 0.0f;
    p.jensen = a->jensen;
    p.out = a->out;
    p.out_dtype = a->out_dtype;
    p.lse = a->lse;
    p.n_split = plan.n_split;
    p.split_tokens = plan.split_tokens;
    p.n_rb = plan.n_rb;
    p.tok_pad = plan.tok_pad;
    p.quota = plan.quota;
    p.work = plan.work;
    p.partial = reinterpret_cast<float *>(a->workspace);
    p.decode = decode ? 1 : 0;
    return kvq::launch_attention(p, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // extern "C"
