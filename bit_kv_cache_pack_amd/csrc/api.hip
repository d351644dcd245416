// C ABI of libkvq (declared and documented in include/kvq.h): argument checks on the host,
// then kernel launches on the caller's stream. Nothing here allocates, frees or waits.
#include <math.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "kvq.h"
#include "kvq_internal.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool half_dtype(int32_t d) { return d == KVQ_F16 || d == KVQ_BF16; }
bool any_dtype(int32_t d) { return d == KVQ_F32 || d == KVQ_F16 || d == KVQ_BF16; }
// the kernels compare the jensen field with these values (JENSEN_ISO, JENSEN_EXACT)
static_assert(KVQ_JENSEN_ISO == 2, "isotropic Jensen form value");
static_assert(KVQ_JENSEN_EXACT == 3, "all-orders Jensen form value");

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
        if (s.k_group_channels != 0 && s.k_group_channels != 32 && s.k_group_channels != 64 &&
            s.k_group_channels != 128)
            return KVQ_ERR_UNSUPPORTED;
        if (s.k_group_channels > s.head_dim) return KVQ_ERR_UNSUPPORTED;
        if (s.comp_rank < 0 || s.comp_rank > 8) return KVQ_ERR_UNSUPPORTED;
        if (s.comp_rank > 0 && s.k_group_channels != 0) return KVQ_ERR_UNSUPPORTED;
    } else if (s.k_group_channels != 0 || s.comp_rank != 0) {
        return KVQ_ERR_UNSUPPORTED;
    }
    return KVQ_OK;
}

kvq_status check_segment_ptrs(const kvq_segment &s) {
    if (!s.k || !s.v || !aligned16(s.k) || !aligned16(s.v)) return KVQ_ERR_ARG;
    if (s.bits != 16) {
        if (!s.k_meta || !s.v_meta || (s.k_group_channels == 0 && !s.kgroup_start)) return KVQ_ERR_ARG;
        if (!aligned16(s.k_meta) || !aligned16(s.v_meta)) return KVQ_ERR_ARG;
        if (s.comp_rank > 0 && (!s.comp_basis || !s.k_comp || !aligned16(s.k_comp) || !aligned16(s.comp_basis)))
            return KVQ_ERR_ARG;
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
    if (a->jensen != KVQ_JENSEN_OFF && a->jensen != KVQ_JENSEN_TAYLOR2 && a->jensen != KVQ_JENSEN_ISO &&
        a->jensen != KVQ_JENSEN_EXACT)
        return KVQ_ERR_UNSUPPORTED;
    if (!any_dtype(a->out_dtype)) return KVQ_ERR_UNSUPPORTED;
    if (!(a->softmax_scale >= 0.0f) || isinf(a->softmax_scale)) return KVQ_ERR_ARG;
    long long n = a->n_cur;
    const kvq_segment *aug = nullptr;   // the first segment with per-token K groups or compensation
    for (int i = 0; i < a->n_segs; ++i) {
        const kvq_segment &s = a->segs[i];
        kvq_status st = check_segment_shape(s);
        if (st != KVQ_OK) return st;
        if (s.elem_dtype != a->dtype) return KVQ_ERR_UNSUPPORTED;
        if (s.batch != a->batch || s.n_kv_heads != a->n_kv_heads || s.head_dim != a->head_dim)
            return KVQ_ERR_ARG;
        if (s.bits != 16 && s.n_tokens > 0 && (s.k_group_channels > 0 || s.comp_rank > 0)) {
            // per-token K groups take the all-orders Jensen form nowhere; segments with extra
            // per-token K columns in one call all use the same kind (and basis)
            if (a->jensen == KVQ_JENSEN_EXACT) return KVQ_ERR_UNSUPPORTED;
            if (aug && (aug->k_group_channels != s.k_group_channels || aug->comp_rank != s.comp_rank ||
                        aug->comp_basis != s.comp_basis))
                return KVQ_ERR_UNSUPPORTED;
            aug = &s;
        }
        n += s.n_tokens;
    }
    if (n < 1 || n > (1ll << 30)) return KVQ_ERR_ARG;
    const long long rows = (long long)a->batch * a->n_q_heads * a->n_q;
    if (rows > (1ll << 31) / a->head_dim) return KVQ_ERR_ARG;
    *n_total = n;
    return KVQ_OK;
}

// Which attention kernel a call runs (the workspace size depends on it).
bool use_decode(const kvq_attn_args *a, long long n_total) {
    int bits[KVQ_MAX_SEGMENTS];
    int n = 0;
    for (int i = 0; i < a->n_segs; ++i) {
        const kvq_segment &s = a->segs[i];
        if (s.n_tokens == 0) continue;
        // per-token K groups and the compensation are chunk-kernel features
        if (s.bits != 16 && (s.k_group_channels > 0 || s.comp_rank > 0)) return false;
        bits[n++] = s.bits;
    }
    return kvq::decode_eligible(a->dtype, a->batch, a->n_q_heads, a->n_kv_heads, a->head_dim, a->n_q, bits, n,
                                a->n_cur, (int)n_total);
}

// Scratch of kvq_chunk_attention_noalloc: the partial results that kvq_chunk_attention
// keeps in the caller's workspace. Every GPU the library runs on holds its own copy of this
// array until the process ends. In host code its name is only a stand-in for the symbol:
// the device address comes from hipGetSymbolAddress, once per device (with that device
// current), and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's address of the scratch array (looked up on its first use).
kvq_status scratch_address(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return KVQ_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return KVQ_ERR_HIP;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return KVQ_OK;
}

kvq_status run_attention(const kvq_attn_args *a, void *stream, bool use_static);

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
    const bool table = s.bits != 16 && s.k_group_channels == 0;   // the segment keeps a K-group table
    if (table && (long long)s.n_kgroups + n_groups > s.kgroup_capacity) return KVQ_ERR_CAPACITY;

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
    p.k_group_channels = s.bits != 16 ? s.k_group_channels : 0;
    p.comp_rank = s.bits != 16 ? s.comp_rank : 0;
    p.comp_basis = s.comp_basis;
    p.k_comp = s.k_comp;
    if (kvq::launch_quant_append(p, s.bits, n_groups, (hipStream_t)stream) != hipSuccess) return KVQ_ERR_HIP;
    s.n_tokens += a->n_new;
    if (table) s.n_kgroups += n_groups;
    return KVQ_OK;
}

kvq_status kvq_window_budget(int32_t n_windows, int32_t pct_fp16, int32_t pct_int4, int32_t *n_fp16,
                             int32_t *n_int4) {
    if (!n_fp16 || !n_int4 || n_windows < 1) return KVQ_ERR_ARG;
    if (pct_fp16 < 0 || pct_int4 < 0 || pct_fp16 > 100 || pct_int4 > 100 || pct_fp16 + pct_int4 > 100)
        return KVQ_ERR_ARG;
    int a = 0, b = 0;
    kvq::window_budget(n_windows, pct_fp16, pct_int4, &a, &b);
    *n_fp16 = a;
    *n_int4 = b;
    return KVQ_OK;
}

kvq_status kvq_assign_windows(const kvq_window_args *a, void *stream) {
    if (!a) return KVQ_ERR_ARG;
    if (!any_dtype(a->k_dtype)) return KVQ_ERR_UNSUPPORTED;
    if (a->head_dim < 1 || a->head_dim > 256) return KVQ_ERR_UNSUPPORTED;
    if (a->n_layers < 1 || a->n_kv_heads < 1 || a->n_tokens < 1 || a->window < 1) return KVQ_ERR_ARG;
    if (a->n_layers > kvq::kMaxWindowLayers) return KVQ_ERR_UNSUPPORTED;
    if (!a->k || !a->text_query || !a->bits_out || !a->order_out || !a->score_out) return KVQ_ERR_ARG;
    const long long W = ((long long)a->n_tokens + a->window - 1) / a->window;
    if (W > kvq::kMaxWindowsPerLayer) return KVQ_ERR_UNSUPPORTED;
    int32_t n16 = 0, n4 = 0;
    kvq_status st = kvq_window_budget((int32_t)W, a->pct_fp16, a->pct_int4, &n16, &n4);
    if (st != KVQ_OK) return st;
    kvq::WindowParams p;
    p.k = a->k;
    p.k_dtype = a->k_dtype;
    p.n_layers = a->n_layers;
    p.n_kv_heads = a->n_kv_heads;
    p.head_dim = a->head_dim;
    p.n_tokens = a->n_tokens;
    p.window = a->window;
    p.n_windows = (int32_t)W;
    p.text = a->text_query;
    p.n_fp16 = n16;
    p.n_int4 = n4;
    p.bits_out = a->bits_out;
    p.order_out = a->order_out;
    p.score = a->score_out;
    p.groups_out = a->groups_out;
    p.class_tokens_out = a->class_tokens_out;
    return kvq::launch_windows(p, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

kvq_status kvq_probe_hbm_read(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
    if (!buf || !sink || !aligned16(buf) || bytes == 0 || bytes % 16 != 0) return KVQ_ERR_ARG;
    return kvq::launch_hbm_read(buf, bytes, sink, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

kvq_status kvq_attention_workspace_size(const kvq_attn_args *a, size_t *bytes) {
    if (!bytes) return KVQ_ERR_ARG;
    long long n_total = 0;
    kvq_status st = check_attention_shape(a, &n_total);
    if (st != KVQ_OK) return st;
    kvq::AttnPlan plan;
    kvq::attention_plan(a->batch, a->n_q_heads, a->n_kv_heads, a->head_dim, a->n_q, (int)n_total, use_decode(a, n_total),
                        &plan);
    *bytes = plan.workspace_bytes;
    return KVQ_OK;
}

kvq_status kvq_chunk_attention(const kvq_attn_args *a, void *stream) {
    return run_attention(a, stream, false);
}

kvq_status kvq_chunk_attention_noalloc(const kvq_attn_args *a, void *stream) {
    return run_attention(a, stream, true);
}

}  // extern "C"

namespace {

// Checks, plan, launches. With use_static the partials go to this device's static scratch
// array instead of the caller's workspace (which is then ignored).
kvq_status run_attention(const kvq_attn_args *a, void *stream, bool use_static) {
    long long n_total = 0;
    kvq_status st = check_attention_shape(a, &n_total);
    if (st != KVQ_OK) return st;
    if (!a->q || !aligned16(a->q) || !a->out || !aligned16(a->out)) return KVQ_ERR_ARG;
    if (a->n_cur > 0 && (!a->k_cur || !a->v_cur || !aligned16(a->k_cur) || !aligned16(a->v_cur)))
        return KVQ_ERR_ARG;
    for (int i = 0; i < a->n_segs; ++i)
        if (a->segs[i].n_tokens > 0 && (st = check_segment_ptrs(a->segs[i])) != KVQ_OK) return st;
    // the optional quantize-append of the current chunk: checked as kvq_quantize_append would
    kvq_segment *dst = a->n_cur > 0 ? a->append_dst : nullptr;
    int app_groups = 0;
    if (dst) {
        if ((st = check_segment_shape(*dst)) != KVQ_OK) return st;
        if ((st = check_segment_ptrs(*dst)) != KVQ_OK) return st;
        if (dst->batch != a->batch || dst->n_kv_heads != a->n_kv_heads || dst->head_dim != a->head_dim)
            return KVQ_ERR_ARG;
        app_groups = (a->n_cur + dst->k_group_tokens - 1) / dst->k_group_tokens;
        if ((long long)dst->n_tokens + a->n_cur > dst->capacity) return KVQ_ERR_CAPACITY;
        if (dst->bits != 16 && dst->k_group_channels == 0 &&
            (long long)dst->n_kgroups + app_groups > dst->kgroup_capacity)
            return KVQ_ERR_CAPACITY;
    }
    const bool decode = use_decode(a, n_total);
    kvq::AttnPlan plan;
    kvq::attention_plan(a->batch, a->n_q_heads, a->n_kv_heads, a->head_dim, a->n_q, (int)n_total, decode, &plan);
    const size_t need = plan.workspace_bytes;
    void *workspace = a->workspace;
    if (use_static) {
        if (need > KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE;
        workspace = nullptr;
        if (need > 0 && (st = scratch_address(&workspace)) != KVQ_OK) return st;
    } else if (need > 0 && (!workspace || a->workspace_bytes < need || !aligned16(workspace))) {
        return KVQ_ERR_WORKSPACE;
    }

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
        v.n_kgroups = s.bits == 16 || s.k_group_channels > 0 ? 0 : s.n_kgroups;
        v.k_group_channels = s.bits == 16 ? 0 : s.k_group_channels;
        v.k_comp = s.bits != 16 && s.comp_rank > 0 ? reinterpret_cast<const uint16_t *>(s.k_comp) : nullptr;
        v.capacity = s.capacity;
        v.kgroup_capacity = s.kgroup_capacity;
        v.v_group_channels = s.v_group_channels;
        v.token_begin = begin;
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
    p.beta_log2 = a->jensen == KVQ_JENSEN_OFF ? 0.0f
                  : a->jensen == KVQ_JENSEN_EXACT ? 1.0f : (float)(scale * scale / 24.0 * log2e);
    p.half_scale = (float)(scale / 2.0);
    p.jensen = a->jensen;
    p.aug = p.aug_kgc = p.aug_rank = 0;
    p.aug_basis = nullptr;
    for (int i = 0; i < a->n_segs; ++i) {
        const kvq_segment &s = a->segs[i];
        if (s.n_tokens == 0 || s.bits == 16) continue;
        if (s.k_group_channels > 0) {
            p.aug = 1;
            p.aug_kgc = s.k_group_channels;
        } else if (s.comp_rank > 0) {
            p.aug = 2;
            p.aug_rank = s.comp_rank;
            p.aug_basis = s.comp_basis;
        }
    }
    p.out = a->out;
    p.out_dtype = a->out_dtype;
    p.lse = a->lse;
    p.n_split = plan.n_split;
    p.split_tokens = plan.split_tokens;
    p.n_rb = plan.n_rb;
    p.tok_pad = plan.tok_pad;
    p.quota = plan.quota;
    p.work = plan.work;
    p.partial = reinterpret_cast<float *>(workspace);
    p.decode = decode ? 1 : 0;
    p.app_bits = p.app_groups = p.n_attn_wg = p.app_per_wg = 0;
    bool append_after = false;
    if (dst) {
        kvq::QuantAppendParams &q = p.app;
        q.k_src = a->k_cur;
        q.v_src = a->v_cur;
        q.src_dtype = a->dtype;
        q.src_tokens = a->n_cur;
        q.n_new = a->n_cur;
        q.src_groups = nullptr;
        q.k_group_tokens = dst->k_group_tokens;
        q.batch = dst->batch;
        q.n_kv_heads = dst->n_kv_heads;
        q.head_dim = dst->head_dim;
        q.capacity = dst->capacity;
        q.kgroup_capacity = dst->kgroup_capacity;
        q.n_tokens = dst->n_tokens;
        q.n_kgroups = dst->n_kgroups;
        q.elem_dtype = dst->elem_dtype;
        q.k_dst = dst->k;
        q.v_dst = dst->v;
        q.k_meta = dst->k_meta;
        q.v_meta = dst->v_meta;
        q.kgroup_start = dst->kgroup_start;
        q.k_group_channels = dst->bits != 16 ? dst->k_group_channels : 0;
        q.comp_rank = dst->bits != 16 ? dst->comp_rank : 0;
        q.comp_basis = dst->comp_basis;
        q.k_comp = dst->k_comp;
        // packed segments of the plain layout go into the chunk kernel's launch; the decode
        // kernel, raw segments, per-token K groups and the compensation take the
        // quantize-append kernel after the attention
        if (!decode && dst->bits != 16 && dst->k_group_channels == 0 && dst->comp_rank == 0) {
            p.app_bits = dst->bits;
            p.app_groups = app_groups;
        } else {
            append_after = true;
        }
    }
    if (kvq::launch_attention(p, (hipStream_t)stream) != hipSuccess) return KVQ_ERR_HIP;
    if (append_after && kvq::launch_quant_append(p.app, dst->bits, app_groups, (hipStream_t)stream) != hipSuccess)
        return KVQ_ERR_HIP;
    if (dst) {
        dst->n_tokens += a->n_cur;
        if (dst->bits != 16 && dst->k_group_channels == 0) dst->n_kgroups += app_groups;
    }
    return KVQ_OK;
}

}  // namespace
