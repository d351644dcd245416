// Drives the library's host code (argument checks, planners, the budget rule) through the
// C ABI on a machine without a GPU, for a build under AddressSanitizer and
// UndefinedBehaviorSanitizer. Every call here is rejected or answered before any launch.
#include <stdio.h>
#include <string.h>

#include "kvq.h"

static int fails = 0;
#define EXPECT(cond) do { if (!(cond)) { fprintf(stderr, "line %d: %s\n", __LINE__, #cond); ++fails; } } while (0)

static kvq_segment seg(int bits, int n_tokens, int n_kgroups) {
    kvq_segment s;
    memset(&s, 0, sizeof(s));
    s.bits = bits; s.elem_dtype = KVQ_BF16; s.batch = 1; s.n_kv_heads = 2; s.head_dim = 128;
    s.capacity = 20000; s.n_tokens = n_tokens; s.k_group_tokens = 128; s.v_group_channels = 32;
    s.kgroup_capacity = 200; s.n_kgroups = n_kgroups;
    void *fake = (void *)0x100000;
    s.k = s.v = s.k_meta = s.v_meta = fake; s.kgroup_start = (int32_t *)fake;
    return s;
}

int main(void) {
    void *fake = (void *)0x100000;
    kvq_segment segs[KVQ_MAX_SEGMENTS + 1];
    for (int i = 0; i <= KVQ_MAX_SEGMENTS; ++i) segs[i] = seg(2, 1000, 8);
    kvq_attn_args a;
    memset(&a, 0, sizeof(a));
    a.q = fake; a.dtype = KVQ_BF16; a.batch = 1; a.n_q_heads = 4; a.n_kv_heads = 2; a.head_dim = 128; a.n_q = 100;
    a.segs = segs; a.n_segs = 3; a.k_cur = a.v_cur = fake; a.n_cur = 50; a.jensen = 1; a.out = fake;
    a.out_dtype = KVQ_F32;
    size_t bytes = 0;
    // planners over many shapes (row blocks, shares, decode splits)
    for (int nq = 1; nq <= 70000; nq = nq * 3 + 1)
        for (int ns = 0; ns <= 3; ++ns) {
            a.n_q = nq; a.n_segs = ns; a.n_cur = ns == 0 ? 17 : 0;
            EXPECT(kvq_attention_workspace_size(&a, &bytes) == KVQ_OK);
        }
    a.n_q = 100; a.n_segs = 3; a.n_cur = 50;
    // rejections before any launch
    a.n_segs = KVQ_MAX_SEGMENTS + 1;
    EXPECT(kvq_chunk_attention(&a, nullptr) == KVQ_ERR_UNSUPPORTED);
    a.n_segs = 3;
    a.jensen = 7;
    EXPECT(kvq_chunk_attention(&a, nullptr) == KVQ_ERR_UNSUPPORTED);
    a.jensen = 1;
    // 2 row blocks of 200 queries: an equal-shares plan, whose partials need a workspace
    EXPECT(kvq_chunk_attention(&a, nullptr) == KVQ_ERR_WORKSPACE);
    segs[1].k_group_channels = 32;
    a.jensen = KVQ_JENSEN_EXACT;
    EXPECT(kvq_chunk_attention(&a, nullptr) == KVQ_ERR_UNSUPPORTED);
    segs[1].k_group_channels = 0;
    a.jensen = 1;
    kvq_segment dst = seg(2, 19990, 8);
    a.append_dst = &dst;
    EXPECT(kvq_chunk_attention(&a, nullptr) == KVQ_ERR_CAPACITY);
    EXPECT(dst.n_tokens == 19990);
    a.append_dst = nullptr;
    EXPECT(kvq_chunk_attention(nullptr, nullptr) == KVQ_ERR_ARG);
    EXPECT(kvq_chunk_attention_noalloc(nullptr, nullptr) == KVQ_ERR_ARG);
    // quantize-append checks
    kvq_append_args ap;
    memset(&ap, 0, sizeof(ap));
    kvq_segment s = seg(2, 19900, 150);
    ap.dst = &s; ap.k_src = ap.v_src = fake; ap.src_dtype = KVQ_BF16; ap.src_tokens = 500; ap.n_new = 500;
    EXPECT(kvq_quantize_append(&ap, nullptr) == KVQ_ERR_CAPACITY);
    s.n_tokens = 0;
    s.n_kgroups = 198;
    EXPECT(kvq_quantize_append(&ap, nullptr) == KVQ_ERR_CAPACITY);
    s.comp_rank = 9;
    EXPECT(kvq_quantize_append(&ap, nullptr) == KVQ_ERR_UNSUPPORTED);
    // windows
    int32_t n16 = 0, n4 = 0;
    for (int W = 1; W <= 20000; W = W * 2 + 1)
        for (int p16 = 0; p16 <= 100; p16 += 25) EXPECT(kvq_window_budget(W, p16, 100 - p16, &n16, &n4) == KVQ_OK);
    EXPECT(kvq_window_budget(10, 60, 50, &n16, &n4) == KVQ_ERR_ARG);
    kvq_window_args w;
    memset(&w, 0, sizeof(w));
    w.k = fake; w.k_dtype = KVQ_F16; w.n_layers = 1; w.n_kv_heads = 2; w.head_dim = 64; w.n_tokens = 16384 * 32 + 1;
    w.window = 32; w.text_query = (const float *)fake; w.bits_out = (int8_t *)fake; w.order_out = (int32_t *)fake;
    w.score_out = (double *)fake;
    EXPECT(kvq_assign_windows(&w, nullptr) == KVQ_ERR_UNSUPPORTED);
    EXPECT(kvq_probe_hbm_read(fake, 1000, (uint32_t *)fake, nullptr) == KVQ_ERR_ARG);
    for (int st = -6; st <= 1; ++st) EXPECT(kvq_status_string((kvq_status)st) != nullptr);
    printf("host driver: %d failures\n", fails);
    return fails != 0;
}
