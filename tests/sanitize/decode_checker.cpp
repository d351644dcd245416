// Host-side check of the decode kernel's memory accesses. It runs the kernel's own walk and
// index functions (decode_walk.cuh) for every workgroup, wave, step and lane of a launch
// plan (decode_plan, as the library makes it), over host buffers of exactly the sizes the
// C ABI gives each array, and reads every element each access would touch. Built with
// AddressSanitizer and UndefinedBehaviorSanitizer, so an index outside a buffer stops the
// run; each access is also checked against its extent explicitly. It also checks that the
// walk visits every token of the range once, that the configurations the kernel was not
// built for are refused by decode_eligible, and the walk alone over a multi-segment table.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "decode_walk.cuh"
#include "kvq.h"   // KVQ_BF16, KVQ_F16: the dtype codes decode_eligible takes

using namespace kvq;
using namespace kvq::dwalk;

static long fails = 0, touched = 0;
#define CHECK(cond, ...)                                         \
    do {                                                         \
        if (!(cond)) {                                           \
            if (fails < 20) {                                    \
                fprintf(stderr, "line %d: %s: ", __LINE__, #cond); \
                fprintf(stderr, __VA_ARGS__);                    \
                fprintf(stderr, "\n");                           \
            }                                                    \
            ++fails;                                             \
        }                                                        \
    } while (0)

struct HostTab {
    static int start(const int32_t *tab, int g) { return tab[g]; }
};

template <class T> struct Buf {
    T *p = nullptr;
    size_t n = 0;
    const char *name = "";
    void alloc(size_t count, const char *nm) {
        n = count;
        name = nm;
        p = static_cast<T *>(malloc(count ? count * sizeof(T) : 1));
        memset(p, 0x5a, count * sizeof(T));
    }
    void release() { free(p); p = nullptr; }
    // every element of [i, i + cnt) exists; reading it lets the sanitizer see the access
    void touch(size_t i, size_t cnt, const char *what) {
        CHECK(i + cnt <= n, "%s: [%zu, %zu) of %zu (%s)", name, i, i + cnt, n, what);
        if (i + cnt <= n) {
            volatile T sink;
            for (size_t k = 0; k < cnt; ++k) sink = p[i + k];
            (void)sink;
            touched += (long)cnt;
        }
    }
};

struct Config {
    const char *name;
    int B, Hq, Hkv, HD, n_q, bits, n_tokens, capacity, Gk, n_cur;
};

// K-group table of a segment appended in groups of Gk, the last one possibly shorter:
// entries [0, n_groups] valid, kgroup_capacity + 1 allocated.
static int build_table(Buf<int32_t> &tab, const Config &c, int kgroup_capacity) {
    tab.alloc((size_t)kgroup_capacity + 1, "kgroup_start");
    int n = 0, g = 0;
    tab.p[0] = 0;
    while (n < c.n_tokens) {
        int len = c.Gk;
        if (c.n_tokens - n < len) len = c.n_tokens - n;
        n += len;
        tab.p[++g] = n;
    }
    return g;
}

template <int HD>
static void check_launch(const Config &c) {
    typedef DGeo<HD> G;
    const int kgroup_capacity = (c.capacity + c.Gk - 1) / c.Gk + 3;
    Buf<int32_t> tab;
    const int n_groups = build_table(tab, c, kgroup_capacity);
    const int wpr = HD * c.bits / 32;
    const size_t BH = (size_t)c.B * c.Hkv;
    Buf<uint32_t> kc, vc, km, vm;
    kc.alloc(BH * c.capacity * wpr, "k codes");
    vc.alloc(BH * c.capacity * wpr, "v codes");
    km.alloc(BH * kgroup_capacity * HD, "k meta");
    vm.alloc(BH * c.capacity * (HD / 32), "v meta");
    Buf<uint16_t> q, kcur, vcur;
    q.alloc((size_t)c.B * c.Hq * c.n_q * HD, "q");
    kcur.alloc(BH * c.n_cur * HD, "k_cur");
    vcur.alloc(BH * c.n_cur * HD, "v_cur");
    Buf<uint16_t> lds;   // one wave's value tile
    lds.alloc(G::VTILE, "LDS value tile");
    Buf<float> epi;      // the same tile read as floats
    epi.alloc(G::VTILE / 2, "LDS epilogue");

    const int n_total = c.n_tokens + c.n_cur;
    const int seg_bits[1] = {c.bits};
    CHECK(decode_eligible(KVQ_BF16, c.B, c.Hq, c.Hkv, HD, c.n_q, seg_bits, 1, c.n_cur, n_total),
          "%s is not a decode case", c.name);
    AttnPlan plan;
    attention_plan(c.B, c.Hq, c.Hkv, HD, c.n_q, n_total, true, &plan);
    const size_t n_rows_total = (size_t)c.B * c.Hq * c.n_q;
    Buf<float> ws, out, lse;
    ws.alloc(plan.workspace_bytes / sizeof(float), "workspace");
    out.alloc(n_rows_total * HD, "out");
    lse.alloc(n_rows_total, "lse");

    AttnParams p;
    memset(&p, 0, sizeof(p));
    p.batch = c.B; p.n_q_heads = c.Hq; p.n_kv_heads = c.Hkv; p.head_dim = HD; p.n_q = c.n_q;
    p.n_segs = 1; p.n_cur = c.n_cur; p.n_total = n_total;
    p.n_split = plan.n_split; p.split_tokens = plan.split_tokens;
    SegmentView &sg = p.segs[0];
    sg.bits = c.bits; sg.n_tokens = c.n_tokens; sg.n_kgroups = n_groups; sg.capacity = c.capacity;
    sg.kgroup_capacity = kgroup_capacity; sg.v_group_channels = 32; sg.token_begin = 0;
    sg.kgroup_start = tab.p;

    const int rows = c.Hq / c.Hkv * c.n_q;
    for (int by = 0; by < c.B * c.Hkv; ++by) {
        const int b = by / c.Hkv, h = by % c.Hkv;
        const size_t bh = (size_t)b * c.Hkv + h;
        long seen = 0;   // tokens this (batch, KV head) visits over all workgroups and waves
        for (int bx = 0; bx < plan.n_split; ++bx) {
            for (int wave = 0; wave < kDWaves; ++wave) {
                // Q operand
                for (int lane = 0; lane < kLanes; ++lane)
                    if (lane % 16 < rows)
                        q.touch(q_elem(HD, out_row(b, h, lane % 16, c.Hq, c.Hkv, c.n_q), lane / 16), HD / 4, "Q");
                for (int i = 0; i < kLanes; ++i)
                    for (int k = i; k < G::VTILE / 8; k += kLanes) lds.touch((size_t)k * 8, 8, "tile clear");
                const int tb = (bx * kDWaves + wave) * p.split_tokens;
                const int te = imin(p.n_total, tb + p.split_tokens);
                Walker<HostTab> wk;
                wk.init();
                int prev_g = -1;
                for (Step st = wk.next(p, tb, te); st.kind != ST_END; st = wk.next(p, tb, te)) {
                    CHECK(st.len >= 1 && st.len <= (st.kind == ST_CUR ? TR : (st.bits == 4 ? TP / 2 : TP)),
                          "%s: step length %d", c.name, st.len);
                    seen += st.len;
                    for (int lane = 0; lane < kLanes; ++lane) {
                        if (st.kind == ST_PACKED) {
                            CHECK(st.g >= 0 && st.g < n_groups, "%s: group %d of %d", c.name, st.g, n_groups);
                            CHECK(st.t >= tab.p[st.g] && st.t + st.len <= tab.p[st.g + 1],
                                  "%s: step [%d, %d) outside group %d", c.name, st.t, st.t + st.len, st.g);
                            const size_t row0 = bh * (size_t)c.capacity + st.t;
                            // every row read is a row of the step: [row0, row0 + len)
                            auto in_step = [&](size_t idx, size_t per_row, const char *what) {
                                const size_t row = idx / per_row;
                                CHECK(row >= row0 && row < row0 + st.len, "%s: %s row %zu outside the step [%zu, %zu)",
                                      c.name, what, row, row0, row0 + st.len);
                            };
                            for (int bb = 0; bb < (st.bits == 2 ? 4 : 2); ++bb) {
                                const size_t kw = k_word(HD, st.bits, row0, st.len, bb, lane);
                                in_step(kw, wpr, "K codes");
                                kc.touch(kw, k_words(HD, st.bits), "K codes");
                            }
                            const size_t vw = v_word(HD, st.bits, row0, st.len, lane);
                            const size_t mw = vm_word(HD, st.bits, row0, st.len, lane);
                            in_step(vw, wpr, "V codes");
                            in_step(mw, HD / 32, "V meta");
                            vc.touch(vw, v_words(HD, st.bits), "V codes");
                            vm.touch(mw, vm_words(HD, st.bits), "V meta");
                            if (st.new_group || st.g != prev_g)
                                km.touch(km_word(HD, bh, kgroup_capacity, st.g, lane), HD / 4, "K meta");
                            if (st.bits == 2)
                                for (int blk = 0; blk < HD / 16; ++blk)
                                    for (int part = 0; part < 2; ++part) lds.touch(vt_int2<HD>(lane, blk, part), 8, "V tile, INT2");
                            else
                                for (int hb = 0; hb < HD / 32; ++hb)
                                    for (int part = 0; part < 2; ++part) lds.touch(vt_int4<HD>(lane, hb, part), 8, "V tile, INT4");
                        } else {
                            const size_t row0 = bh * (size_t)c.n_cur + st.t;
                            const size_t ke = ck_elem(HD, row0, st.len, lane), ve = cv_elem(HD, row0, st.len, lane);
                            CHECK(ke / HD >= row0 && ke / HD < row0 + st.len && ve / HD >= row0 && ve / HD < row0 + st.len,
                                  "%s: current-chunk row outside the step", c.name);
                            kcur.touch(ke, HD / 4, "current K");
                            vcur.touch(ve, HD / 4, "current V");
                            for (int bl = 0; bl < G::NBL; ++bl)
                                for (int part = 0; part < 2; ++part) lds.touch(vt_cur<HD>(lane, bl, part), 8, "V tile, current");
                        }
                        for (int hh = 0; hh < 2; ++hh)
                            for (int db = 0; db < G::DB; ++db) {
                                lds.touch(vt_read<HD>(lane, hh, db), 4, "V tile read");
                                lds.touch(vt_read<HD>(lane, hh, db) + 16 * G::VROW, 4, "V tile read");
                            }
                    }
                    prev_g = st.kind == ST_PACKED ? st.g : prev_g;
                }
                // epilogue: every channel of every row, then m and l
                for (int r = 0; r < 16; ++r) {
                    for (int ch = 0; ch < HD; ++ch) epi.touch(epi_o<HD>(r, ch), 1, "epilogue O");
                    epi.touch(epi_m<HD>(r), 1, "epilogue m");
                    epi.touch(epi_l<HD>(r), 1, "epilogue l");
                }
            }
            for (int r = 0; r < rows; ++r) {
                const size_t qrow = out_row(b, h, r, c.Hq, c.Hkv, c.n_q);
                if (plan.n_split == 1) {
                    out.touch(qrow * HD, HD, "out");
                    lse.touch(qrow, 1, "lse");
                } else {
                    ws.touch(ws_row(bx, n_rows_total, qrow) * (HD + 2), HD + 2, "workspace");
                }
            }
        }
        CHECK(seen == n_total, "%s: (b %d, h %d) walked %ld of %d tokens", c.name, b, h, seen, n_total);
    }
    // the split merge
    if (plan.n_split > 1)
        for (size_t row = 0; row < n_rows_total; ++row) {
            for (int s = 0; s < plan.n_split; ++s) ws.touch(ws_row(s, n_rows_total, row) * (HD + 2), HD + 2, "merge");
            out.touch(row * HD, HD, "merge out");
            lse.touch(row, 1, "merge lse");
        }
    printf("%-34s splits %3d x %4d tokens per wave, %4d K-groups, ok so far: %s\n", c.name, plan.n_split,
           plan.split_tokens, n_groups, fails ? "no" : "yes");
    tab.release(); kc.release(); vc.release(); km.release(); vm.release(); q.release(); kcur.release();
    vcur.release(); lds.release(); epi.release(); ws.release(); out.release(); lse.release();
}

// The walk alone over two packed segments laid out as WindowQuant classes (windows of 32
// tokens, a 16-token last window), head_dim 64: every token once, steps inside their group.
static void check_walk_multi() {
    const int Wn[2] = {184, 368}, last[2] = {32, 16};
    Buf<int32_t> tabs[2];
    AttnParams p;
    memset(&p, 0, sizeof(p));
    int begin = 0;
    for (int s = 0; s < 2; ++s) {
        tabs[s].alloc((size_t)Wn[s] + 1, "window table");
        tabs[s].p[0] = 0;
        for (int w = 0; w < Wn[s]; ++w) tabs[s].p[w + 1] = tabs[s].p[w] + (w == Wn[s] - 1 ? last[s] : 32);
        SegmentView &sg = p.segs[s];
        sg.bits = s == 0 ? 4 : 2; sg.n_kgroups = Wn[s]; sg.n_tokens = tabs[s].p[Wn[s]];
        sg.kgroup_capacity = Wn[s]; sg.token_begin = begin; sg.kgroup_start = tabs[s].p;
        begin += sg.n_tokens;
    }
    p.n_segs = 2; p.n_cur = 0; p.n_total = begin;
    for (int split = 64; split <= 4096; split *= 4) {
        long seen = 0;
        for (int tb = 0; tb < p.n_total; tb += split) {
            Walker<HostTab> wk;
            wk.init();
            for (Step st = wk.next(p, tb, tb + split); st.kind != ST_END; st = wk.next(p, tb, tb + split)) {
                const int32_t *t = tabs[st.seg].p;
                CHECK(st.kind == ST_PACKED && st.t >= t[st.g] && st.t + st.len <= t[st.g + 1],
                      "multi-segment walk: step [%d, %d) of segment %d outside group %d", st.t, st.t + st.len, st.seg,
                      st.g);
                seen += st.len;
            }
        }
        CHECK(seen == p.n_total, "multi-segment walk (split %d): %ld of %d tokens", split, seen, p.n_total);
    }
    tabs[0].release();
    tabs[1].release();
    printf("%-34s ok so far: %s\n", "walk over two window segments", fails ? "no" : "yes");
}

// The value tile's layout: an INT2 step's writes (64 lanes x HD / 16 blocks x 2 parts of 8
// halves) cover each of the tile's 64 token rows at every channel position exactly once and
// never the row padding; an INT4 step's cover rows 0..31 once, a current-chunk step's rows
// 0..15; the PV reads stay inside the rows and the channel positions.
template <int HD>
static void check_tile_layout() {
    typedef DGeo<HD> G;
    static int cnt[G::VTILE];
    auto expect = [&](int n_rows, const char *what) {
        for (int i = 0; i < G::VTILE; ++i)
            CHECK(cnt[i] == (i < n_rows * G::VROW && i % G::VROW < HD ? 1 : 0),
                  "d%d: %s: tile half %d (row %d, position %d) written %d times", HD, what, i, i / G::VROW,
                  i % G::VROW, cnt[i]);
        memset(cnt, 0, sizeof(cnt));
    };
    auto write = [&](int i, const char *what) {
        for (int k = 0; k < 8; ++k) {
            CHECK(i + k >= 0 && i + k < G::VTILE, "d%d: %s write %d outside the tile", HD, what, i + k);
            if (i + k >= 0 && i + k < G::VTILE) ++cnt[i + k];
        }
    };
    memset(cnt, 0, sizeof(cnt));
    for (int lane = 0; lane < kLanes; ++lane)
        for (int blk = 0; blk < HD / 16; ++blk)
            for (int part = 0; part < 2; ++part) write(vt_int2<HD>(lane, blk, part), "INT2");
    expect(TP, "INT2");
    if (HD == 128) {
        for (int lane = 0; lane < kLanes; ++lane)
            for (int hb = 0; hb < HD / 32; ++hb)
                for (int part = 0; part < 2; ++part) write(vt_int4<HD>(lane, hb, part), "INT4");
        expect(TP / 2, "INT4");
    }
    for (int lane = 0; lane < kLanes; ++lane)
        for (int bl = 0; bl < G::NBL; ++bl)
            for (int part = 0; part < 2; ++part) write(vt_cur<HD>(lane, bl, part), "current chunk");
    expect(TR, "current chunk");
    for (int lane = 0; lane < kLanes; ++lane)
        for (int h = 0; h < 2; ++h)
            for (int db = 0; db < G::DB; ++db)
                for (int off = 0; off <= 16 * G::VROW; off += 16 * G::VROW) {
                    const int i = vt_read<HD>(lane, h, db) + off;
                    CHECK(i >= 0 && i + 4 <= TP * G::VROW && i % G::VROW + 4 <= HD, "d%d: PV read %d", HD, i);
                }
    printf("%-34s ok so far: %s\n", HD == 64 ? "value tile layout, head_dim 64" : "value tile layout, head_dim 128",
           fails ? "no" : "yes");
}

int main() {
    check_tile_layout<64>();
    check_tile_layout<128>();
    const Config cases[] = {
        // name, B, Hq, Hkv, HD, n_q, bits, n_tokens, capacity, Gk, n_cur
        {"GQA decode INT2 32k", 8, 32, 8, 128, 1, 2, 32768, 32768, 128, 0},
        {"GQA decode INT4 32k", 8, 32, 8, 128, 1, 4, 32768, 32768, 128, 0},
        {"INT2 d64 ragged", 2, 8, 2, 64, 2, 2, 5003, 6000, 128, 0},
        {"INT2 d64 ragged, full capacity", 2, 8, 2, 64, 2, 2, 5003, 5003, 128, 0},
        {"INT4 d128 ragged, full capacity", 1, 4, 1, 128, 1, 4, 4099, 4099, 128, 0},
        {"INT2 d128 ragged groups of 32", 1, 4, 1, 128, 4, 2, 19601, 19700, 32, 0},
        {"INT4 d128 16 rows", 2, 16, 2, 128, 2, 4, 9000, 9100, 128, 0},
        {"INT2 d128 with current chunk", 64, 16, 8, 128, 2, 2, 700, 800, 128, 37},
        {"INT4 d128 with current chunk", 64, 8, 8, 128, 1, 4, 333, 400, 64, 16},
        {"INT2 d64 one token", 3, 6, 3, 64, 1, 2, 1, 8, 128, 0},
    };
    for (const Config &c : cases) {
        if (c.HD == 64) check_launch<64>(c);
        else check_launch<128>(c);
    }
    check_walk_multi();
    // what the kernel was not built for goes to the chunk kernel: fp16, raw (FP16-window)
    // segments, INT4 at head_dim 64, several segments, and the WindowQuant decode query
    // (14 / 2 heads at head_dim 64 over FP16 + INT4 + INT2 window segments, fp16)
    const int wq[3] = {16, 4, 2}, two[2] = {4, 2}, raw[1] = {16}, int4[1] = {4}, int2[1] = {2};
    CHECK(!decode_eligible(KVQ_F16, 1, 14, 2, 64, 1, wq, 3, 0, 19600), "WindowQuant decode admitted");
    CHECK(!decode_eligible(KVQ_BF16, 1, 14, 2, 64, 1, wq, 3, 0, 19600), "three segments admitted");
    CHECK(!decode_eligible(KVQ_BF16, 1, 14, 2, 64, 1, two, 2, 0, 17648), "two segments admitted");
    CHECK(!decode_eligible(KVQ_BF16, 1, 14, 2, 64, 1, raw, 1, 0, 1952), "raw segment admitted");
    CHECK(!decode_eligible(KVQ_BF16, 1, 14, 2, 64, 1, int4, 1, 0, 5888), "INT4 at head_dim 64 admitted");
    CHECK(!decode_eligible(KVQ_F16, 1, 14, 2, 64, 1, int2, 1, 0, 11760), "fp16 admitted");
    CHECK(!decode_eligible(KVQ_BF16, 1, 34, 2, 128, 1, int2, 1, 0, 100), "17 rows per KV head admitted");
    printf("decode checker: %ld elements touched, %ld failures\n", touched, fails);
    return fails ? 1 : 0;
}
