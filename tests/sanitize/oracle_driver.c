/* Drives the CPU oracle through its entry points on small inputs, for a build under
 * AddressSanitizer and UndefinedBehaviorSanitizer: quantize-append (contiguous, gathered,
 * per-token K groups, compensation, raw), attention with every Jensen form, window scores,
 * assignment and gather lists. Exits 0 when every call returns as expected. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct orc_segment {
    int32_t bits, elem_dtype, capacity, n_tokens, n_kgroups, kgroup_capacity, v_group_channels;
    const uint32_t *k_codes, *v_codes;
    const uint16_t *k_meta, *v_meta;
    const int32_t *kgroup_start;
    const uint16_t *k_raw, *v_raw;
    int32_t k_group_channels, comp_rank;
    const float *comp_basis;
    const uint16_t *k_comp;
} orc_segment;

int orc_append(int bits, int elem_dtype, int B, int H, int d, int cap, int n_tokens, int Gk, int Gv, int kgroup_cap,
               int n_kgroups, uint32_t *k_codes, uint32_t *v_codes, uint16_t *k_meta, uint16_t *v_meta,
               int32_t *kgroup_start, uint16_t *k_raw, uint16_t *v_raw, const float *k_src, const float *v_src,
               int64_t src_tokens, int n_new, const int32_t *groups, int n_groups_in, int kgc, int comp_rank,
               const float *comp_basis, uint16_t *k_comp);
int orc_attention(const float *q, int B, int Hq, int Hkv, int d, int nq, const orc_segment *segs, int n_segs,
                  const float *k_cur, const float *v_cur, int n_cur, double scale, int jensen, int exact,
                  const int32_t *rows, int n_rows, double *out, double *lse, double *mass);
void orc_window_scores(const float *k, int H, int N, int d, int window, const float *text, double *score);
int orc_assign_windows(const double *score, int W, int n_fp16, int n_int4, int8_t *bits, int32_t *order);
void orc_window_groups(const int8_t *bits, const int32_t *order, int W, int N, int window, int32_t *groups,
                       int32_t *class_tokens);
void orc_window_budget(int W, int pct_fp16, int pct_int4, int *n_fp16, int *n_int4);

static float frand(unsigned *s) {
    *s = *s * 1664525u + 1013904223u;
    return ((float)(*s >> 8) / 16777216.0f - 0.5f) * 4.0f;
}

int main(void) {
    enum { B = 1, H = 2, d = 64, N = 150, NC = 20, NQ = 9, CAP = 200 };
    unsigned seed = 7;
    float *k = malloc(sizeof(float) * B * H * N * d), *v = malloc(sizeof(float) * B * H * N * d);
    float *kc = malloc(sizeof(float) * B * H * NC * d), *vc = malloc(sizeof(float) * B * H * NC * d);
    float *q = malloc(sizeof(float) * B * 4 * NQ * d);
    float *U = malloc(sizeof(float) * H * d * 3);
    for (int i = 0; i < B * H * N * d; ++i) { k[i] = frand(&seed); v[i] = frand(&seed); }
    for (int i = 0; i < B * H * NC * d; ++i) { kc[i] = frand(&seed); vc[i] = frand(&seed); }
    for (int i = 0; i < B * 4 * NQ * d; ++i) q[i] = frand(&seed);
    for (int i = 0; i < H * d * 3; ++i) U[i] = frand(&seed) * 0.1f;
    int fails = 0;
    /* four packed segments (plain INT2, gathered INT4, per-token K groups, compensation) and a raw one */
    orc_segment segs[5];
    memset(segs, 0, sizeof(segs));
    const int wpr2 = d * 2 / 32, wpr4 = d * 4 / 32;
    for (int s = 0; s < 4; ++s) {
        const int bits = s == 1 ? 4 : 2, wpr = bits == 2 ? wpr2 : wpr4;
        const int kgc = s == 2 ? 32 : 0, rank = s == 3 ? 3 : 0, kgcap = 8;
        uint32_t *kcod = calloc((size_t)B * H * CAP * wpr, 4), *vcod = calloc((size_t)B * H * CAP * wpr, 4);
        uint16_t *km = calloc((size_t)B * H * (kgc ? CAP * (d / kgc) : kgcap * d) * 2, 2);
        uint16_t *vm = calloc((size_t)B * H * CAP * (d / 32) * 2, 2);
        int32_t *tab = calloc(kgcap + 1, 4);
        uint16_t *comp = rank ? calloc((size_t)B * H * CAP * 8, 2) : NULL;
        int32_t gl[8] = {40, 32, 0, 32, 100, 32, 8, 16};
        const int r = orc_append(bits, 2, B, H, d, CAP, 0, 32, 32, kgcap, 0, kcod, vcod, km, vm, tab, NULL, NULL, k, v,
                                 N, s == 1 ? 112 : N, s == 1 ? gl : NULL, s == 1 ? 4 : 0, kgc, rank, rank ? U : NULL, comp);
        if (r < 0) { fprintf(stderr, "append %d failed\n", s); ++fails; }
        segs[s] = (orc_segment){bits, 2, CAP, s == 1 ? 112 : N, kgc ? 0 : r, kgcap, 32, kcod, vcod, km, vm, tab,
                                NULL, NULL, kgc, rank, rank ? U : NULL, comp};
    }
    uint16_t *kr = calloc((size_t)B * H * CAP * d, 2), *vr = calloc((size_t)B * H * CAP * d, 2);
    if (orc_append(16, 1, B, H, d, CAP, 0, 32, 32, 0, 0, NULL, NULL, NULL, NULL, NULL, kr, vr, k, v, N, 33, NULL, 0,
                   0, 0, NULL, NULL) != 2) { fprintf(stderr, "raw append\n"); ++fails; }
    segs[4] = (orc_segment){16, 1, CAP, 33, 0, 0, 32, NULL, NULL, NULL, NULL, NULL, kr, vr, 0, 0, NULL, NULL};
    segs[4].elem_dtype = 2;
    /* a malformed request is refused without writing */
    if (orc_append(2, 2, B, H, d, CAP, CAP - 10, 32, 32, 8, 0, (uint32_t *)kr, (uint32_t *)vr, kr, vr, NULL, NULL, NULL,
                   k, v, N, 50, NULL, 0, 0, 0, NULL, NULL) != -1) { fprintf(stderr, "capacity\n"); ++fails; }
    double *out = malloc(sizeof(double) * B * 4 * NQ * d), lse[B * 4 * NQ], mass[B * 4 * NQ];
    for (int jensen = 0; jensen <= 3; ++jensen)
        if (orc_attention(q, B, 4, H, d, NQ, segs, 5, kc, vc, NC, 1.0 / 8.0, jensen, 0, NULL, 0, out, lse, mass) != 0) {
            fprintf(stderr, "attention %d\n", jensen); ++fails;
        }
    for (int i = 0; i < B * 4 * NQ * d; ++i) if (!isfinite(out[i])) { fprintf(stderr, "nan\n"); ++fails; break; }
    /* windows */
    const int W = (N + 31) / 32;
    double score[8];
    int8_t wb[8];
    int32_t order[8], groups[16], ct[3];
    int n16, n4;
    orc_window_scores(k, H, N, d, 32, k, score);
    orc_window_budget(W, 10, 30, &n16, &n4);
    if (orc_assign_windows(score, W, n16, n4, wb, order) != 0) { fprintf(stderr, "assign\n"); ++fails; }
    orc_window_groups(wb, order, W, N, 32, groups, ct);
    if (ct[0] + ct[1] + ct[2] != N) { fprintf(stderr, "groups\n"); ++fails; }
    printf("oracle driver: %d failures\n", fails);
    return fails != 0;
}
