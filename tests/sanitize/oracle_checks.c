/* Sanitizer driver for the C oracle (test infrastructure).  Every entry point
 * runs on small seeded inputs, with checks that need no stored values (keep
 * counts, ascending distinct index lists, the r = 1 identities with the dense
 * routines), and every argument error is hit.  tests/test_sanitize.py builds
 * it together with oracle/rmm_oracle.c under -fsanitize=address,undefined; a
 * sanitizer report or a failed check ends the program with a non-zero status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rmm_oracle.h"

static int failures = 0;
#define CHECK(cond)                                                                                    \
    do {                                                                                               \
        if (!(cond)) {                                                                                 \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);                         \
            ++failures;                                                                                \
        }                                                                                              \
    } while (0)

/* xorshift64*: a small seeded generator for the inputs */
static uint64_t rng = 0x9e3779b97f4a7c15ull;
static double uniform(void)
{
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (double)((rng * 0x2545f4914f6cdd1dull) >> 11) * (1.0 / 9007199254740992.0);
}
static float normalish(void) { return (float)(uniform() + uniform() + uniform() - 1.5); }
static uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16); /* truncation is enough for inputs */
}

static void check_ascending(const int32_t *idx, int64_t k, int64_t n)
{
    for (int64_t i = 0; i < k; ++i) {
        CHECK(idx[i] >= 0 && idx[i] < n);
        if (i)
            CHECK(idx[i] > idx[i - 1]);
    }
}

static void linear_checks(int xt)
{
    enum { T = 3, K = 37, LDX = 40, M = 11, LDW = 13, TILE = 2 };
    const int64_t ntiles = (T + TILE - 1) / TILE;
    float xf[T * LDX], wf[K * LDW], c[K];
    uint16_t xb[T * LDX], wb[K * LDW];
    for (int i = 0; i < T * LDX; ++i) {
        xf[i] = normalish();
        xb[i] = to_bf16(xf[i]);
    }
    for (int i = 0; i < K * LDW; ++i) {
        wf[i] = 0.1f * normalish();
        wb[i] = to_bf16(wf[i]);
    }
    for (int j = 0; j < K; ++j)
        c[j] = (float)(0.5 + uniform());
    const void *x = xt ? (const void *)xb : (const void *)xf;
    const void *wt = xt ? (const void *)wb : (const void *)wf;

    float s[ntiles * K];
    CHECK(ora_scores(x, xt, T, K, LDX, c, TILE, s) == 0);
    for (int i = 0; i < ntiles * K; ++i)
        CHECK(s[i] >= 0.0f);

    const double r = 0.3;
    const int64_t k = ora_keep_count(K, r);
    CHECK(k == 12);
    int32_t *idx = (int32_t *)malloc((size_t)(ntiles * k) * sizeof *idx);
    CHECK(ora_select(x, xt, T, K, LDX, c, TILE, r, idx) == 0);
    for (int64_t t = 0; t < ntiles; ++t)
        check_ascending(idx + t * k, k, K);

    double yd[T * M], yref[T * M];
    float y[T * M];
    CHECK(ora_linear(x, xt, T, K, LDX, wt, xt, M, LDW, idx, k, TILE, 0, T, y, M, yd) == 0);
    /* r = 1: the kept list is every slice in order, so the product is the dense one */
    int32_t all[ntiles * K];
    CHECK(ora_select(x, xt, T, K, LDX, c, TILE, 1.0, all) == 0);
    for (int64_t t = 0; t < ntiles; ++t)
        for (int j = 0; j < K; ++j)
            CHECK(all[t * K + j] == j);
    CHECK(ora_linear(x, xt, T, K, LDX, wt, xt, M, LDW, all, K, TILE, 0, T, y, M, yd) == 0);
    CHECK(ora_dense_linear(x, xt, T, K, LDX, wt, xt, M, LDW, 0, T, y, M, yref) == 0);
    for (int i = 0; i < T * M; ++i)
        CHECK(yd[i] == yref[i]);
    free(idx);

    /* argument errors */
    CHECK(ora_scores(x, xt, 0, K, LDX, c, TILE, s) != 0);
    CHECK(ora_select(x, xt, T, K, K - 1, c, TILE, r, all) != 0);
    CHECK(ora_select(x, xt, T, K, LDX, c, TILE, 0.0, all) != 0);
    CHECK(ora_linear(x, xt, T, K, LDX, wt, xt, M, LDW, all, K + 1, TILE, 0, T, y, M, yd) != 0);
    CHECK(ora_linear(x, xt, T, K, LDX, wt, xt, M, LDW, all, K, TILE, 2, 1, y, M, yd) != 0);
    CHECK(ora_dense_linear(x, xt, T, K, LDX, wt, xt, M, M - 1, 0, T, y, M, yd) != 0);
}

static void block_checks(void)
{
    enum { T = 2, K = 64, TILE = 2, BLOCK = 8 };
    uint16_t x[T * K];
    for (int i = 0; i < T * K; ++i)
        x[i] = to_bf16(normalish());
    const int64_t nb = ora_block_keep_count(K / BLOCK, 0.5);
    CHECK(nb == 4);
    int32_t idx[nb * BLOCK];
    CHECK(ora_select_blocks(x, 1, T, K, K, TILE, BLOCK, 0.5, idx) == 0);
    check_ascending(idx, nb * BLOCK, K);
    for (int64_t i = 0; i < nb * BLOCK; i += BLOCK)
        for (int e = 1; e < BLOCK; ++e)
            CHECK(idx[i + e] == idx[i] + e); /* whole blocks */
    CHECK(ora_block_keep_count(0, 0.5) == -1);
    CHECK(ora_select_blocks(x, 1, T, K, K, TILE, 7, 0.5, idx) != 0); /* K not a multiple of the block */
}

static void gate_up_checks(void)
{
    enum { T = 3, H = 16, MI = 24, TILE = 2 };
    uint16_t x[T * H], wg[H * MI], wu[H * MI], h[T * MI];
    float pmax[2 * MI];
    double hd[T * MI];
    for (int i = 0; i < T * H; ++i)
        x[i] = to_bf16(normalish());
    for (int i = 0; i < H * MI; ++i) {
        wg[i] = to_bf16(0.3f * normalish());
        wu[i] = to_bf16(0.3f * normalish());
    }
    CHECK(ora_gate_up(x, T, H, H, wg, wu, MI, MI, TILE, h, MI, pmax, hd) == 0);
    for (int i = 0; i < 2 * MI; ++i)
        CHECK(pmax[i] >= 0.0f);
    CHECK(ora_gate_up(x, T, H, H - 1, wg, wu, MI, MI, TILE, h, MI, pmax, hd) != 0);
}

static void attn_checks(int mode, int with_vn)
{
    enum { B = 2, HQ = 4, HKV = 2, D = 16, S = 37, LD = 40 };
    const int64_t hsel = mode == 0 ? HKV : HQ;
    uint16_t *q = malloc(sizeof(uint16_t) * B * HQ * D), *kt = malloc(sizeof(uint16_t) * B * HKV * D * LD),
             *v = malloc(sizeof(uint16_t) * B * HKV * LD * D);
    float *kn = malloc(sizeof(float) * B * HKV * D), *vn = malloc(sizeof(float) * B * HKV * LD);
    for (int i = 0; i < B * HQ * D; ++i)
        q[i] = to_bf16(normalish());
    for (int i = 0; i < B * HKV * D * LD; ++i)
        kt[i] = to_bf16(normalish());
    for (int i = 0; i < B * HKV * LD * D; ++i)
        v[i] = to_bf16(normalish());
    for (int i = 0; i < B * HKV * D; ++i)
        kn[i] = (float)(0.5 + uniform());
    for (int i = 0; i < B * HKV * LD; ++i)
        vn[i] = (float)(0.5 + uniform());
    const float scale = 0.25f;
    const double r_dim = 0.5, r_pos = 0.3;
    const int64_t kd = ora_keep_count(D, r_dim), ks = ora_keep_count(S, r_pos);
    float out[B * HQ * D], lse[B * HQ];
    int32_t *dim_idx = malloc(sizeof(int32_t) * B * hsel * kd), *pos_idx = malloc(sizeof(int32_t) * B * hsel * ks);
    double *pi = malloc(sizeof(double) * B * hsel * S), *p = malloc(sizeof(double) * B * HQ * S);
    double out_d[B * HQ * D], dense[B * HQ * D];
    CHECK(ora_attn_decode(q, kt, v, kn, B, HQ, HKV, D, S, LD, LD, scale, r_dim, r_pos, mode, out, dim_idx, pos_idx,
                          lse, pi, p, out_d, with_vn ? vn : NULL) == 0);
    for (int64_t i = 0; i < B * hsel; ++i) {
        check_ascending(dim_idx + i * kd, kd, D);
        check_ascending(pos_idx + i * ks, ks, S);
    }
    for (int64_t i = 0; i < B * HQ; ++i) {
        double sum = 0.0;
        for (int s = 0; s < S; ++s)
            sum += p[i * S + s];
        CHECK(fabs(sum - 1.0) < 1e-12); /* full softmax over all positions */
    }
    /* r = 1 on both contractions: dense attention */
    CHECK(ora_attn_decode(q, kt, v, kn, B, HQ, HKV, D, S, LD, LD, scale, 1.0, 1.0, mode, NULL, NULL, NULL, NULL,
                          NULL, NULL, out_d, with_vn ? vn : NULL) == 0);
    CHECK(ora_dense_attn(q, kt, v, B, HQ, HKV, D, S, LD, LD, scale, dense) == 0);
    for (int i = 0; i < B * HQ * D; ++i)
        CHECK(fabs(out_d[i] - dense[i]) <= 1e-12 * (1.0 + fabs(dense[i])));
    /* argument errors */
    CHECK(ora_attn_decode(q, kt, v, kn, B, 3, HKV, D, S, LD, LD, scale, r_dim, r_pos, mode, out, NULL, NULL, NULL,
                          NULL, NULL, NULL, NULL) != 0);
    CHECK(ora_attn_decode(q, kt, v, kn, B, HQ, HKV, D, S, S - 1, LD, scale, r_dim, r_pos, mode, out, NULL, NULL,
                          NULL, NULL, NULL, NULL, NULL) != 0);
    CHECK(ora_attn_decode(q, kt, v, kn, B, HQ, HKV, D, S, LD, LD, scale, r_dim, r_pos, 2, out, NULL, NULL, NULL,
                          NULL, NULL, NULL, NULL) != 0);
    CHECK(ora_dense_attn(q, kt, v, B, HQ, HKV, D, 0, LD, LD, scale, dense) != 0);
    free(q);
    free(kt);
    free(v);
    free(kn);
    free(vn);
    free(dim_idx);
    free(pos_idx);
    free(pi);
    free(p);
}

int main(void)
{
    CHECK(ora_keep_count(10, 0.25) == 3);
    CHECK(ora_keep_count(100, 0.07) == 7);
    CHECK(ora_keep_count(7, 1.0) == 7);
    CHECK(ora_keep_count(5, 0.0) == -1);
    CHECK(ora_keep_count(0, 0.5) == -1);
    CHECK(ora_keep_count(5, NAN) == -1);
    linear_checks(0);
    linear_checks(1);
    block_checks();
    gate_up_checks();
    for (int mode = 0; mode < 2; ++mode)
        for (int with_vn = 0; with_vn < 2; ++with_vn)
            attn_checks(mode, with_vn);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle checks passed\n");
    return 0;
}
