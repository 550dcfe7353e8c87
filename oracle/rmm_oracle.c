/*
 * RMM oracle -- TEST INFRASTRUCTURE ONLY.  See rmm_oracle.h for the sources
 * and the parity status of each function.  Plain C99, single-threaded, built
 * without -ffast-math; every sum is taken in double in ascending index order
 * and rounded once to float at the end.
 */
#include "rmm_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs FLT_EVAL_METHOD == 0 (each float operation rounded to float)"
#endif

static float bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float elem(const void *p, int t, int64_t i)
{
    if (t == ORA_F32)
        return ((const float *)p)[i];
    return bf16_value(((const uint16_t *)p)[i]);
}

/* ---------------------------------------------------------------- keep count
 * Retention ratio r keeps ceil(r*n) slices (paper abstract: "retention-ratio
 * control"; the blog's section 6.1 code keeps max(1, int(n*ratio))).  The
 * product r*n is snapped to an integer when it is within 1e-9 relative of it,
 * so that e.g. 0.07*100 (7.000000000000001 in binary) keeps 7, not 8. */
int64_t ora_keep_count(int64_t n, double r)
{
    if (n < 1 || !(r > 0.0) || !(r <= 1.0))
        return -1;
    double prod = r * (double)n;
    double near = floor(prod + 0.5);
    double scale = prod > 1.0 ? prod : 1.0;
    double k = (fabs(prod - near) <= 1e-9 * scale) ? near : ceil(prod);
    if (k < 1.0)
        k = 1.0;
    if (k > (double)n)
        k = (double)n;
    return (int64_t)k;
}

/* ---------------------------------------------------------------- scorer
 * Blog section 5.1: a cheap gate rates each slice from the current input.
 * Score of slice j for a tile of tokens: the largest |x[t,j]| in the tile,
 * times the slice's weight-row norm c_j (one float multiply). */
int ora_scores(const void *x, int xt, int64_t T, int64_t K, int64_t ldx,
               const float *c, int64_t tile, float *s)
{
    if (T < 1 || K < 1 || tile < 1 || ldx < K)
        return 1;
    int64_t ntiles = (T + tile - 1) / tile;
    for (int64_t tau = 0; tau < ntiles; ++tau) {
        int64_t t0 = tau * tile, t1 = t0 + tile < T ? t0 + tile : T;
        for (int64_t j = 0; j < K; ++j) {
            float a = 0.0f;
            for (int64_t t = t0; t < t1; ++t) {
                float v = fabsf(elem(x, xt, t * ldx + j));
                if (v > a)
                    a = v;
            }
            volatile float prod = a * c[j];
            s[tau * K + j] = prod;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- top-k */
typedef struct {
    double key;
    int64_t pos;
} ora_item;

/* larger key first; equal keys: lower index first */
static int by_key_desc(const void *a, const void *b)
{
    const ora_item *u = (const ora_item *)a, *v = (const ora_item *)b;
    if (u->key > v->key)
        return -1;
    if (u->key < v->key)
        return 1;
    return (u->pos > v->pos) - (u->pos < v->pos);
}

static int by_pos_asc(const void *a, const void *b)
{
    const ora_item *u = (const ora_item *)a, *v = (const ora_item *)b;
    return (u->pos > v->pos) - (u->pos < v->pos);
}

/* Blog sections 5.2 and 6.1: top-k of the scores, the kept indices re-sorted
 * ascending so the compact product keeps the original order. */
static int topk_ascending(const double *key, int64_t n, int64_t k, int32_t *out)
{
    ora_item *it = (ora_item *)malloc((size_t)n * sizeof *it);
    if (!it)
        return 2;
    for (int64_t i = 0; i < n; ++i) {
        it[i].key = key[i] == 0.0 ? 0.0 : key[i]; /* -0 ranks as +0 */
        it[i].pos = i;
    }
    qsort(it, (size_t)n, sizeof *it, by_key_desc);
    qsort(it, (size_t)k, sizeof *it, by_pos_asc);
    for (int64_t i = 0; i < k; ++i)
        out[i] = (int32_t)it[i].pos;
    free(it);
    return 0;
}

int ora_select(const void *x, int xt, int64_t T, int64_t K, int64_t ldx,
               const float *c, int64_t tile, double r, int32_t *idx)
{
    int64_t k = ora_keep_count(K, r);
    if (k < 0 || T < 1 || tile < 1 || ldx < K)
        return 1;
    int64_t ntiles = (T + tile - 1) / tile;
    float *s = (float *)malloc((size_t)(ntiles * K) * sizeof *s);
    double *key = (double *)malloc((size_t)K * sizeof *key);
    if (!s || !key) {
        free(s);
        free(key);
        return 2;
    }
    int rc = ora_scores(x, xt, T, K, ldx, c, tile, s);
    for (int64_t tau = 0; rc == 0 && tau < ntiles; ++tau) {
        for (int64_t j = 0; j < K; ++j)
            key[j] = (double)s[tau * K + j];
        rc = topk_ascending(key, K, k, idx + tau * k);
    }
    free(s);
    free(key);
    return rc;
}

/* ---------------------------------------------------------------- products
 * Blog section 2: Y = X @ W^T; RMM keeps W^T rows (contraction slices) j in J
 * and computes Y ~= X[:,J] @ W^T[J,:].  Output shape is the dense one. */
/* ---------------------------------------------------------------- block variant
 * Blog section 6.1 demo code (ffn_block_reduce): keep_num = max(1,
 * int(num_blocks * keep_ratio)), i.e. the double product truncated, at least 1. */
int64_t ora_block_keep_count(int64_t nb, double keep)
{
    if (nb < 1 || !(keep > 0.0) || !(keep <= 1.0))
        return -1;
    double p = floor((double)nb * keep);
    int64_t k = (int64_t)p;
    if (k < 1)
        k = 1;
    if (k > nb)
        k = nb;
    return k;
}

/* Blog sections 5.1 (block-mean |h| as the block's importance), 5.2 (top-k over
 * blocks, bool mask expanded to neuron indices) and 6.1 (the demo code). */
int ora_select_blocks(const void *x, int xt, int64_t T, int64_t K, int64_t ldx, int64_t tile,
                      int64_t block, double keep, int32_t *idx)
{
    if (T < 1 || K < 1 || tile < 1 || ldx < K || block < 1 || K % block != 0)
        return 1;
    int64_t nb = K / block;
    int64_t nk = ora_block_keep_count(nb, keep);
    if (nk < 0)
        return 1;
    int64_t ntiles = (T + tile - 1) / tile;
    double *score = (double *)malloc((size_t)nb * sizeof *score);
    int32_t *kept = (int32_t *)malloc((size_t)nk * sizeof *kept);
    if (!score || !kept) {
        free(score);
        free(kept);
        return 2;
    }
    int rc = 0;
    for (int64_t tau = 0; rc == 0 && tau < ntiles; ++tau) {
        int64_t t0 = tau * tile, t1 = t0 + tile < T ? t0 + tile : T;
        for (int64_t b = 0; b < nb; ++b) {
            double sum = 0.0;
            for (int64_t e = 0; e < block; ++e) {
                int64_t j = b * block + e;
                float a = 0.0f;
                for (int64_t t = t0; t < t1; ++t) {
                    float v = fabsf(elem(x, xt, t * ldx + j));
                    if (v > a)
                        a = v;
                }
                sum += (double)a;
            }
            score[b] = sum / (double)block;
        }
        rc = topk_ascending(score, nb, nk, kept);
        for (int64_t i = 0; rc == 0 && i < nk; ++i)
            for (int64_t e = 0; e < block; ++e)
                idx[tau * nk * block + i * block + e] = (int32_t)(kept[i] * block + e);
    }
    free(score);
    free(kept);
    return rc;
}

int ora_linear(const void *x, int xt, int64_t T, int64_t K, int64_t ldx,
               const void *wt, int wtt, int64_t M, int64_t ldw,
               const int32_t *idx, int64_t k, int64_t tile, int64_t t0, int64_t t1,
               float *y, int64_t ldy, double *yd)
{
    if (T < 1 || K < 1 || M < 1 || k < 1 || k > K || tile < 1 || ldx < K || ldw < M || ldy < M)
        return 1;
    if (t0 < 0 || t1 > T || t0 > t1)
        return 1;
    double *acc = (double *)malloc((size_t)M * sizeof *acc);
    if (!acc)
        return 2;
    for (int64_t t = t0; t < t1; ++t) {
        const int32_t *J = idx + (t / tile) * k;
        for (int64_t m = 0; m < M; ++m)
            acc[m] = 0.0;
        for (int64_t i = 0; i < k; ++i) {
            int64_t j = J[i];
            double xv = (double)elem(x, xt, t * ldx + j);
            for (int64_t m = 0; m < M; ++m)
                acc[m] += xv * (double)elem(wt, wtt, j * ldw + m);
        }
        for (int64_t m = 0; m < M; ++m) {
            if (y)
                y[t * ldy + m] = (float)acc[m];
            if (yd)
                yd[t * ldy + m] = acc[m];
        }
    }
    free(acc);
    return 0;
}

int ora_dense_linear(const void *x, int xt, int64_t T, int64_t K, int64_t ldx,
                     const void *wt, int wtt, int64_t M, int64_t ldw, int64_t t0, int64_t t1,
                     float *y, int64_t ldy, double *yd)
{
    if (T < 1 || K < 1 || M < 1 || ldx < K || ldw < M || ldy < M || t0 < 0 || t1 > T || t0 > t1)
        return 1;
    for (int64_t t = t0; t < t1; ++t) {
        for (int64_t m = 0; m < M; ++m) {
            double a = 0.0;
            for (int64_t j = 0; j < K; ++j)
                a += (double)elem(x, xt, t * ldx + j) * (double)elem(wt, wtt, j * ldw + m);
            if (y)
                y[t * ldy + m] = (float)a;
            if (yd)
                yd[t * ldy + m] = a;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- FFN producer
 * The gated FFN of the blog's section 6.1 demo code (ffn_full): gate = x W_gate^T,
 * up = x W_up^T, h = silu(gate) * up, which is the down projection's input; the
 * blog's section 5.1 scores the down projection's slices from this activation,
 * and section 6.2 notes that gate and up are computed in full.
 * Double rounded once to bfloat16, to nearest with ties to even, without an
 * intermediate float: the quantum of the result is 2^(e-7) for |d| in
 * [2^e, 2^(e+1)), e >= -126, and 2^-133 below (bfloat16 subnormals). */
static uint16_t bf16_from_double(double d)
{
    if (d != d)
        return 0x7fc0;
    double a = fabs(d);
    double q = a >= ldexp(1.0, -126) ? ldexp(1.0, ilogb(a) - 7) : ldexp(1.0, -133);
    double r = a == 0.0 ? 0.0 : nearbyint(a / q) * q; /* default rounding mode: ties to even */
    uint32_t u;
    if (r >= ldexp(1.0, 128)) {
        u = 0x7f800000u;
    } else {
        float f = (float)r; /* exact: at most 8 significant bits */
        memcpy(&u, &f, sizeof u);
    }
    return (uint16_t)((u >> 16) | (signbit(d) ? 0x8000u : 0u));
}

int ora_gate_up(const uint16_t *x, int64_t T, int64_t H, int64_t ldx,
                const uint16_t *wg, const uint16_t *wu, int64_t ldw, int64_t Mi, int64_t tile,
                uint16_t *h, int64_t ldh, float *pmax, double *hd)
{
    if (T < 1 || H < 1 || Mi < 1 || tile < 1 || ldx < H || ldw < Mi || ldh < Mi)
        return 1;
    const int64_t ntiles = (T + tile - 1) / tile;
    double *g = (double *)malloc((size_t)Mi * sizeof *g), *u = (double *)malloc((size_t)Mi * sizeof *u);
    if (!g || !u) {
        free(g);
        free(u);
        return 2;
    }
    if (pmax)
        for (int64_t i = 0; i < ntiles * Mi; ++i)
            pmax[i] = 0.0f;
    for (int64_t t = 0; t < T; ++t) {
        /* every g[m], u[m] is summed in ascending j */
        for (int64_t m = 0; m < Mi; ++m)
            g[m] = u[m] = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            double xv = (double)bf16_value(x[t * ldx + j]);
            for (int64_t m = 0; m < Mi; ++m) {
                g[m] += xv * (double)bf16_value(wg[j * ldw + m]);
                u[m] += xv * (double)bf16_value(wu[j * ldw + m]);
            }
        }
        for (int64_t m = 0; m < Mi; ++m) {
            double v = g[m] / (1.0 + exp(-g[m])) * u[m];
            uint16_t b = bf16_from_double(v);
            if (h)
                h[t * ldh + m] = b;
            if (hd)
                hd[t * ldh + m] = v;
            if (pmax) {
                float mag = fabsf(bf16_value(b));
                float *pm = pmax + (t / tile) * Mi + m;
                if (mag > *pm)
                    *pm = mag;
            }
        }
    }
    free(g);
    free(u);
    return 0;
}

/* ---------------------------------------------------------------- attention
 * Reduced decode attention for one batch element and one selection group:
 *  1. head_dim slices (the contraction of Q K^T) scored by
 *     fl32( max_{h in group} |q[h,j]| * kn[j] ) and the top k_d kept
 *     (blog section 3.3: reduce inside a head, never drop the head);
 *  2. logits l_h[s] = scale * sum_{j kept} q[h,j] K[s,j]   (all S positions);
 *  3. full softmax over all S positions: p_h[s] = exp(l_h[s]-m_h)/Z_h;
 *  4. key positions (the contraction of P V) scored by max_{h in group} p_h[s],
 *     the top k_s kept (blog section 3.1);
 *  5. out[h,:] = sum_{s kept} p_h[s] V[s,:], with no renormalisation. */
int ora_attn_decode(const uint16_t *q, const uint16_t *kt, const uint16_t *v, const float *kn,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t S,
                    int64_t ldk, int64_t ldv, float scale, double r_dim, double r_pos, int mode,
                    float *out, int32_t *dim_idx, int32_t *pos_idx, float *lse,
                    double *pi, double *p, double *out_d, const float *vn)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || S < 1 || Hq % Hkv != 0 || ldk < S || ldv < S)
        return 1;
    if (mode != 0 && mode != 1)
        return 1;
    int64_t kd = ora_keep_count(D, r_dim), ks = ora_keep_count(S, r_pos);
    if (kd < 0 || ks < 0)
        return 1;
    int64_t G = Hq / Hkv;
    int64_t gsize = mode == 0 ? G : 1;          /* query heads per selection group */
    int64_t Hsel = mode == 0 ? Hkv : Hq;

    double *sig = (double *)malloc((size_t)D * sizeof *sig);
    int32_t *Jd = (int32_t *)malloc((size_t)D * sizeof *Jd);
    double *lg = (double *)malloc((size_t)(gsize * S) * sizeof *lg);
    double *pg = (double *)malloc((size_t)(gsize * S) * sizeof *pg);
    double *pis = (double *)malloc((size_t)S * sizeof *pis);
    int32_t *Js = (int32_t *)malloc((size_t)S * sizeof *Js);
    int rc = 0;
    if (!sig || !Jd || !lg || !pg || !pis || !Js) {
        rc = 2;
        goto done;
    }

    for (int64_t b = 0; b < B; ++b) {
        for (int64_t sg = 0; sg < Hsel; ++sg) {
            int64_t h0 = sg * gsize;               /* first query head of the group */
            int64_t g = h0 / G;                    /* its KV head */
            const uint16_t *K = kt + (b * Hkv + g) * D * ldk;
            const uint16_t *V = v + (b * Hkv + g) * ldv * D;

            /* 1. head_dim scores and selection */
            for (int64_t j = 0; j < D; ++j) {
                float a = 0.0f;
                for (int64_t h = h0; h < h0 + gsize; ++h) {
                    float qa = fabsf(bf16_value(q[(b * Hq + h) * D + j]));
                    if (qa > a)
                        a = qa;
                }
                volatile float prod = a * kn[(b * Hkv + g) * D + j];
                sig[j] = (double)prod;
            }
            rc = topk_ascending(sig, D, kd, Jd);
            if (rc)
                goto done;
            if (dim_idx)
                memcpy(dim_idx + (b * Hsel + sg) * kd, Jd, (size_t)kd * sizeof *Jd);

            /* 2-3. logits over kept dims, full softmax over all positions */
            for (int64_t hh = 0; hh < gsize; ++hh) {
                int64_t h = h0 + hh;
                double *l = lg + hh * S, *ph = pg + hh * S;
                for (int64_t s = 0; s < S; ++s) {
                    double a = 0.0;
                    for (int64_t i = 0; i < kd; ++i) {
                        int64_t j = Jd[i];
                        a += (double)bf16_value(q[(b * Hq + h) * D + j]) * (double)bf16_value(K[j * ldk + s]);
                    }
                    l[s] = (double)scale * a;
                }
                double mx = l[0];
                for (int64_t s = 1; s < S; ++s)
                    if (l[s] > mx)
                        mx = l[s];
                double Z = 0.0;
                for (int64_t s = 0; s < S; ++s)
                    Z += exp(l[s] - mx);
                for (int64_t s = 0; s < S; ++s)
                    ph[s] = exp(l[s] - mx) / Z;
                if (lse)
                    lse[b * Hq + h] = (float)(mx + log(Z));
                if (p)
                    memcpy(p + (b * Hq + h) * S, ph, (size_t)S * sizeof *ph);
            }

            /* 4. position scores and selection; with vn the score is weighted by the
             * norm of the value row, p * ||V_s|| (the analogue of the linear scorer) */
            for (int64_t s = 0; s < S; ++s) {
                double a = pg[s];
                for (int64_t hh = 1; hh < gsize; ++hh)
                    if (pg[hh * S + s] > a)
                        a = pg[hh * S + s];
                pis[s] = vn ? a * (double)vn[(b * Hkv + g) * ldv + s] : a;
            }
            if (pi)
                memcpy(pi + (b * Hsel + sg) * S, pis, (size_t)S * sizeof *pis);
            rc = topk_ascending(pis, S, ks, Js);
            if (rc)
                goto done;
            if (pos_idx)
                memcpy(pos_idx + (b * Hsel + sg) * ks, Js, (size_t)ks * sizeof *Js);

            /* 5. P V over kept positions, no renormalisation */
            for (int64_t hh = 0; hh < gsize; ++hh) {
                int64_t h = h0 + hh;
                for (int64_t d = 0; d < D; ++d) {
                    double a = 0.0;
                    for (int64_t i = 0; i < ks; ++i) {
                        int64_t s = Js[i];
                        a += pg[hh * S + s] * (double)bf16_value(V[s * D + d]);
                    }
                    if (out)
                        out[(b * Hq + h) * D + d] = (float)a;
                    if (out_d)
                        out_d[(b * Hq + h) * D + d] = a;
                }
            }
        }
    }
done:
    free(sig);
    free(Jd);
    free(lg);
    free(pg);
    free(pis);
    free(Js);
    return rc;
}

/* Textbook attention (tangquanwei GEMM notes, section 1), in double. */
int ora_dense_attn(const uint16_t *q, const uint16_t *kt, const uint16_t *v,
                   int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t S,
                   int64_t ldk, int64_t ldv, float scale, double *out_d)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || S < 1 || Hq % Hkv != 0 || ldk < S || ldv < S)
        return 1;
    int64_t G = Hq / Hkv;
    double *l = (double *)malloc((size_t)S * sizeof *l);
    if (!l)
        return 2;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hq; ++h) {
            int64_t g = h / G;
            const uint16_t *K = kt + (b * Hkv + g) * D * ldk;
            const uint16_t *V = v + (b * Hkv + g) * ldv * D;
            double mx = -INFINITY;
            for (int64_t s = 0; s < S; ++s) {
                double a = 0.0;
                for (int64_t j = 0; j < D; ++j)
                    a += (double)bf16_value(q[(b * Hq + h) * D + j]) * (double)bf16_value(K[j * ldk + s]);
                l[s] = (double)scale * a;
                if (l[s] > mx)
                    mx = l[s];
            }
            double Z = 0.0;
            for (int64_t s = 0; s < S; ++s) {
                l[s] = exp(l[s] - mx);
                Z += l[s];
            }
            for (int64_t d = 0; d < D; ++d) {
                double a = 0.0;
                for (int64_t s = 0; s < S; ++s)
                    a += l[s] * (double)bf16_value(V[s * D + d]);
                out_d[(b * Hq + h) * D + d] = a / Z;
            }
        }
    free(l);
    return 0;
}
