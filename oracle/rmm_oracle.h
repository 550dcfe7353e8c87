/*
 * RMM oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded C99 statement of what Reduced Matrix
 * Multiplication computes, used to check the HIP path.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never does, and the two share no code.
 *
 * Sources (cited by page title and section):
 *  - "Reduced Matrix Multiplication: Input-Adaptive Matrix-Product Reduction
 *    for LLM Inference" (opentrain.ai paper listing), abstract: RMM keeps the
 *    informative slices of each product's contraction dimension under a
 *    retention ratio r and leaves the weights unchanged.
 *  - cf-1.com blog on input-adaptive matrix-product reduction, sections 2
 *    (Y = X @ W^T with X [T,H], W [M,H]), 5.1-5.3 (light scorer, top-k, gather,
 *    compact product), 6.1 (code: top-k indices re-sorted ascending; keep
 *    ratio 1.0 reproduces the full product exactly), 6.2 (FLOPs 2*H*active_M).
 *  - tangquanwei GEMM notes, section 1: scores = Q @ K^T, out = softmax(scores) @ V.
 *
 * Parity status of every function is stated next to it.
 */
#ifndef RMM_ORACLE_H
#define RMM_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types of input buffers */
#define ORA_F32 0
#define ORA_BF16 1

/* keep count k = ceil(r*n), with r*n snapped to the nearest integer when it is
 * within 1e-9 relative of it; clamped to [1,n].  -1 if r is not in (0,1] or n<1.
 * Pinned: closed form over exact rationals (tests). */
int64_t ora_keep_count(int64_t n, double r);

/* linear scorer: s[tau*K + j] = fl32( max_{t in tile tau} |x[t,j]| * c[j] ).
 * Pinned: tile=1, c=1 reduces to |x|; order independence; brute force. */
int ora_scores(const void *x, int xt, int64_t T, int64_t K, int64_t ldx,
               const float *c, int64_t tile, float *s);

/* scorer + top-k: idx[tau*k + i], the k = ora_keep_count(K,r) slices of largest
 * score (ties to the lower index), listed in ascending index order.
 * Pinned: brute force over all subsets (K=12), count, ascending. */
int ora_select(const void *x, int xt, int64_t T, int64_t K, int64_t ldx,
               const float *c, int64_t tile, double r, int32_t *idx);

/* block-granular variant (blog section 6.1 demo code, ffn_block_reduce): the
 * contraction dimension in blocks of `block` consecutive slices (K % block == 0);
 * block score = mean over the block's slices, in ascending order and double
 * precision, of max_{t in tile} |x[t,j]|; the nk = ora_block_keep_count(K/block,
 * keep) blocks of largest score are kept (ties to the lower block), in ascending
 * block order, and expanded to their slice indices:
 * idx[tau*nk*block + i*block + e] = b_i*block + e.
 * Pinned: hand example; block=1 equals ora_select with c=1 when the counts agree;
 * brute force over block subsets. */
int64_t ora_block_keep_count(int64_t nb, double keep);
int ora_select_blocks(const void *x, int xt, int64_t T, int64_t K, int64_t ldx, int64_t tile,
                      int64_t block, double keep, int32_t *idx);

/* reduced product over kept slices, rows t in [t0,t1):
 * y[t*ldy+m] = (float) sum_{j in J_tau(t), ascending} (double)x[t,j]*(double)wt[j,m].
 * yd (optional, may be NULL) receives the unrounded double sums.
 * Pinned: r=1 equals ora_dense_linear bitwise and a float64 BLAS matmul;
 * dropped-slice identity against float64 BLAS. */
int ora_linear(const void *x, int xt, int64_t T, int64_t K, int64_t ldx,
               const void *wt, int wtt, int64_t M, int64_t ldw,
               const int32_t *idx, int64_t k, int64_t tile, int64_t t0, int64_t t1,
               float *y, int64_t ldy, double *yd);

/* dense product, triple loop in ascending j (the r=1 reference). */
int ora_dense_linear(const void *x, int xt, int64_t T, int64_t K, int64_t ldx,
                     const void *wt, int wtt, int64_t M, int64_t ldw, int64_t t0, int64_t t1,
                     float *y, int64_t ldy, double *yd);

/* gated FFN producer (blog section 6.1 demo code; 5.1; 6.2): for every token t
 * and intermediate column m < Mi
 *   g = sum_j x[t,j] * wg[j,m],  u = sum_j x[t,j] * wu[j,m]   (double, ascending j)
 *   h[t,m] = bf16( silu(g) * u ),  silu(g) = g / (1 + e^-g)    (double, one rounding)
 *   pmax[tau][m] = max_{t in tile tau} |h[t,m]|               (the scorer's column max)
 * x [T][ldx] bf16; wg, wu [H][ldw] bf16 (W_gate^T and W_up^T, row j = what x_j
 * multiplies); h [T][ldh] bf16; pmax [ceil(T/tile)][Mi] float; hd [T][ldh]
 * double (h before rounding).  Any output may be NULL.
 * Pinned: float64 library products and the logistic function of scipy with the
 * nearest-bfloat16 check, a hand example with silu(+-64), rounding ties and
 * subnormals, tile maxima. */
int ora_gate_up(const uint16_t *x, int64_t T, int64_t H, int64_t ldx,
                const uint16_t *wg, const uint16_t *wu, int64_t ldw, int64_t Mi, int64_t tile,
                uint16_t *h, int64_t ldh, float *pmax, double *hd);

/* reduced GQA attention decode (all bf16 inputs, fp32 kn).
 *  q  [B][Hq][D], kt [B][Hkv][D][ldk] (dim-major keys), v [B][Hkv][ldv][D], kn [B][Hkv][D].
 *  mode 0: one selection per KV head (its G = Hq/Hkv query heads share it);
 *  mode 1: one selection per query head.  Hsel = Hkv (mode 0) or Hq (mode 1).
 * Outputs (any may be NULL): out [B][Hq][D] float, dim_idx [B][Hsel][k_d],
 * pos_idx [B][Hsel][k_s], lse [B][Hq] float, pi [B][Hsel][S] double (the
 * position scores), p [B][Hq][S] double (softmax probabilities),
 * out_d [B][Hq][D] double.
 * vn (may be NULL): [B][Hkv][ldv] fp32 norms of the value rows; when given the
 * position score is max_h p_h[s] * vn[s] instead of max_h p_h[s].
 * Pinned: brute force (D=S=12, with and without vn), softmax sums to 1, r=1
 * equals textbook attention (float64 library), dropped-position identity,
 * vn = 1 equals the probability score. */
int ora_attn_decode(const uint16_t *q, const uint16_t *kt, const uint16_t *v, const float *kn,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t S,
                    int64_t ldk, int64_t ldv, float scale, double r_dim, double r_pos, int mode,
                    float *out, int32_t *dim_idx, int32_t *pos_idx, float *lse,
                    double *pi, double *p, double *out_d, const float *vn);

/* textbook dense attention in double (no reduction): out_d [B][Hq][D]. */
int ora_dense_attn(const uint16_t *q, const uint16_t *kt, const uint16_t *v,
                   int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t S,
                   int64_t ldk, int64_t ldv, float scale, double *out_d);

#ifdef __cplusplus
}
#endif
#endif
