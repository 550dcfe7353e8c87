/*
 * rmm.h -- C ABI of librmm.so, the MI355X (gfx950) hot path of Reduced Matrix
 * Multiplication (RMM).
 *
 * RMM ("Reduced Matrix Multiplication: Input-Adaptive Matrix-Product Reduction
 * for LLM Inference", paper abstract) scores the slices of a matrix product's
 * contraction dimension from the current input, keeps the ceil(r*K) best under
 * a retention ratio r, and multiplies over those slices only; weights are not
 * modified.  The cf-1.com blog on input-adaptive matrix-product reduction gives
 * the problem statement (section 2: Y = X @ W^T, X [T,H], W [M,H]), the flow
 * (sections 5.1-5.3: cheap score, top-k, gather, compact product) and a code
 * sketch (section 6.1: inputs and a keep ratio in, the product and the kept
 * index list out, output shape equal to the dense one).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or equivalent) owned
 *    by the caller; the library never allocates or frees memory and keeps no
 *    per-call state between calls.
 *  - Matrices are row-major with a leading dimension (elements between rows);
 *    a [rows][ld] matrix spans rows*ld elements.  Input matrices (x, W^T, keys,
 *    values, q) must be 16-byte aligned and their leading dimensions a multiple
 *    of 8 elements for bf16 / 4 for fp32; fp32 outputs need only 4-byte
 *    alignment and any leading dimension.
 *  - bf16 data are raw bfloat16 bit patterns (uint16).  fp32 is IEEE binary32.
 *  - Work is enqueued on `stream` (0 = the null stream) and is asynchronous:
 *    results are valid once the stream reaches this point; inputs must stay
 *    unchanged until then.
 *  - Workspace: `ws` is caller-owned device memory of at least the size the
 *    matching *_workspace_size query returns (its first RMM_WS_HEADER_BYTES
 *    bytes are reserved).  Its contents on entry do not matter and need no
 *    initialisation.  The same workspace may serve every entry point, but two
 *    calls in flight at once must not share one workspace.
 *  - Errors: arguments are validated on the host before anything is enqueued;
 *    on any non-OK status nothing has been written.  RMM_EHIP reports a launch
 *    failure (text in rmm_last_error()).  No exception crosses the ABI, and the
 *    library never aborts.  Non-finite inputs give unspecified results.
 */
#ifndef RMM_H
#define RMM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RMM_WS_HEADER_BYTES 4096

/* Each enum below spans the whole int32 range (the _RANGE_ enumerators are not
 * values to pass), so every integer a caller passes is a value of the type and
 * is reported as an argument error when it names nothing, instead of being
 * undefined behaviour in the C++ implementation. */
typedef enum {
    RMM_OK = 0,
    RMM_EINVAL = 1,        /* bad argument: null pointer, size, ratio, stride */
    RMM_EUNSUPPORTED = 2,  /* valid, but no kernel for this shape / dtype / alignment */
    RMM_EWORKSPACE = 3,    /* workspace missing or smaller than the size query */
    RMM_EHIP = 4,          /* a HIP launch failed */
    RMM_STATUS_RANGE_MIN_ = INT32_MIN,
    RMM_STATUS_RANGE_MAX_ = INT32_MAX
} rmm_status_t;

typedef enum {
    RMM_F32 = 0,
    RMM_BF16 = 1,
    RMM_DTYPE_RANGE_MIN_ = INT32_MIN,
    RMM_DTYPE_RANGE_MAX_ = INT32_MAX
} rmm_dtype_t;

/* Selection groups for grouped-query attention.  PER_KV_GROUP: the G = Hq/Hkv
 * query heads sharing one KV head share one head_dim selection and one key
 * position selection (scores take the max over those heads).  PER_Q_HEAD:
 * each query head selects alone (blog section 3.3: reduce inside each head);
 * with G > 1 a KV head's K^T dim rows and V position rows are read once for the
 * union of its query heads' sets, and each head adds only its own kept dims and
 * positions. */
typedef enum {
    RMM_SEL_PER_KV_GROUP = 0,
    RMM_SEL_PER_Q_HEAD = 1,
    RMM_SEL_RANGE_MIN_ = INT32_MIN,
    RMM_SEL_RANGE_MAX_ = INT32_MAX
} rmm_sel_mode_t;

/* ------------------------------------------------------------------ keep count
 * Paper abstract ("retention-ratio control"): k = ceil(r*n) slices are kept.
 * r*n is snapped to the nearest integer when within 1e-9 relative of it, then
 * clamped to [1, n].  Host-only, pure.  Returns -1 if n < 1 or r is not in (0,1]. */
int64_t rmm_keep_count(int64_t n, double r);

/* ------------------------------------------------------------------ select
 * Scorer + top-k selector (blog sections 5.1-5.2; paper abstract).
 * Tokens are grouped into tiles of `tile` consecutive rows, tile tau covering
 * rows [tau*tile, min(T, (tau+1)*tile)); all tokens of a tile share one kept
 * set.  For each tile and slice j < K:
 *     s[j] = fl32( max_{t in tile} |x[t,j]| * c[j] )        (one fp32 multiply)
 * The k = rmm_keep_count(K, r) slices of largest s are kept (equal scores: the
 * lower index wins; -0 ranks as +0) and written in ASCENDING index order.
 *   x    [T][ldx] fp32 or bf16 activations (xt), ldx >= K
 *   c    [K] fp32 per-slice weights, c[j] >= 0 (the norm of W^T row j)
 *   idx  out, int32 [ceil(T/tile)][k]
 * Limits: K <= 32768.  Deterministic: equal inputs give equal outputs. */
size_t rmm_select_workspace_size(int64_t T, int64_t K, int64_t tile, rmm_dtype_t xt);
rmm_status_t rmm_select(const void *x, rmm_dtype_t xt, int64_t T, int64_t K, int64_t ldx,
                        const float *c, int64_t tile, double r,
                        int32_t *idx, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ fused decode step
 * rmm_select followed by rmm_linear for one token, as one launch plus the
 * split-K sum (blog sections 5.1-5.3: score, top-k, compact product; paper
 * abstract).  One workgroup scores and selects; as soon as its first radix
 * pass has run it tells the workgroups that stream W^T which slices are kept
 * for certain, and they start on those rows while it resolves the rest, so the
 * product does not wait for the whole selection.
 *   x    [K] activations of the token (dtype xt), 16-byte aligned; read in
 *        16-byte vectors, so its buffer holds K rounded up to a multiple of 8
 *        (bf16) or 4 (fp32) elements (the padding is read and ignored)
 *   c    [K] fp32 slice weights, c[j] >= 0
 *   wt   [K][ldw] W^T (dtype xt); y out, fp32 [M]
 *   idx  optional out (NULL ok), int32 [k], k = rmm_keep_count(K, r): the kept
 *        slices in ascending order, exactly as rmm_select(x, xt, 1, K, K, c, 1, r, ...)
 *        writes them
 * The kept set is rmm_select's; y is rmm_linear's up to fp32 summation order
 * (each split adds the rows kept for certain before the others).  Deterministic.
 * Workspace: rmm_select_linear_workspace_size(K, M, xt) bytes.  Unlike the
 * other entry points, the first RMM_WS_HEADER_BYTES bytes of this workspace
 * must be zero before the first call that uses it (a zero-filled allocation);
 * every call leaves them zero and no other entry point writes them.
 * Limits: K <= 32768; one token. */
size_t rmm_select_linear_workspace_size(int64_t K, int64_t M, rmm_dtype_t xt);
rmm_status_t rmm_select_linear(const void *x, rmm_dtype_t xt, int64_t K, const float *c, double r,
                               const void *wt, rmm_dtype_t wt_t, int64_t M, int64_t ldw,
                               int32_t *idx, float *y, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ block-granular selection
 * The blog's block variant (section 5.1: a block's importance is the mean
 * absolute activation over its neurons; 5.2: top-k over blocks, the block mask
 * expanded to neuron indices; 6.1: the demo's ffn_block_reduce).  The
 * contraction dimension is cut into nb = K / block blocks of `block`
 * consecutive slices.  Per tile (as in rmm_select) and block b:
 *     score[b] = ( sum_{j in b, ascending} (double) max_{t in tile} |x[t,j]| ) / block
 * (the sum and the division in IEEE double).  The nk = rmm_block_keep_count(nb,
 * keep) blocks of largest score are kept (equal scores: the lower block wins),
 * in ASCENDING block order, each expanded to its `block` slice indices:
 *   idx  out, int32 [ceil(T/tile)][nk*block]: idx[tau][i*block + e] = b_i*block + e
 * The list feeds rmm_linear unchanged (k = nk*block).
 * Limits: K % block == 0 (else RMM_EINVAL), K <= 32768, nb <= 1024.
 * Deterministic. */
int64_t rmm_block_keep_count(int64_t nb, double keep); /* max(1, floor(nb*keep)) clamped to nb; -1 if keep not in (0,1] */
size_t rmm_select_blocks_workspace_size(int64_t T, int64_t K, int64_t tile, int64_t block, rmm_dtype_t xt);
rmm_status_t rmm_select_blocks(const void *x, rmm_dtype_t xt, int64_t T, int64_t K, int64_t ldx,
                               int64_t tile, int64_t block, double keep,
                               int32_t *idx, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ linear
 * Reduced product (blog sections 2 and 5.3; paper abstract):
 *     y[t,m] = sum_{j in idx[t/tile]} x[t,j] * wt[j,m]      (fp32 accumulation)
 * W^T is stored K-major ([K][ldw], row j = the weights slice j multiplies), so
 * every kept slice is one contiguous row; nothing is gathered into a copy of W.
 * Output shape equals the dense one (blog section 6.1).
 *   x   [T][ldx] activations, dtype xt;  wt [K][ldw], dtype must equal xt
 *   idx [ceil(T/tile)][k] int32, strictly ascending, each < K (as rmm_select
 *       writes it; contents are trusted)
 *   y   out, fp32 [T][ldy], ldy >= M
 * bf16 with >= 32 tokens per tile runs on MFMA tiles; otherwise a streaming
 * kernel (any T) runs.  Deterministic. */
size_t rmm_linear_workspace_size(int64_t T, int64_t K, int64_t M, int64_t k, int64_t tile,
                                 rmm_dtype_t xt);
rmm_status_t rmm_linear(const void *x, rmm_dtype_t xt, int64_t T, int64_t K, int64_t ldx,
                        const void *wt, rmm_dtype_t wt_t, int64_t M, int64_t ldw,
                        const int32_t *idx, int64_t k, int64_t tile,
                        float *y, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t stream);

/* rmm_linear for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and results as rmm_linear with the same arguments, with no
 * workspace argument.  Its scratch is a device array of
 * RMM_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, kept until the
 * process ends; the call allocates and frees nothing.  All calls on one GPU
 * share that array, so calls that overlap in time on one GPU (other streams,
 * other threads) race and must be serialised by the caller.  The array needs
 * no initialisation: every call writes the scratch it reads.
 * Errors: as rmm_linear; RMM_EUNSUPPORTED when the product needs more scratch
 * than the array holds (rmm_linear_workspace_size above it: e.g. more than 8
 * tokens per tile times M = 32768 on the streaming path, or T * k above
 * 8 Mi elements on the MFMA path). */
#define RMM_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
rmm_status_t rmm_linear_noalloc(const void *x, rmm_dtype_t xt, int64_t T, int64_t K, int64_t ldx,
                                const void *wt, rmm_dtype_t wt_t, int64_t M, int64_t ldw,
                                const int32_t *idx, int64_t k, int64_t tile,
                                float *y, int64_t ldy, hipStream_t stream);

/* Dense product y = x @ wt over all K slices, by the same kernels without the
 * index list (the r = 1 baseline; blog section 8 asks for a full path next to
 * the compact one).  Same arguments and rules as rmm_linear. */
size_t rmm_linear_dense_workspace_size(int64_t T, int64_t K, int64_t M, rmm_dtype_t xt);
rmm_status_t rmm_linear_dense(const void *x, rmm_dtype_t xt, int64_t T, int64_t K, int64_t ldx,
                              const void *wt, rmm_dtype_t wt_t, int64_t M, int64_t ldw,
                              float *y, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ gated FFN producer
 * The FFN's intermediate activation, the down projection's input (blog section
 * 6.1, the demo's ffn_full: gate = x W_gate^T, up = x W_up^T, h = silu(gate) *
 * up; section 5.1 scores the down projection from h; section 6.2: gate and up
 * stay full).  For every token t and column m < Mi:
 *     g = sum_j x[t,j] * wg[j,m],  u = sum_j x[t,j] * wu[j,m]     (fp32 accumulation)
 *     h[t,m] = bf16( silu(g) * u ),  silu(g) = g / (1 + e^-g)     (fp32, nearest-even)
 *     pmax[tau][m] = max_{t in tile tau} |h[t,m]|                 (optional)
 * pmax is exactly what rmm_select would take as the tile's column maxima, so
 * rmm_select(pmax, RMM_F32, ceil(T/tile), Mi, Mi, c, 1, r, ...) keeps the same
 * slices as rmm_select(h, RMM_BF16, T, Mi, ldh, c, tile, r, ...).
 *   x    bf16 [T][ldx], ldx >= H
 *   wg   bf16 [H][ldw]  W_gate^T, K-major (row j = the weights x[t,j] multiplies)
 *   wu   bf16 [H][ldw]  W_up^T, same layout and pitch
 *   h    out, bf16 [T][ldh], ldh >= Mi, 2-byte aligned
 *   pmax optional out (NULL ok), fp32 [ceil(T/tile)][Mi]
 * Deterministic (fixed-order split reduction). */
size_t rmm_gate_up_workspace_size(int64_t T, int64_t H, int64_t Mi, int64_t tile);
rmm_status_t rmm_gate_up(const void *x, int64_t T, int64_t H, int64_t ldx,
                         const void *wg, const void *wu, int64_t ldw, int64_t Mi, int64_t tile,
                         void *h, int64_t ldh, float *pmax, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/* ------------------------------------------------------------------ attention decode
 * Reduced grouped-query attention for one decode step (blog sections 3.1 and
 * 3.3; GEMM notes section 1: scores = Q K^T, out = softmax(scores) V).
 * Query head h reads KV head g = h / G, G = Hq / Hkv.  Per batch element b and
 * selection group (mode above):
 *  1. head_dim slices: sigma_j = fl32( max_{h in group} |q[b,h,j]| * kn[b,g,j] );
 *     the k_d = rmm_keep_count(D, r_dim) best are kept (ties: lower index);
 *  2. logits l_h[s] = scale * sum_{j kept} q[b,h,j] * K[b,g,s,j], every s < S;
 *  3. full softmax over all S positions: p_h[s] = exp(l_h[s] - lse_h);
 *  4. key positions: pi_s = max_{h in group} p_h[s]; the k_s = rmm_keep_count(S,
 *     r_pos) best are kept, ranked by the log-probability max_h (l_h[s] - lse_h)
 *     evaluated in double and held as a 64-bit fixed-point key (steps of at most
 *     2^-28 nat over [-1056, +1024) nats; every probability below e^-1056, which
 *     is 0 in double, ties); ties: lower index;
 *  5. out[b,h,:] = sum_{s kept} p_h[s] * V[b,g,s,:]  -- no renormalisation.
 *   q   bf16 [B][Hq][D]
 *   kt  bf16 [B][Hkv][D][ldk]  keys stored dim-major: row j holds dim j of every position
 *   v   bf16 [B][Hkv][ldv][D]  values position-major
 *   kn  fp32 [B][Hkv][D]       kn[b,g,j] = L2 norm of K[b,g,0:S,j] (kept by the cache owner)
 *   scale  logit scale (1/sqrt(D) for standard attention; not rescaled by k_d)
 *   out     out, fp32 [B][Hq][D]
 *   dim_idx optional out (NULL ok), int32 [B][Hsel][k_d] ascending
 *   pos_idx optional out (NULL ok), int32 [B][Hsel][k_s] ascending
 *   lse     optional out (NULL ok), fp32 [B][Hq] = log sum_s exp(l_h[s])
 *   Hsel = Hkv (PER_KV_GROUP) or Hq (PER_Q_HEAD).
 * Limits: D == 128, Hq/Hkv in {1,2,4,8}, S <= 2^24, ldk a multiple of 8,
 *   B * Hsel <= 512 and B * Hkv <= 512 (else RMM_EUNSUPPORTED).
 * Deterministic. */
size_t rmm_attn_decode_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t S,
                                      double r_dim, double r_pos, rmm_sel_mode_t mode);
rmm_status_t rmm_attn_decode(const void *q, const void *kt, const void *v, const float *kn,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t S,
                             int64_t ldk, int64_t ldv, float scale,
                             double r_dim, double r_pos, rmm_sel_mode_t mode,
                             float *out, int32_t *dim_idx, int32_t *pos_idx, float *lse,
                             void *ws, size_t ws_bytes, hipStream_t stream);

/* Same as rmm_attn_decode, with the position score optionally weighted by the
 * norm of the value row: step 4 ranks pi_s = max_{h in group} p_h[s] * vn[b,g,s]
 * instead of max_h p_h[s] -- the counterpart, for the PV product, of the linear
 * scorer's |x| * ||W^T row|| (blog section 5.1: a slice's weight is its input
 * magnitude times its weight norm).  Step 5 is unchanged (no renormalisation,
 * p_h[s] unweighted).
 *   vn  NULL, or fp32 [B][Hkv][ldv], 16-byte aligned (ldv then a multiple of 8),
 *       vn[b,g,s] >= 0 for s < S
 *       (vn[b,g,s] = L2 norm of V[b,g,s,:], kept by the cache owner; entries
 *       s >= S are read but ignored)
 * The ranking key holds log(pi_s) - 8 with the same steps and range as the
 * unweighted key (log(pi_s) from -1048 to +1032 nats; a zero norm ranks last).
 * vn = NULL gives exactly rmm_attn_decode's results; the workspace size is
 * rmm_attn_decode's. */
rmm_status_t rmm_attn_decode_ex(const void *q, const void *kt, const void *v, const float *kn,
                                const float *vn,
                                int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t S,
                                int64_t ldk, int64_t ldv, float scale,
                                double r_dim, double r_pos, rmm_sel_mode_t mode,
                                float *out, int32_t *dim_idx, int32_t *pos_idx, float *lse,
                                void *ws, size_t ws_bytes, hipStream_t stream);

/* Paged caches and ragged batches.  Decode servers keep each sequence's KV
 * cache in fixed-size pages and batch sequences of different lengths (GEMM
 * notes section 7: continuous batching and paged attention in decode; blog
 * section 8: batching is the main practical conflict of input-adaptive
 * reduction).  The computation is rmm_attn_decode_ex's, per sequence b over its
 * own S_b = seqlens[b] positions (values outside [1, S] are clamped), with its
 * own kept count k_b = rmm_keep_count(S_b, r_pos).
 *   k_pages  bf16 [num_pages][Hkv][D][page]  dim-major keys: row j of a page holds dim j
 *   v_pages  bf16 [num_pages][Hkv][page][D]
 *   vn_pages NULL, or fp32 [num_pages][Hkv][page] value-row norms (16-byte aligned)
 *   block_table int32 [B][max_pages]: entry i of row b names the page holding
 *            positions [i*page, (i+1)*page) of sequence b; only the first
 *            ceil(S_b/page) entries are read, and their contents are trusted
 *   seqlens  int32 [B] (device memory)
 *   kn       fp32 [B][Hkv][D] key-column norms over each sequence's own positions
 *   S        a bound on every S_b (at most max_pages*page): it sizes the
 *            workspace (rmm_attn_decode_workspace_size with this S) and pos_idx
 *   pos_idx  optional out, int32 [B][Hsel][rmm_keep_count(S, r_pos)]: row (b, .)
 *            holds its k_b kept positions ascending, then -1
 * Limits: page a multiple of 8 in [8, 2^24]; otherwise as rmm_attn_decode. */
rmm_status_t rmm_attn_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                                   const float *kn, const float *vn_pages,
                                   const int32_t *block_table, int64_t max_pages, int64_t page,
                                   const int32_t *seqlens,
                                   int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t S,
                                   float scale, double r_dim, double r_pos, rmm_sel_mode_t mode,
                                   float *out, int32_t *dim_idx, int32_t *pos_idx, float *lse,
                                   void *ws, size_t ws_bytes, hipStream_t stream);

/* Dense decode attention over paged, ragged caches (the r = 1 baseline of
 * rmm_attn_decode_paged): same layouts; workspace from
 * rmm_attn_decode_dense_workspace_size with the same S. */
rmm_status_t rmm_attn_decode_dense_paged(const void *q, const void *k_pages, const void *v_pages,
                                         const int32_t *block_table, int64_t max_pages, int64_t page,
                                         const int32_t *seqlens,
                                         int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t S,
                                         float scale, float *out, float *lse,
                                         void *ws, size_t ws_bytes, hipStream_t stream);

/* Dense decode attention (all D dims, all S positions, online softmax) -- the
 * r = 1 baseline.  Same layouts; lse optional. */
size_t rmm_attn_decode_dense_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t S);
rmm_status_t rmm_attn_decode_dense(const void *q, const void *kt, const void *v,
                                   int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t S,
                                   int64_t ldk, int64_t ldv, float scale,
                                   float *out, float *lse, void *ws, size_t ws_bytes,
                                   hipStream_t stream);

/* ------------------------------------------------------------------ errors */
const char *rmm_status_string(rmm_status_t s);
/* detail of the last non-OK status returned on the calling thread */
const char *rmm_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* RMM_H */
