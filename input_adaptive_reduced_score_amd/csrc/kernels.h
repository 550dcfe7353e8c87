// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// ---- tuning constants (compile-time; override with -D for sweeps)
#ifndef SELECT_DIRECT_ROWS
#define SELECT_DIRECT_ROWS 16 // tiles with at most this many rows are scored inside the select kernel
#endif
#ifndef COLMAX_ROWS
#define COLMAX_ROWS 64 // rows per column-max workgroup for larger tiles
#endif
#define SELECT_MAX_K 32768

#ifndef GEMV_UNROLL
#define GEMV_UNROLL 16     // kept rows in flight per wave
#endif
#ifndef GEMV_TARGET_WGS
#define GEMV_TARGET_WGS 512 // workgroups (8 waves each) the split-K aims for
#endif
#ifndef GEMV_MIN_ROWS
#define GEMV_MIN_ROWS 8 // kept rows per wave below which splitting stops
#endif
#define GEMV_MAX_SPLIT 64
#define MFMA_MIN_TILE_ROWS 32 // bf16 tiles with at least this many tokens use the MFMA GEMM
#ifndef GATEUP_UNROLL
#define GATEUP_UNROLL 8 // rows of each of W_gate^T and W_up^T in flight per wave
#endif
#ifndef GATEUP_TARGET_WGS
#define GATEUP_TARGET_WGS 512
#endif
#ifndef GATEUP_MIN_ROWS
#define GATEUP_MIN_ROWS 8
#endif
#define GATEUP_MAX_SPLIT 64

#define ATTN_D 128
#define ATTN_QK_CHUNK 512   // positions per QK workgroup
#define ATTN_KEY_CHUNK 2048 // positions per key-workgroup chunk
#define ATTN_HIST_BINS 8192 // position-score histogram: half-nat bins outside [-32, 0), 1/128 nat inside
#define ATTN_MAX_GROUPS 512 // B * Hsel and B * Hkv limit of the attention entry points (the range the tests cover)
#define RMM_WS_HEADER_BYTES_INTERNAL 4096

namespace rmm {

// What the selecting workgroup of a fused select-and-product launch publishes
// (select_body.h, gemv.hip), as two 64-bit words in the workspace header (zero
// before the launch, cleared by the launch after it), each carrying a ready bit:
//   sig1: after the first radix pass, the smallest non-zero key mn (keys are
//         re-based as u = key - mn + 1, 0 stays 0) and the undecided digit
//         (digit d of nb bits at bit sh): u above it is kept for certain;
//   sig2: the threshold u and the slice of the last kept key equal to it;
// and offs[p] = kept slices before split p's first slice in the column slice the
// index list is written from (p <= nsplit).  That column slice is cut into a
// short first range of R0 slices (the selecting workgroup's own share, streamed
// after its selection) and nsplit - 1 ranges of R1; the others into ranges of R.
struct SelPub {
    uint64_t *sig1 = nullptr, *sig2 = nullptr, *sig3 = nullptr;
    uint32_t *offs = nullptr;
    int R = 1, R0 = 1, R1 = 1, nsplit = 0;
};
// first slice of split p in the column slice of the index list (p <= nsplit)
__host__ __device__ __forceinline__ int split_start0(const SelPub &pb, int p, int K)
{
    const int q = p == 0 ? 0 : pb.R0 + (p - 1) * pb.R1;
    return q < K ? q : K;
}
__device__ __forceinline__ uint64_t sig1_pack(uint32_t mn, uint32_t d, int sh, int nb)
{
    return ((uint64_t)mn << 32) | ((uint64_t)d << 11) | ((uint64_t)sh << 6) | ((uint64_t)nb << 1) | 1ull;
}
__device__ __forceinline__ uint64_t sig2_pack(uint32_t thr, int jt)
{
    return ((uint64_t)thr << 32) | ((uint64_t)(uint32_t)jt << 1) | 1ull;
}

// select.hip
size_t select_ws_bytes(int64_t T, int64_t K, int64_t tile);
hipError_t launch_select(const void *x, bool bf16, int64_t T, int64_t K, int64_t ldx, const float *c, int64_t tile,
                         int64_t k, int32_t *idx, float *pmax_ws, hipStream_t st);
hipError_t launch_select_blocks(const void *x, bool bf16, int64_t T, int64_t K, int64_t ldx, int64_t tile,
                                int64_t block, int64_t nk, int32_t *idx, float *pmax_ws, hipStream_t st);
#define SELECT_BLOCKS_MAX_NB 1024
void select_init();

// gemv.hip: the fused select + GEMV for one token (workspace after the header;
// its two flags live in the header)
size_t select_gemv_ws_bytes(int64_t K, int64_t M, bool bf16);
bool select_gemv_fits(int64_t K, int64_t M, bool bf16);
hipError_t launch_select_gemv(const void *x, bool bf16, int64_t K, const float *c, int64_t k, const void *wt,
                              int64_t ldw, int64_t M, int32_t *idx, float *y, char *hdr, char *body, hipStream_t st);
int select_per_for(int64_t K);
// gemv.hip
size_t gemv_ws_bytes(int64_t T, int64_t M, int64_t k, int64_t tile, bool bf16);
hipError_t launch_gemv(const void *x, bool bf16, int64_t T, int64_t ldx, const void *wt, int64_t ldw, int64_t M,
                       const int32_t *idx, int64_t k, int64_t tile, bool dense, float *y, int64_t ldy, float *part,
                       hipStream_t st);

// linear.hip
size_t gemm_ws_bytes(int64_t T, int64_t k);
hipError_t launch_gemm(const void *x, int64_t T, int64_t K, int64_t ldx, const void *wt, int64_t ldw, int64_t M,
                       const int32_t *idx, int64_t k, int64_t tile, bool dense, float *y, int64_t ldy, void *xg,
                       hipStream_t st);
void linear_init();

// ffn.hip
size_t gateup_ws_bytes(int64_t T, int64_t H, int64_t Mi, int64_t tile);
int64_t gateup_grid(int64_t T, int64_t H, int64_t Mi, int64_t tile);
hipError_t launch_gateup(const uint16_t *x, int64_t T, int64_t H, int64_t ldx, const uint16_t *wg,
                         const uint16_t *wu, int64_t ldw, int64_t Mi, int64_t tile, uint16_t *h, int64_t ldh,
                         float *pmax, float *part, hipStream_t st);

// attn.hip
struct AttnShape {
    int64_t B, Hq, Hkv, S, ldk, ldv;
    int G;      // query heads per KV head
    int GS;     // query heads per selection group (G or 1)
    int Hsel;   // selection groups per batch element
    int kd, ks; // kept head_dim slices, kept positions
    float scale;
};
struct AttnWs {
    float *logit;     // [B][Hq][Sp] unscaled q.k over kept dims
    float2 *pstat;    // [B][Hq][nqk] (max, sum exp) per QK chunk
    uint16_t *bins;   // [B][Hsel][Sp rounded up to 64] histogram bin of every position's score
    uint32_t *hist;   // [B][Hsel][ATTN_HIST_BINS]
    uint32_t *pcount; // [B][Hsel][npv] kept positions per PV chunk
    uint64_t *sig;    // [B][Hsel][32] words: workgroup counts, threshold bin, threshold rank key
    int32_t *pstage;  // [B][Hsel][Sp] kept positions of each PV chunk, staged at the chunk's start
    float *pvpart;    // [B][Hsel][npv][GS][D]
};
// Where the cache of sequence b keeps position p (contiguous caches, or pages
// named by a block table) and how long each sequence is.
struct KvMap {
    const int32_t *pages;   // block table [B][maxp], or null: contiguous caches with pitches ldk / ldv
    const int32_t *seqlens; // [B] positions per sequence (clamped to [1, S]), or null: every sequence has S
    int64_t maxp;           // block-table row length
    int page;               // positions per page (a multiple of 8)
    double r_pos;           // position keep ratio (per-sequence keep counts)
};
size_t attn_ws_layout(const AttnShape &s, AttnWs *ws, char *base);
hipError_t launch_attn(const AttnShape &s, const KvMap &m, const uint16_t *q, const uint16_t *kt, const uint16_t *v,
                       const float *kn, const float *vn, float *out, int32_t *dim_idx, int32_t *pos_idx, float *lse,
                       const AttnWs &ws, hipStream_t st);
size_t attn_dense_ws_layout(int64_t B, int64_t Hq, int64_t S, char *base, float **part, float2 **stat);
hipError_t launch_attn_dense(const AttnShape &s, const KvMap &m, const uint16_t *q, const uint16_t *kt,
                             const uint16_t *v, float *out, float *lse, float *part, float2 *stat, hipStream_t st);
void attn_init();

} // namespace rmm
