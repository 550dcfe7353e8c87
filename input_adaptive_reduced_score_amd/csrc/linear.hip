// Reduced linear products with many tokens per tile (prefill).
//
// The blog on input-adaptive matrix-product reduction (section 2) reduces
// Y = X @ W^T over the kept contraction slices J: Y ~= X[:,J] @ W^T[J,:];
// section 5.3 gathers the kept slices so the product stays dense, and
// section 8 warns that a gather copy costs bandwidth.  W^T is stored K-major,
// so every kept slice is one contiguous row of W^T: the kernels read kept rows
// in place and never copy W.
//
// gather_kernel + gemm_dma_kernel: the kept columns of the tile's activations
// are packed once (activations are the small operand), then a bf16 MFMA GEMM
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation) brings the packed activations
// and the kept W^T rows through LDS.  (Few tokens per tile: gemv.hip.)
#include "device.h"
#include "kernels.h"

namespace rmm {

// ============================================================================ gather
// xg[t][i] = x[t][idx[t/tile][i]] for i < k, 0 for k <= i < kpad.
// A workgroup takes up to `rows` consecutive token rows of one tile (they share
// the kept list).  Thread t owns packed columns t, t + 256, ...; it loads their
// indices once, with clamped addresses so that every load is issued before the
// first wait, and reuses them for each row.
// With STAGE the rows are first staged in LDS with 16-byte loads, all rows in
// flight together (rows x K elements, K up to GATHER_LDS_MAX_K); without, each
// element is read from global memory.
constexpr int GATHER_LDS_MAX_K = 32768;
constexpr int GATHER_LDS_BUDGET = 16384;  // bytes of staged rows per workgroup (one row may exceed it)
constexpr int GATHER_MAX_ROWS = 8;
constexpr int GATHER_CH_MAX = 4;          // chunks per thread held in registers per pass
template <bool STAGE, int GATHER_CH>
__global__ __launch_bounds__(256) void gather_kernel(const uint16_t *__restrict__ x, int64_t ldx, int T, int K, int tile,
                                                     const int32_t *__restrict__ idx, int k, int kpad, int rows,
                                                     int groups_per_tile, uint16_t *__restrict__ xg)
{
    extern __shared__ uint16_t xrow[];
    const int tau = blockIdx.x / groups_per_tile, grp = blockIdx.x % groups_per_tile;
    const int t0 = tau * tile + grp * rows;
    const int nr = min(rows, min(T, tau * tile + tile) - t0);
    if (nr <= 0)
        return;
    const int32_t *J = idx + (int64_t)tau * k;
    const int K8 = (K + 7) / 8;
    if (STAGE) {
        // ldx is a multiple of 8, so the 16-byte run past K stays inside the row's pitch
        const int per = (K8 + 255) / 256;
        for (int r = 0; r < nr; ++r) {
            const uint16_t *xr = x + (int64_t)(t0 + r) * ldx;
            for (int q = 0; q < per; ++q) {
                const int c = min((int)threadIdx.x + 256 * q, K8 - 1);
                *reinterpret_cast<uint4 *>(xrow + (int64_t)r * K8 * 8 + c * 8) =
                    *reinterpret_cast<const uint4 *>(xr + c * 8);
            }
        }
        __syncthreads();
    }
    // Packed element i of a row is taken by thread i % 256: a wave's 64 reads
    // address 64 consecutive kept columns, 2/r bytes apart on average (few
    // lanes per LDS bank), and its 2-byte stores fill 128 contiguous bytes.  A
    // thread that took 8 consecutive packed elements read 8 kept columns away
    // from its neighbours' addresses: up to 8 lanes per bank.
    constexpr int NJ = 8 * GATHER_CH; // packed elements per thread per pass
    for (int c0 = 0; c0 < kpad; c0 += 256 * NJ) {
        int jv[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            jv[j] = J[min(c0 + (int)threadIdx.x + 256 * j, k - 1)];
        for (int r = 0; r < nr; ++r) {
            const uint16_t *src = STAGE ? xrow + (int64_t)r * K8 * 8 : x + (int64_t)(t0 + r) * ldx;
            uint16_t *dst = xg + (int64_t)(t0 + r) * kpad;
            uint16_t v[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                v[j] = src[jv[j]]; // clamped index: always in bounds
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int i = c0 + (int)threadIdx.x + 256 * j;
                if (i < kpad) // (whole waves: kpad, c0 and 256 j are multiples of 64)
                    dst[i] = i < k ? v[j] : (uint16_t)0;
            }
        }
    }
}

struct GatherPlan {
    int rows, groups_per_tile, ntiles, ch;
    size_t lds;
    bool stage;
};

static GatherPlan gather_plan(int64_t T, int64_t K, int64_t k, int64_t tile)
{
    GatherPlan g;
    const int64_t rowbytes = (K + 7) / 8 * 16;
    // chunk groups of 256 per thread: as many as the packed row needs, up to GATHER_CH_MAX per pass
    const int64_t kpad = (k + 63) / 64 * 64, groups = (kpad / 8 + 255) / 256;
    g.ch = groups <= 1 ? 1 : groups <= 2 ? 2 : GATHER_CH_MAX;
    g.stage = K <= GATHER_LDS_MAX_K;
    int64_t r = g.stage ? GATHER_LDS_BUDGET / rowbytes : GATHER_MAX_ROWS;
    r = r < 1 ? 1 : r > GATHER_MAX_ROWS ? GATHER_MAX_ROWS : r;
    const int64_t trows = tile < T ? tile : T;
    if (r > trows)
        r = trows;
    g.rows = (int)r;
    g.groups_per_tile = (int)((trows + r - 1) / r);
    g.ntiles = (int)((T + tile - 1) / tile);
    g.lds = g.stage ? (size_t)(r * rowbytes) : 0;
    return g;
}

// ============================================================================ MFMA GEMM, register-staged
// The dense product y = x @ W^T when K is not a multiple of 64: the last k
// step is partial and the operands are zero-filled past K on their way through
// registers (the LDS-DMA kernel below needs whole k steps).  Workgroup tile
// 128 x 128, k step 64, 4 waves of 64 x 64 (2 x 2 MFMA 32x32x16).
constexpr int GB_M = 128, GB_N = 128, GB_K = 64;
constexpr int GEMM_THREADS = 256;
constexpr int LPITCH = GB_K + 8; // bf16 per LDS row (pad against bank conflicts)

__global__ __launch_bounds__(GEMM_THREADS) void gemm_kernel(const uint16_t *__restrict__ A, int64_t lda, int T,
                                                            int tile, int mblocks, const uint16_t *__restrict__ wt,
                                                            int64_t ldw, int M, int klim, float *__restrict__ y,
                                                            int64_t ldy)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[2][GB_M * LPITCH];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][GB_N * LPITCH];
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int nb = blockIdx.x, mbk = blockIdx.y;
    const int tau = mbk / mblocks, mm = mbk % mblocks;
    const int row0 = tau * tile + mm * GB_M;
    const int rowend = min(T, tau * tile + tile);
    if (row0 >= rowend)
        return;
    const int n0 = nb * GB_N;
    const int wm = w >> 1, wn = w & 1;

    // A loader: 4 chunks of 8 bf16 per thread: row ar + 32p, k offset 8*ac
    const int ar = tid >> 3, ac = tid & 7;
    // B loader: lane = k row within the step, chunks w + 4p of 8 columns
    uint4 ra[4], rb[4];
    // the W^T row of this lane for a step
    auto jrow = [&](int kk) {
        const int kr = kk + lane;
        return kr < klim ? kr : klim - 1; // rows past K repeat the last one (times zero A)
    };
    auto load_stage = [&](int kk, int j) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = ar + 32 * p;
            const int kc = kk + 8 * ac;
            uint4 v = {0u, 0u, 0u, 0u};
            if (row0 + r < rowend) {
                const uint16_t *src = A + (int64_t)(row0 + r) * lda + kc;
                if (kc + 8 <= klim) {
                    v = *reinterpret_cast<const uint4 *>(src);
                } else if (kc < klim) {
                    uint32_t h[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        h[e] = kc + e < klim ? src[e] : 0u;
                    v.x = h[0] | (h[1] << 16);
                    v.y = h[2] | (h[3] << 16);
                    v.z = h[4] | (h[5] << 16);
                    v.w = h[6] | (h[7] << 16);
                }
            }
            ra[p] = v;
        }
        const uint16_t *wrow = wt + (int64_t)j * ldw;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int nc = n0 + 8 * (w + 4 * p);
            rb[p] = nc < M ? *reinterpret_cast<const uint4 *>(wrow + nc) : uint4{0u, 0u, 0u, 0u};
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
            *reinterpret_cast<uint4 *>(&As[buf][(ar + 32 * p) * LPITCH + 8 * ac]) = ra[p];
        // B^T: transposed on the way into LDS so both operands read as 16-byte k-runs
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int nbase = 8 * (w + 4 * p);
            const uint32_t q[4] = {rb[p].x, rb[p].y, rb[p].z, rb[p].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Bs[buf][(nbase + 2 * e) * LPITCH + lane] = (uint16_t)(q[e] & 0xffffu);
                Bs[buf][(nbase + 2 * e + 1) * LPITCH + lane] = (uint16_t)(q[e] >> 16);
            }
        }
    };
    auto frags = [&](int cur, int ks, bf16x8_t(&a)[2], bf16x8_t(&b)[2]) {
        const int kofs = ks * 16 + 8 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            a[i] = *reinterpret_cast<const bf16x8_t *>(&As[cur][(wm * 64 + i * 32 + (lane & 31)) * LPITCH + kofs]);
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
            b[jn] = *reinterpret_cast<const bf16x8_t *>(&Bs[cur][(wn * 64 + jn * 32 + (lane & 31)) * LPITCH + kofs]);
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][jn][r] = 0.0f;
    auto mma = [&](bf16x8_t(&a)[2], bf16x8_t(&b)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jn = 0; jn < 2; ++jn)
                acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[jn], acc[i][jn], 0, 0, 0);
    };

    const int ksteps = (klim + GB_K - 1) / GB_K;
    load_stage(0, jrow(0));
    int jnext = ksteps > 1 ? jrow(GB_K) : 0;
    store_stage(0);
    __syncthreads();
    for (int s = 0; s < ksteps; ++s) {
        const int cur = s & 1;
        const bool more = s + 1 < ksteps;
        if (more)
            load_stage((s + 1) * GB_K, jnext);
        if (s + 2 < ksteps)
            jnext = jrow((s + 2) * GB_K);
        // fragments of sub-step ks+1 load while sub-step ks multiplies
        bf16x8_t a0[2], b0[2], a1[2], b1[2];
        frags(cur, 0, a0, b0);
        frags(cur, 1, a1, b1);
        mma(a0, b0);
        frags(cur, 2, a0, b0);
        mma(a1, b1);
        frags(cur, 3, a1, b1);
        mma(a0, b0);
        mma(a1, b1);
        if (more)
            store_stage(cur ^ 1);
        __syncthreads();
    }

    // D layout of a 32x32 MFMA: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) {
            const int col = n0 + wn * 64 + jn * 32 + (lane & 31);
            if (col >= M)
                continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < rowend)
                    y[(int64_t)row * ldy + col] = acc[i][jn][r];
            }
        }
}

// ============================================================================ MFMA GEMM, LDS DMA
// The same product for k steps that are whole (packed activations, or a dense
// K that is a multiple of 64).  Workgroup tile 128 x 256, k step 64, one
// workgroup per CU (147 KiB of LDS), 8 waves: 4 compute waves of 128 x 64
// (4 x 2 v_mfma_f32_32x32x16_bf16 per 16-deep slice: they share every A
// fragment and read only their own B columns, which take the slower
// transposing LDS read) and 4 load waves.
//
// Both operands go from global memory straight into LDS (global_load_lds_dwordx4:
// lane l's 16 bytes land at the wave's LDS base + 16 l), three k steps ahead,
// so no registers hold tiles in flight; the kept-row indices of a step travel
// the same way three steps before its rows.  The load waves issue them and wait
// for them: a wave stalled on a full load queue leaves its SIMD to the compute
// wave that shares it.  The compiler drains every outstanding LDS DMA before an
// LDS read it schedules itself, so all LDS reads are inline asm: the compute
// waves' fragment reads come in blocks of 8 interleaved with the 8 MFMAs of the
// previous slice, each block closed by its own lgkmcnt(0); the DMA waits
// (vmcnt) are explicit.
//
// LDS per stage.  A: 128 rows x 128 bytes; the 16-byte chunk c of row r sits
// at chunk c ^ gd_aswz(r) = c ^ ((r >> 1) & 7): the LDS has 64 banks, so a
// 128-byte row pair spans them all and the 16 rows of a 16-lane quarter of a
// 16-byte read must differ in (r & 1, chunk); with c ^ (r & 7) rows r and
// r + 8 collided.  B (kept W^T rows): 64 rows x 512 bytes; chunk c of
// row q sits at chunk c ^ 4(q & 3).  Each spreads a fragment read over the
// banks; the DMA stores a chunk anywhere in its 1 KiB by the choice of the
// lane's source address.
constexpr int GD_M = 128, GD_N = 256, GD_K = 64;
__device__ __forceinline__ int gd_aswz(int r) { return (r >> 1) & 7; }
constexpr int GD_A_STAGE = GD_M * GD_K * 2;            // 16 KiB
constexpr int GD_B_STAGE = GD_K * GD_N * 2;            // 32 KiB
constexpr int GD_B_BASE = 3 * GD_A_STAGE;              // A stages first, then B stages
constexpr int GD_J_BASE = 3 * (GD_A_STAGE + GD_B_STAGE); // then the kept-row indices: [stage][wave][64 words]
constexpr int GD_LDS = GD_J_BASE + 3 * 4 * 256;           // 147 KiB

typedef int gd_v2i __attribute__((ext_vector_type(2)));
typedef int gd_v4i __attribute__((ext_vector_type(4)));

// One 16-deep slice: the 8 MFMAs on fragments a (4 x 32 rows) and b (2 x 32
// columns), with the next slice's fragments read from LDS in between (A rows
// at pa + OA + 4096 i, B halves at pb[jn] + OB and + OB + 2048).  The block
// waits for its own reads.
#define GD_SLICE_OUTS                                                                                             \
    [c00] "+a"(c[0][0]), [c01] "+a"(c[0][1]), [c10] "+a"(c[1][0]), [c11] "+a"(c[1][1]), [c20] "+a"(c[2][0]),     \
        [c21] "+a"(c[2][1]), [c30] "+a"(c[3][0]), [c31] "+a"(c[3][1]), [an0] "=&v"(an[0]), [an1] "=&v"(an[1]),    \
        [an2] "=&v"(an[2]), [an3] "=&v"(an[3]), [bl0] "=&v"(bl[0]), [bh0] "=&v"(bh[0]), [bl1] "=&v"(bl[1]),       \
        [bh1] "=&v"(bh[1])
#define GD_SLICE_INS                                                                                              \
    [a0] "v"(a[0]), [a1] "v"(a[1]), [a2] "v"(a[2]), [a3] "v"(a[3]), [b0] "v"(b[0]), [b1] "v"(b[1]), [pa] "v"(pa), \
        [pb0] "v"(pb[0]), [pb1] "v"(pb[1]), [oa0] "n"(OA), [oa1] "n"(OA + 4096), [oa2] "n"(OA + 8192),           \
        [oa3] "n"(OA + 12288), [ob0] "n"(OB), [ob1] "n"(OB + 2048)
#define GD_SLICE_BODY                                                                                             \
    "s_nop 1\n\t"                                                                                                 \
    "ds_read_b128 %[an0], %[pa] offset:%[oa0]\n\t"                                                                \
    "v_mfma_f32_32x32x16_bf16 %[c00], %[a0], %[b0], %[c00]\n\t"                                                   \
    "ds_read_b128 %[an1], %[pa] offset:%[oa1]\n\t"                                                                \
    "v_mfma_f32_32x32x16_bf16 %[c01], %[a0], %[b1], %[c01]\n\t"                                                   \
    "ds_read_b128 %[an2], %[pa] offset:%[oa2]\n\t"                                                                \
    "v_mfma_f32_32x32x16_bf16 %[c10], %[a1], %[b0], %[c10]\n\t"                                                   \
    "ds_read_b128 %[an3], %[pa] offset:%[oa3]\n\t"                                                                \
    "v_mfma_f32_32x32x16_bf16 %[c11], %[a1], %[b1], %[c11]\n\t"                                                   \
    "ds_read_b64_tr_b16 %[bl0], %[pb0] offset:%[ob0]\n\t"                                                         \
    "ds_read_b64_tr_b16 %[bh0], %[pb0] offset:%[ob1]\n\t"                                                         \
    "v_mfma_f32_32x32x16_bf16 %[c20], %[a2], %[b0], %[c20]\n\t"                                                   \
    "ds_read_b64_tr_b16 %[bl1], %[pb1] offset:%[ob0]\n\t"                                                         \
    "ds_read_b64_tr_b16 %[bh1], %[pb1] offset:%[ob1]\n\t"                                                         \
    "v_mfma_f32_32x32x16_bf16 %[c21], %[a2], %[b1], %[c21]\n\t"

template <int OA, int OB>
__device__ __forceinline__ void gd_slice(f32x16_t (&c)[4][2], const bf16x8_t (&a)[4], const bf16x8_t (&b)[2],
                                         bf16x8_t (&an)[4], gd_v2i (&bl)[2], gd_v2i (&bh)[2], uint32_t pa,
                                         const uint32_t (&pb)[2])
{
    asm volatile(GD_SLICE_BODY "v_mfma_f32_32x32x16_bf16 %[c30], %[a3], %[b0], %[c30]\n\t"
                               "v_mfma_f32_32x32x16_bf16 %[c31], %[a3], %[b1], %[c31]\n\t"
                               "s_waitcnt lgkmcnt(0)"
                 : GD_SLICE_OUTS
                 : GD_SLICE_INS
                 : "memory");
}

// The last slice: MFMAs only.
__device__ __forceinline__ void gd_slice_last(f32x16_t (&c)[4][2], const bf16x8_t (&a)[4], const bf16x8_t (&b)[2])
{
    asm volatile("s_nop 1\n\t"
                 "v_mfma_f32_32x32x16_bf16 %[c00], %[a0], %[b0], %[c00]\n\t"
                 "v_mfma_f32_32x32x16_bf16 %[c01], %[a0], %[b1], %[c01]\n\t"
                 "v_mfma_f32_32x32x16_bf16 %[c10], %[a1], %[b0], %[c10]\n\t"
                 "v_mfma_f32_32x32x16_bf16 %[c11], %[a1], %[b1], %[c11]\n\t"
                 "v_mfma_f32_32x32x16_bf16 %[c20], %[a2], %[b0], %[c20]\n\t"
                 "v_mfma_f32_32x32x16_bf16 %[c21], %[a2], %[b1], %[c21]\n\t"
                 "v_mfma_f32_32x32x16_bf16 %[c30], %[a3], %[b0], %[c30]\n\t"
                 "v_mfma_f32_32x32x16_bf16 %[c31], %[a3], %[b1], %[c31]\n\t"
                 "s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : [c00] "+a"(c[0][0]), [c01] "+a"(c[0][1]), [c10] "+a"(c[1][0]), [c11] "+a"(c[1][1]),
                   [c20] "+a"(c[2][0]), [c21] "+a"(c[2][1]), [c30] "+a"(c[3][0]), [c31] "+a"(c[3][1])
                 : [a0] "v"(a[0]), [a1] "v"(a[1]), [a2] "v"(a[2]), [a3] "v"(a[3]), [b0] "v"(b[0]), [b1] "v"(b[1])
                 : "memory");
}

// The first slice's fragments (reads only).
__device__ __forceinline__ void gd_read(bf16x8_t (&an)[4], gd_v2i (&bl)[2], gd_v2i (&bh)[2], uint32_t pa,
                                        const uint32_t (&pb)[2])
{
    asm volatile("ds_read_b128 %[an0], %[pa]\n\t"
                 "ds_read_b128 %[an1], %[pa] offset:4096\n\t"
                 "ds_read_b128 %[an2], %[pa] offset:8192\n\t"
                 "ds_read_b128 %[an3], %[pa] offset:12288\n\t"
                 "ds_read_b64_tr_b16 %[bl0], %[pb0]\n\t"
                 "ds_read_b64_tr_b16 %[bh0], %[pb0] offset:2048\n\t"
                 "ds_read_b64_tr_b16 %[bl1], %[pb1]\n\t"
                 "ds_read_b64_tr_b16 %[bh1], %[pb1] offset:2048\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : [an0] "=&v"(an[0]), [an1] "=&v"(an[1]), [an2] "=&v"(an[2]), [an3] "=&v"(an[3]),
                   [bl0] "=&v"(bl[0]), [bh0] "=&v"(bh[0]), [bl1] "=&v"(bl[1]), [bh1] "=&v"(bh[1])
                 : [pa] "v"(pa), [pb0] "v"(pb[0]), [pb1] "v"(pb[1])
                 : "memory");
}

__device__ __forceinline__ bf16x8_t gd_cat(gd_v2i lo, gd_v2i hi)
{
    const gd_v4i v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
    return __builtin_bit_cast(bf16x8_t, v);
}

// Wait until at most n vector-memory operations of this wave are outstanding
// (n is one of the counts the pipeline below uses).
__device__ __forceinline__ void gd_wait_vm(int n)
{
    switch (n) {
    case 27: asm volatile("s_waitcnt vmcnt(27)" ::: "memory"); break;
    case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}

// The 16 kept-row indices of a k step from this wave's LDS slot (words 0..15 at
// pj, the same address in every lane).
__device__ __forceinline__ void gd_read_idx(gd_v4i (&jv)[4], uint32_t pj)
{
    asm volatile("ds_read_b128 %[j0], %[pj]\n\t"
                 "ds_read_b128 %[j1], %[pj] offset:16\n\t"
                 "ds_read_b128 %[j2], %[pj] offset:32\n\t"
                 "ds_read_b128 %[j3], %[pj] offset:48\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : [j0] "=&v"(jv[0]), [j1] "=&v"(jv[1]), [j2] "=&v"(jv[2]), [j3] "=&v"(jv[3])
                 : [pj] "v"(pj)
                 : "memory");
}

// 8 waves: waves 0-3 compute (LDS fragment reads and MFMAs only), waves 4-7
// issue the loads and wait for them.  A consumer and a producer share each
// SIMD, so a producer stalled on a full load queue leaves the SIMD to the
// consumer's MFMAs.  One barrier per k step joins the two halves: the
// producers arrive once step s + 1 has landed, the consumers once they have
// read all of step s; after it the consumers read step s + 1 and the producers
// refill step s's stage with step s + 3.
template <bool DENSE>
__global__ __launch_bounds__(512) void gemm_dma_kernel(const uint16_t *__restrict__ A, int64_t lda, int T, int tile,
                                                       int mblocks, int nblocks, const uint16_t *__restrict__ wt,
                                                       int64_t ldw, int M, const int32_t *__restrict__ idx, int k,
                                                       int ksteps, float *__restrict__ y, int64_t ldy)
{
    extern __shared__ __attribute__((aligned(1024))) uint8_t gd_lds[];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x / WAVE);
    const int w = wv & 3; // index within the wave's role
    // Workgroup i runs on XCD i % 8, which gets a contiguous run of lin.  With
    // kept rows the run covers whole row blocks with all their column blocks
    // (the two row blocks of a tile share its kept W^T rows, all column blocks
    // share the activations); dense, it covers whole column blocks with all
    // their row blocks (W^T is the larger operand, read once per XCD).
    int lin = blockIdx.x;
    if ((gridDim.x & 7) == 0)
        lin = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const int nrb = (int)(gridDim.x / nblocks);
    const int nb = DENSE ? lin / nrb : lin % nblocks, rb = DENSE ? lin % nrb : lin / nblocks;
    const int tau = rb / mblocks, mm = rb % mblocks;
    const int row0 = tau * tile + mm * GD_M;
    const int rowend = min(T, tau * tile + tile);
    if (row0 >= rowend)
        return; // the tile's rows end before this block (uniform: before any barrier)
    const int n0 = nb * GD_N;
    const uint32_t lbase = (uint32_t)(uintptr_t)gd_lds;

    if (wv >= 4) {
        // ================================================================ producer
        const int32_t *J = DENSE ? nullptr : idx + (int64_t)tau * k;
        const int klim = DENSE ? ksteps * GD_K : k;
        // A instruction i of wave w fills rows r = 8(4w + i) + lane/8; lane's chunk (lane & 7) holds chunk (lane & 7) ^ gd_aswz(r)
        const uint16_t *pA[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = min(row0 + (4 * w + i) * 8 + (lane >> 3), rowend - 1);
            pA[i] = A + (int64_t)r * lda + (((lane & 7) ^ gd_aswz((4 * w + i) * 8 + (lane >> 3))) * 8);
        }
        // B instruction i of wave w fills rows q = 16w + 2i + lane/32; q & 3 = 2(i & 1) + lane/32
        const int mlast = (M - 1) / 8 * 8;
        int colB[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int c = (lane & 31) ^ (4 * (2 * p + (lane >> 5)));
            colB[p] = min(n0 + 8 * c, mlast);
        }
        // Rows of a k step: a DMA instruction i of wave w fills rows 16w + 2i (lanes
        // 0-31) and 16w + 2i + 1 (lanes 32-63); rr[q] is the W^T row of row 16w + q.
        auto issue = [&](int t, int st, const int (&rr)[16]) {
            const int kk = t * GD_K;
            uint8_t *la = gd_lds + st * GD_A_STAGE + w * 4 * 1024;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_global_load_lds(pA[i] + kk, la + i * 1024, 16, 0, 0);
            uint8_t *lb = gd_lds + GD_B_BASE + st * GD_B_STAGE + w * 8 * 1024;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = (lane >> 5) ? rr[2 * i + 1] : rr[2 * i];
                __builtin_amdgcn_global_load_lds(wt + (int64_t)row * ldw + colB[i & 1], lb + i * 1024, 16, 0, 0);
            }
        };
        auto dense_rows = [&](int t, int (&rr)[16]) {
#pragma unroll
            for (int q = 0; q < 16; ++q)
                rr[q] = min(t * GD_K + 16 * w + q, klim - 1);
        };
        // the kept-row indices of k step t go to LDS slot t % 3 of this wave (lane l: row 16w + l % 16)
        auto issue_idx = [&](int t) {
            if (!DENSE)
                __builtin_amdgcn_global_load_lds(J + min(t * GD_K + 16 * w + (lane & 15), klim - 1),
                                                 gd_lds + GD_J_BASE + ((t % 3) * 4 + w) * 256, 4, 0, 0);
        };
        constexpr int PER_STEP = DENSE ? 12 : 13; // vector-memory operations issued per k step

        // prologue: k steps 0..2 in flight; the indices of step t + 3 travel with step t
        {
            int jr[3] = {0, 0, 0};
            if (!DENSE)
#pragma unroll
                for (int t = 0; t < 3; ++t)
                    jr[t] = J[min(t * GD_K + 16 * w + (lane & 15), klim - 1)];
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                if (t > 0 && t >= ksteps)
                    break;
                int rr[16];
                if (DENSE)
                    dense_rows(t, rr);
                else
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        rr[q] = __builtin_amdgcn_readlane(jr[t], q);
                issue(t, t, rr);
                issue_idx(t + 3);
            }
        }
        // step 0 has landed: the operations issued after it may be outstanding
        gd_wait_vm((PER_STEP - 12) + PER_STEP * (min(ksteps, 3) - 1));
        __builtin_amdgcn_s_barrier();
        const uint32_t pj = lbase + GD_J_BASE + w * 256;
        int st = 0;
        for (int s = 0; s + 1 < ksteps; ++s) {
            // step s + 1 has landed (this wave's loads; the barrier covers the other producers')
            gd_wait_vm((PER_STEP - 12) + (s + 2 < ksteps ? PER_STEP : 0));
            __builtin_amdgcn_s_barrier();
            if (s + 3 < ksteps) {
                int rr[16];
                if (DENSE) {
                    dense_rows(s + 3, rr);
                } else {
                    gd_v4i jv[4];
                    gd_read_idx(jv, pj + st * 4 * 256);
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        rr[q] = jv[q >> 2][q & 3];
                }
                issue(s + 3, st, rr);
                issue_idx(s + 6);
            }
            st = st == 2 ? 0 : st + 1;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); // no load may land after the wave ends
        return;
    }

    // ==================================================================== consumer
    // fragment read addresses: wave w computes all 128 rows x columns 64w .. 64w + 63
    uint32_t pa[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        pa[j] = lbase + (lane & 31) * 128 + (((2 * j + (lane >> 5)) ^ gd_aswz(lane & 31)) * 16);
    const int g = lane >> 4, i16 = lane & 15, trow = 8 * (g >> 1) + (i16 >> 2);
    uint32_t pb[2];
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
        const int c = (w * 8 + jn * 4 + 2 * (g & 1) + ((i16 & 3) >> 1)) ^ (4 * (trow & 3));
        pb[jn] = lbase + GD_B_BASE + trow * 512 + c * 16 + 8 * (i16 & 1);
    }

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][jn][r] = 0.0f;

    __builtin_amdgcn_s_barrier(); // step 0 has landed
    bf16x8_t a[4], b[2], an[4];
    gd_v2i bl[2], bh[2];
    gd_read(an, bl, bh, pa[0], pb);
    auto next = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = an[i];
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
            b[jn] = gd_cat(bl[jn], bh[jn]);
    };
    next();
    // The k steps that have a successor.  Stage addresses are offset at run time
    // (a few adds per step) so that the loop body is one block of code.
    int s = 0, st = 0;
    for (; s + 1 < ksteps; ++s) {
        const int sn = st == 2 ? 0 : st + 1;
        uint32_t pl[4], pbl[2];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            pl[j] = pa[j] + st * GD_A_STAGE;
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
            pbl[jn] = pb[jn] + st * GD_B_STAGE;
        gd_slice<0, 1 * 8192>(acc, a, b, an, bl, bh, pl[1], pbl);
        next();
        gd_slice<0, 2 * 8192>(acc, a, b, an, bl, bh, pl[2], pbl);
        next();
        gd_slice<0, 3 * 8192>(acc, a, b, an, bl, bh, pl[3], pbl);
        next();
        // all of stage st is read (the producers may refill it); step s + 1 has landed after this
        __builtin_amdgcn_s_barrier();
        const uint32_t pn = pa[0] + sn * GD_A_STAGE;
        uint32_t pbn[2];
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
            pbn[jn] = pb[jn] + sn * GD_B_STAGE;
        gd_slice<0, 0>(acc, a, b, an, bl, bh, pn, pbn);
        next();
        st = sn;
    }
    {
        // the last k step
        uint32_t pl[4], pbl[2];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            pl[j] = pa[j] + st * GD_A_STAGE;
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
            pbl[jn] = pb[jn] + st * GD_B_STAGE;
        gd_slice<0, 1 * 8192>(acc, a, b, an, bl, bh, pl[1], pbl);
        next();
        gd_slice<0, 2 * 8192>(acc, a, b, an, bl, bh, pl[2], pbl);
        next();
        gd_slice<0, 3 * 8192>(acc, a, b, an, bl, bh, pl[3], pbl);
        next();
        gd_slice_last(acc, a, b);
    }

    // D layout of a 32x32 MFMA: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) {
            const int col = n0 + w * 64 + jn * 32 + (lane & 31);
            if (col >= M)
                continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < rowend)
                    y[(int64_t)row * ldy + col] = acc[i][jn][r];
            }
        }
}

size_t gemm_ws_bytes(int64_t T, int64_t k)
{
    const int64_t kpad = (k + GB_K - 1) / GB_K * GB_K;
    return (size_t)(T * kpad) * sizeof(uint16_t);
}

hipError_t launch_gemm(const void *x, int64_t T, int64_t K, int64_t ldx, const void *wt, int64_t ldw, int64_t M,
                       const int32_t *idx, int64_t k, int64_t tile, bool dense, float *y, int64_t ldy, void *xg,
                       hipStream_t st)
{
    const int64_t rows = tile < T ? tile : T;
    const int64_t ntiles = (T + tile - 1) / tile;
    if (dense && K % GD_K != 0) {
        // partial last k step: the register-staged kernel zero-fills it
        const int mblocks = (int)((rows + GB_M - 1) / GB_M);
        dim3 grid((unsigned)((M + GB_N - 1) / GB_N), (unsigned)(ntiles * mblocks));
        gemm_kernel<<<grid, GEMM_THREADS, 0, st>>>((const uint16_t *)x, ldx, (int)T, (int)tile, mblocks,
                                                   (const uint16_t *)wt, ldw, (int)M, (int)K, y, ldy);
        return hipGetLastError();
    }
    const int mblocks = (int)((rows + GD_M - 1) / GD_M);
    const int nblocks = (int)((M + GD_N - 1) / GD_N);
    const unsigned grid = (unsigned)(ntiles * mblocks * nblocks);
    if (dense) {
        gemm_dma_kernel<true><<<grid, 512, GD_LDS, st>>>((const uint16_t *)x, ldx, (int)T, (int)tile, mblocks, nblocks,
                                                         (const uint16_t *)wt, ldw, (int)M, nullptr, (int)K,
                                                         (int)(K / GD_K), y, ldy);
        return hipGetLastError();
    }
    const int64_t kpad = (k + GB_K - 1) / GB_K * GB_K;
    const GatherPlan g = gather_plan(T, K, k, tile);
    const unsigned ggrid = (unsigned)((int64_t)g.ntiles * g.groups_per_tile);
#define RMM_GATHER(STG, CH)                                                                                          \
    gather_kernel<STG, CH><<<ggrid, 256, STG ? g.lds : 0, st>>>((const uint16_t *)x, ldx, (int)T, (int)K, (int)tile, \
                                                               idx, (int)k, (int)kpad, g.rows, g.groups_per_tile,   \
                                                               (uint16_t *)xg)
    if (g.stage) {
        if (g.ch == 1)
            RMM_GATHER(true, 1);
        else if (g.ch == 2)
            RMM_GATHER(true, 2);
        else
            RMM_GATHER(true, 4);
    } else {
        RMM_GATHER(false, 4);
    }
#undef RMM_GATHER
    gemm_dma_kernel<false><<<grid, 512, GD_LDS, st>>>((const uint16_t *)xg, kpad, (int)T, (int)tile, mblocks, nblocks,
                                                      (const uint16_t *)wt, ldw, (int)M, idx, (int)k,
                                                      (int)(kpad / GD_K), y, ldy);
    return hipGetLastError();
}

void linear_init()
{
    (void)hipFuncSetAttribute((const void *)gather_kernel<true, 1>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              GATHER_LDS_MAX_K * 2);
    (void)hipFuncSetAttribute((const void *)gather_kernel<true, 2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              GATHER_LDS_MAX_K * 2);
    (void)hipFuncSetAttribute((const void *)gather_kernel<true, 4>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              GATHER_LDS_MAX_K * 2);
    (void)hipFuncSetAttribute((const void *)gemm_dma_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              GD_LDS);
    (void)hipFuncSetAttribute((const void *)gemm_dma_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              GD_LDS);
}

} // namespace rmm
