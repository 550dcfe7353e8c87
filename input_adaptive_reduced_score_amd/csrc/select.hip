// Scorer + top-k selector for the linear path.
//
// Scorer (blog on input-adaptive matrix-product reduction, section 5.1: a cheap
// gate rates every slice from the current input):
//     s[j] = fl32( max_{t in tile} |x[t,j]| * c[j] )
// Selector (section 5.2 top-k; section 6.1 keeps the top-k indices in ascending
// order): radix select of the k-th largest score key over LDS-resident keys,
// then an order-preserving compaction.  Ties go to the lower index.
//
// One workgroup of 1024 threads owns one token tile and all K keys of it
// (K <= 32768 keys of 4 bytes in LDS).  For tiles of many tokens a separate
// column-max kernel first reduces the tile's rows in parallel across the chip.
#include "device.h"
#include "kernels.h"
#include "radix.h"
#include "select_body.h"

namespace rmm {

// Partial column maxima of |x| over row chunks of a tile.
// grid: (ntiles * nrsplit, ceil(K / (64*VEC))); block 256 = 4 waves.
// pmax[(tau*nrsplit + rs)*Kp + j] = max |x[t,j]| over rows t of chunk rs of tile tau.
template <typename TE>
__global__ __launch_bounds__(COLMAX_THREADS) void colmax_kernel(const TE *__restrict__ x, int64_t ldx, int T, int K,
                                                                int tile, int rows_per_chunk, int nrsplit, int Kp,
                                                                float *__restrict__ pmax)
{
    constexpr int VEC = Vec16<TE>::N;
    __shared__ float red[COLMAX_THREADS / WAVE][WAVE * VEC];
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    const int tau = blockIdx.x / nrsplit, rs = blockIdx.x % nrsplit;
    const int col = (blockIdx.y * WAVE + lane) * VEC;
    const int t_end = min(T, (tau + 1) * tile);
    const int r0 = tau * tile + rs * rows_per_chunk;
    const int r1 = min(t_end, r0 + rows_per_chunk);
    float m[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        m[e] = 0.0f;
    if (col < K) {
        // wave w takes rows r0 + w + 4q; all of them are in flight at once (a
        // chunk holds COLMAX_ROWS rows, so q < COLMAX_ROWS / 4).  Rows past the
        // chunk's end repeat its last row, which leaves the maximum unchanged.
        constexpr int NQ = COLMAX_ROWS / 4;
        uint4 u[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            u[q] = Vec16<TE>::raw(x + (int64_t)min(r0 + w + 4 * q, r1 - 1) * ldx + col);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            float v[VEC];
            Vec16<TE>::unpack(u[q], v);
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                m[e] = fmaxf(m[e], fabsf(v[e]));
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        red[w][lane * VEC + e] = m[e];
    __syncthreads();
    float *out = pmax + ((int64_t)tau * nrsplit + rs) * Kp + (int64_t)blockIdx.y * WAVE * VEC;
    for (int i = threadIdx.x; i < WAVE * VEC; i += COLMAX_THREADS) {
        float a = fmaxf(fmaxf(red[0][i], red[1][i]), fmaxf(red[2][i], red[3][i]));
        if ((int64_t)blockIdx.y * WAVE * VEC + i < K)
            out[i] = a;
    }
}

template <typename TE, int PER>
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(const TE *__restrict__ x, int64_t ldx, int T, int K,
                                                             int tile, const float *__restrict__ c,
                                                             const float *__restrict__ pmax, int Kp, int nrsplit,
                                                             int direct, int cvec, int k, int32_t *__restrict__ idx)
{
    select_body<TE, PER, false>(x, ldx, T, K, tile, c, pmax, Kp, nrsplit, direct, cvec, k, (int)blockIdx.x, idx,
                                SelPub{});
}

// Block-granular variant (blog section 5.1 block-mean |h| importance, 5.2
// block top-k with the mask expanded to slice indices, 6.1 demo code): block b
// of `block` consecutive slices scores mean_{j in b} max_{t in tile} |x[t,j]|,
// summed in ascending slice order in double and divided once; the nk best
// blocks (ties to the lower block) are listed in ascending order, expanded to
// their slices.  One workgroup of 1024 threads per tile, one thread per block.
template <typename TE>
__global__ __launch_bounds__(SEL_THREADS) void select_blocks_kernel(const TE *__restrict__ x, int64_t ldx, int T,
                                                                    int K, int tile, const float *__restrict__ pmax,
                                                                    int Kp, int nrsplit, int direct, int block,
                                                                    int nb, int nk, int32_t *__restrict__ idx)
{
    constexpr int NW = SEL_THREADS / WAVE;
    extern __shared__ float mj[]; // K column maxima of the tile
    __shared__ double bs[SEL_THREADS];
    __shared__ uint32_t wk[NW];
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE, tau = blockIdx.x;
    // 1. column maxima (coalesced over j)
    if (direct) {
        const int t0 = tau * tile, t1 = min(T, t0 + tile);
        for (int j = tid; j < K; j += SEL_THREADS) {
            float a = 0.0f;
            for (int t = t0; t < t1; ++t)
                a = fmaxf(a, fabsf(ld_elem(x, (int64_t)t * ldx + j)));
            mj[j] = a;
        }
    } else {
        const float *pm = pmax + (int64_t)tau * nrsplit * Kp;
        for (int j = tid; j < K; j += SEL_THREADS) {
            float a = 0.0f;
            for (int rs = 0; rs < nrsplit; ++rs)
                a = fmaxf(a, pm[(int64_t)rs * Kp + j]);
            mj[j] = a;
        }
    }
    __syncthreads();
    // 2. block means
    if (tid < nb) {
        double sum = 0.0;
        for (int e = 0; e < block; ++e)
            sum += (double)mj[tid * block + e];
        bs[tid] = sum / (double)block;
    }
    __syncthreads();
    // 3. rank by counting: blocks with a larger mean, or an equal mean at a lower index
    uint32_t keep = 0;
    if (tid < nb) {
        const double me = bs[tid];
        uint32_t a0 = 0, a1 = 0;
        int o = 0;
        for (; o + 1 < nb; o += 2) {
            const double v0 = bs[o], v1 = bs[o + 1];
            a0 += (v0 > me) || (v0 == me && o < tid);
            a1 += (v1 > me) || (v1 == me && o + 1 < tid);
        }
        if (o < nb) {
            const double v0 = bs[o];
            a0 += (v0 > me) || (v0 == me && o < tid);
        }
        keep = a0 + a1 < (uint32_t)nk;
    }
    // 4. position among the kept blocks (ascending block order)
    const uint32_t incl = wave_incl_sum(keep);
    if (lane == WAVE - 1)
        wk[w] = incl;
    __syncthreads();
    uint32_t pos = incl - keep;
#pragma unroll
    for (int v = 0; v < NW; ++v)
        pos += v < w ? wk[v] : 0u;
    // 5. expanded slice indices
    if (keep && pos < (uint32_t)nk) {
        int32_t *dst = idx + ((int64_t)tau * nk + pos) * block;
        for (int e = 0; e < block; ++e)
            dst[e] = tid * block + e;
    }
}

hipError_t launch_select_blocks(const void *x, bool bf16, int64_t T, int64_t K, int64_t ldx, int64_t tile,
                                int64_t block, int64_t nk, int32_t *idx, float *pmax_ws, hipStream_t st)
{
    const int ntiles = (int)((T + tile - 1) / tile);
    const int rows = (int)(tile < T ? tile : T);
    const bool direct = rows <= SELECT_DIRECT_ROWS;
    const int Kp = (int)((K + 7) / 8 * 8);
    int nrsplit = 1;
    if (!direct) {
        const int vec = bf16 ? 8 : 4;
        nrsplit = (rows + COLMAX_ROWS - 1) / COLMAX_ROWS;
        dim3 grid(ntiles * nrsplit, (unsigned)((K + WAVE * vec - 1) / (WAVE * vec)));
        if (bf16)
            colmax_kernel<uint16_t><<<grid, COLMAX_THREADS, 0, st>>>((const uint16_t *)x, ldx, (int)T, (int)K,
                                                                      (int)tile, COLMAX_ROWS, nrsplit, Kp, pmax_ws);
        else
            colmax_kernel<float><<<grid, COLMAX_THREADS, 0, st>>>((const float *)x, ldx, (int)T, (int)K, (int)tile,
                                                                   COLMAX_ROWS, nrsplit, Kp, pmax_ws);
    }
    const size_t lds = (size_t)K * sizeof(float);
    const int nb = (int)(K / block);
    if (bf16)
        select_blocks_kernel<uint16_t><<<ntiles, SEL_THREADS, lds, st>>>(
            (const uint16_t *)x, ldx, (int)T, (int)K, (int)tile, pmax_ws, Kp, nrsplit, direct, (int)block, nb,
            (int)nk, idx);
    else
        select_blocks_kernel<float><<<ntiles, SEL_THREADS, lds, st>>>((const float *)x, ldx, (int)T, (int)K,
                                                                       (int)tile, pmax_ws, Kp, nrsplit, direct,
                                                                       (int)block, nb, (int)nk, idx);
    return hipGetLastError();
}

static int per_for(int64_t K)
{
    return K <= 4 * SEL_THREADS ? 4 : K <= 8 * SEL_THREADS ? 8 : K <= 16 * SEL_THREADS ? 16 : 32;
}
int select_per_for(int64_t K) { return per_for(K); }

static int64_t pad8(int64_t n) { return (n + 7) / 8 * 8; }

hipError_t launch_select(const void *x, bool bf16, int64_t T, int64_t K, int64_t ldx, const float *c, int64_t tile,
                         int64_t k, int32_t *idx, float *pmax_ws, hipStream_t st)
{
    const int ntiles = (int)((T + tile - 1) / tile);
    const int rows = (int)(tile < T ? tile : T);
    const bool direct = rows <= SELECT_DIRECT_ROWS;
    const int cvec = ((uintptr_t)c & 15u) == 0u;
    const int Kp = (int)pad8(K);
    int nrsplit = 1;
    if (!direct) {
        const int vec = bf16 ? 8 : 4;
        nrsplit = (rows + COLMAX_ROWS - 1) / COLMAX_ROWS;
        dim3 grid(ntiles * nrsplit, (unsigned)((K + WAVE * vec - 1) / (WAVE * vec)));
        if (bf16)
            colmax_kernel<uint16_t><<<grid, COLMAX_THREADS, 0, st>>>((const uint16_t *)x, ldx, (int)T, (int)K,
                                                                      (int)tile, COLMAX_ROWS, nrsplit, Kp, pmax_ws);
        else
            colmax_kernel<float><<<grid, COLMAX_THREADS, 0, st>>>((const float *)x, ldx, (int)T, (int)K, (int)tile,
                                                                   COLMAX_ROWS, nrsplit, Kp, pmax_ws);
    }
    const size_t lds = (size_t)(k + 3) / 4 * 16;
#define RMM_SEL_LAUNCH(PER)                                                                                        \
    do {                                                                                                           \
        if (bf16)                                                                                                  \
            select_kernel<uint16_t, PER><<<ntiles, SEL_THREADS, lds, st>>>(                                         \
                (const uint16_t *)x, ldx, (int)T, (int)K, (int)tile, c, pmax_ws, Kp, nrsplit, direct, cvec, (int)k, \
                idx);                                                                                              \
        else                                                                                                       \
            select_kernel<float, PER><<<ntiles, SEL_THREADS, lds, st>>>(                                            \
                (const float *)x, ldx, (int)T, (int)K, (int)tile, c, pmax_ws, Kp, nrsplit, direct, cvec, (int)k,   \
                idx);                                                                                              \
    } while (0)
    switch (per_for(K)) {
    case 4:
        RMM_SEL_LAUNCH(4);
        break;
    case 8:
        RMM_SEL_LAUNCH(8);
        break;
    case 16:
        RMM_SEL_LAUNCH(16);
        break;
    default:
        RMM_SEL_LAUNCH(32);
        break;
    }
#undef RMM_SEL_LAUNCH
    return hipGetLastError();
}

size_t select_ws_bytes(int64_t T, int64_t K, int64_t tile)
{
    const int64_t ntiles = (T + tile - 1) / tile;
    const int64_t rows = tile < T ? tile : T;
    if (rows <= SELECT_DIRECT_ROWS)
        return 0;
    const int64_t nrsplit = (rows + COLMAX_ROWS - 1) / COLMAX_ROWS;
    return (size_t)(ntiles * nrsplit * pad8(K)) * sizeof(float);
}

void select_init()
{
    const int lds = SELECT_MAX_K * 4;
    (void)hipFuncSetAttribute((const void *)select_kernel<uint16_t, 4>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute((const void *)select_kernel<float, 4>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute((const void *)select_kernel<uint16_t, 8>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute((const void *)select_kernel<float, 8>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute((const void *)select_kernel<uint16_t, 16>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute((const void *)select_kernel<float, 16>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute((const void *)select_kernel<uint16_t, 32>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute((const void *)select_kernel<float, 32>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute((const void *)select_blocks_kernel<uint16_t>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              SELECT_MAX_K * (int)sizeof(float));
    (void)hipFuncSetAttribute((const void *)select_blocks_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              SELECT_MAX_K * (int)sizeof(float));
}

} // namespace rmm
