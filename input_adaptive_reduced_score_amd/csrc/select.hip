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

namespace rmm {

constexpr int SEL_THREADS = 1024;
constexpr int COLMAX_THREADS = 256;

// Partial column maxima of |x| over row chunks of a tile.
// grid: (ntiles * nrsplit, ceil(K / (64*VEC))); block 256 = 4 waves.
// pmax[(tau*nrsplit + rs)*K + j] = max |x[t,j]| over rows t of chunk rs of tile tau.
template <typename TE>
__global__ __launch_bounds__(COLMAX_THREADS) void colmax_kernel(const TE *__restrict__ x, int64_t ldx, int T, int K,
                                                                int tile, int rows_per_chunk, int nrsplit,
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
        int t = r0 + w;
        // four rows in flight per wave
        for (; t + 3 * 4 < r1; t += 16) {
            uint4 u[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                u[q] = Vec16<TE>::raw(x + (int64_t)(t + 4 * q) * ldx + col);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[VEC];
                Vec16<TE>::unpack(u[q], v);
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    m[e] = fmaxf(m[e], fabsf(v[e]));
            }
        }
        for (; t < r1; t += 4) {
            float v[VEC];
            Vec16<TE>::unpack(Vec16<TE>::raw(x + (int64_t)t * ldx + col), v);
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                m[e] = fmaxf(m[e], fabsf(v[e]));
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        red[w][lane * VEC + e] = m[e];
    __syncthreads();
    float *out = pmax + ((int64_t)tau * nrsplit + rs) * K + (int64_t)blockIdx.y * WAVE * VEC;
    for (int i = threadIdx.x; i < WAVE * VEC; i += COLMAX_THREADS) {
        float a = fmaxf(fmaxf(red[0][i], red[1][i]), fmaxf(red[2][i], red[3][i]));
        if ((int64_t)blockIdx.y * WAVE * VEC + i < K)
            out[i] = a;
    }
}

// Scorer + selector, one workgroup per tile.  direct: score straight from x
// (few rows per tile); otherwise from the column-max partials.
template <typename TE>
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(const TE *__restrict__ x, int64_t ldx, int T, int K,
                                                             int tile, const float *__restrict__ c,
                                                             const float *__restrict__ pmax, int nrsplit, int direct,
                                                             int k, int32_t *__restrict__ idx)
{
    extern __shared__ uint32_t sm[];
    uint32_t *keys = sm;
    uint32_t *hist = sm + ((K + 3) & ~3);
    uint32_t *tmp = hist + SEL_BINS;
    const int tau = blockIdx.x;

    if (direct) {
        const int t0 = tau * tile, t1 = min(T, t0 + tile);
        for (int j = threadIdx.x; j < K; j += SEL_THREADS) {
            float a = 0.0f;
            for (int t = t0; t < t1; ++t)
                a = fmaxf(a, fabsf(ld_elem(x, (int64_t)t * ldx + j)));
            keys[j] = nonneg_key(__fmul_rn(a, c[j]));
        }
    } else {
        const float *pm = pmax + (int64_t)tau * nrsplit * K;
        for (int j = threadIdx.x; j < K; j += SEL_THREADS) {
            float a = 0.0f;
            for (int rs = 0; rs < nrsplit; ++rs)
                a = fmaxf(a, pm[(int64_t)rs * K + j]);
            keys[j] = nonneg_key(__fmul_rn(a, c[j]));
        }
    }
    __syncthreads();

    uint32_t prefix = 0, pmask = 0, krem = (uint32_t)k;
    radix_pass(keys, K, prefix, pmask, 21, 11, krem, hist, tmp);
    radix_pass(keys, K, prefix, pmask, 10, 11, krem, hist, tmp);
    radix_pass(keys, K, prefix, pmask, 0, 10, krem, hist, tmp);
    compact_ascending(keys, K, prefix, krem, idx + (int64_t)tau * k, tmp);
}

size_t select_lds_bytes(int64_t K) { return (size_t)(((K + 3) & ~3) + SEL_BINS + 64) * 4; }

hipError_t launch_select(const void *x, bool bf16, int64_t T, int64_t K, int64_t ldx, const float *c, int64_t tile,
                         int64_t k, int32_t *idx, float *pmax_ws, hipStream_t st)
{
    const int ntiles = (int)((T + tile - 1) / tile);
    const int rows = (int)(tile < T ? tile : T);
    const bool direct = rows <= SELECT_DIRECT_ROWS;
    int nrsplit = 1, rpc = rows;
    if (!direct) {
        const int vec = bf16 ? 8 : 4;
        rpc = COLMAX_ROWS;
        nrsplit = (rows + rpc - 1) / rpc;
        dim3 grid(ntiles * nrsplit, (unsigned)((K + WAVE * vec - 1) / (WAVE * vec)));
        if (bf16)
            colmax_kernel<uint16_t><<<grid, COLMAX_THREADS, 0, st>>>((const uint16_t *)x, ldx, (int)T, (int)K,
                                                                      (int)tile, rpc, nrsplit, pmax_ws);
        else
            colmax_kernel<float><<<grid, COLMAX_THREADS, 0, st>>>((const float *)x, ldx, (int)T, (int)K, (int)tile,
                                                                   rpc, nrsplit, pmax_ws);
    }
    const size_t lds = select_lds_bytes(K);
    if (bf16)
        select_kernel<uint16_t><<<ntiles, SEL_THREADS, lds, st>>>((const uint16_t *)x, ldx, (int)T, (int)K, (int)tile,
                                                                  c, pmax_ws, nrsplit, direct, (int)k, idx);
    else
        select_kernel<float><<<ntiles, SEL_THREADS, lds, st>>>((const float *)x, ldx, (int)T, (int)K, (int)tile, c,
                                                               pmax_ws, nrsplit, direct, (int)k, idx);
    return hipGetLastError();
}

size_t select_ws_bytes(int64_t T, int64_t K, int64_t tile)
{
    const int64_t ntiles = (T + tile - 1) / tile;
    const int64_t rows = tile < T ? tile : T;
    if (rows <= SELECT_DIRECT_ROWS)
        return 0;
    const int64_t nrsplit = (rows + COLMAX_ROWS - 1) / COLMAX_ROWS;
    return (size_t)(ntiles * nrsplit * K) * sizeof(float);
}

void select_init()
{
    (void)hipFuncSetAttribute((const void *)select_kernel<uint16_t>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)select_lds_bytes(SELECT_MAX_K));
    (void)hipFuncSetAttribute((const void *)select_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)select_lds_bytes(SELECT_MAX_K));
}

} // namespace rmm
