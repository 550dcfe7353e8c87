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
    float *out = pmax + ((int64_t)tau * nrsplit + rs) * Kp + (int64_t)blockIdx.y * WAVE * VEC;
    for (int i = threadIdx.x; i < WAVE * VEC; i += COLMAX_THREADS) {
        float a = fmaxf(fmaxf(red[0][i], red[1][i]), fmaxf(red[2][i], red[3][i]));
        if ((int64_t)blockIdx.y * WAVE * VEC + i < K)
            out[i] = a;
    }
}

// Histogram bins are stored with one pad word per 32 bins so that wave 0,
// whose lane l reads 32 consecutive bins, touches distinct LDS banks.
__device__ __forceinline__ int hpad(int b) { return b + (b >> 5); }
constexpr int SEL_HIST_WORDS = SEL_BINS + SEL_BINS / 32;

// Wave 0 finds the digit holding the krem-th largest key (lane l covers bins
// 2047-32l down to 2016-32l), clears the histogram and publishes
// (digit, rank inside the digit) in res[0..1].
__device__ __forceinline__ void wave0_crossing(uint32_t *hist, uint32_t krem, uint32_t *res)
{
    const int lane = threadIdx.x & (WAVE - 1);
    uint32_t h[32];
    const int top = SEL_BINS - 1 - 32 * lane;
    uint32_t tot = 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        h[e] = hist[hpad(top - e)];
        tot += h[e];
    }
#pragma unroll
    for (int e = 0; e < 32; ++e)
        hist[hpad(top - e)] = 0;
    const uint32_t incl = wave_incl_sum(tot);
    uint32_t run = incl - tot;
    if (run < krem && krem <= incl) {
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            if (run < krem && krem <= run + h[e]) {
                res[0] = (uint32_t)(top - e);
                res[1] = krem - run;
            }
            run += h[e];
        }
    }
}

// Scorer + selector, one workgroup of 1024 threads (16 waves) per tile.
// Wave w owns the contiguous block of slices [w*BW, (w+1)*BW); lane l handles
// slices w*BW + 64*i + l (coalesced loads); keys live in LDS at their slice
// index.  Keys are re-based as u = key - (smallest non-zero key) + 1 (0 stays
// 0), an order-preserving map, so the first radix digit spans the keys' actual
// range instead of the few float exponents they share.  The kept list is
// written in ascending order by per-wave ballots after one exchange of wave
// totals.  direct: score straight from x (few rows per tile); otherwise from
// the column-max partials (row pitch Kp).
template <typename TE, int PER>
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(const TE *__restrict__ x, int64_t ldx, int T, int K,
                                                             int tile, const float *__restrict__ c,
                                                             const float *__restrict__ pmax, int Kp, int nrsplit,
                                                             int direct, int k, int32_t *__restrict__ idx)
{
    constexpr int NW = SEL_THREADS / WAVE;
    constexpr int LB = PER < 16 ? PER : 16; // loads in flight per lane per batch
    extern __shared__ uint32_t kl[];        // keys, then re-based keys, at slice index
    __shared__ uint32_t hist[SEL_HIST_WORDS];
    __shared__ uint32_t wmin[NW], wmax[NW], wgt[NW], weq[NW];
    __shared__ uint32_t res[2];
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE, tau = blockIdx.x;
    const int jb = w * (PER * WAVE) + lane; // slice of element i: jb + 64*i

    for (int i = tid; i < SEL_HIST_WORDS; i += SEL_THREADS)
        hist[i] = 0;
    if (tid == 0) {
        res[0] = 0;
        res[1] = 1;
    }

    // 1. scores -> keys, in batches of LB loads per lane
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int i0 = 0; i0 < PER; i0 += LB) {
        float a[LB];
#pragma unroll
        for (int i = 0; i < LB; ++i)
            a[i] = 0.0f;
        if (direct) {
            const int t0 = tau * tile, t1 = min(T, t0 + tile);
            for (int t = t0; t < t1; ++t) {
                const TE *xr = x + (int64_t)t * ldx;
                float f[LB];
#pragma unroll
                for (int i = 0; i < LB; ++i) {
                    const int j = jb + 64 * (i0 + i);
                    f[i] = j < K ? ld_elem(xr, j) : 0.0f;
                }
#pragma unroll
                for (int i = 0; i < LB; ++i)
                    a[i] = fmaxf(a[i], fabsf(f[i]));
            }
        } else {
            const float *pm = pmax + (int64_t)tau * nrsplit * Kp;
            for (int rs = 0; rs < nrsplit; ++rs) {
                float f[LB];
#pragma unroll
                for (int i = 0; i < LB; ++i) {
                    const int j = jb + 64 * (i0 + i);
                    f[i] = j < K ? pm[(int64_t)rs * Kp + j] : 0.0f;
                }
#pragma unroll
                for (int i = 0; i < LB; ++i)
                    a[i] = fmaxf(a[i], f[i]);
            }
        }
        float cw[LB];
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            const int j = jb + 64 * (i0 + i);
            cw[i] = j < K ? c[j] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            const int j = jb + 64 * (i0 + i);
            if (j < K) {
                const uint32_t key = nonneg_key(__fmul_rn(a[i], cw[i]));
                kl[j] = key;
                if (key != 0u)
                    mn = min(mn, key);
                mx = max(mx, key);
            }
        }
    }
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (lane == 0) {
        wmin[w] = mn;
        wmax[w] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        mn = min(mn, wmin[i]);
        mx = max(mx, wmax[i]);
    }
    // re-base in place: u = key - mn + 1 for key > 0, 0 stays 0 (mn = smallest non-zero key)
    const uint32_t umax = mx == 0u ? 0u : mx - mn + 1u;
    for (int i = 0; i < PER; ++i) {
        const int j = jb + 64 * i;
        if (j < K) {
            const uint32_t key = kl[j];
            kl[j] = key == 0u ? 0u : key - mn + 1u;
        }
    }
    const int L = umax == 0u ? 0 : 32 - __clz(umax);

    // 2. radix passes from the top bit of umax, up to 11 bits each
    uint32_t prefix = 0, pmask = 0, krem = (uint32_t)k;
    int top = L;
    while (top > 0) {
        const int nb = top < 11 ? top : 11;
        const int sh = top - nb;
        const uint32_t dm = (1u << nb) - 1u;
#pragma unroll 4
        for (int i = 0; i < PER; ++i) {
            const int j = jb + 64 * i;
            if (j < K) {
                const uint32_t uu = kl[j];
                if ((uu & pmask) == prefix)
                    atomicAdd(&hist[hpad((int)((uu >> sh) & dm))], 1u);
            }
        }
        __syncthreads();
        if (w == 0)
            wave0_crossing(hist, krem, res);
        __syncthreads();
        prefix |= res[0] << sh;
        pmask |= dm << sh;
        krem = res[1];
        top = sh;
    }
    // (L == 0: every key is zero; prefix 0 and krem = k ties)

    // 3. order-preserving compaction: per-wave counts, one exchange, ballot-ranked stores
    uint32_t gt = 0, eq = 0;
#pragma unroll 4
    for (int i = 0; i < PER; ++i) {
        const int j = jb + 64 * i;
        const uint32_t uu = j < K ? kl[j] : 0u;
        gt += __popcll(__ballot(j < K && uu > prefix));
        eq += __popcll(__ballot(j < K && uu == prefix));
    }
    if (lane == 0) {
        wgt[w] = gt;
        weq[w] = eq;
    }
    __syncthreads();
    uint32_t gtb = 0, eqb = 0;
    for (int i = 0; i < w; ++i) {
        gtb += wgt[i];
        eqb += weq[i];
    }
    const uint64_t lt = lanemask_lt();
    int32_t *dst = idx + (int64_t)tau * k;
#pragma unroll 2
    for (int i = 0; i < PER; ++i) {
        const int j = jb + 64 * i;
        const uint32_t uu = j < K ? kl[j] : 0u;
        const bool g = j < K && uu > prefix, e = j < K && uu == prefix;
        const uint64_t mg = __ballot(g), me = __ballot(e);
        const uint32_t tie_rank = eqb + __popcll(me & lt);
        const bool keep = g || (e && tie_rank < krem);
        const uint64_t mk = __ballot(keep);
        const uint32_t pos = gtb + min(eqb, krem) + __popcll(mk & lt);
        if (keep && pos < (uint32_t)k)
            dst[pos] = j;
        gtb += __popcll(mg);
        eqb += __popcll(me);
    }
}

size_t select_lds_bytes(int64_t K) { return (size_t)K * 4; }

static int64_t pad8(int64_t n) { return (n + 7) / 8 * 8; }

hipError_t launch_select(const void *x, bool bf16, int64_t T, int64_t K, int64_t ldx, const float *c, int64_t tile,
                         int64_t k, int32_t *idx, float *pmax_ws, hipStream_t st)
{
    const int ntiles = (int)((T + tile - 1) / tile);
    const int rows = (int)(tile < T ? tile : T);
    const bool direct = rows <= SELECT_DIRECT_ROWS;
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
#define RMM_SEL_LAUNCH(TE, PER)                                                                                    \
    select_kernel<TE, PER><<<ntiles, SEL_THREADS, select_lds_bytes(K), st>>>(                                      \
        (const TE *)x, ldx, (int)T, (int)K, (int)tile, c, pmax_ws, Kp, nrsplit, direct, (int)k, idx)
    if (K <= 4 * SEL_THREADS) {
        if (bf16)
            RMM_SEL_LAUNCH(uint16_t, 4);
        else
            RMM_SEL_LAUNCH(float, 4);
    } else if (K <= 16 * SEL_THREADS) {
        if (bf16)
            RMM_SEL_LAUNCH(uint16_t, 16);
        else
            RMM_SEL_LAUNCH(float, 16);
    } else {
        if (bf16)
            RMM_SEL_LAUNCH(uint16_t, 32);
        else
            RMM_SEL_LAUNCH(float, 32);
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
    const int lds = (int)select_lds_bytes(SELECT_MAX_K);
    (void)hipFuncSetAttribute((const void *)select_kernel<uint16_t, 32>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute((const void *)select_kernel<float, 32>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute((const void *)select_kernel<uint16_t, 16>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute((const void *)select_kernel<float, 16>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
}

} // namespace rmm
