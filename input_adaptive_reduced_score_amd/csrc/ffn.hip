// Gated FFN producer (decode).
//
// The blog on input-adaptive matrix-product reduction computes the FFN's
// intermediate activation as h = silu(x W_gate^T) * (x W_up^T) (section 6.1,
// the demo's ffn_full); section 5.1 scores the down projection's slices from
// that activation, and section 6.2 notes that the gate and up products stay
// full.  This producer streams W_gate^T and W_up^T (both K-major [H][ldw]) once,
// split over H like the reduced GEMV, and forms h in the fixed-order split
// reduction, together with the scorer's column maxima over each token tile.
// The down projection's selector then reads those maxima (exactly the values it
// would compute from h), so h is not read again for scoring.
//
//  * gateup_kernel: workgroup (token group, column slice, split of H); 8 waves,
//    wave w streams a contiguous run of the split's rows of both matrices over
//    the slice (64 lanes x 16 bytes each), rows broadcast with readlane as in
//    the GEMV; the waves' sums meet in LDS in wave order and go to the
//    workspace as (gate, up) partials.
//  * gateup_reduce_kernel: workgroup (tile, 64 columns); sums the partials in
//    split order, applies silu(g) * u in fp32, rounds to bf16 (nearest even),
//    writes h and max_{t in tile} |h| for its columns.
#include "device.h"
#include "kernels.h"

namespace rmm {

constexpr int GU_WAVES = 8;
constexpr int GU_THREADS = GU_WAVES * WAVE;
constexpr int GU_VEC = 8;               // bf16 columns per lane
constexpr int GU_CW = WAVE * GU_VEC;    // columns per slice
constexpr int GU_U = GATEUP_UNROLL;     // rows of each matrix in flight per wave
constexpr int GU_RED_CHUNK = WAVE;      // columns per reduce workgroup

template <int NT>
__global__ __launch_bounds__(GU_THREADS) void gateup_kernel(const uint16_t *__restrict__ x, int64_t ldx, int T,
                                                            int tile, const uint16_t *__restrict__ wg,
                                                            const uint16_t *__restrict__ wu, int64_t ldw, int H,
                                                            int Mi, int groups_per_tile, int nslices, int nsplit,
                                                            float *__restrict__ part)
{
    __shared__ float red[GU_WAVES][NT][GU_CW];
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;

    int bid = blockIdx.x;
    const int slice = bid % nslices;
    bid /= nslices;
    const int split = bid % nsplit;
    const int grp = bid / nsplit;
    const int tau = grp / groups_per_tile, sub = grp % groups_per_tile;
    const int t0 = tau * tile + sub * NT;
    const int nt = min(NT, min(T, tau * tile + tile) - t0);
    if (nt <= 0)
        return;

    const int i0 = (int)((int64_t)H * split / nsplit), i1 = (int)((int64_t)H * (split + 1) / nsplit);
    const int n = i1 - i0;
    const int r0 = i0 + (int)((int64_t)n * w / GU_WAVES), r1 = i0 + (int)((int64_t)n * (w + 1) / GU_WAVES);
    const int col = slice * GU_CW + lane * GU_VEC;
    const bool active = col < Mi;

    float ag[NT][GU_VEC], au[NT][GU_VEC];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < GU_VEC; ++e)
            ag[t][e] = au[t][e] = 0.0f;

    for (int b0 = r0; b0 < r1; b0 += WAVE) {
        const int nb = min(WAVE, r1 - b0);
        float xv[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
            xv[t] = 0.0f;
        if (lane < nb) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                if (t < nt)
                    xv[t] = bf16_to_f32(x[(int64_t)(t0 + t) * ldx + b0 + lane]);
        }
        for (int c0 = 0; c0 < nb; c0 += GU_U) {
            uint4 ug[GU_U], uu[GU_U];
#pragma unroll
            for (int q = 0; q < GU_U; ++q) {
                if (c0 + q < nb && active) {
                    const int64_t off = (int64_t)(b0 + c0 + q) * ldw + col;
                    ug[q] = *reinterpret_cast<const uint4 *>(wg + off);
                    uu[q] = *reinterpret_cast<const uint4 *>(wu + off);
                }
            }
#pragma unroll
            for (int q = 0; q < GU_U; ++q) {
                if (c0 + q < nb) {
                    float vg[GU_VEC], vu[GU_VEC];
                    Vec16<uint16_t>::unpack(ug[q], vg);
                    Vec16<uint16_t>::unpack(uu[q], vu);
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const float xs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xv[t]), c0 + q));
#pragma unroll
                        for (int e = 0; e < GU_VEC; ++e) {
                            ag[t][e] = fmaf(xs, vg[e], ag[t][e]);
                            au[t][e] = fmaf(xs, vu[e], au[t][e]);
                        }
                    }
                }
            }
        }
    }

    // waves meet in LDS in wave order, gate then up
    float *dst = part + (((int64_t)grp * nslices + slice) * nsplit + split) * (2 * NT * GU_CW);
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) {
        if (m2)
            __syncthreads();
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < GU_VEC; ++e)
                red[w][t][lane * GU_VEC + e] = m2 ? au[t][e] : ag[t][e];
        __syncthreads();
        for (int i = threadIdx.x; i < NT * GU_CW; i += GU_THREADS) {
            const int t = i / GU_CW, cc = i % GU_CW;
            float s = red[0][t][cc];
#pragma unroll
            for (int ww = 1; ww < GU_WAVES; ++ww)
                s += red[ww][t][cc];
            dst[m2 * NT * GU_CW + i] = s;
        }
    }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v)
{
    const uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return 0x7fc0;
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// silu(g) = g / (1 + e^-g), written with e^-|g| so that it neither overflows nor
// loses the negative branch's tiny values
__device__ __forceinline__ float silu_f32(float g)
{
    const float e = expf(-fabsf(g));
    return g >= 0.0f ? g / (1.0f + e) : g * e / (1.0f + e);
}

template <int NT>
__global__ __launch_bounds__(GU_THREADS) void gateup_reduce_kernel(const float *__restrict__ part, int T, int tile,
                                                                   int groups_per_tile, int nslices, int nsplit,
                                                                   int Mi, uint16_t *__restrict__ h, int64_t ldh,
                                                                   float *__restrict__ pmax)
{
    constexpr int CHUNKS = GU_CW / GU_RED_CHUNK;
    constexpr int MAXS = (GATEUP_MAX_SPLIT + GU_WAVES - 1) / GU_WAVES;
    __shared__ float red[GU_WAVES][2][NT][GU_RED_CHUNK];
    __shared__ float mag[GU_WAVES][GU_RED_CHUNK];
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    const int chunk = blockIdx.x % CHUNKS;
    const int rest = blockIdx.x / CHUNKS;
    const int slice = rest % nslices, tau = rest / nslices;
    const int m = slice * GU_CW + chunk * GU_RED_CHUNK + lane;
    const int s0 = nsplit * w / GU_WAVES, s1 = nsplit * (w + 1) / GU_WAVES;
    const int tend = min(T, tau * tile + tile);
    float tmax = 0.0f; // wave 0: running max of |h| over the tile's tokens

    for (int sub = 0; sub < groups_per_tile; ++sub) {
        const int t0 = tau * tile + sub * NT;
        if (t0 >= tend)
            break;
        const int grp = tau * groups_per_tile + sub;
        const float *p = part + ((int64_t)grp * nslices + slice) * nsplit * (2 * NT * GU_CW) + chunk * GU_RED_CHUNK +
                         lane;
        // wave w: its share of the splits, in split order, for every (matrix, token)
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                float v[MAXS];
#pragma unroll
                for (int q = 0; q < MAXS; ++q)
                    v[q] = s0 + q < s1 ? p[(int64_t)(s0 + q) * (2 * NT * GU_CW) + (m2 * NT + t) * GU_CW] : 0.0f;
                float a = 0.0f;
#pragma unroll
                for (int q = 0; q < MAXS; ++q)
                    a += v[q];
                red[w][m2][t][lane] = a;
            }
        }
        __syncthreads();
        // wave t (< NT) finishes token t0 + t: wave sums in wave order, then the epilogue
        float hm = 0.0f;
        if (w < NT) {
            const int t = w;
            float g = 0.0f, u = 0.0f;
#pragma unroll
            for (int q = 0; q < GU_WAVES; ++q) {
                g += red[q][0][t][lane];
                u += red[q][1][t][lane];
            }
            if (t0 + t < tend && m < Mi) {
                const uint16_t hb = f32_to_bf16_rne(silu_f32(g) * u);
                h[(int64_t)(t0 + t) * ldh + m] = hb;
                hm = fabsf(bf16_to_f32(hb));
            }
        }
        mag[w][lane] = hm;
        __syncthreads();
        if (w == 0) {
#pragma unroll
            for (int q = 0; q < GU_WAVES; ++q)
                tmax = fmaxf(tmax, mag[q][lane]);
        }
        __syncthreads();
    }
    if (w == 0 && pmax && m < Mi)
        pmax[(int64_t)tau * Mi + m] = tmax;
}

struct GateUpPlan {
    int nt, groups_per_tile, nslices, nsplit, ngroups, ntiles;
};

static int gu_nt_for(int64_t rows)
{
    return rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : 8;
}

static GateUpPlan gateup_plan(int64_t T, int64_t H, int64_t Mi, int64_t tile)
{
    GateUpPlan p;
    const int64_t rows = tile < T ? tile : T;
    p.nt = gu_nt_for(rows);
    p.groups_per_tile = (int)((rows + p.nt - 1) / p.nt);
    p.ntiles = (int)((T + tile - 1) / tile);
    p.ngroups = p.ntiles * p.groups_per_tile;
    p.nslices = (int)((Mi + GU_CW - 1) / GU_CW);
    const int64_t base = (int64_t)p.ngroups * p.nslices;
    // as many splits as keep the grid within one round of resident workgroups:
    // a partial second round runs at the latency of a whole workgroup
    int64_t ns = GATEUP_TARGET_WGS / base;
    const int64_t by_rows = (H + GU_WAVES * GATEUP_MIN_ROWS - 1) / (GU_WAVES * GATEUP_MIN_ROWS);
    if (ns > by_rows)
        ns = by_rows;
    if (ns > GATEUP_MAX_SPLIT)
        ns = GATEUP_MAX_SPLIT;
    if (ns < 1)
        ns = 1;
    p.nsplit = (int)ns;
    return p;
}

size_t gateup_ws_bytes(int64_t T, int64_t H, int64_t Mi, int64_t tile)
{
    const GateUpPlan p = gateup_plan(T, H, Mi, tile);
    return (size_t)p.ngroups * p.nslices * p.nsplit * 2 * p.nt * GU_CW * sizeof(float);
}

int64_t gateup_grid(int64_t T, int64_t H, int64_t Mi, int64_t tile)
{
    const GateUpPlan p = gateup_plan(T, H, Mi, tile);
    return (int64_t)p.ngroups * p.nslices * p.nsplit;
}

hipError_t launch_gateup(const uint16_t *x, int64_t T, int64_t H, int64_t ldx, const uint16_t *wg,
                         const uint16_t *wu, int64_t ldw, int64_t Mi, int64_t tile, uint16_t *h, int64_t ldh,
                         float *pmax, float *part, hipStream_t st)
{
    const GateUpPlan p = gateup_plan(T, H, Mi, tile);
    const dim3 grid((unsigned)((int64_t)p.ngroups * p.nslices * p.nsplit));
    const dim3 rgrid((unsigned)((int64_t)p.ntiles * p.nslices * (GU_CW / GU_RED_CHUNK)));
#define RMM_GU_CASE(NTV)                                                                                           \
    case NTV:                                                                                                      \
        gateup_kernel<NTV><<<grid, GU_THREADS, 0, st>>>(x, ldx, (int)T, (int)tile, wg, wu, ldw, (int)H, (int)Mi,   \
                                                        p.groups_per_tile, p.nslices, p.nsplit, part);             \
        gateup_reduce_kernel<NTV><<<rgrid, GU_THREADS, 0, st>>>(part, (int)T, (int)tile, p.groups_per_tile,        \
                                                                p.nslices, p.nsplit, (int)Mi, h, ldh, pmax);       \
        break;
    switch (p.nt) {
        RMM_GU_CASE(1)
        RMM_GU_CASE(2)
        RMM_GU_CASE(4)
        RMM_GU_CASE(8)
    default:
        return hipErrorInvalidValue;
    }
#undef RMM_GU_CASE
    return hipGetLastError();
}

} // namespace rmm
