// Reduced linear products with few tokens per tile (decode).
//
// The blog on input-adaptive matrix-product reduction (section 2) reduces
// Y = X @ W^T over the kept contraction slices J: Y ~= X[:,J] @ W^T[J,:];
// section 5.3 gathers the kept slices so the product stays dense, and
// section 8 warns that a gather copy costs bandwidth.  W^T is stored K-major,
// so every kept slice is one contiguous row of W^T: the kernels read kept rows
// in place and never copy W.
//
// gemv_kernel + gemv_reduce_kernel: HBM-streaming split-K over the kept rows;
// the partials are summed in a fixed order by a second small kernel, so results
// are deterministic.  (Many tokens per tile: linear.hip.)
#include "device.h"
#include "kernels.h"

namespace rmm {

// ============================================================================ GEMV
// Split-K over the kept list.  Workgroup (token group, column slice, split):
// 8 waves; wave w streams a contiguous run of the split's kept rows over the
// slice (64 lanes x 16 bytes).  The wave loads its run's indices and the
// tokens' activations with one vector load per 64 rows and broadcasts them
// with readlane, so each row load has a scalar base address and U rows are in
// flight per wave.  Waves are summed through LDS in a fixed order; with more
// than one split the partials go to the workspace and gemv_reduce_kernel sums
// them in split order (a kernel boundary instead of per-workgroup fences).
constexpr int GEMV_WAVES = 8;
constexpr int GEMV_THREADS = GEMV_WAVES * WAVE;

template <typename TE, int NT, bool DENSE>
__global__ __launch_bounds__(GEMV_THREADS) void gemv_kernel(
    const TE *__restrict__ x, int64_t ldx, int T, int tile, const TE *__restrict__ wt, int64_t ldw, int M,
    const int32_t *__restrict__ idx, int k, int groups_per_tile, int nslices, int nsplit, float *__restrict__ part,
    float *__restrict__ y, int64_t ldy)
{
    constexpr int VEC = Vec16<TE>::N;
    constexpr int CW = WAVE * VEC; // columns per slice
    constexpr int U = GEMV_UNROLL; // kept rows in flight per wave
    __shared__ float red[GEMV_WAVES][NT][CW];
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;

    int bid = blockIdx.x;
    const int slice = bid % nslices;
    bid /= nslices;
    const int split = bid % nsplit;
    const int grp = bid / nsplit;
    const int tau = grp / groups_per_tile, sub = grp % groups_per_tile;
    const int t0 = tau * tile + sub * NT;
    const int tend = min(T, tau * tile + tile);
    const int nt = min(NT, tend - t0);
    if (nt <= 0)
        return;

    const int i0 = (int)((int64_t)k * split / nsplit), i1 = (int)((int64_t)k * (split + 1) / nsplit);
    const int n = i1 - i0;
    const int r0 = i0 + (int)((int64_t)n * w / GEMV_WAVES), r1 = i0 + (int)((int64_t)n * (w + 1) / GEMV_WAVES);
    const int32_t *J = DENSE ? nullptr : idx + (int64_t)tau * k;
    const int col = slice * CW + lane * VEC;
    const bool active = col < M;

    float acc[NT][VEC];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            acc[t][e] = 0.0f;

    for (int b0 = r0; b0 < r1; b0 += WAVE) {
        const int nb = min(WAVE, r1 - b0);
        int jv = 0;
        float xv[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
            xv[t] = 0.0f;
        if (lane < nb) {
            jv = DENSE ? b0 + lane : J[b0 + lane];
#pragma unroll
            for (int t = 0; t < NT; ++t)
                if (t < nt)
                    xv[t] = ld_elem(x, (int64_t)(t0 + t) * ldx + jv);
        }
        for (int c0 = 0; c0 < nb; c0 += U) {
            uint4 u[U];
#pragma unroll
            for (int q = 0; q < U; ++q) {
                if (c0 + q < nb) {
                    const int j = __builtin_amdgcn_readlane(jv, c0 + q); // wave-uniform row index
                    if (active)
                        u[q] = Vec16<TE>::raw(wt + (int64_t)j * ldw + col);
                }
            }
#pragma unroll
            for (int q = 0; q < U; ++q) {
                if (c0 + q < nb) {
                    float v[VEC];
                    Vec16<TE>::unpack(u[q], v);
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const float xs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xv[t]), c0 + q));
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            acc[t][e] = fmaf(xs, v[e], acc[t][e]);
                    }
                }
            }
        }
    }

#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            red[w][t][lane * VEC + e] = acc[t][e];
    __syncthreads();
    for (int i = threadIdx.x; i < NT * CW; i += GEMV_THREADS) {
        const int t = i / CW, cc = i % CW;
        float s = red[0][t][cc];
#pragma unroll
        for (int ww = 1; ww < GEMV_WAVES; ++ww)
            s += red[ww][t][cc];
        if (nsplit == 1) {
            if (t < nt && slice * CW + cc < M)
                y[(int64_t)(t0 + t) * ldy + slice * CW + cc] = s;
        } else {
            part[(((int64_t)grp * nslices + slice) * nsplit + split) * (NT * CW) + i] = s;
        }
    }
}

// y[t0+t][slice*CW + cc] = sum over splits of the partials, in a fixed order.
// Workgroup = 64 consecutive partial elements of one (group, slice); wave w sums
// the w-th eighth of the splits in split order, then wave 0 adds the eight
// wave sums in wave order.
constexpr int RED_WAVES = 8;
template <int NT, int CW>
__global__ __launch_bounds__(RED_WAVES * WAVE) void gemv_reduce_kernel(const float *__restrict__ part, int T,
                                                                       int tile, int groups_per_tile, int nslices,
                                                                       int nsplit, int M, float *__restrict__ y,
                                                                       int64_t ldy)
{
    constexpr int CHUNKS = NT * CW / WAVE;
    __shared__ float red[RED_WAVES][WAVE];
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    const int chunk = blockIdx.x % CHUNKS;
    const int gs = blockIdx.x / CHUNKS;
    const int slice = gs % nslices, grp = gs / nslices;
    const int i = chunk * WAVE + lane;
    const float *p = part + (int64_t)gs * nsplit * (NT * CW) + i;
    const int s0 = nsplit * w / RED_WAVES, s1 = nsplit * (w + 1) / RED_WAVES;
    constexpr int MAXS = (GEMV_MAX_SPLIT + RED_WAVES - 1) / RED_WAVES;
    float v[MAXS];
#pragma unroll
    for (int q = 0; q < MAXS; ++q)
        v[q] = s0 + q < s1 ? p[(int64_t)(s0 + q) * (NT * CW)] : 0.0f;
    float a = 0.0f;
#pragma unroll
    for (int q = 0; q < MAXS; ++q)
        a += v[q];
    red[w][lane] = a;
    __syncthreads();
    if (w != 0)
        return;
    float sum = 0.0f;
#pragma unroll
    for (int q = 0; q < RED_WAVES; ++q)
        sum += red[q][lane];
    const int tau = grp / groups_per_tile, sub = grp % groups_per_tile;
    const int t0 = tau * tile + sub * NT;
    const int t = i / CW, cc = i % CW;
    const int tend = min(T, tau * tile + tile);
    if (t0 + t < tend && slice * CW + cc < M)
        y[(int64_t)(t0 + t) * ldy + slice * CW + cc] = sum;
}

struct GemvPlan {
    int nt, groups_per_tile, nslices, nsplit, ngroups;
};

static int nt_for(int64_t rows)
{
    return rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : 8;
}

static GemvPlan gemv_plan(int64_t T, int64_t M, int64_t k, int64_t tile, bool bf16)
{
    GemvPlan p;
    const int64_t rows = tile < T ? tile : T;
    p.nt = nt_for(rows);
    p.groups_per_tile = (int)((rows + p.nt - 1) / p.nt);
    const int64_t ntiles = (T + tile - 1) / tile;
    p.ngroups = (int)(ntiles * p.groups_per_tile);
    const int cw = WAVE * (bf16 ? 8 : 4);
    p.nslices = (int)((M + cw - 1) / cw);
    const int64_t base = (int64_t)p.ngroups * p.nslices;
    // as many splits as keep the grid within one round of resident workgroups:
    // a partial second round runs at the latency of a whole workgroup
    int64_t ns = GEMV_TARGET_WGS / base;
    const int64_t by_rows = (k + GEMV_WAVES * GEMV_MIN_ROWS - 1) / (GEMV_WAVES * GEMV_MIN_ROWS);
    if (ns > by_rows)
        ns = by_rows;
    if (ns > GEMV_MAX_SPLIT)
        ns = GEMV_MAX_SPLIT;
    if (ns < 1)
        ns = 1;
    p.nsplit = (int)ns;
    return p;
}

size_t gemv_ws_bytes(int64_t T, int64_t M, int64_t k, int64_t tile, bool bf16)
{
    GemvPlan p = gemv_plan(T, M, k, tile, bf16);
    if (p.nsplit == 1)
        return 0;
    const int cw = WAVE * (bf16 ? 8 : 4);
    return (size_t)p.ngroups * p.nslices * p.nsplit * p.nt * cw * sizeof(float);
}

template <typename TE, bool DENSE>
static hipError_t gemv_dispatch(const GemvPlan &p, const void *x, int64_t ldx, int64_t T, int64_t tile,
                                const void *wt, int64_t ldw, int64_t M, const int32_t *idx, int64_t k, float *part,
                                float *y, int64_t ldy, hipStream_t st)
{
    constexpr int CW = WAVE * Vec16<TE>::N;
    dim3 grid((unsigned)((int64_t)p.ngroups * p.nslices * p.nsplit));
    dim3 rgrid((unsigned)((int64_t)p.ngroups * p.nslices * (p.nt * CW / WAVE)));
#define RMM_GEMV_CASE(NTV)                                                                                         \
    case NTV:                                                                                                      \
        gemv_kernel<TE, NTV, DENSE><<<grid, GEMV_THREADS, 0, st>>>(                                                \
            (const TE *)x, ldx, (int)T, (int)tile, (const TE *)wt, ldw, (int)M, idx, (int)k, p.groups_per_tile,     \
            p.nslices, p.nsplit, part, y, ldy);                                                                    \
        if (p.nsplit > 1)                                                                                          \
            gemv_reduce_kernel<NTV, CW><<<rgrid, RED_WAVES * WAVE, 0, st>>>(part, (int)T, (int)tile, p.groups_per_tile,          \
                                                                p.nslices, p.nsplit, (int)M, y, ldy);              \
        break;
    switch (p.nt) {
        RMM_GEMV_CASE(1)
        RMM_GEMV_CASE(2)
        RMM_GEMV_CASE(4)
        RMM_GEMV_CASE(8)
    default:
        return hipErrorInvalidValue;
    }
#undef RMM_GEMV_CASE
    return hipGetLastError();
}

hipError_t launch_gemv(const void *x, bool bf16, int64_t T, int64_t ldx, const void *wt, int64_t ldw, int64_t M,
                       const int32_t *idx, int64_t k, int64_t tile, bool dense, float *y, int64_t ldy, float *part,
                       hipStream_t st)
{
    GemvPlan p = gemv_plan(T, M, k, tile, bf16);
    if (bf16)
        return dense ? gemv_dispatch<uint16_t, true>(p, x, ldx, T, tile, wt, ldw, M, idx, k, part, y, ldy, st)
                     : gemv_dispatch<uint16_t, false>(p, x, ldx, T, tile, wt, ldw, M, idx, k, part, y, ldy, st);
    return dense ? gemv_dispatch<float, true>(p, x, ldx, T, tile, wt, ldw, M, idx, k, part, y, ldy, st)
                 : gemv_dispatch<float, false>(p, x, ldx, T, tile, wt, ldw, M, idx, k, part, y, ldy, st);
}

} // namespace rmm
