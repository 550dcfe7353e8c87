// Reduced linear products.
//
// The blog on input-adaptive matrix-product reduction (section 2) reduces
// Y = X @ W^T over the kept contraction slices J: Y ~= X[:,J] @ W^T[J,:];
// section 5.3 gathers the kept slices so the product stays dense, and
// section 8 warns that a gather copy costs bandwidth.  W^T is stored K-major,
// so every kept slice is one contiguous row of W^T: the kernels read kept rows
// in place and never copy W.
//
//  * gemv_kernel (+ gemv_reduce_kernel): few tokens per tile (decode).
//    HBM-streaming split-K over the kept rows; partials are summed in a fixed
//    order by a second small kernel, so results are deterministic.
//  * gather_kernel + gemm_kernel: many tokens per tile (prefill).  The kept
//    columns of the tile's activations are packed once (activations are the
//    small operand), then a bf16 MFMA GEMM (v_mfma_f32_32x32x16_bf16, fp32
//    accumulation) stages A tiles and the kept W^T rows through LDS.
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
                       uint32_t *cnt, hipStream_t st)
{
    (void)cnt;
    GemvPlan p = gemv_plan(T, M, k, tile, bf16);
    if (bf16)
        return dense ? gemv_dispatch<uint16_t, true>(p, x, ldx, T, tile, wt, ldw, M, idx, k, part, y, ldy, st)
                     : gemv_dispatch<uint16_t, false>(p, x, ldx, T, tile, wt, ldw, M, idx, k, part, y, ldy, st);
    return dense ? gemv_dispatch<float, true>(p, x, ldx, T, tile, wt, ldw, M, idx, k, part, y, ldy, st)
                 : gemv_dispatch<float, false>(p, x, ldx, T, tile, wt, ldw, M, idx, k, part, y, ldy, st);
}

// ============================================================================ gather
// xg[t][i] = x[t][idx[t/tile][i]] for i < k, 0 for k <= i < kpad.  One workgroup
// per token row: with STAGE the row is staged in LDS with 16-byte loads (rows up
// to GATHER_LDS_MAX_K elements), then gathered; without, gathered from HBM.
constexpr int GATHER_LDS_MAX_K = 32768;
template <bool STAGE>
__global__ __launch_bounds__(256) void gather_kernel(const uint16_t *__restrict__ x, int64_t ldx, int K, int tile,
                                                     const int32_t *__restrict__ idx, int k, int kpad,
                                                     uint16_t *__restrict__ xg)
{
    extern __shared__ uint16_t xrow[];
    const int t = blockIdx.x;
    const uint16_t *xr = x + (int64_t)t * ldx;
    if (STAGE) {
        // ldx is a multiple of 8, so the 16-byte run past K stays inside the row's pitch
        for (int c = threadIdx.x * 8; c < K; c += 256 * 8)
            *reinterpret_cast<uint4 *>(xrow + c) = *reinterpret_cast<const uint4 *>(xr + c);
        __syncthreads();
    }
    const int32_t *J = idx + (int64_t)(t / tile) * k;
    for (int ch = threadIdx.x; ch < kpad / 8; ch += 256) {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = ch * 8 + e;
            h[e] = i < k ? (STAGE ? xrow[J[i]] : xr[J[i]]) : 0u;
        }
        uint4 o;
        o.x = h[0] | (h[1] << 16);
        o.y = h[2] | (h[3] << 16);
        o.z = h[4] | (h[5] << 16);
        o.w = h[6] | (h[7] << 16);
        *reinterpret_cast<uint4 *>(xg + (int64_t)t * kpad + ch * 8) = o;
    }
}

// ============================================================================ MFMA GEMM
// C[t][n] = sum_i A[t][i] * W^T[row(i)][n], A = packed kept activations
// (or x itself when dense), row(i) = idx[tile(t)][i] (or i when dense).
// Workgroup tile 128 x 128, k step 64, 4 waves of 64 x 64 (2 x 2 MFMA 32x32x16).
constexpr int GB_M = 128, GB_N = 128, GB_K = 64;
constexpr int GEMM_THREADS = 256;
constexpr int LPITCH = GB_K + 8; // bf16 per LDS row (pad against bank conflicts)

template <bool DENSE>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_kernel(const uint16_t *__restrict__ A, int64_t lda, int T,
                                                            int tile, int mblocks, const uint16_t *__restrict__ wt,
                                                            int64_t ldw, int M, const int32_t *__restrict__ idx,
                                                            int k, int klim, float *__restrict__ y, int64_t ldy)
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
    const int32_t *J = DENSE ? nullptr : idx + (int64_t)tau * k;
    const int wm = w >> 1, wn = w & 1;

    // A loader: 4 chunks of 8 bf16 per thread: row ar + 32p, k offset 8*ac
    const int ar = tid >> 3, ac = tid & 7;
    // B loader: lane = k row within the step, chunks w + 4p of 8 columns
    uint4 ra[4], rb[4];
    // the W^T row index of this lane for a step, loaded one step before its rows are
    auto jrow = [&](int kk) {
        int kr = kk + lane;
        kr = kr < klim ? kr : klim - 1; // padded steps reuse a valid row (times zero A)
        return DENSE ? kr : J[kr];
    };
    auto load_stage = [&](int kk, int j) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = ar + 32 * p;
            const int kc = kk + 8 * ac;
            uint4 v = {0u, 0u, 0u, 0u};
            if (row0 + r < rowend) {
                const uint16_t *src = A + (int64_t)(row0 + r) * lda + kc;
                if (!DENSE || kc + 8 <= klim) {
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
    const int mblocks = (int)((rows + GB_M - 1) / GB_M);
    const int64_t ntiles = (T + tile - 1) / tile;
    dim3 grid((unsigned)((M + GB_N - 1) / GB_N), (unsigned)(ntiles * mblocks));
    if (dense) {
        gemm_kernel<true><<<grid, GEMM_THREADS, 0, st>>>((const uint16_t *)x, ldx, (int)T, (int)tile, mblocks,
                                                         (const uint16_t *)wt, ldw, (int)M, nullptr, (int)K, (int)K,
                                                         y, ldy);
        return hipGetLastError();
    }
    const int64_t kpad = (k + GB_K - 1) / GB_K * GB_K;
    if (K <= GATHER_LDS_MAX_K)
        gather_kernel<true><<<(unsigned)T, 256, (size_t)(K + 7) / 8 * 16, st>>>(
            (const uint16_t *)x, ldx, (int)K, (int)tile, idx, (int)k, (int)kpad, (uint16_t *)xg);
    else
        gather_kernel<false><<<(unsigned)T, 256, 0, st>>>((const uint16_t *)x, ldx, (int)K, (int)tile, idx, (int)k,
                                                          (int)kpad, (uint16_t *)xg);
    gemm_kernel<false><<<grid, GEMM_THREADS, 0, st>>>((const uint16_t *)xg, kpad, (int)T, (int)tile, mblocks,
                                                      (const uint16_t *)wt, ldw, (int)M, idx, (int)k, (int)k, y, ldy);
    return hipGetLastError();
}

void linear_init()
{
    (void)hipFuncSetAttribute((const void *)gather_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              GATHER_LDS_MAX_K * 2);
}

} // namespace rmm
