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
#include "select_body.h"

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
                                                                       int64_t ldy, uint64_t *__restrict__ clear1 = nullptr,
                                                                       uint64_t *__restrict__ clear2 = nullptr,
                                                                       uint64_t *__restrict__ clear3 = nullptr)
{
    if (clear1 && blockIdx.x == 0 && threadIdx.x == 0) {
        // the fused launch before this one has finished: its flags return to zero
        __hip_atomic_store(clear1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(clear2, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(clear3, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
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

// ============================================================================ fused select + GEMV (one token)
// One launch selects and multiplies.  Workgroup 0 runs the tile's selection
// (select_body with PUB) and publishes, in two steps, which slices are kept
// (then, for the kept list, each split's offset in it);
// every workgroup (0 included, after its selection) owns a column slice and a
// range of R slice indices, 16 waves of up to 64 slices each.  Every other
// workgroup first estimates the threshold key from its own slices' keys
// (estimate_edge) and streams the rows of its slices at or above it while
// workgroup 0 still selects.  Once both flags are out a wave streams, in one
// pass, the kept rows it has not taken yet and takes back (adds with the
// opposite sign) those it took that are not kept; the waves of column slice 0
// write their kept slices once the offsets are out.  The kept set is the
// selection's in every case; the estimate only moves work earlier.  Each wave
// adds its rows in that fixed order, the waves are summed in order, and
// gemv_reduce_kernel sums the splits in order, so the result is
// deterministic.  Workgroup 0 is dispatched first and waits on no other
// workgroup, so the waits end whatever the residency; each wait is bounded all
// the same, and a wait that runs out poisons the output with NaN.
constexpr int FUSED_WAVES = SEL_THREADS / WAVE; // 16
constexpr int FUSED_SPIN = 1 << 20;             // polls (about 1 s) before a wait gives up
constexpr double EST_FRAC = 0.9;               // the estimate aims at this fraction of the kept count
constexpr int EST_BITS = 11;                    // its histogram: the top 11 bits of the 31-bit key
constexpr int EST_BINS = 1 << EST_BITS;

// The early estimate, taken by each workgroup but the selecting one from the
// keys of its own slices (which its waves hold for the selection anyway), so no
// further load and no hand-off: an LDS histogram of their top EST_BITS bits (8
// bins per octave), and E = the upper edge of the bin holding the key of rank
// EST_FRAC * k * ns / K from the top, ns the workgroup's slice count.  Keys at or
// above E are kept for all but a range that misleads; the caller streams those
// rows before the selection is known and corrects the rest after it.  h holds
// EST_BINS + FUSED_WAVES + 1 words of LDS.  Contains barriers: every thread of
// the workgroup calls it.
__device__ uint32_t estimate_edge(uint32_t key, bool valid, int ns, int K, int k, uint32_t *h)
{
    const int tid = threadIdx.x;
    for (int i = tid; i < EST_BINS; i += SEL_THREADS)
        h[i] = 0;
    if (tid == 0)
        h[EST_BINS + FUSED_WAVES] = 0xffffffffu; // no slices: nothing early
    __syncthreads();
    if (valid)
        atomicAdd(&h[key >> (31 - EST_BITS)], 1u);
    __syncthreads();
    // thread t holds bins B-1-BPT*t down to B-BPT-BPT*t (B bins); exactly one
    // bin holds the target rank when 1 <= want <= ns
    constexpr int BPT = EST_BINS / SEL_THREADS;
    const uint32_t want = max(1u, (uint32_t)(EST_FRAC * (double)k * (double)ns / (double)K));
    uint32_t hc[BPT], tot = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        hc[i] = h[EST_BINS - 1 - BPT * tid - i];
        tot += hc[i];
    }
    const uint32_t incl = block_incl_scan(tot, h + EST_BINS); // (barriers inside)
    uint32_t run = incl - tot;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        if (run < want && want <= run + hc[i])
            h[EST_BINS + FUSED_WAVES] = (uint32_t)(EST_BINS - BPT * tid - i) << (31 - EST_BITS);
        run += hc[i];
    }
    __syncthreads();
    return h[EST_BINS + FUSED_WAVES];
}

// Polls a published word until its ready bit is set; 0 if it never is.
__device__ __forceinline__ uint64_t wait_sig(const uint64_t *sig)
{
    for (int it = 0; it < FUSED_SPIN; ++it) {
        const uint64_t v = pub_load64(sig);
        if (v & 1ull)
            return v;
        __builtin_amdgcn_s_sleep(2);
    }
    return 0ull;
}

template <typename TE, int PER>
__global__ __launch_bounds__(SEL_THREADS) void select_gemv_kernel(const TE *__restrict__ x, const float *__restrict__ c,
                                                                  int K, int k, int cvec, const TE *__restrict__ wt,
                                                                  int64_t ldw, int M, int nslices, SelPub pub,
                                                                  float *__restrict__ part, int32_t *__restrict__ idx)
{
    constexpr int VEC = Vec16<TE>::N;
    constexpr int CW = WAVE * VEC; // columns per slice
    constexpr int U = GEMV_UNROLL; // kept rows in flight per wave
    __shared__ union {
        float red[FUSED_WAVES][CW];             // the waves' partial sums
        uint32_t est[EST_BINS + FUSED_WAVES + 1]; // the early estimate's histogram
    } lds;
    float(&red)[FUSED_WAVES][CW] = lds.red;
    __shared__ uint64_t sig[3];
    __shared__ uint32_t wcnt[FUSED_WAVES];
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    if (blockIdx.x == 0)
        select_body<TE, PER, true>(x, 0, 1, K, 1, c, nullptr, 0, 1, 1, cvec, k, 0, nullptr, pub);

    const int slice = (int)blockIdx.x % nslices, split = (int)blockIdx.x / nslices;
    // this workgroup's slice range: column slice 0 starts with the selecting workgroup's short range
    int ws0, ws1;
    if (slice == 0) {
        ws0 = split_start0(pub, split, K);
        ws1 = split_start0(pub, split + 1, K);
    } else {
        ws0 = min(split * pub.R, K);
        ws1 = min(ws0 + pub.R, K);
    }
    const int RW = (ws1 - ws0 + FUSED_WAVES - 1) / FUSED_WAVES; // <= 64 slices per wave
    const int lo = ws0 + w * RW;
    const int hi = min(lo + RW, ws1);
    const int n = hi > lo ? hi - lo : 0;
    const int col = slice * CW + lane * VEC;
    const bool active = col < M;
    // this lane's slice: activation and score key (the selecting workgroup's
    // arithmetic: one fp32 multiply of |x| by the slice weight), loaded before the wait
    float xj = 0.0f, cj = 0.0f;
    if (lane < n) {
        xj = ld_elem(x, lo + lane);
        cj = c[lo + lane];
    }
    const uint32_t key0 = lane < n ? nonneg_key(__fmul_rn(fabsf(xj), cj)) : 0u;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        acc[e] = 0.0f;
    // rows of the slices lo + b for the set bits b of two disjoint wave-uniform
    // masks, ascending, U in flight: added for `plus`, taken back (added with
    // the opposite sign) for `minus`
    auto stream = [&](uint64_t plus, uint64_t minus) {
        uint64_t m = plus | minus;
        while (m) {
            uint4 u[U];
            float xs[U];
            int cnt = 0;
#pragma unroll
            for (int q = 0; q < U; ++q) {
                if (m) {
                    const int b = __builtin_ctzll(m);
                    m &= m - 1ull;
                    const float xb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xj), b));
                    xs[q] = ((minus >> b) & 1ull) ? -xb : xb;
                    if (active)
                        u[q] = Vec16<TE>::raw(wt + (int64_t)(lo + b) * ldw + col);
                    cnt = q + 1;
                }
            }
#pragma unroll
            for (int q = 0; q < U; ++q) {
                if (q < cnt) {
                    float v[VEC];
                    Vec16<TE>::unpack(u[q], v);
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        acc[e] = fmaf(xs[q], v[e], acc[e]);
                }
            }
        }
    };

    // 0. rows at or above the early estimate (every workgroup but the selecting one)
    uint64_t spec = 0;
    if (blockIdx.x != 0) {
        const uint32_t est = estimate_edge(key0, lane < n, ws1 - ws0, K, k, lds.est);
        spec = __ballot(lane < n && key0 >= est);
        stream(spec, 0ull);
    }
    // 1. the selection: the undecided digit and the slices above it (flag1), the
    // threshold within the digit (flag2)
    if (tid == 0) {
        sig[0] = wait_sig(pub.sig1);
        sig[1] = wait_sig(pub.sig2);
    }
    __syncthreads();
    const uint64_t s1 = sig[0], s2 = sig[1];
    const uint32_t mn = (uint32_t)(s1 >> 32), dg = (uint32_t)(s1 >> 11) & 0x1fffffu;
    const int sh = (int)(s1 >> 6) & 31, nb = (int)(s1 >> 1) & 31;
    const uint32_t pm = ((1u << nb) - 1u) << sh, pfx = dg << sh;
    const uint32_t key = key0 == 0u ? 0u : key0 - mn + 1u; // re-based as the selecting workgroup does
    const uint32_t thr = (uint32_t)(s2 >> 32);
    const int jt = (int)((uint32_t)s2 >> 1);
    const bool cand = lane < n && (key & pm) == pfx;
    const uint64_t sure = __ballot(lane < n && (key & pm) > pfx);
    const uint64_t keptc = __ballot(cand && (key > thr || (key == thr && lo + lane <= jt)));
    const uint64_t kept = sure | keptc;
    // 2. the kept rows not taken early, and those taken early that are not kept, in one pass
    stream(kept & ~spec, spec & ~kept);
    if (!(s1 & s2 & 1ull)) {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            acc[e] = __builtin_nanf("");
    }
    // kept list (ascending): the waves of column slice 0 write their kept slices
    // once the per-split offsets are out
    if (idx && slice == 0) {
        if (tid == 0)
            sig[2] = wait_sig(pub.sig3);
        if (lane == 0)
            wcnt[w] = (uint32_t)__popcll(kept);
        __syncthreads();
        if (!(sig[2] & 1ull)) {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                acc[e] = __builtin_nanf("");
        }
        uint32_t off = pub_load(pub.offs + split);
        for (int i = 0; i < w; ++i)
            off += wcnt[i];
        const uint32_t at = off + (uint32_t)__popcll(kept & lanemask_lt());
        if (((kept >> lane) & 1ull) && at < (uint32_t)k)
            idx[at] = lo + lane;
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        red[w][lane * VEC + e] = acc[e];
    __syncthreads();
    for (int i = tid; i < CW; i += SEL_THREADS) {
        float sum = red[0][i];
#pragma unroll
        for (int ww = 1; ww < FUSED_WAVES; ++ww)
            sum += red[ww][i];
        part[((int64_t)slice * pub.nsplit + split) * CW + i] = sum;
    }
}

struct FusedPlan {
    int nslices, nsplit, R, R0, R1;
};
static FusedPlan fused_plan(int64_t K, int64_t M, bool bf16)
{
    FusedPlan p;
    const int cw = WAVE * (bf16 ? 8 : 4);
    const int64_t cap = 64 * FUSED_WAVES; // at most 64 slices per wave
    p.nslices = (int)((M + cw - 1) / cw);
    int64_t ns = 256 / p.nslices; // one workgroup per CU
    if (ns > GEMV_MAX_SPLIT)
        ns = GEMV_MAX_SPLIT;
    if (ns > K)
        ns = K;
    if (ns < 1)
        ns = 1;
    // column slice 0: the selecting workgroup (split 0) takes an eighth of a range, since it
    // starts streaming only after its selection; splits 1 .. nsplit-1 share the rest
    for (;; ++ns) {
        p.nsplit = (int)ns;
        p.R = (int)((K + ns - 1) / ns);
        if (ns == 1) {
            p.R0 = (int)K;
            p.R1 = 1;
        } else {
            p.R0 = (p.R + 7) / 8;
            p.R1 = (int)((K - p.R0 + ns - 2) / (ns - 1));
        }
        if ((p.R <= cap && p.R0 <= cap && p.R1 <= cap) || ns >= GEMV_MAX_SPLIT || ns >= K)
            break;
    }
    return p;
}

static inline size_t al256(size_t n) { return (n + 255) & ~(size_t)255; }

size_t select_gemv_ws_bytes(int64_t K, int64_t M, bool bf16)
{
    const FusedPlan p = fused_plan(K, M, bf16);
    const int cw = WAVE * (bf16 ? 8 : 4);
    return al256((size_t)(p.nsplit + 1) * 4) + (size_t)p.nslices * p.nsplit * cw * sizeof(float);
}

bool select_gemv_fits(int64_t K, int64_t M, bool bf16)
{
    const FusedPlan p = fused_plan(K, M, bf16);
    return (int64_t)p.R <= 64 * FUSED_WAVES && (int64_t)p.R0 <= 64 * FUSED_WAVES &&
           (int64_t)p.R1 <= 64 * FUSED_WAVES && p.nsplit <= GEMV_MAX_SPLIT;
}

template <typename TE>
static hipError_t select_gemv_dispatch(const FusedPlan &p, const TE *x, int64_t K, const float *c, int cvec, int64_t k,
                                       const TE *wt, int64_t ldw, int64_t M, int32_t *idx, float *y, char *hdr,
                                       char *body, hipStream_t st)
{
    constexpr int CW = WAVE * Vec16<TE>::N;
    SelPub pub;
    pub.sig1 = reinterpret_cast<uint64_t *>(hdr);
    pub.sig2 = reinterpret_cast<uint64_t *>(hdr + 128);
    pub.sig3 = reinterpret_cast<uint64_t *>(hdr + 256);
    pub.offs = idx ? reinterpret_cast<uint32_t *>(body) : nullptr; // the offsets serve the kept list only
    pub.R = p.R;
    pub.R0 = p.R0;
    pub.R1 = p.R1;
    pub.nsplit = p.nsplit;
    float *part = reinterpret_cast<float *>(body + al256((size_t)(p.nsplit + 1) * 4));
    const dim3 grid((unsigned)(p.nslices * p.nsplit));
#define RMM_FUSED_CASE(PERV)                                                                                       \
    case PERV:                                                                                                     \
        select_gemv_kernel<TE, PERV><<<grid, SEL_THREADS, 0, st>>>(x, c, (int)K, (int)k, cvec, wt, ldw, (int)M,    \
                                                                   p.nslices, pub, part, idx);                     \
        break;
    switch (select_per_for(K)) {
        RMM_FUSED_CASE(4)
        RMM_FUSED_CASE(8)
        RMM_FUSED_CASE(16)
        RMM_FUSED_CASE(32)
    default:
        return hipErrorInvalidValue;
    }
#undef RMM_FUSED_CASE
    const dim3 rgrid((unsigned)(p.nslices * (CW / WAVE)));
    gemv_reduce_kernel<1, CW><<<rgrid, RED_WAVES * WAVE, 0, st>>>(part, 1, 1, 1, p.nslices, p.nsplit, (int)M, y,
                                                                 (int64_t)M, pub.sig1, pub.sig2, pub.sig3);
    return hipGetLastError();
}

hipError_t launch_select_gemv(const void *x, bool bf16, int64_t K, const float *c, int64_t k, const void *wt,
                              int64_t ldw, int64_t M, int32_t *idx, float *y, char *hdr, char *body, hipStream_t st)
{
    const FusedPlan p = fused_plan(K, M, bf16);
    const int cvec = ((uintptr_t)c & 15u) == 0u;
    if (bf16)
        return select_gemv_dispatch<uint16_t>(p, (const uint16_t *)x, K, c, cvec, k, (const uint16_t *)wt, ldw, M,
                                              idx, y, hdr, body, st);
    return select_gemv_dispatch<float>(p, (const float *)x, K, c, cvec, k, (const float *)wt, ldw, M, idx, y, hdr,
                                       body, st);
}

} // namespace rmm
