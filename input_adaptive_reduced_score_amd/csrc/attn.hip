// Reduced grouped-query attention decode.
//
// Blog on input-adaptive matrix-product reduction: section 3.1 (most past keys
// matter little to the current query: skip low-contribution work along the
// sequence), section 3.3 (reduce inside each head, never drop a head);
// paper abstract (keep informative slices of each product's contraction
// dimension: head_dim for Q K^T, key positions for P V).  GEMM notes section 1:
// scores = Q K^T, out = softmax(scores) V.
//
// Pipeline per (batch element, selection group), five launches on one stream
// (a sixth writes the kept-position lists when they are asked for):
//  qk    : head_dim selection (one wave, bitwise search over ballots), then
//          unscaled logits over the kept dims for 8 positions per lane from
//          dim-major keys (a kept dim is one contiguous row), and per-chunk
//          softmax statistics (max, sum of exponentials); the first chunk's
//          workgroup clears the group's score histogram.
//  keys  : every workgroup merges the chunk statistics into lse (double), then
//          scores its positions by max_h (scale*a_h - lse_h) in double, stores
//          each position's histogram bin and adds it to the group histogram.
//  select: one workgroup per group resolves the group's exact threshold from
//          the histogram and the bins.
//  pv    : each workgroup keeps its chunk's positions at or above the
//          threshold (order-preserving), streams their V rows and accumulates
//          p*V into a per-chunk partial.
//  reduce: the chunk partials are summed in a fixed order.
#include "device.h"
#include "kernels.h"

namespace rmm {

constexpr int D = ATTN_D;
constexpr int QK_U = 16;      // kept key rows in flight per lane
constexpr int QK_THREADS = 256; // 4 waves split the kept dims of one chunk

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, WAVE));
    return v;
}
template <typename F> __device__ __forceinline__ F wave_sum(F v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, WAVE);
    return v;
}

// ---- cache addressing (contiguous or paged) and per-sequence lengths
__device__ __forceinline__ int seq_len(const AttnShape &s, const KvMap &m, int b)
{
    if (!m.seqlens)
        return (int)s.S;
    const int v = m.seqlens[b];
    return v < 1 ? 1 : (v > (int)s.S ? (int)s.S : v);
}

// The keep count of the C ABI (paper abstract, retention-ratio control) for a
// sequence length known only on the device: ceil(r*n), r*n snapped to the
// nearest integer within 1e-9 relative, clamped to [1, n]; the same IEEE
// double operations as on the host.
__device__ __forceinline__ int keep_count_dev(int n, double r)
{
    const double prod = r * (double)n;
    const double near = rint(prod);
    const double tol = 1e-9 * (prod > 1.0 ? prod : 1.0);
    double kk = fabs(prod - near) <= tol ? near : ceil(prod);
    kk = kk < 1.0 ? 1.0 : kk;
    kk = kk > (double)n ? (double)n : kk;
    return (int)kk;
}

__device__ __forceinline__ int seq_keep(const AttnShape &s, const KvMap &m, int Sb)
{
    return m.seqlens ? keep_count_dev(Sb, m.r_pos) : s.ks;
}

// Row of position p of KV head g of sequence b: the V row (times D elements)
// and the value-norm entry share this index.  Needs p < the sequence's length
// (block-table entries beyond it are never read).
__device__ __forceinline__ int64_t kv_row(const AttnShape &s, const KvMap &m, int b, int g, int p)
{
    if (!m.pages)
        return ((int64_t)b * s.Hkv + g) * s.ldv + p;
    const int64_t pg = m.pages[(int64_t)b * m.maxp + p / m.page];
    return (pg * s.Hkv + g) * m.page + p % m.page;
}

// Element offset of dim 0 at position p in the dim-major keys of (b, g), and
// the pitch between dims.  p is a multiple of 8, so p .. p + 7 share a page.
__device__ __forceinline__ int64_t kt_off(const AttnShape &s, const KvMap &m, int b, int g, int p, int64_t &pitch)
{
    if (!m.pages) {
        pitch = s.ldk;
        return ((int64_t)b * s.Hkv + g) * D * s.ldk + p;
    }
    const int64_t pg = m.pages[(int64_t)b * m.maxp + p / m.page];
    pitch = m.page;
    return (pg * s.Hkv + g) * D * m.page + p % m.page;
}

// Keeps the kd largest of 128 keys held two per lane (j = lane, lane + 64),
// ties to the lower index, and writes the kept indices in ascending order.
__device__ __forceinline__ void wave_select128(uint32_t key0, uint32_t key1, int kd, int *jd)
{
    const int lane = threadIdx.x & (WAVE - 1);
    // largest v with #(key >= v) >= kd: the kd-th largest key
    uint32_t v = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = v | (1u << bit);
        const int c = __popcll(__ballot(key0 >= cand)) + __popcll(__ballot(key1 >= cand));
        if (c >= kd)
            v = cand;
    }
    const int gt = __popcll(__ballot(key0 > v)) + __popcll(__ballot(key1 > v));
    const int quota = kd - gt;
    const uint64_t e0 = __ballot(key0 == v), e1 = __ballot(key1 == v);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int r0 = __popcll(e0 & lt), r1 = __popcll(e0) + __popcll(e1 & lt);
    const bool keep0 = key0 > v || (key0 == v && r0 < quota);
    const bool keep1 = key1 > v || (key1 == v && r1 < quota);
    const uint64_t k0 = __ballot(keep0), k1 = __ballot(keep1);
    if (keep0)
        jd[__popcll(k0 & lt)] = lane;
    if (keep1)
        jd[__popcll(k0) + __popcll(k1 & lt)] = lane + WAVE;
}

// ------------------------------------------------------------------ qk
template <int GS>
__global__ __launch_bounds__(QK_THREADS) void attn_qk_kernel(AttnShape s, KvMap m, int Sp, const uint16_t *__restrict__ q,
                                                             const uint16_t *__restrict__ kt,
                                                             const float *__restrict__ kn, float *__restrict__ logit,
                                                             float2 *__restrict__ pstat,
                                                             int32_t *__restrict__ dim_idx_out,
                                                             uint32_t *__restrict__ hist)
{
    constexpr int NWQ = QK_THREADS / WAVE;
    __shared__ int jd[D];
    __shared__ float qs[GS][D];
    __shared__ float part[NWQ][GS][ATTN_QK_CHUNK];
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int grp = blockIdx.y, b = grp / s.Hsel, sg = grp % s.Hsel;
    const int h0 = sg * s.GS, g = h0 / s.G;
    const int chunk = blockIdx.x, nchunk = gridDim.x;
    const int Sb = seq_len(s, m, b);
    if (chunk * ATTN_QK_CHUNK >= Sb)
        return; // past this sequence's end: its statistics are never read
    const uint16_t *qb = q + ((int64_t)b * s.Hq + h0) * D;
    // this lane's key columns (the page lookup overlaps the staging and selection below)
    const int sp = chunk * ATTN_QK_CHUNK + lane * 8;
    const bool act = sp < Sb;
    int64_t kpitch = 0;
    const int64_t koff = act ? kt_off(s, m, b, g, sp, kpitch) : 0;

    // q of the group's heads, staged once (one 16-byte load per thread; q is
    // 16-byte aligned and D = 128) while wave 0 selects
    __shared__ float qall[GS][D];
    static_assert(GS * D / 8 <= QK_THREADS, "one 16-byte vector of q per thread");
    if (tid < GS * D / 8) {
        float v[8];
        Vec16<uint16_t>::unpack(*reinterpret_cast<const uint4 *>(qb + tid * 8), v);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            qall[(tid * 8 + e) / D][(tid * 8 + e) % D] = v[e];
    }
    // 1. head_dim selection (wave 0): sigma_j = fl32(max_h |q_h[j]| * kn[j])
    if (w == 0) {
        uint32_t key[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int j = lane + WAVE * half;
            float a = 0.0f;
#pragma unroll
            for (int hh = 0; hh < GS; ++hh)
                a = fmaxf(a, fabsf(bf16_to_f32(qb[hh * D + j])));
            key[half] = nonneg_key(__fmul_rn(a, kn[((int64_t)b * s.Hkv + g) * D + j]));
        }
        wave_select128(key[0], key[1], s.kd, jd);
    }
    __syncthreads();
    for (int i = tid; i < s.kd; i += QK_THREADS) {
        const int j = jd[i];
#pragma unroll
        for (int hh = 0; hh < GS; ++hh)
            qs[hh][i] = qall[hh][j];
        if (chunk == 0 && dim_idx_out)
            dim_idx_out[(int64_t)grp * s.kd + i] = j;
    }
    __syncthreads();

    // 2. partial dot products: wave w takes kept dims [i0, i1) (ascending), 8 positions per lane
    const int i0 = s.kd * w / NWQ, i1 = s.kd * (w + 1) / NWQ;
    float acc[GS][8];
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[hh][e] = 0.0f;
    if (act) {
        const uint16_t *kbase = kt + koff;
        for (int ib = i0; ib < i1; ib += QK_U) {
            // the rows' indices first, then every load (past the wave's last
            // dim they repeat it, unused): all loads in flight before the first wait
            int jr[QK_U];
#pragma unroll
            for (int qq = 0; qq < QK_U; ++qq)
                jr[qq] = jd[min(ib + qq, i1 - 1)];
            uint4 u[QK_U];
#pragma unroll
            for (int qq = 0; qq < QK_U; ++qq)
                u[qq] = *reinterpret_cast<const uint4 *>(kbase + (int64_t)jr[qq] * kpitch);
#pragma unroll
            for (int qq = 0; qq < QK_U; ++qq) {
                if (ib + qq < i1) {
                    float v[8];
                    Vec16<uint16_t>::unpack(u[qq], v);
#pragma unroll
                    for (int hh = 0; hh < GS; ++hh) {
                        const float qv = qs[hh][ib + qq];
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[hh][e] = fmaf(qv, v[e], acc[hh][e]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            part[w][hh][lane * 8 + e] = acc[hh][e];
    __syncthreads();

    // 3. logits (the waves' partials added in wave order) and per-chunk softmax
    // statistics (max, sum exp) per head; wave w handles heads w, w + NWQ, ...
    for (int hh = w; hh < GS; hh += NWQ) {
        float a8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = part[0][hh][lane * 8 + e];
#pragma unroll
            for (int ww = 1; ww < NWQ; ++ww)
                x += part[ww][hh][lane * 8 + e];
            a8[e] = x;
        }
        if (act) {
            float *dst = logit + ((int64_t)b * s.Hq + h0 + hh) * Sp + sp;
            reinterpret_cast<f32x4_t *>(dst)[0] = f32x4_t{a8[0], a8[1], a8[2], a8[3]};
            reinterpret_cast<f32x4_t *>(dst)[1] = f32x4_t{a8[4], a8[5], a8[6], a8[7]};
        }
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (sp + e < Sb)
                mx = fmaxf(mx, a8[e]);
        mx = wave_max(mx);
        float z = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (sp + e < Sb)
                z += expf(s.scale * (a8[e] - mx));
        z = wave_sum(z);
        if (lane == 0)
            pstat[((int64_t)b * s.Hq + h0 + hh) * nchunk + chunk] = make_float2(mx, z);
    }

    // 4. the first chunk's workgroup clears the group's key histogram for the key kernel
    if (chunk == 0)
        for (int i = tid; i < ATTN_HIST_BINS; i += QK_THREADS)
            hist[(int64_t)grp * ATTN_HIST_BINS + i] = 0;
}

// ------------------------------------------------------------------ position scores
// A position's selection score is L' = max over the group's heads of the
// log-probability scale*a_h[s] - lse_h (the log of max_h p_h[s]), plus
// log vn[s] - 8 when the score is weighted by the value-row norm (the shift puts
// log(p * ||V_s||) of typical rows in the same window as log p).  Every kernel
// evaluates it with this one function, in IEEE double without contraction, so a
// position gets the same value wherever it is scored.
template <int GS>
__device__ __forceinline__ double pos_score(const float (&a)[GS], const double (&lse)[GS], double sc, bool has_vn,
                                            float vnv)
{
#pragma clang fp contract(off)
    double lp = sc * (double)a[0] - lse[0];
#pragma unroll
    for (int hh = 1; hh < GS; ++hh)
        lp = fmax(lp, sc * (double)a[hh] - lse[hh]);
    if (has_vn)
        lp += log((double)vnv) - 8.0;
    return lp;
}

// Order key of a score: floor((L' + 1056) * 2^52), clamped to 64 bits and
// non-decreasing in L'.  Over [-1056, 1024) its step (2^-52 nat) is finer than
// the doubles it is computed from; every score below -1056 maps to 0 (the
// probabilities there underflow to 0 in double as well).
constexpr uint64_t KEY_NAT = 1ull << 52;
constexpr uint64_t KEY_M32 = 1024ull * KEY_NAT; // L' = -32
constexpr uint64_t KEY_0 = 1056ull * KEY_NAT;   // L' = 0
__device__ __forceinline__ uint64_t pos_key(double lp)
{
#pragma clang fp contract(off)
    const double y = (lp + 1056.0) * 4503599627370496.0;
    if (!(y > 0.0))
        return 0ull;
    if (y >= 18446744073709549568.0) // the largest double below 2^64
        return ~0ull;
    return (uint64_t)y;
}

// Histogram bin of a key (ATTN_HIST_BINS = 8192 bins, non-decreasing in the
// key): [0, 2048) half-nat bins for L' in [-1056, -32); [2048, 6144) bins of
// 1/128 nat for L' in [-32, 0), where the threshold of a decode softmax usually
// lies; [6144, 8192) half-nat bins for L' >= 0, the last one open-ended.
__device__ __forceinline__ uint32_t key_bin(uint64_t k)
{
    if (k < KEY_M32)
        return (uint32_t)(k >> 51);
    if (k < KEY_0)
        return 2048u + (uint32_t)((k - KEY_M32) >> 45);
    const uint64_t t = (k - KEY_0) >> 51;
    return t < 2047u ? 6144u + (uint32_t)t : 8191u;
}

// Rank key of a position whose key lies in bin d: the key's offset inside the
// bin cut to 39 bits (a step of at most 2^-28 nat), then the complemented
// position in the low 24 bits.  A larger rank key comes earlier in the
// selection order (score descending, then position ascending), no two positions
// share one, and every rank key is below 2^63.
__device__ __forceinline__ uint64_t rank_key(uint64_t k, uint32_t d, int pos)
{
    uint64_t base;
    int sh;
    if (d < 2048u) {
        base = (uint64_t)d << 51;
        sh = 12;
    } else if (d < 6144u) {
        base = KEY_M32 + ((uint64_t)(d - 2048u) << 45);
        sh = 6;
    } else if (d < 8191u) {
        base = KEY_0 + ((uint64_t)(d - 6144u) << 51);
        sh = 12;
    } else {
        base = KEY_0 + (2047ull << 51);
        sh = 24;
    }
    return (((k - base) >> sh) << 24) | (uint64_t)(0xffffffu - (uint32_t)pos);
}

// ------------------------------------------------------------------ keys
// Every workgroup merges the group's chunk statistics into lse (double, fixed
// order), scores its positions, stores each position's histogram bin (2 bytes)
// and adds the bins to the group's histogram (LDS, then global atomics; the QK
// kernel cleared it).
template <int GS>
__global__ __launch_bounds__(256) void attn_key_kernel(AttnShape s, KvMap m, int Sp, int nqk_all, int nsub,
                                                       const float *__restrict__ logit,
                                                       const float2 *__restrict__ pstat, double *__restrict__ lse_ws,
                                                       float *__restrict__ lse_out, const float *__restrict__ vn,
                                                       uint16_t *__restrict__ bins, uint32_t *__restrict__ hist)
{
    __shared__ uint32_t lh[ATTN_HIST_BINS];
    __shared__ float smax[GS][4];
    __shared__ double ssum[GS][4];
    __shared__ double lse_s[GS];
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int grp = blockIdx.y, b = grp / s.Hsel, sg = grp % s.Hsel, h0 = sg * s.GS;
    const int Sb = seq_len(s, m, b);
    // the workgroup takes nsub consecutive chunks of ATTN_KEY_CHUNK positions
    // (long sequences: fewer workgroups, fewer statistics merges and fewer
    // global histogram atomics)
    const int c0 = blockIdx.x * nsub;
    if (c0 * ATTN_KEY_CHUNK >= Sb)
        return;
    const int nqk = (Sb + ATTN_QK_CHUNK - 1) / ATTN_QK_CHUNK; // this sequence's QK chunks
    for (int i = tid; i < ATTN_HIST_BINS; i += 256)
        lh[i] = 0;
    // this thread's logits are loaded first so their latency overlaps the statistics merge
    f32x4_t a[GS][2], an[GS][2];
    auto load_logits = [&](f32x4_t (&dst)[GS][2], int sp) {
        if (sp < Sb) {
#pragma unroll
            for (int hh = 0; hh < GS; ++hh) {
                const f32x4_t *src = reinterpret_cast<const f32x4_t *>(logit + ((int64_t)b * s.Hq + h0 + hh) * Sp + sp);
                dst[hh][0] = src[0];
                dst[hh][1] = src[1];
            }
        }
    };
    load_logits(a, c0 * ATTN_KEY_CHUNK + threadIdx.x * 8);
    // merge the per-chunk softmax statistics of the group's heads into lse (double, fixed order)
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
        const float2 *ps = pstat + ((int64_t)b * s.Hq + h0 + hh) * nqk_all;
        float mx = -INFINITY;
        for (int i = tid; i < nqk; i += 256)
            mx = fmaxf(mx, ps[i].x);
        mx = wave_max(mx);
        if (lane == 0)
            smax[hh][w] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
        const float M = fmaxf(fmaxf(smax[hh][0], smax[hh][1]), fmaxf(smax[hh][2], smax[hh][3]));
        const float2 *ps = pstat + ((int64_t)b * s.Hq + h0 + hh) * nqk_all;
        double z = 0.0;
        for (int i = tid; i < nqk; i += 256) {
            const float2 st = ps[i];
            z += (double)st.y * exp((double)s.scale * ((double)st.x - (double)M));
        }
        z = wave_sum(z);
        if (lane == 0)
            ssum[hh][w] = z;
    }
    __syncthreads();
    if (tid < GS) {
        const float M = fmaxf(fmaxf(smax[tid][0], smax[tid][1]), fmaxf(smax[tid][2], smax[tid][3]));
        const double z = ((ssum[tid][0] + ssum[tid][1]) + ssum[tid][2]) + ssum[tid][3];
        const double l = (double)s.scale * (double)M + log(z);
        lse_s[tid] = l;
        if (blockIdx.x == 0) {
            lse_ws[(int64_t)b * s.Hq + h0 + tid] = l;
            if (lse_out)
                lse_out[(int64_t)b * s.Hq + h0 + tid] = (float)l;
        }
    }
    __syncthreads();
    double lse[GS];
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
        lse[hh] = lse_s[hh];
    const double sc = (double)s.scale;
    for (int sub = 0; sub < nsub; ++sub) {
        const int sp = (c0 + sub) * ATTN_KEY_CHUNK + threadIdx.x * 8;
        if (sp >= Sb)
            break; // (per thread: later chunks start further on)
        if (sub + 1 < nsub)
            load_logits(an, sp + ATTN_KEY_CHUNK); // the next chunk's logits load while this one is scored
        // value-row norms of the 8 positions (one page or row: pitches and pages are multiples of 8)
        f32x4_t nv[2] = {{1.f, 1.f, 1.f, 1.f}, {1.f, 1.f, 1.f, 1.f}};
        if (vn) {
            const f32x4_t *src = reinterpret_cast<const f32x4_t *>(vn + kv_row(s, m, b, h0 / s.G, sp));
            nv[0] = src[0];
            nv[1] = src[1];
        }
        uint32_t bn[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float av[GS];
#pragma unroll
            for (int hh = 0; hh < GS; ++hh)
                av[hh] = a[hh][e >> 2][e & 3];
            const uint32_t bb = key_bin(pos_key(pos_score<GS>(av, lse, sc, vn != nullptr, nv[e >> 2][e & 3])));
            if (sp + e < Sb) {
                atomicAdd(&lh[bb], 1u);
                bn[e] = bb;
            } else {
                bn[e] = 0u; // past the sequence's end: never read as a position
            }
        }
        *reinterpret_cast<uint4 *>(bins + (int64_t)grp * Sp + sp) =
            make_uint4(bn[0] | bn[1] << 16, bn[2] | bn[3] << 16, bn[4] | bn[5] << 16, bn[6] | bn[7] << 16);
#pragma unroll
        for (int hh = 0; hh < GS; ++hh) {
            a[hh][0] = an[hh][0];
            a[hh][1] = an[hh][1];
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < ATTN_HIST_BINS; i += 256)
        if (lh[i])
            atomicAdd(&hist[(int64_t)grp * ATTN_HIST_BINS + i], lh[i]);
}

// ------------------------------------------------------------------ position selection helpers
constexpr int ASEL_THREADS = 512;       // threshold workgroup (one per group)
constexpr int PV_THREADS = 256;
constexpr int PV_WAVES = PV_THREADS / WAVE;
constexpr int PV_PASS = 2 * PV_THREADS; // positions per PV pass (2 per thread)
constexpr int PV_MAX_CHUNKS = 64;
constexpr int PV_U = 16;                // kept V rows in flight per lane
constexpr int SEL_CAP = 2048;           // candidates of the threshold bin ranked in LDS
constexpr int SEL_FEW = 64;             // a radix digit with at most this many keys is ranked by one wave

// The krem-th largest (1-based) of a set of distinct keys below 2^63, which
// each_key(f) visits (every thread calls f(key) for its share of the set): 8-bit
// radix digits from the top; once the crossing digit holds at most SEL_FEW keys
// they are gathered and wave 0 ranks them.  Every thread of the block calls it.
struct RadixLds {
    uint32_t h[256];
    uint32_t tmp[64];
    uint64_t few[SEL_FEW];
    uint32_t nfew;
    uint32_t res[3];
    uint64_t found;
};
template <typename EachKey>
__device__ uint64_t radix_select_u64(EachKey each_key, uint32_t krem, RadixLds &R)
{
    const int tid = threadIdx.x, lane = tid & (WAVE - 1);
    uint64_t prefix = 0, pmask = 0;
    for (int shift = 56;; shift -= 8) {
        for (int i = tid; i < 256; i += blockDim.x)
            R.h[i] = 0;
        if (tid == 0) {
            R.res[0] = 0;
            R.res[1] = 1;
            R.res[2] = 0;
        }
        __syncthreads();
        each_key([&](uint64_t key) {
            if ((key & pmask) == prefix)
                atomicAdd(&R.h[(uint32_t)(key >> shift) & 255u], 1u);
        });
        __syncthreads();
        // crossing digit in descending order: thread t < 256 holds digit 255 - t
        const uint32_t cnt = tid < 256 ? R.h[255 - tid] : 0u;
        const uint32_t incl = block_incl_scan(cnt, R.tmp);
        if (tid < 256 && incl - cnt < krem && krem <= incl) {
            R.res[0] = 255u - (uint32_t)tid;
            R.res[1] = krem - (incl - cnt);
            R.res[2] = cnt;
        }
        __syncthreads();
        const uint32_t dig = R.res[0], n = R.res[2];
        krem = R.res[1];
        prefix |= (uint64_t)dig << shift;
        pmask |= 0xffull << shift;
        __syncthreads();
        if (n <= (uint32_t)SEL_FEW || shift == 0) {
            if (tid == 0) {
                R.nfew = 0;
                R.found = 0;
            }
            __syncthreads();
            each_key([&](uint64_t key) {
                if ((key & pmask) == prefix) {
                    const uint32_t sl = atomicAdd(&R.nfew, 1u);
                    if (sl < (uint32_t)SEL_FEW)
                        R.few[sl] = key;
                }
            });
            __syncthreads();
            if (tid < WAVE) {
                const uint32_t nn = min(R.nfew, (uint32_t)SEL_FEW);
                const uint64_t me = (uint32_t)lane < nn ? R.few[lane] : 0ull;
                uint32_t above = 0;
                for (uint32_t j = 0; j < nn; ++j)
                    above += R.few[j] > me ? 1u : 0u;
                if ((uint32_t)lane < nn && above + 1u == krem)
                    R.found = me;
            }
            __syncthreads();
            return R.found;
        }
    }
}

// ------------------------------------------------------------------ select
// One workgroup per group finds the group's exact threshold: the 8192-bin
// histogram of scores gives the bin d holding the ks-th largest score and its
// rank krem inside the bin; one pass over the 2-byte bins of all positions
// gathers bin d's positions, whose rank keys (recomputed from the logits) are
// radix-selected for the krem-th largest.  Past SEL_CAP candidates the radix
// passes recompute the rank keys instead of holding them in LDS.  Output per
// group: (d, threshold rank key).  A position is kept iff its bin is above d,
// or it is in bin d with a rank key at least the threshold's: exactly the ks
// first positions of the order (score descending, position ascending).
struct AttnSel {
    uint32_t d, pad;
    uint64_t thr;
};
struct SelLds {
    uint64_t key[SEL_CAP];
    int32_t pos[SEL_CAP];
    RadixLds rad;
    uint32_t tmp[64];
    uint32_t ncand;
    uint32_t bres[3];
};

template <int GS>
__global__ __launch_bounds__(ASEL_THREADS) void attn_select_kernel(AttnShape s, KvMap m, int Sp,
                                                                   const float *__restrict__ logit,
                                                                   const double *__restrict__ lse_ws,
                                                                   const uint16_t *__restrict__ bins,
                                                                   const uint32_t *__restrict__ hist,
                                                                   const float *__restrict__ vn,
                                                                   AttnSel *__restrict__ sel)
{
    __shared__ SelLds L;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1);
    const int grp = blockIdx.x, b = grp / s.Hsel, sg = grp % s.Hsel, h0 = sg * s.GS, g = h0 / s.G;
    const int Sb = seq_len(s, m, b), ksb = seq_keep(s, m, Sb);
    const float *Lg = logit + ((int64_t)b * s.Hq + h0) * Sp; // head hh at Lg + hh * Sp
    const uint4 *B4 = reinterpret_cast<const uint4 *>(bins + (int64_t)grp * Sp);
    const int n8 = (Sb + 7) / 8; // 8-position groups of bins
    const double sc = (double)s.scale;
    double lsed[GS];
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
        lsed[hh] = lse_ws[(int64_t)b * s.Hq + h0 + hh];
    // rank key of position p (its bin is d): score recomputed from the logits
    auto rank_of = [&](int p, uint32_t d) -> uint64_t {
        float av[GS];
#pragma unroll
        for (int hh = 0; hh < GS; ++hh)
            av[hh] = Lg[(int64_t)hh * Sp + p];
        const float vv = vn ? vn[kv_row(s, m, b, g, p)] : 1.0f;
        return rank_key(pos_key(pos_score<GS>(av, lsed, sc, vn != nullptr, vv)), d, p);
    };

    // the histogram's loads, then the first batch of bins (it does not depend on the
    // threshold bin), so both are in flight together
    static_assert(ATTN_HIST_BINS == 16 * ASEL_THREADS, "16 histogram bins per thread");
    constexpr int UB = 4; // 16-byte loads of bins in flight per thread
    uint4 q[4];
    {
        const uint4 *h4 = reinterpret_cast<const uint4 *>(hist + (int64_t)grp * ATTN_HIST_BINS + ATTN_HIST_BINS -
                                                          16 * (tid + 1));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            q[i] = h4[i];
    }
    uint4 u[UB];
#pragma unroll
    for (int j = 0; j < UB; ++j) {
        const int i = tid + j * ASEL_THREADS;
        u[j] = i < n8 ? B4[i] : make_uint4(0u, 0u, 0u, 0u);
    }
    // threshold bin: thread t holds bins 8191-16t down to 8176-16t
    uint32_t hc[16];
    {
        const uint32_t asc[16] = {q[0].x, q[0].y, q[0].z, q[0].w, q[1].x, q[1].y, q[1].z, q[1].w,
                                  q[2].x, q[2].y, q[2].z, q[2].w, q[3].x, q[3].y, q[3].z, q[3].w};
#pragma unroll
        for (int i = 0; i < 16; ++i)
            hc[i] = asc[15 - i];
    }
    if (tid == 0) {
        L.bres[0] = 0;
        L.bres[1] = 1;
        L.bres[2] = 0;
        L.ncand = 0;
    }
    uint32_t tot = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        tot += hc[i];
    const uint32_t incl = block_incl_scan(tot, L.tmp); // (barriers inside)
    {
        const uint32_t top = ATTN_HIST_BINS - 1 - 16 * tid, want = (uint32_t)ksb;
        uint32_t run = incl - tot;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (run < want && want <= run + hc[i]) {
                L.bres[0] = top - i;
                L.bres[1] = want - run;
                L.bres[2] = hc[i];
            }
            run += hc[i];
        }
    }
    __syncthreads();
    const uint32_t d = L.bres[0], krem = L.bres[1], nbin = L.bres[2];

    uint64_t thr;
    if (nbin <= (uint32_t)SEL_CAP) {
        // gather bin d's positions: per-lane bit masks, one slot reservation per wave
        for (int i0 = tid; i0 - lane < n8; i0 += UB * ASEL_THREADS) {
            if (i0 != tid) {
#pragma unroll
                for (int j = 0; j < UB; ++j) {
                    const int i = i0 + j * ASEL_THREADS;
                    u[j] = i < n8 ? B4[i] : make_uint4(0u, 0u, 0u, 0u);
                }
            }
            uint32_t cm = 0;
#pragma unroll
            for (int j = 0; j < UB; ++j) {
                const uint32_t wd[4] = {u[j].x, u[j].y, u[j].z, u[j].w};
                const int pb = 8 * (i0 + j * ASEL_THREADS);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t bn = (e & 1) ? wd[e >> 1] >> 16 : wd[e >> 1] & 0xffffu;
                    cm |= (uint32_t)((bn == d) & (pb + e < Sb)) << (8 * j + e);
                }
            }
            const uint32_t cl = (uint32_t)__popc(cm);
            const uint32_t cincl = wave_incl_sum(cl);
            const uint32_t wcount = (uint32_t)__builtin_amdgcn_readlane((int)cincl, WAVE - 1);
            uint32_t base = 0;
            if (lane == 0 && wcount != 0u)
                base = atomicAdd(&L.ncand, wcount);
            base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
            uint32_t slot = base + cincl - cl;
            while (cm) {
                const int bit = __builtin_ctz(cm);
                cm &= cm - 1u;
                if (slot < (uint32_t)SEL_CAP)
                    L.pos[slot] = 8 * (i0 + (bit >> 3) * ASEL_THREADS) + (bit & 7);
                ++slot;
            }
        }
        __syncthreads();
        const int nc = (int)min(L.ncand, (uint32_t)SEL_CAP);
        for (int i = tid; i < nc; i += ASEL_THREADS)
            L.key[i] = rank_of(L.pos[i], d);
        __syncthreads();
        thr = radix_select_u64(
            [&](auto f) {
                for (int i = tid; i < nc; i += ASEL_THREADS)
                    f(L.key[i]);
            },
            krem, L.rad);
    } else {
        // a crowded bin: every radix pass recomputes the rank keys of bin d's positions
        thr = radix_select_u64(
            [&](auto f) {
                for (int i = tid; i < n8; i += ASEL_THREADS) {
                    const uint4 w4 = B4[i];
                    const uint32_t wd[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t bn = (e & 1) ? wd[e >> 1] >> 16 : wd[e >> 1] & 0xffffu;
                        const int p = 8 * i + e;
                        if (bn == d && p < Sb)
                            f(rank_of(p, d));
                    }
                }
            },
            krem, L.rad);
    }
    if (tid == 0) {
        AttnSel r;
        r.d = d;
        r.pad = 0;
        r.thr = thr;
        sel[grp] = r;
    }
}

// ------------------------------------------------------------------ pv
// One workgroup per (chunk of P positions, group), 4 waves.  The group's
// threshold and the first pass's bins and logits are loaded together; each
// pass examines PV_PASS positions (2 per thread), keeps those at or above the
// threshold (bin above d, or bin d with a rank key at least the threshold's,
// recomputed from the logits already loaded), stages their V rows and
// probabilities in LDS in position order, and streams the rows, 16 in flight
// per lane (a 16-lane quarter wave per 256-byte row), into p * V partial sums.
template <int GS>
__global__ __launch_bounds__(PV_THREADS) void attn_pv_kernel(AttnShape s, KvMap m, int Sp, int P,
                                                             const uint16_t *__restrict__ v,
                                                             const float *__restrict__ logit,
                                                             const double *__restrict__ lse_ws,
                                                             const uint16_t *__restrict__ bins,
                                                             const float *__restrict__ vn,
                                                             const AttnSel *__restrict__ sel,
                                                             int32_t *__restrict__ pstage,
                                                             uint32_t *__restrict__ pcount, float *__restrict__ part)
{
    __shared__ int64_t rows[PV_PASS]; // V row index of each kept position of the pass
    __shared__ float pr[GS][PV_PASS];
    __shared__ uint32_t wk[PV_WAVES];
    __shared__ float red[PV_WAVES][GS][D];
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int grp = blockIdx.y, b = grp / s.Hsel, sg = grp % s.Hsel, h0 = sg * s.GS, g = h0 / s.G;
    const int c = blockIdx.x, npv = gridDim.x;
    const int Sb = seq_len(s, m, b);
    const int p0 = c * P, p1 = min(Sb, p0 + P);
    const float *Lg = logit + ((int64_t)b * s.Hq + h0) * Sp;
    const uint16_t *Bn = bins + (int64_t)grp * Sp;
    const double sc = (double)s.scale;
    float acc[GS][8];
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[hh][e] = 0.0f;
    uint32_t chunk_kept = 0;
    if (p0 < p1) { // (uniform over the workgroup) chunks past the sequence's end write zeros
        // this thread's positions of the first pass, loaded with the threshold
        auto load_pass = [&](int sb, uint32_t &bw, float2 (&lg)[GS], int64_t &vrow) {
            const int j0 = sb + 2 * tid;
            bw = 0;
            vrow = 0;
#pragma unroll
            for (int hh = 0; hh < GS; ++hh)
                lg[hh] = make_float2(0.0f, 0.0f);
            if (j0 < p1) {
                vrow = kv_row(s, m, b, g, j0);
                bw = *reinterpret_cast<const uint32_t *>(Bn + j0);
#pragma unroll
                for (int hh = 0; hh < GS; ++hh)
                    lg[hh] = *reinterpret_cast<const float2 *>(Lg + (int64_t)hh * Sp + j0);
            }
        };
        uint32_t bw;
        float2 lg[GS];
        int64_t vrow;
        load_pass(p0, bw, lg, vrow);
        const AttnSel st = sel[grp];
        double lsed[GS];
        float lsef[GS];
#pragma unroll
        for (int hh = 0; hh < GS; ++hh) {
            lsed[hh] = lse_ws[(int64_t)b * s.Hq + h0 + hh];
            lsef[hh] = (float)lsed[hh];
        }
        const uint32_t d = st.d;
        const uint64_t thr = st.thr;
        const int quarter = lane >> 4, dl = lane & 15, slot = w * 4 + quarter;
        constexpr int NSLOT = PV_WAVES * 4;
        for (int sb = p0; sb < p1; sb += PV_PASS) {
            if (sb != p0)
                load_pass(sb, bw, lg, vrow);
            // thread tid holds positions j0, j0 + 1 (j0 even and Sp a multiple of 8: j0 < Sb keeps both in
            // the row; pages hold a multiple of 8 positions, so both share j0's page)
            const int j0 = sb + 2 * tid;
            const uint32_t ba = bw & 0xffffu, bb = bw >> 16;
            uint32_t ka = (uint32_t)(j0 < p1) & (uint32_t)(ba > d);
            uint32_t kb = (uint32_t)(j0 + 1 < p1) & (uint32_t)(bb > d);
            if (j0 < p1 && ba == d) {
                float av[GS];
#pragma unroll
                for (int hh = 0; hh < GS; ++hh)
                    av[hh] = lg[hh].x;
                const float vv = vn ? vn[vrow] : 1.0f;
                ka = rank_key(pos_key(pos_score<GS>(av, lsed, sc, vn != nullptr, vv)), d, j0) >= thr;
            }
            if (j0 + 1 < p1 && bb == d) {
                float av[GS];
#pragma unroll
                for (int hh = 0; hh < GS; ++hh)
                    av[hh] = lg[hh].y;
                const float vv = vn ? vn[vrow + 1] : 1.0f;
                kb = rank_key(pos_key(pos_score<GS>(av, lsed, sc, vn != nullptr, vv)), d, j0 + 1) >= thr;
            }
            const uint32_t ki = wave_incl_sum(ka + kb);
            if (lane == WAVE - 1)
                wk[w] = ki;
            __syncthreads();
            uint32_t before = 0, nkept = 0;
#pragma unroll
            for (int i = 0; i < PV_WAVES; ++i) {
                before += i < w ? wk[i] : 0u;
                nkept += wk[i];
            }
            const uint32_t sa = before + ki - (ka + kb), sbb = sa + ka; // pass-local slots
            if (ka) {
                rows[sa] = vrow;
#pragma unroll
                for (int hh = 0; hh < GS; ++hh)
                    pr[hh][sa] = expf(fmaf(s.scale, lg[hh].x, -lsef[hh]));
                if (pstage)
                    pstage[(int64_t)grp * Sp + p0 + chunk_kept + sa] = j0;
            }
            if (kb) {
                rows[sbb] = vrow + 1;
#pragma unroll
                for (int hh = 0; hh < GS; ++hh)
                    pr[hh][sbb] = expf(fmaf(s.scale, lg[hh].y, -lsef[hh]));
                if (pstage)
                    pstage[(int64_t)grp * Sp + p0 + chunk_kept + sbb] = j0 + 1;
            }
            __syncthreads();
            const int nk = (int)nkept;
            for (int r0 = slot; r0 < nk; r0 += NSLOT * PV_U) {
                uint4 u[PV_U];
#pragma unroll
                for (int qq = 0; qq < PV_U; ++qq) {
                    const int r = r0 + NSLOT * qq;
                    if (r < nk)
                        u[qq] = *reinterpret_cast<const uint4 *>(v + rows[r] * D + dl * 8);
                }
#pragma unroll
                for (int qq = 0; qq < PV_U; ++qq) {
                    const int r = r0 + NSLOT * qq;
                    if (r < nk) {
                        float vv[8];
                        Vec16<uint16_t>::unpack(u[qq], vv);
#pragma unroll
                        for (int hh = 0; hh < GS; ++hh) {
                            const float pv = pr[hh][r];
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                acc[hh][e] = fmaf(pv, vv[e], acc[hh][e]);
                        }
                    }
                }
            }
            chunk_kept += nkept;
            __syncthreads();
        }
    }

    // reduce the four quarters of each wave, then the waves (fixed order)
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = acc[hh][e];
            x += __shfl_xor(x, 16, WAVE);
            x += __shfl_xor(x, 32, WAVE);
            acc[hh][e] = x;
        }
    if ((lane >> 4) == 0) {
#pragma unroll
        for (int hh = 0; hh < GS; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                red[w][hh][(lane & 15) * 8 + e] = acc[hh][e];
    }
    __syncthreads();
    float *mine = part + ((int64_t)grp * npv + c) * GS * D;
    for (int i = tid; i < GS * D; i += PV_THREADS) {
        const int hh = i / D, dd = i % D;
        float x = red[0][hh][dd];
#pragma unroll
        for (int ww = 1; ww < PV_WAVES; ++ww)
            x += red[ww][hh][dd];
        mine[i] = x;
    }
    if (pcount && tid == 0)
        pcount[(int64_t)grp * npv + c] = chunk_kept;
}

// out[b, h0 + hh, :] = sum over the PV chunks of the chunk partials, in a fixed
// order.  Workgroup = 64 consecutive outputs of one group (GS*D/64 workgroups
// per group, so the partials are read by many CUs at once); wave w sums the
// w-th quarter of the chunks in chunk order, then wave 0 adds the four wave
// sums in wave order.
constexpr int PVR_WAVES = 4;
template <int GS>
__global__ __launch_bounds__(PVR_WAVES * WAVE) void attn_pv_reduce_kernel(AttnShape s, int npv,
                                                                         const float *__restrict__ part,
                                                                         float *__restrict__ out)
{
    constexpr int PIECES = GS * D / WAVE;
    constexpr int MAXQ = (PV_MAX_CHUNKS + PVR_WAVES - 1) / PVR_WAVES;
    __shared__ float red[PVR_WAVES][WAVE];
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    const int grp = blockIdx.x / PIECES, i = (blockIdx.x % PIECES) * WAVE + lane;
    const float *pb = part + (int64_t)grp * npv * GS * D + i;
    const int c0 = npv * w / PVR_WAVES, c1 = npv * (w + 1) / PVR_WAVES;
    float vals[MAXQ];
#pragma unroll
    for (int q = 0; q < MAXQ; ++q)
        vals[q] = c0 + q < c1 ? pb[(int64_t)(c0 + q) * GS * D] : 0.0f;
    float a = 0.0f;
#pragma unroll
    for (int q = 0; q < MAXQ; ++q)
        a += vals[q];
    red[w][lane] = a;
    __syncthreads();
    if (w != 0)
        return;
    float sum = red[0][lane];
#pragma unroll
    for (int q = 1; q < PVR_WAVES; ++q)
        sum += red[q][lane];
    const int b = grp / s.Hsel, h0 = (grp % s.Hsel) * s.GS;
    out[((int64_t)b * s.Hq + h0 + i / D) * D + i % D] = sum;
}

// Kept-position lists: workgroup (chunk c, group) copies the chunk's staged
// kept positions (ascending) to the group's list after the kept positions of
// chunks 0 .. c-1; chunk 0 also fills the entries past a shorter sequence's
// keep count with -1.
__global__ __launch_bounds__(256) void attn_pos_kernel(AttnShape s, KvMap m, int Sp, int P,
                                                       const uint32_t *__restrict__ pcount,
                                                       const int32_t *__restrict__ pstage,
                                                       int32_t *__restrict__ pos_out)
{
    __shared__ uint32_t off_s;
    const int grp = blockIdx.y, c = blockIdx.x, npv = gridDim.x;
    const int tid = threadIdx.x;
    const int Sb = seq_len(s, m, grp / s.Hsel), ksb = seq_keep(s, m, Sb);
    const uint32_t *pc = pcount + (int64_t)grp * npv;
    if (tid < WAVE) { // npv <= PV_MAX_CHUNKS = 64: one chunk per lane
        const uint32_t x = tid < c ? pc[tid] : 0u;
        const uint32_t tot = wave_incl_sum(x);
        if (tid == WAVE - 1)
            off_s = tot;
    }
    __syncthreads();
    const uint32_t off = off_s, n = c * P < Sb ? pc[c] : 0u;
    int32_t *dst = pos_out + (int64_t)grp * s.ks;
    const int32_t *src = pstage + (int64_t)grp * Sp + (int64_t)c * P;
    for (uint32_t i = tid; i < n; i += 256)
        if (off + i < (uint32_t)s.ks)
            dst[off + i] = src[i];
    if (c == 0)
        for (int i = ksb + tid; i < s.ks; i += 256)
            dst[i] = -1;
}

// ------------------------------------------------------------------ host side
// PV chunks: at most PV_MAX_CHUNKS per group, each a whole number of passes.
static void pv_chunks(int64_t S, int *P, int *npv)
{
    int64_t n = (S + PV_PASS - 1) / PV_PASS;
    if (n > PV_MAX_CHUNKS)
        n = PV_MAX_CHUNKS;
    int64_t per = (S + n - 1) / n;
    per = (per + PV_PASS - 1) / PV_PASS * PV_PASS;
    *P = (int)per;
    *npv = (int)((S + per - 1) / per);
}

static inline char *align256(char *p) { return (char *)(((uintptr_t)p + 255) & ~(uintptr_t)255); }

size_t attn_ws_layout(const AttnShape &s, AttnWs *ws, char *base)
{
    const int64_t Sp = (s.S + 7) / 8 * 8;
    const int64_t nqk = (s.S + ATTN_QK_CHUNK - 1) / ATTN_QK_CHUNK;
    const int64_t G = s.B * s.Hsel;
    int P, npv;
    pv_chunks(s.S, &P, &npv);
    char *p = base + RMM_WS_HEADER_BYTES_INTERNAL;
    AttnWs w;
    w.logit = (float *)p;
    p = align256(p + (size_t)(s.B * s.Hq * Sp) * 4);
    w.pstat = (float2 *)p;
    p = align256(p + (size_t)(s.B * s.Hq * nqk) * 8);
    w.lse = (double *)p;
    p = align256(p + (size_t)(s.B * s.Hq) * 8);
    w.bins = (uint16_t *)p;
    p = align256(p + (size_t)(G * Sp) * 2);
    w.hist = (uint32_t *)p;
    p = align256(p + (size_t)(G * ATTN_HIST_BINS) * 4);
    w.pcount = (uint32_t *)p;
    p = align256(p + (size_t)(G * npv) * 4);
    w.sel = p;
    p = align256(p + (size_t)G * sizeof(AttnSel));
    w.pstage = (int32_t *)p;
    p = align256(p + (size_t)(G * Sp) * 4);
    w.pvpart = (float *)p;
    p = align256(p + (size_t)(G * npv * s.GS * D) * 4);
    if (ws)
        *ws = w;
    return (size_t)(p - base);
}

// Key chunks per workgroup: one up to 32K positions, more for longer sequences
// (at 128K x 4 sequences, 2048 workgroups of one chunk spent most of their time
// in global histogram atomics).
static int key_chunks_per_wg(int64_t S)
{
    const int64_t n = S / 32768;
    return n < 1 ? 1 : n > 4 ? 4 : (int)n;
}

template <int GS>
static hipError_t attn_run(const AttnShape &s, const KvMap &m, const uint16_t *q, const uint16_t *kt,
                           const uint16_t *v, const float *kn, const float *vn, float *out, int32_t *dim_idx, int32_t *pos_idx, float *lse,
                           const AttnWs &ws, hipStream_t st)
{
    const int Sp = (int)((s.S + 7) / 8 * 8);
    const int G = (int)(s.B * s.Hsel);
    const int nqk = (int)((s.S + ATTN_QK_CHUNK - 1) / ATTN_QK_CHUNK);
    int P, npv;
    pv_chunks(s.S, &P, &npv);
    AttnSel *sel = reinterpret_cast<AttnSel *>(ws.sel);
    attn_qk_kernel<GS><<<dim3(nqk, G), QK_THREADS, 0, st>>>(s, m, Sp, q, kt, kn, ws.logit, ws.pstat, dim_idx,
                                                             ws.hist);
    const int nkc = (int)((s.S + ATTN_KEY_CHUNK - 1) / ATTN_KEY_CHUNK);
    const int nsub = key_chunks_per_wg(s.S);
    attn_key_kernel<GS><<<dim3((nkc + nsub - 1) / nsub, G), 256, 0, st>>>(
        s, m, Sp, nqk, nsub, ws.logit, ws.pstat, ws.lse, lse, vn, ws.bins, ws.hist);
    attn_select_kernel<GS><<<G, ASEL_THREADS, 0, st>>>(s, m, Sp, ws.logit, ws.lse, ws.bins, ws.hist, vn, sel);
    attn_pv_kernel<GS><<<dim3(npv, G), PV_THREADS, 0, st>>>(s, m, Sp, P, v, ws.logit, ws.lse, ws.bins, vn, sel,
                                                            pos_idx ? ws.pstage : nullptr,
                                                            pos_idx ? ws.pcount : nullptr, ws.pvpart);
    attn_pv_reduce_kernel<GS><<<G * (GS * D / WAVE), PVR_WAVES * WAVE, 0, st>>>(s, npv, ws.pvpart, out);
    if (pos_idx)
        attn_pos_kernel<<<dim3(npv, G), 256, 0, st>>>(s, m, Sp, P, ws.pcount, ws.pstage, pos_idx);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnShape &s, const KvMap &m, const uint16_t *q, const uint16_t *kt, const uint16_t *v,
                       const float *kn, const float *vn, float *out, int32_t *dim_idx, int32_t *pos_idx, float *lse,
                       const AttnWs &ws, hipStream_t st)
{
    switch (s.GS) {
    case 1:
        return attn_run<1>(s, m, q, kt, v, kn, vn, out, dim_idx, pos_idx, lse, ws, st);
    case 2:
        return attn_run<2>(s, m, q, kt, v, kn, vn, out, dim_idx, pos_idx, lse, ws, st);
    case 4:
        return attn_run<4>(s, m, q, kt, v, kn, vn, out, dim_idx, pos_idx, lse, ws, st);
    case 8:
        return attn_run<8>(s, m, q, kt, v, kn, vn, out, dim_idx, pos_idx, lse, ws, st);
    default:
        return hipErrorInvalidValue;
    }
}

// ------------------------------------------------------------------ dense flash decode (r = 1 baseline)
// One workgroup per (span of positions, KV head): QK over all D dims (waves
// split the dims), online softmax over 512-position sub-chunks, P V; partial
// (max, sum, o) per span; a second launch rescales and sums them in a fixed order.
constexpr int DN_SUB = 512;
constexpr int DN_MAX_SPANS = 64;

template <int G>
__global__ __launch_bounds__(256) void attn_dense_kernel(AttnShape s, KvMap m, int span, const uint16_t *__restrict__ q,
                                                         const uint16_t *__restrict__ kt, const uint16_t *__restrict__ v,
                                                         float *__restrict__ part, float2 *__restrict__ stat)
{
    __shared__ float qs[G][D];
    __shared__ float lg[4][G][DN_SUB]; // per-wave partial dots, then wave 0's slot holds the sums
    __shared__ float red[4][G][D];
    __shared__ float mrun[G], zrun[G], fac[G];
    __shared__ int64_t vrow[DN_SUB]; // V row index of each position of the sub-chunk
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int grp = blockIdx.y, b = grp / s.Hkv, g = grp % s.Hkv, h0 = g * G;
    const int c = blockIdx.x, nspan = gridDim.x;
    for (int i = tid; i < G * D; i += 256)
        qs[i / D][i % D] = bf16_to_f32(q[((int64_t)b * s.Hq + h0) * D + i]);
    if (tid < G) {
        mrun[tid] = -INFINITY;
        zrun[tid] = 0.0f;
    }
    const int Sb = seq_len(s, m, b);
    const int quarter = lane >> 4, dl = lane & 15;
    float o[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            o[hh][e] = 0.0f;
    __syncthreads();
    const int p0 = c * span, p1 = min(Sb, p0 + span);
    for (int sb = p0; sb < p1; sb += DN_SUB) {
        // QK: wave w takes dims [32w, 32w+32) for 8 positions per lane
        const int sp = sb + lane * 8;
        float a[G][8];
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                a[hh][e] = 0.0f;
        for (int i = tid; i < min(DN_SUB, p1 - sb); i += 256)
            vrow[i] = kv_row(s, m, b, g, sb + i);
        if (sp < p1) {
            int64_t kpitch;
            const uint16_t *kb = kt + kt_off(s, m, b, g, sp, kpitch);
            for (int j0 = 32 * w; j0 < 32 * w + 32; j0 += 16) {
                uint4 u[16];
#pragma unroll
                for (int qq = 0; qq < 16; ++qq)
                    u[qq] = *reinterpret_cast<const uint4 *>(kb + (int64_t)(j0 + qq) * kpitch);
#pragma unroll
                for (int qq = 0; qq < 16; ++qq) {
                    float kv[8];
                    Vec16<uint16_t>::unpack(u[qq], kv);
#pragma unroll
                    for (int hh = 0; hh < G; ++hh) {
                        const float qv = qs[hh][j0 + qq];
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            a[hh][e] = fmaf(qv, kv[e], a[hh][e]);
                    }
                }
            }
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                lg[w][hh][lane * 8 + e] = a[hh][e];
        __syncthreads();
        // logits (scaled), sub-chunk max per head, new running max
        for (int i = tid; i < G * DN_SUB; i += 256) {
            const int hh = i / DN_SUB, r = i % DN_SUB;
            const float l = ((lg[0][hh][r] + lg[1][hh][r]) + lg[2][hh][r]) + lg[3][hh][r];
            lg[0][hh][r] = sb + r < p1 ? s.scale * l : -INFINITY;
        }
        __syncthreads();
        for (int hh = w; hh < G; hh += 4) {
            float m = -INFINITY;
            for (int r = lane; r < DN_SUB; r += WAVE)
                m = fmaxf(m, lg[0][hh][r]);
            m = wave_max(m);
            if (lane == 0) {
                const float mn = fmaxf(mrun[hh], m);
                fac[hh] = expf(mrun[hh] - mn);
                mrun[hh] = mn;
            }
        }
        __syncthreads();
        for (int i = tid; i < G * DN_SUB; i += 256) {
            const int hh = i / DN_SUB, r = i % DN_SUB;
            lg[1][hh][r] = expf(lg[0][hh][r] - mrun[hh]);
        }
        __syncthreads();
        for (int hh = w; hh < G; hh += 4) {
            float z = 0.0f;
            for (int r = lane; r < DN_SUB; r += WAVE)
                z += lg[1][hh][r];
            z = wave_sum(z);
            if (lane == 0)
                zrun[hh] = zrun[hh] * fac[hh] + z;
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o[hh][e] *= fac[hh];
        // P V over this sub-chunk's rows
        const int nr = min(DN_SUB, p1 - sb);
        // 8 rows in flight per lane: rows r0 + 16 qq
        for (int r0 = w * 4 + quarter; r0 < nr; r0 += 128) {
            uint4 u[8];
#pragma unroll
            for (int qq = 0; qq < 8; ++qq) {
                const int r = r0 + 16 * qq;
                if (r < nr)
                    u[qq] = *reinterpret_cast<const uint4 *>(v + vrow[r] * D + dl * 8);
            }
#pragma unroll
            for (int qq = 0; qq < 8; ++qq) {
                const int r = r0 + 16 * qq;
                if (r < nr) {
                    float vv[8];
                    Vec16<uint16_t>::unpack(u[qq], vv);
#pragma unroll
                    for (int hh = 0; hh < G; ++hh) {
                        const float p = lg[1][hh][r];
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            o[hh][e] = fmaf(p, vv[e], o[hh][e]);
                    }
                }
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = o[hh][e];
            x += __shfl_xor(x, 16, WAVE);
            x += __shfl_xor(x, 32, WAVE);
            o[hh][e] = x;
        }
    if (quarter == 0) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                red[w][hh][dl * 8 + e] = o[hh][e];
    }
    __syncthreads();
    float *mine = part + ((int64_t)grp * nspan + c) * G * D;
    for (int i = tid; i < G * D; i += 256) {
        const int hh = i / D, dd = i % D;
        mine[i] = ((red[0][hh][dd] + red[1][hh][dd]) + red[2][hh][dd]) + red[3][hh][dd];
    }
    if (tid < G)
        stat[((int64_t)grp * nspan + c) * G + tid] = make_float2(mrun[tid], zrun[tid]);
}

// Rescales every span's partial to the largest running max and sums them in
// span order.  One workgroup per (group, head), one thread per dim.  The
// partials (DN_MAX_SPANS deep) are loaded first, so they are in flight with the
// span statistics; wave 0 holds one span per lane, finds the largest max and
// sums the rescaled denominators with a fixed wave reduction.
template <int G>
__global__ __launch_bounds__(D) void attn_dense_reduce_kernel(AttnShape s, int nspan, const float *__restrict__ part,
                                                              const float2 *__restrict__ stat,
                                                              float *__restrict__ out, float *__restrict__ lse_out)
{
    __shared__ float fs[DN_MAX_SPANS];
    __shared__ float Ms, dens;
    const int grp = blockIdx.x, hh = blockIdx.y, b = grp / s.Hkv, g = grp % s.Hkv, h0 = g * G;
    const int dd = threadIdx.x;
    const float *pp = part + (int64_t)grp * nspan * G * D + hh * D + dd;
    float v[DN_MAX_SPANS];
#pragma unroll
    for (int cc = 0; cc < DN_MAX_SPANS; ++cc)
        v[cc] = cc < nspan ? pp[(int64_t)cc * G * D] : 0.0f;
    const float2 *st = stat + (int64_t)grp * nspan * G + hh;
    if (dd < WAVE) {
        // nspan <= DN_MAX_SPANS = 64
        const float2 mine = dd < nspan ? st[(int64_t)dd * G] : make_float2(-INFINITY, 0.0f);
        const float M = wave_max(mine.x);
        const float f = dd < nspan ? expf(mine.x - M) : 0.0f;
        fs[dd] = f;
        const float den = wave_sum(f * mine.y);
        if (dd == 0) {
            Ms = M;
            dens = den;
        }
    }
    __syncthreads();
    float num = 0.0f;
#pragma unroll
    for (int cc = 0; cc < DN_MAX_SPANS; ++cc)
        num += fs[cc] * v[cc];
    out[((int64_t)b * s.Hq + h0 + hh) * D + dd] = num / dens;
    if (lse_out && dd == 0)
        lse_out[(int64_t)b * s.Hq + h0 + hh] = Ms + logf(dens);
}

static void dense_spans(int64_t S, int *span, int *nspan)
{
    int64_t n = (S + DN_SUB - 1) / DN_SUB;
    if (n > DN_MAX_SPANS)
        n = DN_MAX_SPANS;
    int64_t per = (S + n - 1) / n;
    per = (per + DN_SUB - 1) / DN_SUB * DN_SUB;
    *span = (int)per;
    *nspan = (int)((S + per - 1) / per);
}

size_t attn_dense_ws_layout(int64_t B, int64_t Hq, int64_t S, char *base, float **part, float2 **stat)
{
    int span, nspan;
    dense_spans(S, &span, &nspan);
    char *p = base + RMM_WS_HEADER_BYTES_INTERNAL;
    if (part)
        *part = (float *)p;
    p = align256(p + (size_t)(B * Hq * nspan * D) * 4);
    if (stat)
        *stat = (float2 *)p;
    p = align256(p + (size_t)(B * Hq * nspan) * 8);
    return (size_t)(p - base);
}

hipError_t launch_attn_dense(const AttnShape &s, const KvMap &m, const uint16_t *q, const uint16_t *kt,
                             const uint16_t *v, float *out, float *lse, float *part, float2 *stat, hipStream_t st)
{
    int span, nspan;
    dense_spans(s.S, &span, &nspan);
    dim3 grid(nspan, (unsigned)(s.B * s.Hkv));
    const unsigned ng = (unsigned)(s.B * s.Hkv);
#define RMM_DENSE_CASE(GV)                                                                                         \
    case GV:                                                                                                       \
        attn_dense_kernel<GV><<<grid, 256, 0, st>>>(s, m, span, q, kt, v, part, stat);                             \
        attn_dense_reduce_kernel<GV><<<dim3(ng, GV), D, 0, st>>>(s, nspan, part, stat, out, lse);                   \
        break;
    switch (s.G) {
        RMM_DENSE_CASE(1)
        RMM_DENSE_CASE(2)
        RMM_DENSE_CASE(4)
        RMM_DENSE_CASE(8)
    default:
        return hipErrorInvalidValue;
    }
#undef RMM_DENSE_CASE
    return hipGetLastError();
}

void attn_init() {}

} // namespace rmm
