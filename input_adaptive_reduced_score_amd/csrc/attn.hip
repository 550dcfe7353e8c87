// Reduced grouped-query attention decode.
//
// Blog on input-adaptive matrix-product reduction: section 3.1 (most past keys
// matter little to the current query: skip low-contribution work along the
// sequence), section 3.3 (reduce inside each head, never drop a head);
// paper abstract (keep informative slices of each product's contraction
// dimension: head_dim for Q K^T, key positions for P V).  GEMM notes section 1:
// scores = Q K^T, out = softmax(scores) V.
//
// Pipeline per (batch element, selection group), five launches on one stream:
//  qk    : head_dim selection (one wave, bitwise search over ballots), then
//          unscaled logits over the kept dims for 8 positions per lane from
//          dim-major keys (a kept dim is one contiguous row), and per-chunk
//          softmax statistics (max, sum of exponentials); the first chunk's
//          workgroup clears the group's key histogram.
//  keys  : every workgroup merges the chunk statistics into lse (double), then
//          scores its positions by max_h (scale*a_h[s] - lse_h), stores each as
//          a fixed-point log-probability key and adds the top bits to a
//          4096-bin histogram.
//  select: one workgroup per group: threshold bin from the histogram, exact
//          ranking of the crossing bin's keys, then kept/tie counts per PV chunk.
//  pv    : each workgroup takes a chunk of positions, keeps the selected ones
//          (order-preserving), streams their V rows and accumulates p*V into
//          a per-chunk partial.
//  reduce: the chunk partials are summed in a fixed order.
#include "device.h"
#include "kernels.h"
#include "radix.h"

namespace rmm {

constexpr int D = ATTN_D;
constexpr int QK_U = 16;      // kept key rows in flight per lane
constexpr int QK_THREADS = 256; // 4 waves split the kept dims of one chunk
constexpr int PV_SUB = 512;   // positions examined per PV pass (2 per thread)
constexpr int PV_MAX_CHUNKS = 64;
constexpr int PV_U = 16;      // kept V rows in flight per lane

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

// ------------------------------------------------------------------ keys
// Position key: max over the group's heads of the log-probability
// scale*a_h[s] - lse_h (double), plus log ||V_s|| when the score is weighted by
// the value-row norm, as fixed point floor((L + off) * 2^25), clamped to 32 bits.
// off = 128 covers L in [-128, 0) (plain probabilities); off = 120 covers
// [-120, 8) (probability times a norm below e^8).
__device__ __forceinline__ uint32_t logprob_key(double L, double off)
{
    const double t = (L + off) * 33554432.0;
    if (!(t > 0.0))
        return 0u;
    if (t >= 4294967295.0)
        return 0xffffffffu;
    return (uint32_t)t;
}

// Histogram bin of a position key: 4096 bins of 1/128 nat over (L + off) in
// [96, 128), i.e. log-probabilities in [-32, 0) (or [-24, 8) with value norms);
// every key below that window falls into bin 0.  Bin d >= 1 holds exactly the
// keys with kk >> 18 == d + KEY_BIN_BASE.
constexpr uint32_t KEY_BIN_BASE = 96u << 7; // (96 * 2^25) >> 18
__device__ __forceinline__ uint32_t key_bin(uint32_t kk)
{
    const uint32_t t = kk >> 18;
    return t > KEY_BIN_BASE ? t - KEY_BIN_BASE : 0u;
}

template <int GS>
__global__ __launch_bounds__(256) void attn_key_kernel(AttnShape s, KvMap m, int Sp, int nqk_all, int nsub,
                                                       const float *__restrict__ logit,
                                                       const float2 *__restrict__ pstat, double *__restrict__ lse_ws,
                                                       float *__restrict__ lse_out, const float *__restrict__ vn,
                                                       uint32_t *__restrict__ keys, uint32_t *__restrict__ hist)
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
    __syncthreads();
    for (int sub = 0; sub < nsub; ++sub) {
        const int sp = (c0 + sub) * ATTN_KEY_CHUNK + threadIdx.x * 8;
        if (sp >= Sb)
            break; // (per thread: later chunks start further on)
        if (sub + 1 < nsub)
            load_logits(an, sp + ATTN_KEY_CHUNK); // the next chunk's logits load while this one is keyed
        uint32_t kk[8];
        const double sc = (double)s.scale;
        // value-row norms of the 8 positions (one page or row: pitches and pages are multiples of 8)
        f32x4_t nv[2] = {{1.f, 1.f, 1.f, 1.f}, {1.f, 1.f, 1.f, 1.f}};
        const double off = vn ? 120.0 : 128.0;
        if (vn) {
            const f32x4_t *src = reinterpret_cast<const f32x4_t *>(vn + kv_row(s, m, b, h0 / s.G, sp));
            nv[0] = src[0];
            nv[1] = src[1];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            double lp = sc * (double)a[0][e >> 2][e & 3] - lse[0];
#pragma unroll
            for (int hh = 1; hh < GS; ++hh)
                lp = fmax(lp, sc * (double)a[hh][e >> 2][e & 3] - lse[hh]);
            if (vn)
                lp += log((double)nv[e >> 2][e & 3]);
            kk[e] = logprob_key(lp, off);
            if (sp + e < Sb)
                atomicAdd(&lh[key_bin(kk[e])], 1u);
            else
                kk[e] = 0u; // past the sequence's end: the lowest key, in no bin above 0
        }
        uint4 *dst = reinterpret_cast<uint4 *>(keys + (int64_t)grp * Sp + sp);
        dst[0] = uint4{kk[0], kk[1], kk[2], kk[3]};
        dst[1] = uint4{kk[4], kk[5], kk[6], kk[7]};
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

// ------------------------------------------------------------------ select
// Threshold key thr and tie quota of the group, then per PV chunk c (P
// positions): info[c] = (kept before the chunk, ties at thr before the chunk).
// Fast path: the 4096-bin histogram (1/128 nat per bin, key_bin) names the bin
// d holding the k-th key; one pass over the keys counts, per chunk, the keys in
// higher bins and gathers the bin's keys (candidates) into LDS.  Up to
// SEL_RANK_MAX candidates are ranked exactly (key descending, position
// ascending); up to CAND_CAP the last 18 key bits are resolved by two radix
// passes over the candidates (ranking costs O(n^2) LDS reads); beyond that the
// radix passes and a counting pass run over all keys, over all 32 bits when the
// k-th key lies below the histogram's window (bin 0).
struct SelInfo {
    uint32_t thr, quota;
};
constexpr int CAND_CAP = 8192;
constexpr int SEL_RANK_MAX = 256;
constexpr int SEL_KB = 8; // 16-byte key loads in flight per thread

__global__ __launch_bounds__(1024) void attn_select_kernel(AttnShape s, KvMap m, int Sp, int P, int npv,
                                                           const uint32_t *__restrict__ keys,
                                                           const uint32_t *__restrict__ hist, SelInfo *__restrict__ sel,
                                                           uint2 *__restrict__ info, int32_t *__restrict__ pos_out)
{
    __shared__ uint32_t h2[SEL_BINS];
    __shared__ uint32_t tmp[64];
    __shared__ uint32_t cgt[PV_MAX_CHUNKS], ceq[PV_MAX_CHUNKS];
    __shared__ uint32_t ckey[CAND_CAP];
    __shared__ int cpos[CAND_CAP];
    __shared__ uint32_t rk_above[1024]; // one slot per thread: (part, candidate)
    __shared__ uint64_t ck64[SEL_RANK_MAX];
    __shared__ uint32_t ncand, nquota, res[2];
    const int grp = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const uint32_t *K = keys + (int64_t)grp * Sp;
    const uint32_t *H = hist + (int64_t)grp * ATTN_HIST_BINS;
    const int Sb = seq_len(s, m, grp / (int)s.Hsel);
    const int ksb = seq_keep(s, m, Sb);
    // a shorter sequence keeps fewer positions: the rest of its index row is -1
    if (pos_out)
        for (int i = ksb + tid; i < s.ks; i += 1024)
            pos_out[(int64_t)grp * s.ks + i] = -1;
    uint32_t krem = (uint32_t)ksb;
    // the histogram's loads first, then the first batch of keys (it does not depend on
    // the threshold bin), so the key loads stay in flight through the histogram phase
    static_assert(ATTN_HIST_BINS == 4 * 1024, "four histogram bins per thread");
    uint32_t hc[4];
    hist_counts<4>(H, hc);
    const uint4 *k4 = reinterpret_cast<const uint4 *>(K);
    const int n4 = (int)((Sb + 3) / 4), step = 1024;
    uint4 u[SEL_KB];
#pragma unroll
    for (int q = 0; q < SEL_KB; ++q) { // unconditional loads (an in-range address), zeroed past n4
        const int ii = tid + q * step;
        const uint4 t = k4[min(ii, n4 - 1)];
        const uint32_t keep = 0u - ilt(ii, n4);
        u[q] = make_uint4(t.x & keep, t.y & keep, t.z & keep, t.w & keep);
    }
    uint32_t nbin;
    const uint32_t d = crossing_from_counts<4>(hc, krem, tmp, &nbin);
    if (tid < PV_MAX_CHUNKS) {
        cgt[tid] = 0;
        ceq[tid] = 0;
    }
    if (tid == 0) {
        ncand = 0;
        nquota = 0;
        res[0] = 0;
        res[1] = 0;
    }
    __syncthreads();
    const uint32_t tD = d + KEY_BIN_BASE; // kk >> 18 of the crossing bin's keys (d >= 1)
    uint32_t thr, quota;
    if (d > 0 && nbin <= (uint32_t)CAND_CAP) {
        for (int i0 = tid; i0 - lane < n4; i0 += SEL_KB * step) {
            if (i0 != tid) {
#pragma unroll
                for (int q = 0; q < SEL_KB; ++q)
                    u[q] = i0 + q * step < n4 ? k4[i0 + q * step] : make_uint4(0u, 0u, 0u, 0u);
            }
            // predicates as integer arithmetic (bins are 14-bit): per element, in bin tD
            // (a candidate) or above it; candidates also as a bit mask.  Keys past the
            // sequence's end (up to the 8-position boundary the loads reach) are 0, in
            // neither; loads past n4 give 0 as well.
            uint32_t cl = 0, cmask = 0, ngt[SEL_KB];
#pragma unroll
            for (int q = 0; q < SEL_KB; ++q) {
                const uint32_t kk[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
                ngt[q] = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t top = kk[e] >> 18;
                    const uint32_t g = (tD - top) >> 31, ge = (tD - 1u - top) >> 31; // top > tD, top >= tD
                    const uint32_t c = ge - g;
                    cl += c;
                    cmask |= c << (4 * q + e);
                    ngt[q] += g;
                }
            }
            // candidates: per-lane count, wave scan, one slot reservation per wave
            const uint32_t cincl = wave_incl_sum(cl);
            const uint32_t wcount = (uint32_t)__builtin_amdgcn_readlane((int)cincl, WAVE - 1);
            uint32_t base = 0;
            if (lane == 0 && wcount != 0u)
                base = atomicAdd(&ncand, wcount);
            base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
            uint32_t slot = base + cincl - cl;
            while (cmask) { // rare: the bin holds ~1/100 of the keys
                const int b = __builtin_ctz(cmask);
                cmask &= cmask - 1u;
                const int q = b >> 2, e = b & 3;
                uint32_t kv = 0; // u[q] selected with compile-time indices (no private-memory copy of u)
#pragma unroll
                for (int qq = 0; qq < SEL_KB; ++qq)
                    if (qq == q)
                        kv = e == 0 ? u[qq].x : e == 1 ? u[qq].y : e == 2 ? u[qq].z : u[qq].w;
                if (slot < (uint32_t)CAND_CAP) {
                    ckey[slot] = kv;
                    cpos[slot] = 4 * (i0 + q * step) + e;
                }
                ++slot;
            }
            // keys above the bin, per PV chunk (one wave load covers 256 consecutive positions: one chunk)
#pragma unroll
            for (int q = 0; q < SEL_KB; ++q) {
                const int i = i0 + q * step;
                const uint32_t wgt = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_sum(ngt[q]), WAVE - 1);
                if (lane == 0 && wgt != 0u)
                    atomicAdd(&cgt[(4 * (i - lane)) / P], wgt);
            }
        }
        __syncthreads();
        const uint32_t nc = min(nbin, (uint32_t)CAND_CAP);
        if (nc <= (uint32_t)SEL_RANK_MAX) {
            // Rank by one 64-bit order key per candidate: the 18 key bits under the bin
            // (candidates share its top 14), then the complemented position (< 2^24), so
            // larger means earlier in the total order and no two are equal.  Thread t
            // counts the candidates above candidate t % 256 among every fourth one.
            const uint32_t kb = tD << 18;
            for (int i = tid; i < (int)nc; i += 1024)
                ck64[i] = ((uint64_t)(ckey[i] - kb) << 24) | (uint64_t)(0xffffffu - (uint32_t)cpos[i]);
            __syncthreads();
            constexpr uint32_t RS = SEL_RANK_MAX, split = 1024u / RS;
            const uint32_t me_i = (uint32_t)tid % RS, part = (uint32_t)tid / RS;
            if (me_i < nc) {
                const uint64_t mk = ck64[me_i];
                // 8 independent comparisons per step keep the LDS reads pipelined; a
                // difference of two keys below 2^42 has its top bit set iff the other is larger
                uint32_t ab[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                uint32_t i = part;
                for (; i + 7 * split < nc; i += 8 * split) {
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        ab[u] += (uint32_t)((mk - ck64[i + u * split]) >> 63);
                }
                for (; i < nc; i += split)
                    ab[0] += (uint32_t)((mk - ck64[i]) >> 63);
                rk_above[tid] = ((ab[0] + ab[1]) + (ab[2] + ab[3])) + ((ab[4] + ab[5]) + (ab[6] + ab[7]));
            }
            __syncthreads();
            if ((uint32_t)tid < nc) {
                uint32_t above = 0;
#pragma unroll
                for (uint32_t q = 0; q < split; ++q)
                    above += rk_above[q * RS + tid];
                if (above + 1u == krem) { // the krem-th candidate: the threshold key and its position
                    res[0] = ckey[tid];
                    res[1] = (uint32_t)cpos[tid];
                }
            }
            __syncthreads();
            thr = res[0];
            // quota: the threshold's rank among its ties, i.e. equal keys at positions <= its own
            const uint32_t pk = res[1];
            for (int i = tid; i < (int)nc; i += 1024)
                if (ckey[i] == thr && (uint32_t)cpos[i] <= pk)
                    atomicAdd(&nquota, 1u);
            __syncthreads();
            quota = nquota;
        } else {
            uint32_t prefix = tD << 18, pmask = 0xfffc0000u;
#pragma clang loop unroll(disable)
            for (int ps = 0; ps < 2; ++ps) // bits 9..17, then 0..8 (one copy of the pass: smaller code)
                radix_pass(ckey, (int)nc, prefix, pmask, 9 - 9 * ps, 9, krem, h2, tmp);
            thr = prefix;
            quota = krem;
        }
        for (int i = tid; i < (int)nc; i += 1024) {
            if (ckey[i] > thr)
                atomicAdd(&cgt[cpos[i] / P], 1u);
            else if (ckey[i] == thr)
                atomicAdd(&ceq[cpos[i] / P], 1u);
        }
    } else {
        // a crowded bin: the 18 bits under it (9 + 9); a threshold below the histogram's
        // window (bin 0): all 32 bits (11 + 11 + 10)
        const bool full = d == 0;
        uint32_t prefix = full ? 0u : tD << 18, pmask = full ? 0u : 0xfffc0000u;
        if (full)
            krem = (uint32_t)ksb;
        const int npass = full ? 3 : 2;
#pragma clang loop unroll(disable)
        for (int ps = 0; ps < npass; ++ps) {
            const int shift = full ? (ps == 0 ? 21 : ps == 1 ? 10 : 0) : (ps == 0 ? 9 : 0);
            const int nbits = full ? (ps == 2 ? 10 : 11) : 9;
            radix_pass_v4(K, Sb, prefix, pmask, shift, nbits, krem, h2, tmp);
        }
        thr = prefix;
        quota = krem;
        for (int i0 = tid; i0 - lane < n4; i0 += SEL_KB * step) {
            uint4 u[SEL_KB];
#pragma unroll
            for (int q = 0; q < SEL_KB; ++q)
                u[q] = i0 + q * step < n4 ? k4[i0 + q * step] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int q = 0; q < SEL_KB; ++q) {
                const int i = i0 + q * step;
                const uint32_t kk[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
                uint32_t ngt = 0, neq = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool ok = 4 * i + e < Sb;
                    ngt += ok & (kk[e] > thr);
                    neq += ok & (kk[e] == thr);
                }
                const uint32_t wgt = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_sum(ngt), WAVE - 1);
                const uint32_t weq = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_sum(neq), WAVE - 1);
                if (lane == 0) {
                    if (wgt)
                        atomicAdd(&cgt[(4 * (i - lane)) / P], wgt);
                    if (weq)
                        atomicAdd(&ceq[(4 * (i - lane)) / P], weq);
                }
            }
        }
    }
    __syncthreads();
    if (w == 0) {
        // per chunk: kept and tied positions before it (npv <= 64 chunks: one lane each, DPP scans)
        const uint32_t cg = lane < npv ? cgt[lane] : 0u, ce = lane < npv ? ceq[lane] : 0u;
        const uint32_t gex = wave_incl_sum(cg) - cg, eex = wave_incl_sum(ce) - ce;
        if (lane < npv)
            info[(int64_t)grp * npv + lane] = make_uint2(gex + min(eex, quota), eex);
        if (lane == 0) {
            sel[grp].thr = thr;
            sel[grp].quota = quota;
        }
    }
}

// ------------------------------------------------------------------ pv
// One workgroup per (chunk of P positions, group).  4 waves; each wave
// quarter (16 lanes) holds one 256-byte V row, 8 dims per lane.
template <int GS>
__global__ __launch_bounds__(256) void attn_pv_kernel(AttnShape s, KvMap m, int Sp, int P, const uint16_t *__restrict__ v,
                                                      const float *__restrict__ logit, const double *__restrict__ lse_ws,
                                                      const uint32_t *__restrict__ keys, const SelInfo *__restrict__ sel,
                                                      const uint2 *__restrict__ info, int32_t *__restrict__ pos_out,
                                                      float *__restrict__ part)
{
    __shared__ int64_t rows[PV_SUB]; // V row index of each kept position of the pass
    __shared__ float pr[GS][PV_SUB];
    __shared__ uint32_t wgt[4], weq[4];
    __shared__ float red[4][GS][D];
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int grp = blockIdx.y, b = grp / s.Hsel, sg = grp % s.Hsel, h0 = sg * s.GS, g = h0 / s.G;
    const int c = blockIdx.x, npv = gridDim.x;
    const uint32_t thr = sel[grp].thr, quota = sel[grp].quota;
    const uint2 inf = info[(int64_t)grp * npv + c];
    uint32_t kept_before = inf.x, ties_before = inf.y;
    float lsef[GS];
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
        lsef[hh] = (float)lse_ws[(int64_t)b * s.Hq + h0 + hh];
    const uint32_t *K = keys + (int64_t)grp * Sp;
    const float *L = logit + ((int64_t)b * s.Hq + h0) * Sp;
    const int Sb = seq_len(s, m, b), ksb = seq_keep(s, m, Sb);
    const int quarter = lane >> 4, dl = lane & 15, slot = w * 4 + quarter;

    float acc[GS][8];
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[hh][e] = 0.0f;

    const int p0 = c * P, p1 = min(Sb, p0 + P);
    for (int sb = p0; sb < p1; sb += PV_SUB) {
        // thread tid holds positions j0, j0+1 (j0 even and Sp a multiple of 8: j0 < S keeps both in the row;
        // pages hold a multiple of 8 positions, so both share j0's page)
        const int j0 = sb + 2 * tid;
        uint2 kk = make_uint2(0u, 0u);
        float2 lg[GS];
        int64_t vrow = 0;
#pragma unroll
        for (int hh = 0; hh < GS; ++hh)
            lg[hh] = make_float2(0.0f, 0.0f);
        if (j0 < p1) {
            vrow = kv_row(s, m, b, g, j0);
            kk = *reinterpret_cast<const uint2 *>(K + j0);
#pragma unroll
            for (int hh = 0; hh < GS; ++hh)
                lg[hh] = *reinterpret_cast<const float2 *>(L + (int64_t)hh * Sp + j0);
        }
        const uint32_t va = j0 < p1, vb1 = j0 + 1 < p1;
        const uint32_t ga = va & (kk.x > thr), gb = vb1 & (kk.y > thr);
        const uint32_t ea = va & (kk.x == thr), eb = vb1 & (kk.y == thr);
        // kept before a position = greater before + min(equal before, quota): one scan of each
        const uint32_t gi = wave_incl_sum(ga + gb), ei = wave_incl_sum(ea + eb);
        if (lane == WAVE - 1) {
            wgt[w] = gi;
            weq[w] = ei;
        }
        __syncthreads();
        uint32_t gbw = 0, ebw = 0, gtot = 0, etot = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            gbw += i < w ? wgt[i] : 0u;
            ebw += i < w ? weq[i] : 0u;
            gtot += wgt[i];
            etot += weq[i];
        }
        const uint32_t gpa = gbw + gi - (ga + gb), epa = ties_before + ebw + ei - (ea + eb); // before position a
        const uint32_t gpb = gpa + ga, epb = epa + ea;
        const uint32_t base0 = min(ties_before, quota); // kept ties before this pass
        const uint32_t keepa = ga | (ea & (epa < quota)), keepb = gb | (eb & (epb < quota));
        const uint32_t la = gpa + min(epa, quota) - base0, lb = gpb + min(epb, quota) - base0; // pass-local slots
        const uint32_t nkept = gtot + min(ties_before + etot, quota) - base0;
        if (keepa && la < PV_SUB) {
            rows[la] = vrow;
#pragma unroll
            for (int hh = 0; hh < GS; ++hh)
                pr[hh][la] = expf(fmaf(s.scale, lg[hh].x, -lsef[hh]));
            if (pos_out && kept_before + la < (uint32_t)ksb)
                pos_out[(int64_t)grp * s.ks + kept_before + la] = j0;
        }
        if (keepb && lb < PV_SUB) {
            rows[lb] = vrow + 1;
#pragma unroll
            for (int hh = 0; hh < GS; ++hh)
                pr[hh][lb] = expf(fmaf(s.scale, lg[hh].y, -lsef[hh]));
            if (pos_out && kept_before + lb < (uint32_t)ksb)
                pos_out[(int64_t)grp * s.ks + kept_before + lb] = j0 + 1;
        }
        __syncthreads();
        // stream kept V rows: slot (wave, quarter) takes rows slot + 16 m, PV_U rows in flight per lane
        const int nk = (int)min(nkept, (uint32_t)PV_SUB);
        for (int r0 = slot; r0 < nk; r0 += 16 * PV_U) {
            uint4 u[PV_U];
#pragma unroll
            for (int qq = 0; qq < PV_U; ++qq) {
                const int r = r0 + 16 * qq;
                if (r < nk)
                    u[qq] = *reinterpret_cast<const uint4 *>(v + rows[r] * D + dl * 8);
            }
#pragma unroll
            for (int qq = 0; qq < PV_U; ++qq) {
                const int r = r0 + 16 * qq;
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
        kept_before += nkept;
        ties_before += etot;
        __syncthreads();
    }

    // reduce the four quarters of each wave, then the four waves (fixed order)
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = acc[hh][e];
            x += __shfl_xor(x, 16, WAVE);
            x += __shfl_xor(x, 32, WAVE);
            acc[hh][e] = x;
        }
    if (quarter == 0) {
#pragma unroll
        for (int hh = 0; hh < GS; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                red[w][hh][dl * 8 + e] = acc[hh][e];
    }
    __syncthreads();
    float *mine = part + ((int64_t)grp * npv + c) * GS * D;
    for (int i = tid; i < GS * D; i += 256) {
        const int hh = i / D, dd = i % D;
        mine[i] = ((red[0][hh][dd] + red[1][hh][dd]) + red[2][hh][dd]) + red[3][hh][dd];
    }
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

// ------------------------------------------------------------------ host side
static void pv_chunks(int64_t S, int *P, int *npv)
{
    int64_t n = (S + PV_SUB - 1) / PV_SUB;
    if (n > PV_MAX_CHUNKS)
        n = PV_MAX_CHUNKS;
    int64_t per = (S + n - 1) / n;
    per = (per + PV_SUB - 1) / PV_SUB * PV_SUB;
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
    w.keys = (uint32_t *)p;
    p = align256(p + (size_t)(G * Sp) * 4);
    w.hist = (uint32_t *)p;
    p = align256(p + (size_t)(G * ATTN_HIST_BINS) * 4);
    w.pos = (int32_t *)p; // SelInfo [G] then chunk info [G][npv]
    p = align256(p + (size_t)G * sizeof(SelInfo) + (size_t)(G * npv) * sizeof(uint2) + 256);
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
    SelInfo *sel = reinterpret_cast<SelInfo *>(ws.pos);
    uint2 *info = reinterpret_cast<uint2 *>(align256((char *)(sel + G)));
    attn_qk_kernel<GS><<<dim3(nqk, G), QK_THREADS, 0, st>>>(s, m, Sp, q, kt, kn, ws.logit, ws.pstat, dim_idx,
                                                             ws.hist);
    const int nkc = (int)((s.S + ATTN_KEY_CHUNK - 1) / ATTN_KEY_CHUNK);
    const int nsub = key_chunks_per_wg(s.S);
    attn_key_kernel<GS><<<dim3((nkc + nsub - 1) / nsub, G), 256, 0, st>>>(
        s, m, Sp, nqk, nsub, ws.logit, ws.pstat, ws.lse, lse, vn, ws.keys, ws.hist);
    attn_select_kernel<<<G, 1024, 0, st>>>(s, m, Sp, P, npv, ws.keys, ws.hist, sel, info, pos_idx);
    attn_pv_kernel<GS><<<dim3(npv, G), 256, 0, st>>>(s, m, Sp, P, v, ws.logit, ws.lse, ws.keys, sel, info, pos_idx,
                                                     ws.pvpart);
    attn_pv_reduce_kernel<GS><<<G * (GS * D / WAVE), PVR_WAVES * WAVE, 0, st>>>(s, npv, ws.pvpart, out);
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
