// Reduced grouped-query attention decode.
//
// Blog on input-adaptive matrix-product reduction: section 3.1 (most past keys
// matter little to the current query: skip low-contribution work along the
// sequence), section 3.3 (reduce inside each head, never drop a head);
// paper abstract (keep informative slices of each product's contraction
// dimension: head_dim for Q K^T, key positions for P V).  GEMM notes section 1:
// scores = Q K^T, out = softmax(scores) V.
//
// Pipeline per (batch element, selection group), three launches on one stream
// (a fourth writes the kept-position lists when they are asked for):
//  qk    : head_dim selection (one wave, bitwise search over ballots), then
//          unscaled logits over the kept dims for 8 positions per lane from
//          dim-major keys (a kept dim is one contiguous row), and per-chunk
//          softmax statistics (max, sum of exponentials); the first chunk's
//          workgroup clears the group's score histogram and signal words.
//  fused : one launch of two workgroup roles.  Key workgroups merge the
//          chunk statistics into lse (double), score their positions by
//          max_h (scale*a_h - lse_h) in double, store each one's histogram bin
//          and add them to the group's score histogram; the group's last key
//          workgroup finds and publishes the bin holding the threshold, then
//          ranks that bin's positions and publishes the exact threshold.  PV
//          workgroups score their own chunk's positions the same way and
//          stream the V rows of those above the threshold bin into p*V
//          partial sums while the rank is resolved, then those in the bin at
//          or above the threshold.
//  reduce: the chunk partials are summed in a fixed order.
// When the fused launch would hold more workgroups than the device keeps
// resident (long or many sequences), the key role runs as a launch of its own,
// attn_select_kernel resolves each group's threshold, and attn_pv_split_kernel
// does PV with the thresholds known.  Per-query-head selection with several
// query heads per KV head reads each KV row once for the union of the heads'
// sets (attn_qk_kernel<G, true>, the key role per head, attn_pv_union_kernel).
#include "device.h"
#include "kernels.h"

namespace rmm {

constexpr int D = ATTN_D;
constexpr int QK_U = 16;      // kept key rows in flight per lane
constexpr int QK_THREADS = 256; // 4 waves split the kept dims of one chunk

// Wave reductions on DPP moves (VALU only, no LDS round trip per step): the
// row-scan pattern of wave_scan_dpp, whose last lane then holds the result in a
// fixed order of operations, read back into every lane.  Doubles move as two
// 32-bit halves.
template <int CTRL, int RMASK> __device__ __forceinline__ float dpp_f32(float ident, float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(ident), __float_as_int(v), CTRL, RMASK, 0xf, false));
}
template <int CTRL, int RMASK> __device__ __forceinline__ double dpp_f64(double v) // identity 0.0
{
    const int64_t u = __double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, RMASK, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, RMASK, 0xf, false);
    return __longlong_as_double((int64_t)((uint64_t)hi << 32 | lo));
}
__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp_f32<RMM_DPP_ROW_SHR(1), 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<RMM_DPP_ROW_SHR(2), 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<RMM_DPP_ROW_SHR(4), 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<RMM_DPP_ROW_SHR(8), 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<RMM_DPP_ROW_BCAST15, 0xa>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<RMM_DPP_ROW_BCAST31, 0xc>(-INFINITY, v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), WAVE - 1));
}
template <typename F> __device__ __forceinline__ F wave_sum(F v)
{
    if constexpr (sizeof(F) == 8) {
        v += dpp_f64<RMM_DPP_ROW_SHR(1), 0xf>(v);
        v += dpp_f64<RMM_DPP_ROW_SHR(2), 0xf>(v);
        v += dpp_f64<RMM_DPP_ROW_SHR(4), 0xf>(v);
        v += dpp_f64<RMM_DPP_ROW_SHR(8), 0xf>(v);
        v += dpp_f64<RMM_DPP_ROW_BCAST15, 0xa>(v);
        v += dpp_f64<RMM_DPP_ROW_BCAST31, 0xc>(v);
        const int64_t u = __double_as_longlong(v);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, WAVE - 1);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), WAVE - 1);
        return __longlong_as_double((int64_t)((uint64_t)hi << 32 | lo));
    } else {
        v += dpp_f32<RMM_DPP_ROW_SHR(1), 0xf>(0.0f, v);
        v += dpp_f32<RMM_DPP_ROW_SHR(2), 0xf>(0.0f, v);
        v += dpp_f32<RMM_DPP_ROW_SHR(4), 0xf>(0.0f, v);
        v += dpp_f32<RMM_DPP_ROW_SHR(8), 0xf>(0.0f, v);
        v += dpp_f32<RMM_DPP_ROW_BCAST15, 0xa>(0.0f, v);
        v += dpp_f32<RMM_DPP_ROW_BCAST31, 0xc>(0.0f, v);
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), WAVE - 1));
    }
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
__device__ __forceinline__ void wave_select128(uint32_t key0, uint32_t key1, int kd, int *jd, uint64_t *kmask = nullptr)
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
    if (kmask && lane == 0) {
        kmask[0] = k0;
        kmask[1] = k1;
    }
    if (keep0)
        jd[__popcll(k0 & lt)] = lane;
    if (keep1)
        jd[__popcll(k0) + __popcll(k1 & lt)] = lane + WAVE;
}

// ------------------------------------------------------------------ signals between the roles
// Per group, 256 bytes of the workspace.  First cache line: the count of key
// workgroups done (32-bit, word 0).  Second line, polled: the threshold bin
// (word 16: d << 40 | krem << 2 | all-of-bin-d-kept << 1 | ready) and the
// threshold rank key (word 17: thr << 1 | ready).  The QK kernel clears them;
// the fused kernel writes them with agent-scope stores and atomics, which every
// XCD sees once they complete.
constexpr int SIG_WORDS = 32;
constexpr int SIG_KCNT = 0, SIG_D = 16, SIG_THR = 17, SIG_LSE = 18; // SIG_LSE: GS doubles (split launches)
constexpr int ATTN_SPIN = 1 << 20; // polls (about a second) before a wait gives up

// ------------------------------------------------------------------ qk
// One workgroup per (chunk of ATTN_QK_CHUNK positions, group).  PH = false: the
// group is a selection group whose GS heads share one kept dim set.  PH = true
// (per-query-head selection with G > 1): the group is a KV head, each of its GS
// = G query heads selects its own dims, the union of the heads' dims is read
// once, and a head's logits add only its own dims (q is zero on the others).
template <int GS, bool PH>
__global__ __launch_bounds__(QK_THREADS) void attn_qk_kernel(AttnShape s, KvMap m, int Sp, const uint16_t *__restrict__ q,
                                                             const uint16_t *__restrict__ kt,
                                                             const float *__restrict__ kn, float *__restrict__ logit,
                                                             float2 *__restrict__ pstat,
                                                             int32_t *__restrict__ dim_idx_out,
                                                             uint32_t *__restrict__ hist, uint64_t *__restrict__ sig)
{
    constexpr int NWQ = QK_THREADS / WAVE;
    __shared__ int jd[D]; // the dims read, ascending
    __shared__ float qs[GS][D];
    __shared__ float part[NWQ][GS][ATTN_QK_CHUNK];
    __shared__ int jh[PH ? GS : 1][D];          // PH: each head's kept dims
    __shared__ uint64_t hm[PH ? GS : 1][2];     // PH: each head's kept dims as two 64-bit masks
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int grp = blockIdx.y;
    const int b = PH ? grp / (int)s.Hkv : grp / s.Hsel;
    const int h0 = PH ? (grp % (int)s.Hkv) * s.G : (grp % s.Hsel) * s.GS, g = h0 / s.G;
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
    int nsel = s.kd; // dims read
    if constexpr (!PH) {
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
    } else {
        // 1. each head's selection (wave w takes heads w, w + 4, ...):
        // sigma_j = fl32(|q_h[j]| * kn[j])
        for (int hh = w; hh < GS; hh += NWQ) {
            uint32_t key[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int j = lane + WAVE * half;
                key[half] = nonneg_key(
                    __fmul_rn(fabsf(bf16_to_f32(qb[hh * D + j])), kn[((int64_t)b * s.Hkv + g) * D + j]));
            }
            wave_select128(key[0], key[1], s.kd, jh[hh], hm[hh]);
        }
        __syncthreads();
        // the union of the heads' dims, ascending; q of a head is zero on the dims it dropped
        uint64_t u0 = 0, u1 = 0;
#pragma unroll
        for (int hh = 0; hh < GS; ++hh) {
            u0 |= hm[hh][0];
            u1 |= hm[hh][1];
        }
        nsel = __popcll(u0) + __popcll(u1);
        if (tid < D) {
            const int j = tid, hf = j / WAVE, bit = j % WAVE;
            const uint64_t um = hf ? u1 : u0;
            if ((um >> bit) & 1ull) {
                const uint64_t below = bit ? (um & (~0ull >> (WAVE - bit))) : 0ull;
                const int i = (hf ? __popcll(u0) : 0) + __popcll(below);
                jd[i] = j;
#pragma unroll
                for (int hh = 0; hh < GS; ++hh)
                    qs[hh][i] = ((hm[hh][hf] >> bit) & 1ull) ? qall[hh][j] : 0.0f;
            }
        }
        if (chunk == 0 && dim_idx_out)
            for (int i = tid; i < GS * s.kd; i += QK_THREADS)
                dim_idx_out[((int64_t)b * s.Hq + h0 + i / s.kd) * s.kd + i % s.kd] = jh[i / s.kd][i % s.kd];
    }
    __syncthreads();

    // 2. partial dot products: wave w takes kept dims [i0, i1) (ascending), 8 positions per lane
    const int i0 = nsel * w / NWQ, i1 = nsel * (w + 1) / NWQ;
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

    // 4. the first chunk's workgroup clears the score histograms and signal words
    // of the group's selection groups (PH: one per head) for the next launch
    if (chunk == 0) {
        const int nsg = PH ? GS : 1;
        const int64_t sg0 = PH ? (int64_t)b * s.Hq + h0 : grp;
        for (int i = tid; i < nsg * ATTN_HIST_BINS; i += QK_THREADS)
            hist[sg0 * ATTN_HIST_BINS + i] = 0;
        if (tid < nsg) {
            uint64_t *sw = sig + (sg0 + tid) * SIG_WORDS;
            pub_store64(sw + SIG_KCNT, 0ull);
            pub_store64(sw + SIG_D, 0ull);
            pub_store64(sw + SIG_THR, 0ull);
        }
    }
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

// ------------------------------------------------------------------ group log-sum-exp
// lse_h for each of the group's heads: scale*M + log(sum over the QK chunks of
// z_c * exp(scale*(m_c - M))), M the largest chunk maximum, in double.  Each
// thread merges its share of the chunk statistics online, then the block merges
// the threads' pairs in a fixed order, so every workgroup that calls this
// function (256 threads; barriers inside) holds the same bits.  The caller loads
// the thread's first statistic of each head early (ld_stats), ahead of its other
// loads.
struct LseLds {
    float smax[8][4];
    double ssum[8][4];
};
template <int GS>
__device__ __forceinline__ void ld_stats(const AttnShape &s, int b, int h0, int nqk_all, int nqk,
                                         const float2 *__restrict__ pstat, float2 (&pst)[GS])
{
    const int tid = threadIdx.x;
    // Every thread loads, at a clamped index (nqk_all >= 1); group_lse replaces
    // the statistic of threads past the sequence's chunks by the empty one.  A
    // select here, or a load under a per-thread branch, would be waited for at
    // once: one round trip per head before the logits are even requested.
    const int i = max(0, min(tid, nqk - 1));
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
        pst[hh] = pstat[((int64_t)b * s.Hq + h0 + hh) * nqk_all + i];
}
template <int GS>
__device__ void group_lse(const AttnShape &s, int b, int h0, int nqk_all, int nqk, const float2 *__restrict__ pstat,
                          const float2 (&pst)[GS], LseLds &L, double (&lse)[GS])
{
#pragma clang fp contract(off)
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const double sc = (double)s.scale;
    float mt[GS];
    double zt[GS];
    // threads past the sequence's chunks take the empty statistic (-inf, 0),
    // blended in with a mask the optimizer cannot turn back into a branch
    int okm = tid < nqk ? -1 : 0;
    asm volatile("" : "+v"(okm));
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
        mt[hh] = __int_as_float((__float_as_int(pst[hh].x) & okm) | (int)(0xff800000u & ~(uint32_t)okm));
        zt[hh] = (double)__int_as_float(__float_as_int(pst[hh].y) & okm);
    }
    for (int i = tid + 256; i < nqk; i += 256) { // sequences of more than 256 QK chunks
#pragma unroll
        for (int hh = 0; hh < GS; ++hh) {
            const float2 st = pstat[((int64_t)b * s.Hq + h0 + hh) * nqk_all + i];
            if (st.x > mt[hh]) {
                zt[hh] = zt[hh] * exp(sc * ((double)mt[hh] - (double)st.x)) + (double)st.y;
                mt[hh] = st.x;
            } else {
                zt[hh] += (double)st.y * exp(sc * ((double)st.x - (double)mt[hh]));
            }
        }
    }
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
        const float mx = wave_max(mt[hh]);
        if (lane == 0)
            L.smax[hh][w] = mx;
    }
    __syncthreads();
    float M[GS];
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
        M[hh] = fmaxf(fmaxf(L.smax[hh][0], L.smax[hh][1]), fmaxf(L.smax[hh][2], L.smax[hh][3]));
        const double z = mt[hh] == -INFINITY ? 0.0 : zt[hh] * exp(sc * ((double)mt[hh] - (double)M[hh]));
        const double zs = wave_sum(z);
        if (lane == 0)
            L.ssum[hh][w] = zs;
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
        lse[hh] = sc * (double)M[hh] + log(((L.ssum[hh][0] + L.ssum[hh][1]) + L.ssum[hh][2]) + L.ssum[hh][3]);
}

__device__ __forceinline__ uint64_t wait_ready(const uint64_t *p)
{
    for (int it = 0; it < ATTN_SPIN; ++it) {
        const uint64_t v = pub_load64(p);
        if (v & 1ull)
            return v;
        __builtin_amdgcn_s_sleep(2);
    }
    return 0ull;
}

// ------------------------------------------------------------------ position selection helpers
constexpr int PV_WAVES = 4;
constexpr int PV_THREADS = PV_WAVES * WAVE; // every role of the fused kernel: 256 threads
constexpr int PV_PASS = 2 * PV_THREADS;     // positions per PV pass (2 per thread)
constexpr int PV_STAGE = 2 * PV_PASS;       // kept rows staged in LDS before they are streamed
constexpr int PV_MAX_CHUNKS = 32;
constexpr int PV_U = 16;                    // kept V rows in flight per lane
constexpr int PV_CAND = PV_THREADS;         // threshold-bin positions a PV chunk keeps in LDS for its second phase
constexpr int SEL_CAP = 2048;               // threshold-bin candidates of a group ranked in LDS
constexpr int SEL_FEW = 64;                 // a radix digit with at most this many keys is ranked by one wave
static_assert(PV_MAX_CHUNKS <= PV_THREADS, "one chunk count per thread");

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

// ------------------------------------------------------------------ key role and threshold
// A key workgroup takes nsub consecutive chunks of ATTN_KEY_CHUNK positions of
// one group: it scores them (lse from the chunk statistics), stores each
// position's 2-byte histogram bin (agent-scope stores) and adds the bins to the
// group's histogram (LDS, then global atomics; the QK kernel cleared it), then
// counts itself.  The group's last key workgroup to count (every histogram
// atomic and bin store of the group has then completed) resolves the
// threshold: the histogram gives the bin d holding the ks-th largest score and
// the rank krem of that score inside the bin; d is published at once (with a
// flag when all of bin d is kept, which makes the threshold rank key 0), so
// the PV workgroups start on the positions above it.  Then bin d's positions
// are gathered from the bins, their rank keys are recomputed from the logits,
// and the krem-th largest is radix-selected and published.  Past SEL_CAP
// candidates the radix passes recompute the rank keys instead of holding them
// in LDS.  No key workgroup waits on another.
//
// The last workgroup reads the histogram and the bins with plain loads: the
// atomics are performed in memory and the bins written through to it with
// agent-scope stores before their workgroups count themselves, and no
// workgroup reads a group's histogram or bins before that group's last count
// (each group's bins row is padded to whole 128-byte lines), so no XCD's cache
// holds an older copy of them.
constexpr int SEL_UB = 16;  // 16-byte words of bins per thread per pass
constexpr int BIN_ROW = 64; // positions a group's bins row is padded to (128 bytes)
template <int CAP> struct KeyLdsT {
    union {
        uint32_t lh[ATTN_HIST_BINS];
        struct {
            uint64_t key[CAP];
            int32_t pos[CAP];
        } c;
    };
    RadixLds rad;
    uint32_t ncand;
    uint32_t bres[3];
    uint32_t last;
};
using KeyLds = KeyLdsT<SEL_CAP>;
static_assert(ATTN_HIST_BINS == 32 * PV_THREADS, "32 histogram bins per thread");

__device__ __forceinline__ uint32_t bin_of(const uint4 &w, int e)
{
    const uint32_t wd = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
    return (e & 1) ? wd >> 16 : wd & 0xffffu;
}

template <int GS, int NT, int CAP>
__device__ void publish_select(const AttnShape &s, const KvMap &m, int Sp, int Spb, int grp,
                               const float *__restrict__ logit, const double (&lsed)[GS],
                               const float *__restrict__ vn, const uint16_t *bins, const uint32_t *hg,
                               uint64_t *sg, KeyLdsT<CAP> &L)
{
    constexpr int T = NT;                    // threads of the workgroup
    constexpr int BPT = ATTN_HIST_BINS / NT; // histogram bins per thread
    static_assert(BPT % 4 == 0 && BPT * NT == ATTN_HIST_BINS, "whole 16-byte words of bins per thread");
    const int tid = threadIdx.x, lane = tid & (WAVE - 1);
    const int b = grp / s.Hsel, h0 = (grp % s.Hsel) * s.GS, g = h0 / s.G;
    const int Sb = seq_len(s, m, b), ksb = seq_keep(s, m, Sb);
    const float *Lg = logit + ((int64_t)b * s.Hq + h0) * Sp; // head hh at Lg + hh * Sp
    const uint4 *B16 = reinterpret_cast<const uint4 *>(bins + (int64_t)grp * Spb);
    const int n8 = (Sb + 7) / 8; // 8-position words of bins
    const double sc = (double)s.scale;
    auto rank_of = [&](int p, uint32_t d) -> uint64_t {
        float av[GS];
#pragma unroll
        for (int hh = 0; hh < GS; ++hh)
            av[hh] = Lg[(int64_t)hh * Sp + p];
        const float vv = vn ? vn[kv_row(s, m, b, g, p)] : 1.0f;
        return rank_key(pos_key(pos_score<GS>(av, lsed, sc, vn != nullptr, vv)), d, p);
    };
    // threshold bin: thread t holds bins 8191-BPT*t down to 8192-BPT*(t+1)
    uint32_t hc[BPT];
    {
        const uint4 *h4 = reinterpret_cast<const uint4 *>(hg + ATTN_HIST_BINS - BPT * (tid + 1));
        uint4 q[BPT / 4];
#pragma unroll
        for (int i = 0; i < BPT / 4; ++i)
            q[i] = h4[i];
#pragma unroll
        for (int i = 0; i < BPT / 4; ++i) {
            hc[BPT - 1 - 4 * i] = q[i].x;
            hc[BPT - 2 - 4 * i] = q[i].y;
            hc[BPT - 3 - 4 * i] = q[i].z;
            hc[BPT - 4 - 4 * i] = q[i].w;
        }
    }
    if (tid == 0) {
        L.bres[0] = 0;
        L.bres[1] = 1;
        L.bres[2] = 0;
        L.ncand = 0;
    }
    uint32_t tot = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i)
        tot += hc[i];
    const uint32_t incl = block_incl_scan(tot, L.rad.tmp); // (barriers inside)
    {
        const uint32_t top = ATTN_HIST_BINS - 1 - BPT * tid, want = (uint32_t)ksb;
        uint32_t run = incl - tot;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
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
    if (tid == 0)
        pub_store64(sg + SIG_D, (uint64_t)d << 40 | (uint64_t)krem << 2 | (krem == nbin ? 2ull : 0ull) | 1ull);
    if (krem == nbin)
        return; // all of bin d is kept

    uint64_t thr;
    if (nbin <= (uint32_t)CAP) {
        // gather bin d's positions: per-lane bit masks of 4 words, one slot reservation per wave
        for (int base = 0; base < n8; base += SEL_UB * T) {
            uint4 u[SEL_UB];
#pragma unroll
            for (int j = 0; j < SEL_UB; ++j) {
                const int i = base + tid + j * T;
                u[j] = i < n8 ? B16[i] : make_uint4(0u, 0u, 0u, 0u);
            }
            // the positions of bin d, two per 32-bit word at a time: a 16-bit half h of
            // word ^ (d, d) is zero iff bit 15 of ((h & 0x7fff) + 0x7fff) | h is clear (no
            // carry crosses the halves)
            const uint32_t dd = d | d << 16;
            auto eq2 = [&](uint32_t wd) -> uint32_t { // bit 0: low half is d, bit 1: high half
                const uint32_t a = wd ^ dd;
                const uint32_t nz = (((a & 0x7fff7fffu) + 0x7fff7fffu) | a) & 0x80008000u;
                const uint32_t z = ~nz & 0x80008000u;
                return (z >> 15 & 1u) | z >> 30;
            };
#pragma unroll
            for (int j0 = 0; j0 < SEL_UB; j0 += 4) {
                uint32_t cm = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = base + tid + (j0 + j) * T;
                    const uint4 &wv = u[j0 + j];
                    uint32_t m8 = eq2(wv.x) | eq2(wv.y) << 2 | eq2(wv.z) << 4 | eq2(wv.w) << 6;
                    const int left = Sb - 8 * i; // positions of the word inside the sequence
                    m8 &= left >= 8 ? 0xffu : left > 0 ? (1u << left) - 1u : 0u;
                    cm |= m8 << (8 * j);
                }
                const uint32_t cl = (uint32_t)__popc(cm);
                const uint32_t cincl = wave_incl_sum(cl);
                const uint32_t wcount = (uint32_t)__builtin_amdgcn_readlane((int)cincl, WAVE - 1);
                uint32_t sbase = 0;
                if (lane == 0 && wcount != 0u)
                    sbase = atomicAdd(&L.ncand, wcount);
                sbase = (uint32_t)__builtin_amdgcn_readfirstlane((int)sbase);
                uint32_t slot = sbase + cincl - cl;
                while (cm) {
                    const int bit = __builtin_ctz(cm);
                    cm &= cm - 1u;
                    if (slot < (uint32_t)CAP)
                        L.c.pos[slot] = 8 * (base + tid + (j0 + (bit >> 3)) * T) + (bit & 7);
                    ++slot;
                }
            }
        }
        __syncthreads();
        const int nc = (int)min(L.ncand, (uint32_t)CAP);
        // the candidates' rank keys, the logits of RB candidates per thread in flight together
        // (one at a time in the fused launch, whose registers the key role shares with PV)
        constexpr int RB = NT >= 1024 ? 4 : 1;
        for (int i0 = tid; i0 < nc; i0 += T * RB) {
            int pp[RB];
            float av[RB][GS], vv[RB];
#pragma unroll
            for (int u = 0; u < RB; ++u) {
                const int i = i0 + u * T;
                pp[u] = i < nc ? L.c.pos[i] : -1;
                vv[u] = 1.0f;
#pragma unroll
                for (int hh = 0; hh < GS; ++hh)
                    av[u][hh] = pp[u] >= 0 ? Lg[(int64_t)hh * Sp + pp[u]] : 0.0f;
                if (vn && pp[u] >= 0)
                    vv[u] = vn[kv_row(s, m, b, g, pp[u])];
            }
#pragma unroll
            for (int u = 0; u < RB; ++u)
                if (pp[u] >= 0)
                    L.c.key[i0 + u * T] =
                        rank_key(pos_key(pos_score<GS>(av[u], lsed, sc, vn != nullptr, vv[u])), d, pp[u]);
        }
        __syncthreads();
        thr = radix_select_u64(
            [&](auto f) {
                for (int i = tid; i < nc; i += T)
                    f(L.c.key[i]);
            },
            krem, L.rad);
    } else {
        // a crowded bin: every radix pass recomputes the rank keys of bin d's positions
        thr = radix_select_u64(
            [&](auto f) {
                for (int i = tid; i < n8; i += T) {
                    const uint4 w4 = B16[i];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int p = 8 * i + e;
                        if (bin_of(w4, e) == d && p < Sb)
                            f(rank_of(p, d));
                    }
                }
            },
            krem, L.rad);
    }
    if (tid == 0)
        pub_store64(sg + SIG_THR, thr << 1 | 1ull);
}

template <int GS>
__device__ void key_role(const AttnShape &s, const KvMap &m, int Sp, int Spb, int nqk_all, int nsub, int nkw, int grp,
                         int kx, bool resolve, const float *__restrict__ logit, const float2 *__restrict__ pstat,
                         float *__restrict__ lse_out, const float *__restrict__ vn, uint16_t *bins,
                         uint32_t *__restrict__ hist, uint64_t *sg, KeyLds &L, LseLds &LL)
{
    const int tid = threadIdx.x;
    const int b = grp / s.Hsel, h0 = (grp % s.Hsel) * s.GS;
    const int Sb = seq_len(s, m, b);
    const int nqk = (Sb + ATTN_QK_CHUNK - 1) / ATTN_QK_CHUNK; // this sequence's QK chunks
    const int c0 = kx * nsub;
    uint32_t *hg = hist + (int64_t)grp * ATTN_HIST_BINS;
    double lse[GS];
    float2 pst[GS];
    ld_stats<GS>(s, b, h0, nqk_all, nqk, pstat, pst);
    if (c0 * ATTN_KEY_CHUNK < Sb) { // (uniform) workgroups past the sequence's end only count themselves
        for (int i = tid; i < ATTN_HIST_BINS; i += PV_THREADS)
            L.lh[i] = 0;
        // this thread's logits load behind the statistics, so their latency overlaps the merge
        f32x4_t a[GS][2], an[GS][2];
        auto load_logits = [&](f32x4_t (&dst)[GS][2], int sp) {
            if (sp < Sb) {
#pragma unroll
                for (int hh = 0; hh < GS; ++hh) {
                    const f32x4_t *src =
                        reinterpret_cast<const f32x4_t *>(logit + ((int64_t)b * s.Hq + h0 + hh) * Sp + sp);
                    dst[hh][0] = src[0];
                    dst[hh][1] = src[1];
                }
            }
        };
        load_logits(a, c0 * ATTN_KEY_CHUNK + tid * 8);
        group_lse<GS>(s, b, h0, nqk_all, nqk, pstat, pst, LL, lse); // (its barriers order the clearing of lh)
        if (kx == 0 && lse_out) {
#pragma unroll
            for (int hh = 0; hh < GS; ++hh)
                if (tid == hh)
                    lse_out[(int64_t)b * s.Hq + h0 + hh] = (float)lse[hh];
        }
        const double sc = (double)s.scale;
        uint64_t *bg = reinterpret_cast<uint64_t *>(bins + (int64_t)grp * Spb);
        for (int sub = 0; sub < nsub; ++sub) {
            const int sp = (c0 + sub) * ATTN_KEY_CHUNK + tid * 8;
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
                    atomicAdd(&L.lh[bb], 1u);
                    bn[e] = bb;
                } else {
                    bn[e] = 0u; // past the sequence's end: never read as a position
                }
            }
            pub_store64(bg + sp / 4, (uint64_t)(bn[0] | bn[1] << 16) | (uint64_t)(bn[2] | bn[3] << 16) << 32);
            pub_store64(bg + sp / 4 + 1, (uint64_t)(bn[4] | bn[5] << 16) | (uint64_t)(bn[6] | bn[7] << 16) << 32);
#pragma unroll
            for (int hh = 0; hh < GS; ++hh) {
                a[hh][0] = an[hh][0];
                a[hh][1] = an[hh][1];
            }
        }
        __syncthreads();
        for (int i = tid; i < ATTN_HIST_BINS; i += PV_THREADS)
            if (L.lh[i])
                atomicAdd(&hg[i], L.lh[i]);
    }
    // every histogram atomic and bin store of the workgroup has completed before it counts itself
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t before = __hip_atomic_fetch_add(reinterpret_cast<uint32_t *>(sg + SIG_KCNT), 1u,
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        L.last = before == (uint32_t)(nkw - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (!L.last)
        return;
    if (c0 * ATTN_KEY_CHUNK >= Sb) // (uniform) a workgroup past the end merges lse only when it is the last
        group_lse<GS>(s, b, h0, nqk_all, nqk, pstat, pst, LL, lse);
    if (!resolve) {
        // the threshold is resolved by attn_select_kernel after this launch: it takes the lse from here
#pragma unroll
        for (int hh = 0; hh < GS; ++hh)
            if (tid == hh)
                pub_store64(sg + SIG_LSE + hh, (uint64_t)__double_as_longlong(lse[hh]));
        return;
    }
    publish_select<GS, PV_THREADS, SEL_CAP>(s, m, Sp, Spb, grp, logit, lse, vn, bins, hg, sg, L);
}

// ------------------------------------------------------------------ pv role
// One workgroup per (chunk of P positions, group).  It loads its first pass's
// logits and merges the group's lse, stores every position's histogram bin and
// counts itself; the group's last chunk to count resolves the threshold.  Then
// it waits for the threshold bin d (its first pass's scores stay in
// registers).  Phase one: every pass keeps the positions above bin d
// (order-preserving), stages their V rows and probabilities in LDS and streams
// the rows, 16 in flight per lane (a 16-lane quarter wave per 256-byte row),
// into p*V partial sums; the chunk's bin-d positions go to an LDS list with
// their rank keys.  Phase two (only chunks holding bin-d positions wait for the
// threshold rank key): the listed positions at or above it are streamed the
// same way.  The order of the additions does not depend on the optional
// outputs.
template <int GS> struct PvLds {
    int64_t rows[PV_STAGE]; // V row index of each staged kept position
    union {
        float pr[GS][PV_STAGE];
        float red[PV_WAVES][GS][D];
    };
    int32_t cpos[PV_CAND];
    uint64_t crank[PV_CAND];
    uint32_t wk[PV_WAVES];
};
static_assert(PV_STAGE >= PV_WAVES * D, "the wave partials reuse the probability staging");

template <int GS> struct FusedLds {
    LseLds ls;
    uint64_t sigv;
    union {
        KeyLds key;
        PvLds<GS> pv;
    };
};

template <int GS>
__device__ void pv_role(const AttnShape &s, const KvMap &m, int Sp, int nqk_all, int P, int npv, int grp, int c,
                        const uint16_t *__restrict__ v, const float *__restrict__ logit,
                        const float2 *__restrict__ pstat, const float *__restrict__ vn, uint64_t *sg,
                        int32_t *__restrict__ pstage, uint32_t *__restrict__ pcount, float *__restrict__ part,
                        FusedLds<GS> &LF)
{
    PvLds<GS> &L = LF.pv;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int b = grp / s.Hsel, h0 = (grp % s.Hsel) * s.GS, g = h0 / s.G;
    const int Sb = seq_len(s, m, b);
    const int p0 = c * P, p1 = min(Sb, p0 + P);
    const float *Lg = logit + ((int64_t)b * s.Hq + h0) * Sp;
    const double sc = (double)s.scale;
    const int quarter = lane >> 4, dl = lane & 15, slot = w * 4 + quarter;
    constexpr int NSLOT = PV_WAVES * 4;
    float acc[GS][8];
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[hh][e] = 0.0f;
    uint32_t chunk_kept = 0;
    bool poison = false;

    // the nk rows staged in L.rows / L.pr, into acc
    auto stream = [&](int nk) {
        for (int r0 = slot; r0 < nk; r0 += NSLOT * PV_U) {
            uint4 uu[PV_U];
#pragma unroll
            for (int qq = 0; qq < PV_U; ++qq) {
                const int r = r0 + NSLOT * qq;
                if (r < nk)
                    uu[qq] = *reinterpret_cast<const uint4 *>(v + L.rows[r] * D + dl * 8);
            }
#pragma unroll
            for (int qq = 0; qq < PV_U; ++qq) {
                const int r = r0 + NSLOT * qq;
                if (r < nk) {
                    float vv[8];
                    Vec16<uint16_t>::unpack(uu[qq], vv);
#pragma unroll
                    for (int hh = 0; hh < GS; ++hh) {
                        const float pv = L.pr[hh][r];
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[hh][e] = fmaf(pv, vv[e], acc[hh][e]);
                    }
                }
            }
        }
    };
    // exclusive slot of this thread's n among the pass (wave scan plus the wave
    // totals in LDS); returns the block total.  A barrier must separate two calls.
    auto pass_slots = [&](uint32_t n, uint32_t &excl) -> uint32_t {
        const uint32_t ki = wave_incl_sum(n);
        if (lane == WAVE - 1)
            L.wk[w] = ki;
        __syncthreads();
        uint32_t before = 0, tot = 0;
#pragma unroll
        for (int i = 0; i < PV_WAVES; ++i) {
            before += i < w ? L.wk[i] : 0u;
            tot += L.wk[i];
        }
        excl = before + ki - n;
        return tot;
    };

    if (p0 < p1) { // (uniform over the workgroup) chunks past the sequence's end write zeros
        // this thread's two positions of a pass: j0 even and Sp a multiple of 8, so
        // j0 < Sb keeps both in the row, and pages hold a multiple of 8 positions,
        // so both share j0's page
        int j0 = 0;
        uint32_t va = 0, vb = 0;
        int64_t vrow = 0;
        float2 lg[GS], nv = make_float2(1.0f, 1.0f);
        double lsed[GS];
        float lsef[GS];
        uint64_t ka = 0, kb = 0;
        auto load_pass = [&](int sb) {
            j0 = sb + 2 * tid;
            va = (uint32_t)(j0 < p1);
            vb = (uint32_t)(j0 + 1 < p1);
            vrow = 0;
#pragma unroll
            for (int hh = 0; hh < GS; ++hh)
                lg[hh] = make_float2(0.0f, 0.0f);
            nv = make_float2(1.0f, 1.0f);
            if (va) {
                vrow = kv_row(s, m, b, g, j0);
#pragma unroll
                for (int hh = 0; hh < GS; ++hh)
                    lg[hh] = *reinterpret_cast<const float2 *>(Lg + (int64_t)hh * Sp + j0);
                if (vn)
                    nv = *reinterpret_cast<const float2 *>(vn + vrow);
            }
        };
        // the next pass's logits, value norms and row, loaded while this pass's rows stream
        int j0n = 0;
        uint32_t van = 0, vbn = 0;
        int64_t vrown = 0;
        float2 lgn[GS], nvn = make_float2(1.0f, 1.0f);
        auto load_next = [&](int sb) {
            j0n = sb + 2 * tid;
            van = (uint32_t)(j0n < p1);
            vbn = (uint32_t)(j0n + 1 < p1);
            vrown = 0;
#pragma unroll
            for (int hh = 0; hh < GS; ++hh)
                lgn[hh] = make_float2(0.0f, 0.0f);
            nvn = make_float2(1.0f, 1.0f);
            if (van) {
                vrown = kv_row(s, m, b, g, j0n);
#pragma unroll
                for (int hh = 0; hh < GS; ++hh)
                    lgn[hh] = *reinterpret_cast<const float2 *>(Lg + (int64_t)hh * Sp + j0n);
                if (vn)
                    nvn = *reinterpret_cast<const float2 *>(vn + vrown);
            }
        };
        auto take_next = [&]() {
            j0 = j0n;
            va = van;
            vb = vbn;
            vrow = vrown;
#pragma unroll
            for (int hh = 0; hh < GS; ++hh)
                lg[hh] = lgn[hh];
            nv = nvn;
        };
        auto score_pass = [&]() {
            float ax[GS], ay[GS];
#pragma unroll
            for (int hh = 0; hh < GS; ++hh) {
                ax[hh] = lg[hh].x;
                ay[hh] = lg[hh].y;
            }
            ka = pos_key(pos_score<GS>(ax, lsed, sc, vn != nullptr, nv.x));
            kb = pos_key(pos_score<GS>(ay, lsed, sc, vn != nullptr, nv.y));
        };
        auto stage = [&](uint32_t so, bool second) {
            L.rows[so] = vrow + (second ? 1 : 0);
#pragma unroll
            for (int hh = 0; hh < GS; ++hh)
                L.pr[hh][so] = expf(fmaf(s.scale, second ? lg[hh].y : lg[hh].x, -lsef[hh]));
        };
        const int nqk = (Sb + ATTN_QK_CHUNK - 1) / ATTN_QK_CHUNK;
        float2 pst[GS];
        ld_stats<GS>(s, b, h0, nqk_all, nqk, pstat, pst);
        load_pass(p0);
        group_lse<GS>(s, b, h0, nqk_all, nqk, pstat, pst, LF.ls, lsed);
#pragma unroll
        for (int hh = 0; hh < GS; ++hh)
            lsef[hh] = (float)lsed[hh];
        score_pass();
        // the threshold bin, from the group's last key workgroup
        if (tid == 0)
            LF.sigv = wait_ready(sg + SIG_D);
        __syncthreads();
        const uint64_t s1 = LF.sigv;
        poison = !(s1 & 1ull);
        const uint32_t d = (uint32_t)(s1 >> 40);
        const bool all_kept = (s1 & 2ull) != 0ull; // every bin-d position is kept: threshold rank key 0
        uint64_t thr = 0;
        uint32_t ncand = 0;
        // phase one: positions above bin d, staged over passes in LDS and
        // streamed when the stage would overflow or the chunk ends; the bin-d
        // positions go to the LDS list
        if (!poison) {
            uint32_t nst = 0; // rows staged and not yet streamed
            for (int sb = p0; sb < p1; sb += PV_PASS) {
                if (sb != p0) {
                    take_next();
                    score_pass();
                }
                const uint32_t ba = key_bin(ka), bb = key_bin(kb);
                const uint32_t ya = va & (uint32_t)(ba > d), yb = vb & (uint32_t)(bb > d);
                const uint32_t ca = va & (uint32_t)(ba == d), cb = vb & (uint32_t)(bb == d);
                const uint32_t n = (ya + yb) | (ca + cb) << 16;
                uint32_t ex;
                const uint32_t tot = pass_slots(n, ex);
                uint32_t so = nst + (ex & 0xffffu), co = ncand + (ex >> 16);
                if (ya)
                    stage(so++, false);
                if (yb)
                    stage(so, true);
                if (ca) {
                    if (co < (uint32_t)PV_CAND) {
                        L.cpos[co] = j0;
                        L.crank[co] = rank_key(ka, d, j0);
                    }
                    ++co;
                }
                if (cb && co < (uint32_t)PV_CAND) {
                    L.cpos[co] = j0 + 1;
                    L.crank[co] = rank_key(kb, d, j0 + 1);
                }
                nst += tot & 0xffffu;
                chunk_kept += tot & 0xffffu;
                ncand += tot >> 16;
                __syncthreads();
                if (sb + PV_PASS < p1)
                    load_next(sb + PV_PASS);
                // (uniform) a further pass could overflow the stage, or this is the last pass
                if (nst > (uint32_t)(PV_STAGE - PV_PASS) || sb + PV_PASS >= p1) {
                    stream((int)nst);
                    nst = 0;
                }
                __syncthreads();
            }
        }
        // phase two: the bin-d positions at or above the threshold
        if (ncand != 0u && !poison && !all_kept) {
            if (tid == 0)
                LF.sigv = wait_ready(sg + SIG_THR);
            __syncthreads();
            const uint64_t s2 = LF.sigv;
            poison = !(s2 & 1ull);
            thr = s2 >> 1;
        }
        if (ncand != 0u && !poison) {
            if (ncand <= (uint32_t)PV_CAND) {
                const uint32_t keep = (uint32_t)((uint32_t)tid < ncand) & (uint32_t)(L.crank[tid] >= thr);
                uint32_t ex;
                const uint32_t tot = pass_slots(keep, ex);
                if (keep) {
                    const int p = L.cpos[tid];
                    L.rows[ex] = kv_row(s, m, b, g, p);
#pragma unroll
                    for (int hh = 0; hh < GS; ++hh)
                        L.pr[hh][ex] = expf(fmaf(s.scale, Lg[(int64_t)hh * Sp + p], -lsef[hh]));
                }
                __syncthreads();
                stream((int)tot);
                chunk_kept += tot;
                __syncthreads();
            } else {
                // more bin-d positions than the list holds: the passes are scored again
                for (int sb = p0; sb < p1; sb += PV_PASS) {
                    load_pass(sb);
                    score_pass();
                    const uint32_t ya = va & (uint32_t)(key_bin(ka) == d) & (uint32_t)(rank_key(ka, d, j0) >= thr);
                    const uint32_t yb =
                        vb & (uint32_t)(key_bin(kb) == d) & (uint32_t)(rank_key(kb, d, j0 + 1) >= thr);
                    uint32_t ex;
                    const uint32_t tot = pass_slots(ya + yb, ex);
                    if (ya)
                        stage(ex++, false);
                    if (yb)
                        stage(ex, true);
                    __syncthreads();
                    stream((int)tot);
                    chunk_kept += tot;
                    __syncthreads();
                }
            }
        }
        // kept positions in ascending order, for the kept-position lists
        if (pstage && !poison) {
            uint32_t off = 0;
            for (int sb = p0; sb < p1; sb += PV_PASS) {
                load_pass(sb);
                score_pass();
                const uint32_t ba = key_bin(ka), bb = key_bin(kb);
                const uint32_t ya =
                    va & ((uint32_t)(ba > d) | ((uint32_t)(ba == d) & (uint32_t)(rank_key(ka, d, j0) >= thr)));
                const uint32_t yb =
                    vb & ((uint32_t)(bb > d) | ((uint32_t)(bb == d) & (uint32_t)(rank_key(kb, d, j0 + 1) >= thr)));
                uint32_t ex;
                const uint32_t tot = pass_slots(ya + yb, ex);
                int32_t *dst = pstage + (int64_t)grp * Sp + p0 + off + ex;
                if (ya)
                    *dst++ = j0;
                if (yb)
                    *dst = j0 + 1;
                off += tot;
                __syncthreads();
            }
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
    __syncthreads(); // (the partials reuse the probability staging)
    if ((lane >> 4) == 0) {
#pragma unroll
        for (int hh = 0; hh < GS; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                L.red[w][hh][(lane & 15) * 8 + e] = acc[hh][e];
    }
    __syncthreads();
    float *mine = part + ((int64_t)grp * npv + c) * GS * D;
    for (int i = tid; i < GS * D; i += PV_THREADS) {
        const int hh = i / D, dd = i % D;
        float x = L.red[0][hh][dd];
#pragma unroll
        for (int ww = 1; ww < PV_WAVES; ++ww)
            x += L.red[ww][hh][dd];
        mine[i] = poison ? __builtin_nanf("") : x;
    }
    if (pcount && tid == 0)
        pcount[(int64_t)grp * npv + c] = chunk_kept;
}

// ------------------------------------------------------------------ fused key / pv launch
// Workgroups take their role from their index: [0, nkw*G) key workgroups
// (group-major), then npv*G PV workgroups (group-major).  Only PV workgroups
// wait, and only for the words the group's last key workgroup publishes; key
// workgroups wait on nobody and have lower indices.  The dispatcher starts
// workgroups in index order on each XCD, so every key workgroup has started
// before any PV workgroup and the waits end whatever the residency.  Each wait
// is bounded all the same, and one that runs out poisons the group's output
// with NaN.
template <int GS, bool KEY_ONLY = false>
__global__ __launch_bounds__(PV_THREADS) void attn_fused_kernel(
    AttnShape s, KvMap m, int Sp, int nqk_all, int nsub, int nkw, int P, int npv, const uint16_t *__restrict__ v,
    const float *__restrict__ logit, const float2 *__restrict__ pstat, float *__restrict__ lse_out,
    const float *__restrict__ vn, uint16_t *__restrict__ bins, uint32_t *__restrict__ hist,
    uint64_t *__restrict__ sig, int32_t *__restrict__ pstage, uint32_t *__restrict__ pcount, float *__restrict__ part,
    int resolve)
{
    __shared__ FusedLds<GS> L;
    const int G = (int)(s.B * s.Hsel);
    const int Spb = (Sp + BIN_ROW - 1) / BIN_ROW * BIN_ROW;
    int bid = (int)blockIdx.x;
    if (bid < nkw * G) {
        const int grp = bid / nkw;
        key_role<GS>(s, m, Sp, Spb, nqk_all, nsub, nkw, grp, bid % nkw, resolve != 0, logit, pstat, lse_out, vn, bins,
                     hist,
                     sig + (int64_t)grp * SIG_WORDS, L.key, L.ls);
        return;
    }
    if constexpr (!KEY_ONLY) { // (the key-only instance leaves out the PV role and its registers)
        bid -= nkw * G;
        const int grp = bid / npv;
        pv_role<GS>(s, m, Sp, nqk_all, P, npv, grp, bid % npv, v, logit, pstat, vn, sig + (int64_t)grp * SIG_WORDS,
                    pstage, pcount, part, L);
    }
}

// ------------------------------------------------------------------ threshold of split launches
// When the key role runs as a launch of its own (see attn_pv_split_kernel),
// one workgroup of SELK_THREADS per group resolves the group's threshold after
// it, exactly as the key role's last workgroup does in the fused launch
// (publish_select, with the lse that workgroup left in the signal words), with
// four times the threads and four times the candidates in LDS: the stored bins
// of up to 128K positions are gathered in one round trip.
constexpr int SELK_THREADS = 1024;
constexpr int SELK_CAP = 8192; // threshold-bin candidates held in LDS (96 KB)
template <int GS>
__global__ __launch_bounds__(SELK_THREADS) void attn_select_kernel(AttnShape s, KvMap m, int Sp,
                                                                   const float *__restrict__ logit,
                                                                   const float *__restrict__ vn,
                                                                   const uint16_t *__restrict__ bins,
                                                                   const uint32_t *__restrict__ hist, uint64_t *sig)
{
    __shared__ KeyLdsT<SELK_CAP> L;
    const int grp = blockIdx.x;
    const int Spb = (Sp + BIN_ROW - 1) / BIN_ROW * BIN_ROW;
    uint64_t *sg = sig + (int64_t)grp * SIG_WORDS;
    double lse[GS];
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
        lse[hh] = __longlong_as_double((long long)pub_load64(sg + SIG_LSE + hh));
    publish_select<GS, SELK_THREADS, SELK_CAP>(s, m, Sp, Spb, grp, logit, lse, vn, bins,
                                               hist + (int64_t)grp * ATTN_HIST_BINS, sg, L);
}

// ------------------------------------------------------------------ PV after the threshold (large launches)
// When the fused launch holds more workgroups than the device keeps resident,
// its PV workgroups would only start as key workgroups retire and run two to a
// CU.  Then the key role runs alone, and this kernel does PV once every
// group's threshold is out: one workgroup per (chunk of P positions, group),
// every position decided in one pass from its stored histogram bin (above bin
// d: kept; bin d: its rank key from the logits against the published one), the
// kept rows staged and streamed as in the fused kernel, PVU rows in flight per
// lane (fewer registers, more resident workgroups).
template <int GS, int PVU>
__global__ __launch_bounds__(PV_THREADS) __attribute__((amdgpu_waves_per_eu(4))) void attn_pv_split_kernel(AttnShape s, KvMap m, int Sp, int nqk_all, int P,
                                                                   const uint16_t *__restrict__ v,
                                                                   const float *__restrict__ logit,
                                                                   const float2 *__restrict__ pstat,
                                                                   const float *__restrict__ vn,
                                                                   const uint16_t *__restrict__ bins,
                                                                   const uint64_t *__restrict__ sig,
                                                                   int32_t *__restrict__ pstage,
                                                                   uint32_t *__restrict__ pcount,
                                                                   float *__restrict__ part)
{
    __shared__ LseLds LL;
    __shared__ int64_t rows[PV_STAGE];
    __shared__ union {
        float pr[GS][PV_STAGE];
        float red[PV_WAVES][GS][D];
    } U;
    __shared__ uint32_t wk[PV_WAVES];
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int grp = blockIdx.y, c = blockIdx.x, npv = gridDim.x;
    const int b = grp / s.Hsel, h0 = (grp % s.Hsel) * s.GS, g = h0 / s.G;
    const int Sb = seq_len(s, m, b);
    const int p0 = c * P, p1 = min(Sb, p0 + P);
    const float *Lg = logit + ((int64_t)b * s.Hq + h0) * Sp;
    const int Spb = (Sp + BIN_ROW - 1) / BIN_ROW * BIN_ROW;
    const uint16_t *Bg = bins + (int64_t)grp * Spb;
    const double sc = (double)s.scale;
    const int quarter = lane >> 4, dl = lane & 15, slot = w * 4 + quarter;
    constexpr int NSLOT = PV_WAVES * 4;
    float acc[GS][8];
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[hh][e] = 0.0f;
    bool poison = false;
    uint32_t kept_n = 0;

    auto stream = [&](int nk) {
        for (int r0 = slot; r0 < nk; r0 += NSLOT * PVU) {
            uint4 uu[PVU];
#pragma unroll
            for (int qq = 0; qq < PVU; ++qq) {
                const int r = r0 + NSLOT * qq;
                if (r < nk)
                    uu[qq] = *reinterpret_cast<const uint4 *>(v + rows[r] * D + dl * 8);
            }
#pragma unroll
            for (int qq = 0; qq < PVU; ++qq) {
                const int r = r0 + NSLOT * qq;
                if (r < nk) {
                    float vv[8];
                    Vec16<uint16_t>::unpack(uu[qq], vv);
#pragma unroll
                    for (int hh = 0; hh < GS; ++hh) {
                        const float pv = U.pr[hh][r];
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[hh][e] = fmaf(pv, vv[e], acc[hh][e]);
                    }
                }
            }
        }
    };
    // exclusive slot of this thread's n; returns the block total.  A barrier must separate two calls.
    auto pass_slots = [&](uint32_t n, uint32_t &excl) -> uint32_t {
        const uint32_t ki = wave_incl_sum(n);
        if (lane == WAVE - 1)
            wk[w] = ki;
        __syncthreads();
        uint32_t before = 0, tot = 0;
#pragma unroll
        for (int i = 0; i < PV_WAVES; ++i) {
            before += i < w ? wk[i] : 0u;
            tot += wk[i];
        }
        excl = before + ki - n;
        return tot;
    };

    if (p0 < p1) { // (uniform) chunks past the sequence's end write zeros
        const uint64_t *sw = sig + (int64_t)grp * SIG_WORDS;
        const uint64_t w1 = sw[SIG_D], w2 = sw[SIG_THR];
        const bool all = (w1 & 2ull) != 0ull;
        poison = !(w1 & 1ull) || (!all && !(w2 & 1ull));
        const uint32_t d = (uint32_t)(w1 >> 40);
        const uint64_t thr = all ? 0ull : w2 >> 1;
        const int nqk = (Sb + ATTN_QK_CHUNK - 1) / ATTN_QK_CHUNK;
        float2 pst[GS];
        double lsed[GS];
        float lsef[GS];
        ld_stats<GS>(s, b, h0, nqk_all, nqk, pstat, pst);
        // this thread's two positions of a pass: bins, logits, value norms and row,
        // the next pass's loaded while this one is decided and streamed
        int j0 = 0;
        uint32_t bw = 0;
        float2 lg[GS], nv = make_float2(1.0f, 1.0f);
        int64_t vrow = 0;
        auto load = [&](int sb, int &jj, uint32_t &bb, float2 (&ll)[GS], float2 &nn, int64_t &vr) {
            jj = sb + 2 * tid;
            bb = 0;
            vr = 0;
            nn = make_float2(1.0f, 1.0f);
#pragma unroll
            for (int hh = 0; hh < GS; ++hh)
                ll[hh] = make_float2(0.0f, 0.0f);
            if (jj < p1) {
                vr = kv_row(s, m, b, g, jj);
                bb = *reinterpret_cast<const uint32_t *>(Bg + jj);
#pragma unroll
                for (int hh = 0; hh < GS; ++hh)
                    ll[hh] = *reinterpret_cast<const float2 *>(Lg + (int64_t)hh * Sp + jj);
                if (vn)
                    nn = *reinterpret_cast<const float2 *>(vn + vr);
            }
        };
        load(p0, j0, bw, lg, nv, vrow);
        group_lse<GS>(s, b, h0, nqk_all, nqk, pstat, pst, LL, lsed);
#pragma unroll
        for (int hh = 0; hh < GS; ++hh)
            lsef[hh] = (float)lsed[hh];
        if (!poison) {
            uint32_t nst = 0, off = 0;
            for (int sb = p0; sb < p1; sb += PV_PASS) {
                int j0n = 0;
                uint32_t bwn = 0;
                float2 lgn[GS], nvn = make_float2(1.0f, 1.0f);
                int64_t vrown = 0;
                if (sb + PV_PASS < p1)
                    load(sb + PV_PASS, j0n, bwn, lgn, nvn, vrown);
                const bool va = j0 < p1, vb = j0 + 1 < p1;
                const uint32_t ba = bw & 0xffffu, bb = bw >> 16;
                bool ka = va && ba > d, kb = vb && bb > d;
                if (va && ba == d) {
                    float ax[GS];
#pragma unroll
                    for (int hh = 0; hh < GS; ++hh)
                        ax[hh] = lg[hh].x;
                    ka = rank_key(pos_key(pos_score<GS>(ax, lsed, sc, vn != nullptr, nv.x)), d, j0) >= thr;
                }
                if (vb && bb == d) {
                    float ay[GS];
#pragma unroll
                    for (int hh = 0; hh < GS; ++hh)
                        ay[hh] = lg[hh].y;
                    kb = rank_key(pos_key(pos_score<GS>(ay, lsed, sc, vn != nullptr, nv.y)), d, j0 + 1) >= thr;
                }
                uint32_t ex;
                const uint32_t tot = pass_slots((uint32_t)ka + (uint32_t)kb, ex);
                uint32_t so = nst + ex;
                if (ka) {
                    rows[so] = vrow;
#pragma unroll
                    for (int hh = 0; hh < GS; ++hh)
                        U.pr[hh][so] = expf(fmaf(s.scale, lg[hh].x, -lsef[hh]));
                    ++so;
                }
                if (kb) {
                    rows[so] = vrow + 1;
#pragma unroll
                    for (int hh = 0; hh < GS; ++hh)
                        U.pr[hh][so] = expf(fmaf(s.scale, lg[hh].y, -lsef[hh]));
                }
                if (pstage) {
                    int32_t *dst = pstage + (int64_t)grp * Sp + p0 + off + ex;
                    if (ka)
                        *dst++ = j0;
                    if (kb)
                        *dst = j0 + 1;
                }
                nst += tot;
                off += tot;
                kept_n += tot;
                __syncthreads();
                // (uniform) a further pass could overflow the stage, or this is the last pass
                if (nst > (uint32_t)(PV_STAGE - PV_PASS) || sb + PV_PASS >= p1) {
                    stream((int)nst);
                    nst = 0;
                }
                __syncthreads();
                j0 = j0n;
                bw = bwn;
                vrow = vrown;
                nv = nvn;
#pragma unroll
                for (int hh = 0; hh < GS; ++hh)
                    lg[hh] = lgn[hh];
            }
        }
        if (pcount && tid == 0)
            pcount[(int64_t)grp * npv + c] = poison ? 0u : kept_n;
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
    __syncthreads(); // (the partials reuse the probability staging)
    if ((lane >> 4) == 0) {
#pragma unroll
        for (int hh = 0; hh < GS; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                U.red[w][hh][(lane & 15) * 8 + e] = acc[hh][e];
    }
    __syncthreads();
    float *mine = part + ((int64_t)grp * npv + c) * GS * D;
    for (int i = tid; i < GS * D; i += PV_THREADS) {
        const int hh = i / D, dd = i % D;
        float x = U.red[0][hh][dd];
#pragma unroll
        for (int ww = 1; ww < PV_WAVES; ++ww)
            x += U.red[ww][hh][dd];
        mine[i] = poison ? __builtin_nanf("") : x;
    }
}

// ------------------------------------------------------------------ per-query-head PV over the union of rows
// Per-query-head selection with G > 1: after the key launch has published every
// head's threshold, one workgroup per (chunk of P positions, KV head) decides
// for each position and each of the G heads whether that head keeps it (the
// head's own score, bin and rank key, as its key workgroups computed them),
// and streams every position some head keeps once, each head adding p_h * V
// for the positions it keeps (0 for the others).  Partials per (KV head,
// chunk, head) as the grouped path writes them; the kept positions per head go
// to the staging lists.
template <int GS>
__global__ __launch_bounds__(PV_THREADS) void attn_pv_union_kernel(AttnShape s, KvMap m, int Sp, int nqk_all, int P,
                                                                   const uint16_t *__restrict__ v,
                                                                   const float *__restrict__ logit,
                                                                   const float2 *__restrict__ pstat,
                                                                   const float *__restrict__ vn,
                                                                   const uint64_t *__restrict__ sig,
                                                                   int32_t *__restrict__ pstage,
                                                                   uint32_t *__restrict__ pcount,
                                                                   float *__restrict__ part)
{
    __shared__ LseLds LL;
    __shared__ PvLds<GS> L;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int grp = blockIdx.y, c = blockIdx.x, npv = gridDim.x;
    const int b = grp / (int)s.Hkv, g = grp % (int)s.Hkv, h0 = g * s.G;
    const int Sb = seq_len(s, m, b);
    const int p0 = c * P, p1 = min(Sb, p0 + P);
    const float *Lg = logit + ((int64_t)b * s.Hq + h0) * Sp;
    const double sc = (double)s.scale;
    const int quarter = lane >> 4, dl = lane & 15, slot = w * 4 + quarter;
    constexpr int NSLOT = PV_WAVES * 4;
    float acc[GS][8];
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[hh][e] = 0.0f;
    bool poison = false;
    uint32_t kept_h[GS];
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
        kept_h[hh] = 0;

    auto stream = [&](int nk) {
        for (int r0 = slot; r0 < nk; r0 += NSLOT * PV_U) {
            uint4 uu[PV_U];
#pragma unroll
            for (int qq = 0; qq < PV_U; ++qq) {
                const int r = r0 + NSLOT * qq;
                if (r < nk)
                    uu[qq] = *reinterpret_cast<const uint4 *>(v + L.rows[r] * D + dl * 8);
            }
#pragma unroll
            for (int qq = 0; qq < PV_U; ++qq) {
                const int r = r0 + NSLOT * qq;
                if (r < nk) {
                    float vv[8];
                    Vec16<uint16_t>::unpack(uu[qq], vv);
#pragma unroll
                    for (int hh = 0; hh < GS; ++hh) {
                        const float pv = L.pr[hh][r];
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[hh][e] = fmaf(pv, vv[e], acc[hh][e]);
                    }
                }
            }
        }
    };
    // exclusive slot of this thread's n (wave scan plus the wave totals in LDS);
    // returns the block total.  A barrier must separate two calls.
    auto pass_slots = [&](uint32_t n, uint32_t &excl) -> uint32_t {
        const uint32_t ki = wave_incl_sum(n);
        if (lane == WAVE - 1)
            L.wk[w] = ki;
        __syncthreads();
        uint32_t before = 0, tot = 0;
#pragma unroll
        for (int i = 0; i < PV_WAVES; ++i) {
            before += i < w ? L.wk[i] : 0u;
            tot += L.wk[i];
        }
        excl = before + ki - n;
        return tot;
    };

    if (p0 < p1) { // (uniform) chunks past the sequence's end write zeros
        // every head's threshold: bin d, all-of-bin-d flag, rank key (the key launch has finished)
        uint32_t dh[GS];
        uint64_t th[GS];
#pragma unroll
        for (int hh = 0; hh < GS; ++hh) {
            const uint64_t *sw = sig + ((int64_t)b * s.Hq + h0 + hh) * SIG_WORDS;
            const uint64_t w1 = sw[SIG_D], w2 = sw[SIG_THR];
            const bool all = (w1 & 2ull) != 0ull;
            poison |= !(w1 & 1ull) || (!all && !(w2 & 1ull));
            dh[hh] = (uint32_t)(w1 >> 40);
            th[hh] = all ? 0ull : w2 >> 1;
        }
        const int nqk = (Sb + ATTN_QK_CHUNK - 1) / ATTN_QK_CHUNK;
        float2 pst[GS];
        double lsed[GS];
        float lsef[GS];
        ld_stats<GS>(s, b, h0, nqk_all, nqk, pstat, pst);
        group_lse<GS>(s, b, h0, nqk_all, nqk, pstat, pst, LL, lsed);
#pragma unroll
        for (int hh = 0; hh < GS; ++hh)
            lsef[hh] = (float)lsed[hh];
        if (!poison) {
            uint32_t nst = 0;
            uint32_t off[GS]; // kept positions of each head staged so far (pstage)
#pragma unroll
            for (int hh = 0; hh < GS; ++hh)
                off[hh] = 0;
            for (int sb = p0; sb < p1; sb += PV_PASS) {
                // this thread's two positions (j0 even, Sp a multiple of 8, pages hold a multiple of 8)
                const int j0 = sb + 2 * tid;
                const bool va = j0 < p1, vb = j0 + 1 < p1;
                float2 lg[GS];
                float2 nv = make_float2(1.0f, 1.0f);
                int64_t vrow = 0;
#pragma unroll
                for (int hh = 0; hh < GS; ++hh)
                    lg[hh] = make_float2(0.0f, 0.0f);
                if (va) {
                    vrow = kv_row(s, m, b, g, j0);
#pragma unroll
                    for (int hh = 0; hh < GS; ++hh)
                        lg[hh] = *reinterpret_cast<const float2 *>(Lg + (int64_t)hh * Sp + j0);
                    if (vn)
                        nv = *reinterpret_cast<const float2 *>(vn + vrow);
                }
                // which heads keep each position: the head's own score key against its threshold
                uint32_t ma = 0, mb = 0;
#pragma unroll
                for (int hh = 0; hh < GS; ++hh) {
                    const float ax[1] = {lg[hh].x}, ay[1] = {lg[hh].y};
                    const double lh[1] = {lsed[hh]};
                    const uint64_t ka = pos_key(pos_score<1>(ax, lh, sc, vn != nullptr, nv.x));
                    const uint64_t kb = pos_key(pos_score<1>(ay, lh, sc, vn != nullptr, nv.y));
                    const uint32_t ba = key_bin(ka), bb = key_bin(kb);
                    const bool keepa = va && (ba > dh[hh] || (ba == dh[hh] && rank_key(ka, dh[hh], j0) >= th[hh]));
                    const bool keepb =
                        vb && (bb > dh[hh] || (bb == dh[hh] && rank_key(kb, dh[hh], j0 + 1) >= th[hh]));
                    ma |= (uint32_t)keepa << hh;
                    mb |= (uint32_t)keepb << hh;
                }
                uint32_t ex;
                const uint32_t tot = pass_slots((uint32_t)(ma != 0u) + (uint32_t)(mb != 0u), ex);
                uint32_t so = nst + ex;
                if (ma) {
                    L.rows[so] = vrow;
#pragma unroll
                    for (int hh = 0; hh < GS; ++hh)
                        L.pr[hh][so] = ((ma >> hh) & 1u) ? expf(fmaf(s.scale, lg[hh].x, -lsef[hh])) : 0.0f;
                    ++so;
                }
                if (mb) {
                    L.rows[so] = vrow + 1;
#pragma unroll
                    for (int hh = 0; hh < GS; ++hh)
                        L.pr[hh][so] = ((mb >> hh) & 1u) ? expf(fmaf(s.scale, lg[hh].y, -lsef[hh])) : 0.0f;
                }
                nst += tot;
                __syncthreads();
                // each head's kept positions, ascending, for the kept-position lists
                if (pstage) {
#pragma unroll
                    for (int hh = 0; hh < GS; ++hh) {
                        const uint32_t ka = (ma >> hh) & 1u, kb = (mb >> hh) & 1u;
                        uint32_t e2;
                        const uint32_t t2 = pass_slots(ka + kb, e2);
                        int32_t *dst = pstage + ((int64_t)b * s.Hq + h0 + hh) * Sp + p0 + off[hh] + e2;
                        if (ka)
                            *dst++ = j0;
                        if (kb)
                            *dst = j0 + 1;
                        off[hh] += t2;
                        __syncthreads();
                    }
                }
#pragma unroll
                for (int hh = 0; hh < GS; ++hh)
                    kept_h[hh] += ((ma >> hh) & 1u) + ((mb >> hh) & 1u);
                // (uniform) a further pass could overflow the stage, or this is the last pass
                if (nst > (uint32_t)(PV_STAGE - PV_PASS) || sb + PV_PASS >= p1) {
                    stream((int)nst);
                    nst = 0;
                }
                __syncthreads();
            }
        }
        if (pcount) {
            // this chunk's kept count per head (block sums of the threads' counts)
#pragma unroll
            for (int hh = 0; hh < GS; ++hh) {
                uint32_t e3;
                const uint32_t t3 = pass_slots(kept_h[hh], e3);
                if (tid == 0)
                    pcount[((int64_t)b * s.Hq + h0 + hh) * npv + c] = poison ? 0u : t3;
                __syncthreads();
            }
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
    __syncthreads(); // (the partials reuse the probability staging)
    if ((lane >> 4) == 0) {
#pragma unroll
        for (int hh = 0; hh < GS; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                L.red[w][hh][(lane & 15) * 8 + e] = acc[hh][e];
    }
    __syncthreads();
    float *mine = part + ((int64_t)grp * npv + c) * GS * D;
    for (int i = tid; i < GS * D; i += PV_THREADS) {
        const int hh = i / D, dd = i % D;
        float x = L.red[0][hh][dd];
#pragma unroll
        for (int ww = 1; ww < PV_WAVES; ++ww)
            x += L.red[ww][hh][dd];
        mine[i] = poison ? __builtin_nanf("") : x;
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
    w.bins = (uint16_t *)p;
    p = align256(p + (size_t)(G * ((Sp + BIN_ROW - 1) / BIN_ROW * BIN_ROW)) * 2);
    w.hist = (uint32_t *)p;
    p = align256(p + (size_t)(G * ATTN_HIST_BINS) * 4);
    w.pcount = (uint32_t *)p;
    p = align256(p + (size_t)(G * npv) * 4);
    w.sig = (uint64_t *)p;
    p = align256(p + (size_t)(G * SIG_WORDS) * 8);
    w.pstage = (int32_t *)p;
    p = align256(p + (size_t)(G * Sp) * 4);
    w.pvpart = (float *)p;
    p = align256(p + (size_t)(G * npv * s.GS * D) * 4);
    if (ws)
        *ws = w;
    return (size_t)(p - base);
}

// Key chunks per workgroup: one up to 32K positions, more for longer sequences
// (fewer workgroups, fewer statistics merges and fewer global histogram atomics).
static int key_chunks_per_wg(int64_t S)
{
    const int64_t n = S / 32768;
    return n < 1 ? 1 : n > 4 ? 4 : (int)n;
}

// Workgroups of the fused kernel the current device holds at once (occupancy
// times compute units), per device.
template <int GS> static int64_t fused_resident()
{
    static int64_t cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 0;
    if (cached[dev] == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_fused_kernel<GS>, PV_THREADS, 0) !=
                hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cached[dev] = (int64_t)per_cu * cus;
    }
    return cached[dev];
}
constexpr int ATTN_SPLIT_PVU = 8; // V rows in flight per lane in the split PV kernel

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
    attn_qk_kernel<GS, false><<<dim3(nqk, G), QK_THREADS, 0, st>>>(s, m, Sp, q, kt, kn, ws.logit, ws.pstat,
                                                                    dim_idx, ws.hist, ws.sig);
    const int nkc = (int)((s.S + ATTN_KEY_CHUNK - 1) / ATTN_KEY_CHUNK);
    const int nsub = key_chunks_per_wg(s.S);
    const int nkw = (nkc + nsub - 1) / nsub;
    int32_t *pst = pos_idx ? ws.pstage : nullptr;
    uint32_t *pcn = pos_idx ? ws.pcount : nullptr;
    if ((int64_t)(nkw + npv) * G <= fused_resident<GS>()) {
        attn_fused_kernel<GS><<<(unsigned)((int64_t)(nkw + npv) * G), PV_THREADS, 0, st>>>(
            s, m, Sp, nqk, nsub, nkw, P, npv, v, ws.logit, ws.pstat, lse, vn, ws.bins, ws.hist, ws.sig, pst, pcn,
            ws.pvpart, 1);
    } else {
        // more workgroups than stay resident: the key role alone, the thresholds, then PV
        attn_fused_kernel<GS, true><<<(unsigned)((int64_t)nkw * G), PV_THREADS, 0, st>>>(
            s, m, Sp, nqk, nsub, nkw, P, npv, v, ws.logit, ws.pstat, lse, vn, ws.bins, ws.hist, ws.sig, pst, pcn,
            ws.pvpart, 0);
        attn_select_kernel<GS><<<G, SELK_THREADS, 0, st>>>(s, m, Sp, ws.logit, vn, ws.bins, ws.hist, ws.sig);
        attn_pv_split_kernel<GS, ATTN_SPLIT_PVU><<<dim3(npv, G), PV_THREADS, 0, st>>>(
            s, m, Sp, nqk, P, v, ws.logit, ws.pstat, vn, ws.bins, ws.sig, pst, pcn, ws.pvpart);
    }
    attn_pv_reduce_kernel<GS><<<G * (GS * D / WAVE), PVR_WAVES * WAVE, 0, st>>>(s, npv, ws.pvpart, out);
    if (pos_idx)
        attn_pos_kernel<<<dim3(npv, G), 256, 0, st>>>(s, m, Sp, P, ws.pcount, ws.pstage, pos_idx);
    return hipGetLastError();
}

// Per-query-head selection with G > 1 query heads per KV head: QK over the
// union of the heads' kept dims (one launch per KV head and chunk), the key
// role per head (the fused kernel with no PV workgroups), PV over the union of
// the heads' kept positions, the fixed-order reduce per KV head.
template <int G>
static hipError_t attn_run_union(const AttnShape &s, const KvMap &m, const uint16_t *q, const uint16_t *kt,
                                 const uint16_t *v, const float *kn, const float *vn, float *out, int32_t *dim_idx,
                                 int32_t *pos_idx, float *lse, const AttnWs &ws, hipStream_t st)
{
    const int Sp = (int)((s.S + 7) / 8 * 8);
    const int Gsel = (int)(s.B * s.Hsel); // one selection group per query head
    const int Gkv = (int)(s.B * s.Hkv);
    const int nqk = (int)((s.S + ATTN_QK_CHUNK - 1) / ATTN_QK_CHUNK);
    int P, npv;
    pv_chunks(s.S, &P, &npv);
    attn_qk_kernel<G, true><<<dim3(nqk, Gkv), QK_THREADS, 0, st>>>(s, m, Sp, q, kt, kn, ws.logit, ws.pstat,
                                                                    dim_idx, ws.hist, ws.sig);
    const int nkc = (int)((s.S + ATTN_KEY_CHUNK - 1) / ATTN_KEY_CHUNK);
    const int nsub = key_chunks_per_wg(s.S);
    const int nkw = (nkc + nsub - 1) / nsub;
    attn_fused_kernel<1, true><<<(unsigned)((int64_t)nkw * Gsel), PV_THREADS, 0, st>>>(
        s, m, Sp, nqk, nsub, nkw, P, npv, v, ws.logit, ws.pstat, lse, vn, ws.bins, ws.hist, ws.sig, nullptr, nullptr,
        ws.pvpart, 1);
    attn_pv_union_kernel<G><<<dim3(npv, Gkv), PV_THREADS, 0, st>>>(s, m, Sp, nqk, P, v, ws.logit, ws.pstat, vn,
                                                                   ws.sig, pos_idx ? ws.pstage : nullptr,
                                                                   pos_idx ? ws.pcount : nullptr, ws.pvpart);
    AttnShape su = s; // the partials are laid out per KV head with its G heads
    su.GS = G;
    su.Hsel = (int)s.Hkv;
    attn_pv_reduce_kernel<G><<<Gkv * (G * D / WAVE), PVR_WAVES * WAVE, 0, st>>>(su, npv, ws.pvpart, out);
    if (pos_idx)
        attn_pos_kernel<<<dim3(npv, Gsel), 256, 0, st>>>(s, m, Sp, P, ws.pcount, ws.pstage, pos_idx);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnShape &s, const KvMap &m, const uint16_t *q, const uint16_t *kt, const uint16_t *v,
                       const float *kn, const float *vn, float *out, int32_t *dim_idx, int32_t *pos_idx, float *lse,
                       const AttnWs &ws, hipStream_t st)
{
    if (s.GS == 1 && s.G > 1) {
        switch (s.G) {
        case 2:
            return attn_run_union<2>(s, m, q, kt, v, kn, vn, out, dim_idx, pos_idx, lse, ws, st);
        case 4:
            return attn_run_union<4>(s, m, q, kt, v, kn, vn, out, dim_idx, pos_idx, lse, ws, st);
        case 8:
            return attn_run_union<8>(s, m, q, kt, v, kn, vn, out, dim_idx, pos_idx, lse, ws, st);
        default:
            return hipErrorInvalidValue;
        }
    }
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
