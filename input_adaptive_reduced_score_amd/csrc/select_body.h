// The one-workgroup selection of a tile (scorer + top-k), shared by the
// selector kernel (select.hip) and the fused select-and-product kernel
// (gemv.hip).  See select_body.
#pragma once

#include "device.h"
#include "kernels.h"
#include "radix.h"

namespace rmm {

constexpr int SEL_THREADS = 1024;
constexpr uint32_t SEL_CAND_CAP = 256; // crossing-digit keys ranked directly
constexpr int SEL_RANK_SPLIT = SEL_THREADS / SEL_CAND_CAP; // threads per candidate in the ranking
constexpr int COLMAX_THREADS = 256;

// 8 consecutive elements from p as floats; `avail` of them are in range.  The
// 16-byte vector holding the first element is always read (row pitches are
// multiples of 16 bytes); for fp32 the second only if it holds one in range.
__device__ __forceinline__ void load8(const uint16_t *p, int avail, float (&v)[8])
{
    (void)avail;
    Vec16<uint16_t>::unpack(*reinterpret_cast<const uint4 *>(p), v);
}
__device__ __forceinline__ void load8(const float *p, int avail, float (&v)[8])
{
    const uint4 lo = *reinterpret_cast<const uint4 *>(p);
    const uint4 hi = avail > 4 ? *reinterpret_cast<const uint4 *>(p + 4) : make_uint4(0u, 0u, 0u, 0u);
    v[0] = __uint_as_float(lo.x); v[1] = __uint_as_float(lo.y); v[2] = __uint_as_float(lo.z); v[3] = __uint_as_float(lo.w);
    v[4] = __uint_as_float(hi.x); v[5] = __uint_as_float(hi.y); v[6] = __uint_as_float(hi.z); v[7] = __uint_as_float(hi.w);
}

// 0/1 predicates computed with integer arithmetic on values below 2^31 (keys,
// slice indices, counts): they stay in vector registers, whereas comparisons
// combined with && / || become lane-mask logic on the one scalar unit the
// workgroup's 16 waves share.
// Histogram bins are stored with one pad word per 32 bins: bin 32g+e sits at
// word 33g+e, so the 32 bins of group g are contiguous and the 64 groups that
// wave 0's lanes read start in distinct LDS banks.
__device__ __forceinline__ int hpad(int b) { return b + (b >> 5); }
constexpr int SEL_HIST_WORDS = SEL_BINS + SEL_BINS / 32;
constexpr int SEL_DUMMY = SEL_HIST_WORDS; // + lane: per-lane sink for masked-off histogram atomics

// The whole block finds the digit holding the krem-th largest key, clears the
// histogram and publishes (digit, rank inside the digit, keys in the digit) in
// res[0..2].  Thread t owns bins 2047-2t and 2046-2t, so threads in ascending
// order walk the bins from the top: a wave scan plus one exchange of wave
// totals gives every thread the count above its bins.  Contains barriers.
__device__ __forceinline__ void block_crossing(uint32_t *hist, uint32_t krem, uint32_t *wtot, uint32_t *res)
{
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int b0 = SEL_BINS - 1 - 2 * tid; // the higher of the thread's two bins
    const uint32_t h0 = hist[hpad(b0)], h1 = hist[hpad(b0 - 1)];
    hist[hpad(b0)] = 0;
    hist[hpad(b0 - 1)] = 0;
    const uint32_t sum = h0 + h1;
    const uint32_t incl = wave_incl_sum(sum);
    if (lane == WAVE - 1)
        wtot[w] = incl;
    __syncthreads();
    uint32_t above = incl - sum;
#pragma unroll
    for (int v = 0; v < SEL_THREADS / WAVE; ++v)
        above += v < w ? wtot[v] : 0u;
    if (above < krem && krem <= above + sum) {
        const bool hi = krem <= above + h0;
        res[0] = (uint32_t)(hi ? b0 : b0 - 1);
        res[1] = hi ? krem - above : krem - above - h0;
        res[2] = hi ? h0 : h1;
    }
    __syncthreads();
}

// Scorer + selector, one workgroup of 1024 threads (16 waves) per tile.
// Thread t scores slices t*PER .. t*PER+PER-1 (16-byte loads) and keeps their
// keys in registers for the whole kernel; threads in ascending order hold the
// slices in ascending order, so every ordered count is a per-lane count plus a
// wave scan plus one exchange of wave totals (vector ALU work, no per-element
// ballots).  Slots past K hold key 0: they rank after every real key (value 0,
// highest indices) and k <= K, so they are never kept.  Keys are re-based as
// u = key - (smallest non-zero key) + 1 (0 stays 0), an order-preserving map,
// so the first radix digit spans the keys' actual range instead of the few
// float exponents they share.  direct: score straight from x (few rows per
// tile); otherwise from the column-max partials (row pitch Kp).
// The selection of one tile by one workgroup of SEL_THREADS.  Without PUB it
// writes the tile's kept list to idx.  With PUB it publishes to the other
// workgroups of a fused select-and-product launch (SelPub): after the first
// radix pass, the re-basing minimum and the digit whose keys are still
// undecided (sig1; keys above it are kept for certain), then the exact
// threshold and the slice of the last kept key equal to it (sig2: as soon as
// the crossing digit's candidates are ranked, else after the compaction), and
// each split's count of kept slices before it (complete before sig3 is
// stored; only when pub.offs is given).  Published words are agent-scope stores (coherent across XCDs
// without cache write-backs).
template <typename TE, int PER, bool PUB>
__device__ __forceinline__ void select_body(const TE *__restrict__ x, int64_t ldx, int T, int K, int tile,
                                            const float *__restrict__ c, const float *__restrict__ pmax, int Kp,
                                            int nrsplit, int direct, int cvec, int k, int tau,
                                            int32_t *__restrict__ idx, const SelPub &pub)
{
    static_assert(PER == 4 || PER % 8 == 0, "slices per thread: 4, or 8-slice chunks");
    constexpr int NW = SEL_THREADS / WAVE;
    constexpr int CH = PER / 8; // chunks per thread (PER = 4: one 4-slice run, loaded separately)
    __shared__ uint32_t hist[SEL_HIST_WORDS + WAVE];
    __shared__ uint32_t wmin[NW], wmax[NW], wgt[NW], weq[NW], wtot[NW];
    __shared__ uint2 cand[SEL_CAND_CAP];
    __shared__ uint32_t rk_above[SEL_RANK_SPLIT][SEL_CAND_CAP], rk_tie[SEL_RANK_SPLIT][SEL_CAND_CAP];
    __shared__ uint32_t res[6], ncand;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
    const int j0 = tid * PER; // first slice of this thread
    const int lim = K - j0;   // registers i < lim hold real slices

    for (int i = tid; i < SEL_HIST_WORDS; i += SEL_THREADS)
        hist[i] = 0;
    if (tid == 0) {
        res[0] = 0;
        res[1] = 1;
        res[2] = 0;
        res[3] = 0;
        res[4] = 0;
        res[5] = 0;
        ncand = 0;
    }

    // 1. scores -> keys
    float a[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i)
        a[i] = 0.0f;
    if constexpr (PER == 4) {
        // four slices per thread (K <= 4096): one 8-byte (bf16) or 16-byte (fp32) run
        if (j0 < K) {
            if (direct) {
                const int t0 = tau * tile, t1 = min(T, t0 + tile);
                for (int t = t0; t < t1; ++t) {
                    const TE *xr = x + (int64_t)t * ldx + j0;
                    float f[4];
                    if constexpr (sizeof(TE) == 2) {
                        const uint2 u = *reinterpret_cast<const uint2 *>(xr);
                        f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
                    } else {
                        const uint4 u = *reinterpret_cast<const uint4 *>(xr);
                        f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
                        f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        a[e] = fmaxf(a[e], fabsf(f[e]));
                }
            } else {
                const float *pm = pmax + (int64_t)tau * nrsplit * Kp + j0;
                for (int rs = 0; rs < nrsplit; ++rs) {
                    const uint4 u = *reinterpret_cast<const uint4 *>(pm + (int64_t)rs * Kp);
                    a[0] = fmaxf(a[0], __uint_as_float(u.x)); a[1] = fmaxf(a[1], __uint_as_float(u.y));
                    a[2] = fmaxf(a[2], __uint_as_float(u.z)); a[3] = fmaxf(a[3], __uint_as_float(u.w));
                }
            }
        }
    } else {
        if (direct) {
            const int t0 = tau * tile, t1 = min(T, t0 + tile);
            for (int t = t0; t < t1; ++t) {
                const TE *xr = x + (int64_t)t * ldx;
    #pragma unroll
                for (int m = 0; m < CH; ++m) {
                    const int jc = j0 + 8 * m;
                    if (jc < K) {
                        float f[8];
                        load8(xr + jc, K - jc, f);
    #pragma unroll
                        for (int e = 0; e < 8; ++e)
                            a[8 * m + e] = fmaxf(a[8 * m + e], fabsf(f[e]));
                    }
                }
            }
        } else {
            const float *pm = pmax + (int64_t)tau * nrsplit * Kp;
            for (int rs = 0; rs < nrsplit; ++rs) {
    #pragma unroll
                for (int m = 0; m < CH; ++m) {
                    const int jc = j0 + 8 * m;
                    if (jc < K) {
                        float f[8];
                        load8(pm + (int64_t)rs * Kp + jc, K - jc, f);
    #pragma unroll
                        for (int e = 0; e < 8; ++e)
                            a[8 * m + e] = fmaxf(a[8 * m + e], f[e]);
                    }
                }
            }
        }
    }
    uint32_t uk[PER];
    uint32_t mn = 0xffffffffu, mx = 0u;
    if constexpr (PER == 4) {
        const int avail = K - j0; // <= 0 past the end
        float cw[4];
        if (cvec && avail >= 4) {
            const uint4 u = *reinterpret_cast<const uint4 *>(c + j0);
            cw[0] = __uint_as_float(u.x); cw[1] = __uint_as_float(u.y);
            cw[2] = __uint_as_float(u.z); cw[3] = __uint_as_float(u.w);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                cw[e] = e < avail ? c[j0 + e] : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t key = e < avail ? nonneg_key(__fmul_rn(a[e], cw[e])) : 0u;
            uk[e] = key;
            mn = min(mn, key == 0u ? 0xffffffffu : key);
            mx = max(mx, key);
        }
    }
#pragma unroll
    for (int m = 0; m < CH; ++m) {
        const int jc = j0 + 8 * m;
        const int avail = K - jc; // <= 0 past the end
        float cw[8];
        if (cvec && avail >= 8) {
            load8(c + jc, 8, cw);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                cw[e] = e < avail ? c[jc + e] : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t key = e < avail ? nonneg_key(__fmul_rn(a[8 * m + e], cw[e])) : 0u;
            uk[8 * m + e] = key;
            mn = min(mn, key == 0u ? 0xffffffffu : key);
            mx = max(mx, key);
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
    // re-base: u = key - mn + 1 for key > 0, 0 stays 0 (mn = smallest non-zero key)
    const uint32_t umax = mx == 0u ? 0u : mx - mn + 1u;
    const int L = umax == 0u ? 0 : 32 - __clz(umax);
#pragma unroll
    for (int i = 0; i < PER; ++i)
        uk[i] = uk[i] == 0u ? 0u : uk[i] - mn + 1u;
    bool published1 = false, published2 = false;

    // 2. radix passes from the top bit of umax, up to 11 bits each.  After a
    // pass, if few keys share the crossing digit they are gathered and ranked
    // exactly (key descending, then slice ascending), which settles the rest.
    uint32_t prefix = 0, pmask = 0, krem = (uint32_t)k;
    int top = L;
    while (top > 0) {
        opaque_all(uk);
        const int nb = top < 11 ? top : 11;
        const int sh = top - nb;
        const uint32_t dm = (1u << nb) - 1u;
        // zero keys (all in bin 0) are counted per lane and added once per
        // wave: same-address LDS atomics serialise.  The first pass (every key
        // eligible) adds unconditionally, masked-off lanes into their own sink.
        uint32_t zc = 0;
        if (pmask == 0u) {
            const int lim1 = opaque(lim);
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const uint32_t real = ilt(i, lim1), nz = lt31(0u, uk[i]);
                const uint32_t in = real & nz;
                zc += real - in;
                const uint32_t word = in * (uint32_t)hpad((int)((uk[i] >> sh) & dm)) + (1u - in) * (SEL_DUMMY + lane);
                atomicAdd(&hist[word], 1u);
            }
        } else {
            const int lim2 = opaque(lim);
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                if (i < lim2 && (uk[i] & pmask) == prefix) {
                    if (uk[i] == 0u)
                        ++zc;
                    else
                        atomicAdd(&hist[hpad((int)((uk[i] >> sh) & dm))], 1u);
                }
            }
        }
        if (prefix == 0u) {
            const uint32_t zw = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_sum(zc), WAVE - 1);
            if (lane == 0 && zw != 0u)
                atomicAdd(&hist[hpad(0)], zw);
        }
        __syncthreads();
        block_crossing(hist, krem, wtot, res);
        prefix |= res[0] << sh;
        pmask |= dm << sh;
        krem = res[1];
        const uint32_t nc = res[2];
        top = sh;
        if constexpr (PUB) {
            if (!published1) { // keys whose digit lies above the crossing digit are kept for certain
                if (tid == 0)
                    pub_store64(pub.sig1, sig1_pack(mn, res[0], sh, nb));
                published1 = true;
            }
        }
        if (top > 0 && nc <= SEL_CAND_CAP) {
            // gather the crossing digit's keys (any order): per-lane count, wave
            // scan, one slot reservation per wave
            // (the lane's candidates as a bit mask; only set bits are visited below)
            opaque_all(uk);
            const int limc = opaque(lim);
            uint32_t cmask = 0;
#pragma unroll
            for (int i = 0; i < PER; ++i)
                cmask |= (ilt(i, limc) & eq31(uk[i] & pmask, prefix)) << i;
            const uint32_t cl = (uint32_t)__popc(cmask);
            const uint32_t cincl = wave_incl_sum(cl);
            const uint32_t wcount = (uint32_t)__builtin_amdgcn_readlane((int)cincl, WAVE - 1);
            uint32_t base = 0;
            if (lane == 0 && wcount != 0u)
                base = atomicAdd(&ncand, wcount);
            base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
            uint32_t slot = base + cincl - cl;
            while (cmask) {
                const int b = __builtin_ctz(cmask);
                cmask &= cmask - 1u;
                uint32_t kv = 0; // uk[b] through compile-time indices (no private-memory copy of uk)
#pragma unroll
                for (int q = 0; q < PER; ++q)
                    kv = q == b ? uk[q] : kv;
                if (slot < SEL_CAND_CAP)
                    cand[slot] = make_uint2(kv, (uint32_t)(j0 + b));
                ++slot;
            }
            __syncthreads();
            // the candidate ranked krem-th fixes the threshold key and how many
            // keys equal to it (lowest slices first) are kept.  Thread t compares
            // candidate t % CAP with every SEL_RANK_SPLIT-th other candidate.
            {
                const uint32_t me_i = (uint32_t)tid % SEL_CAND_CAP, part = (uint32_t)tid / SEL_CAND_CAP;
                if (me_i < nc) {
                    const uint2 me = cand[me_i];
                    uint32_t ab0 = 0, ab1 = 0, ti0 = 0, ti1 = 0;
                    uint32_t i = part;
                    // o ranks above me: larger key, or equal key at a lower slice;
                    // tie_upto counts equal keys at slices <= me's
                    for (; i + SEL_RANK_SPLIT < nc; i += 2 * SEL_RANK_SPLIT) {
                        const uint2 o0 = cand[i], o1 = cand[i + SEL_RANK_SPLIT];
                        const uint32_t e0 = eq31(o0.x, me.x), e1 = eq31(o1.x, me.x);
                        ab0 += lt31(me.x, o0.x) | (e0 & lt31(o0.y, me.y));
                        ti0 += e0 & (1u - lt31(me.y, o0.y));
                        ab1 += lt31(me.x, o1.x) | (e1 & lt31(o1.y, me.y));
                        ti1 += e1 & (1u - lt31(me.y, o1.y));
                    }
                    if (i < nc) {
                        const uint2 o0 = cand[i];
                        const uint32_t e0 = eq31(o0.x, me.x);
                        ab0 += lt31(me.x, o0.x) | (e0 & lt31(o0.y, me.y));
                        ti0 += e0 & (1u - lt31(me.y, o0.y));
                    }
                    rk_above[part][me_i] = ab0 + ab1;
                    rk_tie[part][me_i] = ti0 + ti1;
                }
            }
            __syncthreads();
            if (tid < (int)nc) {
                uint32_t above = 0, tie_upto = 0;
#pragma unroll
                for (int q = 0; q < SEL_RANK_SPLIT; ++q) {
                    above += rk_above[q][tid];
                    tie_upto += rk_tie[q][tid];
                }
                if (above + 1u == krem) {
                    res[3] = cand[tid].x;
                    res[4] = tie_upto;
                    res[5] = cand[tid].y; // the last kept slice
                }
            }
            __syncthreads();
            prefix = res[3];
            krem = res[4];
            if constexpr (PUB) {
                // the threshold is out before the compaction; the offsets follow (sig3)
                if (tid == 0)
                    pub_store64(pub.sig2, sig2_pack(prefix, (int)res[5]));
                published2 = true;
            }
            break;
        }
    }
    // (L == 0: every key is zero; prefix 0 and krem = k ties)
    if constexpr (PUB) {
        if (published2 && !pub.offs)
            return; // the threshold is out and no kept list is asked for
    }

    // 3. order-preserving compaction.  Kept: u > prefix, or u == prefix among
    // the first krem such slices.  Output position of a slice = slices kept
    // before it = (greater before) + min(equal before, krem).
    // The lane's greater and equal slices as bit masks (masked-off registers hold 0,
    // which is never above the threshold; a zero threshold is matched only by real
    // slices); only kept bits are visited when writing.
    opaque_all(uk);
    const int limk = opaque(lim);
    uint32_t gmask = 0, emask = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const uint32_t real = ilt(i, limk);
        gmask |= (real & lt31(prefix, uk[i])) << i;
        emask |= (real & eq31(uk[i], prefix)) << i;
    }
    const uint32_t gl = (uint32_t)__popc(gmask), el = (uint32_t)__popc(emask);
    const uint32_t gincl = wave_incl_sum(gl), eincl = wave_incl_sum(el);
    if (lane == WAVE - 1) {
        wgt[w] = gincl;
        weq[w] = eincl;
    }
    __syncthreads();
    uint32_t gb = gincl - gl, eb = eincl - el;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        gb += v < w ? wgt[v] : 0u;
        eb += v < w ? weq[v] : 0u;
    }
    // kept: every greater slice, and equal slices while fewer than krem equal ones precede them
    uint32_t kmask = gmask;
    {
        uint32_t em = emask, ebr = eb;
        while (em) { // rare: usually only the threshold's own slice
            const int b = __builtin_ctz(em);
            em &= em - 1u;
            kmask |= lt31(ebr, krem) << b;
            ++ebr;
        }
    }
    // in ascending slice order from the count of slices kept before this thread
    uint32_t pos = gb + min(eb, krem);
    if constexpr (PUB) {
        if (!published1 && tid == 0)
            pub_store64(pub.sig1, sig1_pack(mn, 0u, 0, 0)); // every key zero: all of them undecided
        // the slice of the krem-th key equal to the threshold (the last one kept)
        __shared__ int jt_s;
        if (eb < krem && krem <= eb + el) {
            uint32_t em = emask;
            for (uint32_t q = krem - eb; q > 1u; --q)
                em &= em - 1u;
            jt_s = j0 + __builtin_ctz(em);
        }
        // kept slices before each split's first slice that falls in this thread's slices: split
        // 0 starts at slice 0, split p >= 1 at R0 + (p - 1) * R1 (splits starting at K: all k)
        auto put_off = [&](int p) {
            const int bq = split_start0(pub, p, K) - j0;
            const uint32_t below = bq >= 32 ? kmask : (kmask & ((1u << bq) - 1u));
            pub_store(pub.offs + p, pos + (uint32_t)__popc(below));
        };
        if (pub.offs && j0 == 0 && K > 0)
            put_off(0);
        if (pub.offs && pub.nsplit >= 1 && K > pub.R0 && j0 + PER > pub.R0 && j0 < K) {
            const int a = j0 > pub.R0 ? (j0 - pub.R0 + pub.R1 - 1) / pub.R1 : 0; // first p - 1 with start >= j0
            const int b = (min(j0 + PER, K) - 1 - pub.R0) / pub.R1;              // last p - 1 with start < j0 + PER
            for (int p = 1 + a; p <= 1 + b && p <= pub.nsplit; ++p)
                put_off(p);
        }
        if (pub.offs && tid == 0) { // first split starting at K: 1 + ceil((K - R0) / R1)
            const int pend = K > pub.R0 ? 1 + (K - pub.R0 + pub.R1 - 1) / pub.R1 : 1;
            for (int p = pend; p <= pub.nsplit; ++p)
                pub_store(pub.offs + p, (uint32_t)k);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            if (!published2)
                pub_store64(pub.sig2, sig2_pack(prefix, jt_s));
            if (pub.offs)
                pub_store64(pub.sig3, 1ull);
        }
    } else {
        extern __shared__ int32_t outl[]; // k entries: the kept list before it is written out
        while (kmask) {
            const int b = __builtin_ctz(kmask);
            kmask &= kmask - 1u;
            if (pos < (uint32_t)k)
                outl[pos] = j0 + b;
            ++pos;
        }
        // the list is staged in LDS, then written with coalesced stores
        __syncthreads();
        int32_t *dst = idx + (int64_t)tau * k;
        for (int p = tid; p < k; p += SEL_THREADS)
            dst[p] = outl[p];
    }
}

} // namespace rmm
