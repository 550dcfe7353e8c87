// Block-wide radix selection helpers (top-k by key, ties to the lower index).
#pragma once

#include "device.h"

namespace rmm {

constexpr int SEL_BINS = 2048;

// One radix pass over `n` keys (LDS or global), restricted to keys whose bits
// under `pmask` equal `prefix`.  Finds the digit (bits [shift, shift+nbits)) of
// the krem-th largest key and returns it through `res`; updates krem.
// Every thread of the block calls it.  `hist` holds SEL_BINS words of LDS,
// `tmp` 64 words.
__device__ __forceinline__ void radix_pass(const uint32_t *keys, int n, uint32_t &prefix, uint32_t &pmask,
                                           int shift, int nbits, uint32_t &krem, uint32_t *hist, uint32_t *tmp)
{
    const uint32_t dm = (1u << nbits) - 1u;
    for (int i = threadIdx.x; i < SEL_BINS; i += blockDim.x)
        hist[i] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += blockDim.x) {
        uint32_t key = keys[j];
        if ((key & pmask) == prefix)
            atomicAdd(&hist[(key >> shift) & dm], 1u);
    }
    __syncthreads();
    // thread t covers bins hb = 2047-2t (higher) and hb-1, i.e. descending digit order
    const int hb = SEL_BINS - 1 - 2 * (int)threadIdx.x;
    uint32_t ch = 0, cl = 0;
    if (hb >= 1) {
        ch = hist[hb];
        cl = hist[hb - 1];
    }
    uint32_t incl = block_incl_scan(ch + cl, tmp);
    uint32_t excl = incl - ch - cl;
    if (hb >= 1) {
        if (excl < krem && krem <= excl + ch) {
            tmp[32] = (uint32_t)hb;
            tmp[33] = krem - excl;
        } else if (excl + ch < krem && krem <= incl) {
            tmp[32] = (uint32_t)(hb - 1);
            tmp[33] = krem - excl - ch;
        }
    }
    __syncthreads();
    prefix |= tmp[32] << shift;
    pmask |= dm << shift;
    krem = tmp[33];
    __syncthreads();
}

// Order-preserving compaction: writes, in ascending j, every j with
// key > thr, plus the first `quota` (in index order) with key == thr.
// Threads own contiguous index ranges.  Every thread of the block calls it.
// n <= 65535 is not required: counts are packed as gt | eq << 16 only when
// n <= 32768; larger n uses two scans.
__device__ __forceinline__ void compact_ascending(const uint32_t *keys, int n, uint32_t thr, uint32_t quota,
                                                  int32_t *out, uint32_t *tmp)
{
    const int chunk = (n + (int)blockDim.x - 1) / (int)blockDim.x;
    const int j0 = min(n, (int)threadIdx.x * chunk), j1 = min(n, j0 + chunk);
    uint32_t gt = 0, eq = 0;
    for (int j = j0; j < j1; ++j) {
        uint32_t key = keys[j];
        gt += key > thr;
        eq += key == thr;
    }
    uint32_t gt_b, eq_b;
    if (n <= 32768) {
        uint32_t packed = gt | (eq << 16);
        uint32_t ex = block_incl_scan(packed, tmp) - packed;
        gt_b = ex & 0xffffu;
        eq_b = ex >> 16;
    } else {
        gt_b = block_incl_scan(gt, tmp) - gt;
        eq_b = block_incl_scan(eq, tmp) - eq;
    }
    uint32_t pos = gt_b + min(eq_b, quota);
    for (int j = j0; j < j1; ++j) {
        uint32_t key = keys[j];
        if (key > thr || (key == thr && eq_b++ < quota))
            out[pos++] = j;
    }
}


// Finds, in a histogram of `nbins` digit counts (nbins a multiple of
// blockDim.x, at most 8 per thread; LDS or global), the digit holding the
// krem-th largest key; returns it, updates krem to the rank inside that digit
// and, if `count` is given, sets it to that digit's count.  Each count is read
// once (a global histogram costs one round trip).  Every thread calls it.
__device__ __forceinline__ uint32_t hist_crossing(const uint32_t *hist, int nbins, uint32_t &krem, uint32_t *tmp,
                                                  uint32_t *count = nullptr)
{
    constexpr int MAXPER = 8;
    const int per = nbins / (int)blockDim.x;
    const int top = nbins - 1 - (int)threadIdx.x * per; // this thread covers bins top, top-1, ..., top-per+1
    uint32_t c[MAXPER];
    uint32_t tot = 0;
#pragma unroll
    for (int q = 0; q < MAXPER; ++q) {
        c[q] = q < per ? hist[top - q] : 0u;
        tot += c[q];
    }
    const uint32_t incl = block_incl_scan(tot, tmp);
    uint32_t run = incl - tot;
#pragma unroll
    for (int q = 0; q < MAXPER; ++q) {
        if (q < per && run < krem && krem <= run + c[q]) {
            tmp[32] = (uint32_t)(top - q);
            tmp[33] = krem - run;
            tmp[34] = c[q];
        }
        run += c[q];
    }
    __syncthreads();
    const uint32_t d = tmp[32];
    krem = tmp[33];
    if (count)
        *count = tmp[34];
    __syncthreads();
    return d;
}

// hist_crossing in two steps, so that other loads can be issued between the
// histogram's loads and their use: hist_counts loads this thread's PER bins
// (nbins == PER * blockDim.x), crossing_from_counts finishes as hist_crossing.
template <int PER> __device__ __forceinline__ void hist_counts(const uint32_t *hist, uint32_t (&c)[PER])
{
    const int top = PER * (int)blockDim.x - 1 - (int)threadIdx.x * PER;
#pragma unroll
    for (int q = 0; q < PER; ++q)
        c[q] = hist[top - q];
}
template <int PER>
__device__ __forceinline__ uint32_t crossing_from_counts(const uint32_t (&c)[PER], uint32_t &krem, uint32_t *tmp,
                                                         uint32_t *count)
{
    const int top = PER * (int)blockDim.x - 1 - (int)threadIdx.x * PER;
    uint32_t tot = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q)
        tot += c[q];
    const uint32_t incl = block_incl_scan(tot, tmp);
    uint32_t run = incl - tot;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        if (run < krem && krem <= run + c[q]) {
            tmp[32] = (uint32_t)(top - q);
            tmp[33] = krem - run;
            tmp[34] = c[q];
        }
        run += c[q];
    }
    __syncthreads();
    const uint32_t d = tmp[32];
    krem = tmp[33];
    *count = tmp[34];
    __syncthreads();
    return d;
}

// radix_pass over a 16-byte aligned key array in global memory: 8 independent
// 16-byte loads per thread per batch so one workgroup keeps enough bytes in
// flight.  Same contract as radix_pass.
__device__ __forceinline__ void radix_pass_v4(const uint32_t *keys, int n, uint32_t &prefix, uint32_t &pmask,
                                              int shift, int nbits, uint32_t &krem, uint32_t *hist, uint32_t *tmp)
{
    const uint32_t dm = (1u << nbits) - 1u;
    for (int i = threadIdx.x; i < SEL_BINS; i += blockDim.x)
        hist[i] = 0;
    __syncthreads();
    const uint4 *k4 = reinterpret_cast<const uint4 *>(keys);
    const int n4 = (n + 3) / 4, step = (int)blockDim.x;
    for (int i0 = threadIdx.x; i0 < n4; i0 += 8 * step) {
        uint4 u[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (i0 + q * step < n4)
                u[q] = k4[i0 + q * step];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int i = i0 + q * step;
            if (i < n4) {
                const uint32_t kk[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * i + e < n && (kk[e] & pmask) == prefix)
                        atomicAdd(&hist[(kk[e] >> shift) & dm], 1u);
            }
        }
    }
    __syncthreads();
    const uint32_t d = hist_crossing(hist, SEL_BINS, krem, tmp);
    prefix |= d << shift;
    pmask |= dm << shift;
}

} // namespace rmm
