// Device helpers for the RMM kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmm {

constexpr int WAVE = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// element loads for the two storage types (bf16 bits in uint16_t, or float)
__device__ __forceinline__ float ld_elem(const uint16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float ld_elem(const float *p, int64_t i) { return p[i]; }

// 16-byte vector of a row: 8 bf16 or 4 fp32 values, unpacked to float
template <typename TE> struct Vec16;
template <> struct Vec16<uint16_t> {
    static constexpr int N = 8;
    __device__ __forceinline__ static void load(const uint16_t *p, float (&v)[8]) {
        uint4 u = *reinterpret_cast<const uint4 *>(p);
        v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x);
        v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
        v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z);
        v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
    }
    __device__ __forceinline__ static uint4 raw(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ static void unpack(uint4 u, float (&v)[8]) {
        v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x);
        v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
        v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z);
        v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
    }
};
template <> struct Vec16<float> {
    static constexpr int N = 4;
    __device__ __forceinline__ static uint4 raw(const float *p) { return *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ static void unpack(uint4 u, float (&v)[4]) {
        v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
        v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
    }
};

// Predicates as integer arithmetic (0 or 1) on the vector ALU: a compare would
// produce a lane mask in scalar registers, and combining masks runs on the
// scalar ALU, which the 16 waves of a 1024-thread workgroup share.
// lt31 and eq31 need a, b < 2^31; ilt needs |a - b| < 2^31.
__device__ __forceinline__ uint32_t lt31(uint32_t a, uint32_t b) { return (a - b) >> 31; }        // a < b
__device__ __forceinline__ uint32_t eq31(uint32_t a, uint32_t b) { return ((a ^ b) - 1u) >> 31; } // a == b
__device__ __forceinline__ uint32_t ilt(int a, int b) { return ((uint32_t)a - (uint32_t)b) >> 31; } // a < b
// A copy of v the compiler cannot see through: predicates built from it stay in
// the phase that uses them instead of being hoisted (and held in registers)
// across the whole kernel.
__device__ __forceinline__ int opaque(int v)
{
    asm volatile("" : "+v"(v));
    return v;
}
template <int N> __device__ __forceinline__ void opaque_all(uint32_t (&v)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i)
        asm volatile("" : "+v"(v[i]));
}

// Inclusive prefix sum over the whole block (blockDim.x threads, multiple of 64).
// `tmp` holds at least blockDim.x/64 words of LDS.  Contains barriers: every
// thread of the block must call it.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t *tmp)
{
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE, nw = blockDim.x / WAVE;
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        uint32_t n = __shfl_up(v, off, WAVE);
        if (lane >= off)
            v += n;
    }
    if (lane == WAVE - 1)
        tmp[w] = v;
    __syncthreads();
    uint32_t add = 0;
    for (int i = 0; i < w && i < nw; ++i)
        add += tmp[i];
    __syncthreads();
    return v + add;
}

// Non-negative float -> order-preserving uint32 key; -0 ranks as +0.
__device__ __forceinline__ uint32_t nonneg_key(float s) { return __float_as_uint(s) & 0x7fffffffu; }

// ---- wave64 DPP reductions and scans (GFX9 row_shr / row_bcast controls)
// update_dpp(old, src, ctrl, row_mask, bank_mask, bound_ctrl): lanes without a
// source (or outside row_mask) keep `old`, which is the operation's identity.
#define RMM_DPP_ROW_SHR(n) (0x110 + (n))
#define RMM_DPP_ROW_BCAST15 0x142
#define RMM_DPP_ROW_BCAST31 0x143

template <typename Op>
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t v, uint32_t ident, Op op)
{
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, RMM_DPP_ROW_SHR(1), 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, RMM_DPP_ROW_SHR(2), 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, RMM_DPP_ROW_SHR(4), 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, RMM_DPP_ROW_SHR(8), 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, RMM_DPP_ROW_BCAST15, 0xa, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, RMM_DPP_ROW_BCAST31, 0xc, 0xf, false));
    return v; // inclusive prefix over lanes 0..lane
}
struct OpAdd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct OpMax { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; } };
struct OpMin { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; } };

__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) { return wave_scan_dpp(v, 0u, OpAdd()); }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_dpp(v, 0u, OpMax()), WAVE - 1);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_dpp(v, 0xffffffffu, OpMin()), WAVE - 1);
}
__device__ __forceinline__ uint64_t lanemask_lt()
{
    const int lane = threadIdx.x & (WAVE - 1);
    return lane == 0 ? 0ull : (~0ull >> (WAVE - lane));
}

// Agent-scope stores and loads of published words (coherent across XCDs when complete).
__device__ __forceinline__ void pub_store(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t pub_load(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void pub_store64(uint64_t *p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t pub_load64(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

} // namespace rmm
