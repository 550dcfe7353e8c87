// C ABI of librmm.so: argument validation, workspace carving and dispatch.
// Semantics of every entry point are documented in include/rmm.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/rmm.h"
#include "kernels.h"

static_assert(RMM_WS_HEADER_BYTES == RMM_WS_HEADER_BYTES_INTERNAL, "workspace header size");

namespace {

thread_local char g_err[512];

rmm_status_t fail(rmm_status_t st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

rmm_status_t ok()
{
    g_err[0] = 0;
    return RMM_OK;
}

std::once_flag g_init;
void init_once()
{
    std::call_once(g_init, [] {
        rmm::select_init();
        rmm::linear_init();
        rmm::attn_init();
        (void)hipGetLastError();
    });
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
int vec_elems(rmm_dtype_t t) { return t == RMM_BF16 ? 8 : 4; }
size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

rmm_status_t launch_status(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(RMM_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Keep count (paper abstract: retention-ratio control): ceil(r*n) with r*n
// snapped to the nearest integer within 1e-9 relative, clamped to [1, n].
int64_t keep_count(int64_t n, double r)
{
    if (n < 1 || !(r > 0.0) || !(r <= 1.0))
        return -1;
    const double prod = r * (double)n;
    const double near = nearbyint(prod);
    const double tol = 1e-9 * (prod > 1.0 ? prod : 1.0);
    double kk = fabs(prod - near) <= tol ? near : ceil(prod);
    if (kk < 1.0)
        kk = 1.0;
    if (kk > (double)n)
        kk = (double)n;
    return (int64_t)kk;
}

bool use_mfma(int64_t T, int64_t tile, rmm_dtype_t xt)
{
    const int64_t rows = tile < T ? tile : T;
    return xt == RMM_BF16 && rows >= MFMA_MIN_TILE_ROWS;
}

size_t linear_ws(int64_t T, int64_t K, int64_t M, int64_t k, int64_t tile, rmm_dtype_t xt, bool dense)
{
    size_t n = RMM_WS_HEADER_BYTES;
    if (use_mfma(T, dense ? T : tile, xt))
        n += dense ? 0 : round256(rmm::gemm_ws_bytes(T, k));
    else
        n += round256(rmm::gemv_ws_bytes(T, M, k, dense ? T : tile, xt == RMM_BF16));
    (void)K;
    return n;
}

rmm_status_t check_linear(const void *x, rmm_dtype_t xt, int64_t T, int64_t K, int64_t ldx, const void *wt,
                          rmm_dtype_t wt_t, int64_t M, int64_t ldw, float *y, int64_t ldy)
{
    if (!x || !wt || !y)
        return fail(RMM_EINVAL, "null pointer (x=%p wt=%p y=%p)", x, wt, (void *)y);
    if (T < 1 || K < 1 || M < 1)
        return fail(RMM_EINVAL, "sizes must be positive (T=%lld K=%lld M=%lld)", (long long)T, (long long)K,
                    (long long)M);
    if (xt != RMM_F32 && xt != RMM_BF16)
        return fail(RMM_EINVAL, "unknown dtype %d", (int)xt);
    if (wt_t != xt)
        return fail(RMM_EINVAL, "x and W^T dtypes differ (%d vs %d)", (int)xt, (int)wt_t);
    if (ldx < K || ldw < M || ldy < M)
        return fail(RMM_EINVAL, "leading dimension too small (ldx=%lld K=%lld, ldw=%lld ldy=%lld M=%lld)",
                    (long long)ldx, (long long)K, (long long)ldw, (long long)ldy, (long long)M);
    if (K > INT32_MAX || M > INT32_MAX || T > INT32_MAX)
        return fail(RMM_EUNSUPPORTED, "sizes beyond 2^31");
    const int ve = vec_elems(xt);
    if (!aligned16(x) || !aligned16(wt) || ldx % ve || ldw % ve || ((uintptr_t)y & 3u))
        return fail(RMM_EUNSUPPORTED,
                    "x and W^T must be 16-byte aligned with ldx/ldw multiples of %d elements, y 4-byte aligned", ve);
    return RMM_OK;
}

} // namespace

extern "C" {

int64_t rmm_keep_count(int64_t n, double r) { return keep_count(n, r); }

const char *rmm_status_string(rmm_status_t s)
{
    switch (s) {
    case RMM_OK:
        return "RMM_OK";
    case RMM_EINVAL:
        return "RMM_EINVAL: invalid argument";
    case RMM_EUNSUPPORTED:
        return "RMM_EUNSUPPORTED: no kernel for this shape, dtype or alignment";
    case RMM_EWORKSPACE:
        return "RMM_EWORKSPACE: workspace missing or too small";
    case RMM_EHIP:
        return "RMM_EHIP: HIP launch failed";
    default:
        break;
    }
    return "unknown rmm_status_t";
}

const char *rmm_last_error(void) { return g_err; }

// ------------------------------------------------------------------ select
size_t rmm_select_workspace_size(int64_t T, int64_t K, int64_t tile, rmm_dtype_t xt)
{
    (void)xt;
    if (T < 1 || K < 1 || tile < 1)
        return 0;
    return RMM_WS_HEADER_BYTES + round256(rmm::select_ws_bytes(T, K, tile));
}

rmm_status_t rmm_select(const void *x, rmm_dtype_t xt, int64_t T, int64_t K, int64_t ldx, const float *c,
                        int64_t tile, double r, int32_t *idx, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (!x || !c || !idx)
        return fail(RMM_EINVAL, "null pointer (x=%p c=%p idx=%p)", x, (const void *)c, (void *)idx);
    if (T < 1 || K < 1 || tile < 1)
        return fail(RMM_EINVAL, "sizes must be positive (T=%lld K=%lld tile=%lld)", (long long)T, (long long)K,
                    (long long)tile);
    if (xt != RMM_F32 && xt != RMM_BF16)
        return fail(RMM_EINVAL, "unknown dtype %d", (int)xt);
    if (ldx < K)
        return fail(RMM_EINVAL, "ldx (%lld) < K (%lld)", (long long)ldx, (long long)K);
    const int64_t k = keep_count(K, r);
    if (k < 0)
        return fail(RMM_EINVAL, "retention ratio %g not in (0, 1]", r);
    if (K > SELECT_MAX_K)
        return fail(RMM_EUNSUPPORTED, "K = %lld above the single-workgroup selector limit %d", (long long)K,
                    SELECT_MAX_K);
    if (T > INT32_MAX)
        return fail(RMM_EUNSUPPORTED, "T beyond 2^31");
    const int ve = vec_elems(xt);
    if (!aligned16(x) || ldx % ve)
        return fail(RMM_EUNSUPPORTED, "x must be 16-byte aligned with ldx a multiple of %d elements", ve);
    const size_t need = rmm_select_workspace_size(T, K, tile, xt);
    if (!ws || ws_bytes < need)
        return fail(RMM_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    init_once();
    float *pmax = (float *)((char *)ws + RMM_WS_HEADER_BYTES);
    return launch_status(rmm::launch_select(x, xt == RMM_BF16, T, K, ldx, c, tile, k, idx, pmax, stream), "select");
}

// ------------------------------------------------------------------ fused decode step
size_t rmm_select_linear_workspace_size(int64_t K, int64_t M, rmm_dtype_t xt)
{
    if (K < 1 || M < 1 || K > SELECT_MAX_K || M > INT32_MAX || (xt != RMM_F32 && xt != RMM_BF16))
        return 0;
    if (!rmm::select_gemv_fits(K, M, xt == RMM_BF16))
        return 0;
    return RMM_WS_HEADER_BYTES + round256(rmm::select_gemv_ws_bytes(K, M, xt == RMM_BF16));
}

rmm_status_t rmm_select_linear(const void *x, rmm_dtype_t xt, int64_t K, const float *c, double r, const void *wt,
                               rmm_dtype_t wt_t, int64_t M, int64_t ldw, int32_t *idx, float *y, void *ws,
                               size_t ws_bytes, hipStream_t stream)
{
    if (!x || !c || !wt || !y)
        return fail(RMM_EINVAL, "null pointer (x=%p c=%p wt=%p y=%p)", x, (const void *)c, wt, (void *)y);
    if (K < 1 || M < 1)
        return fail(RMM_EINVAL, "sizes must be positive (K=%lld M=%lld)", (long long)K, (long long)M);
    if (xt != RMM_F32 && xt != RMM_BF16)
        return fail(RMM_EINVAL, "unknown dtype %d", (int)xt);
    if (wt_t != xt)
        return fail(RMM_EINVAL, "x and W^T dtypes differ (%d vs %d)", (int)xt, (int)wt_t);
    if (ldw < M)
        return fail(RMM_EINVAL, "ldw (%lld) < M (%lld)", (long long)ldw, (long long)M);
    const int64_t k = keep_count(K, r);
    if (k < 0)
        return fail(RMM_EINVAL, "retention ratio %g not in (0, 1]", r);
    if (K > SELECT_MAX_K || M > INT32_MAX)
        return fail(RMM_EUNSUPPORTED, "K = %lld above the selector limit %d or M beyond 2^31", (long long)K,
                    SELECT_MAX_K);
    const int ve = vec_elems(xt);
    if (!aligned16(x) || !aligned16(wt) || ldw % ve || ((uintptr_t)y & 3u) || ((uintptr_t)idx & 3u))
        return fail(RMM_EUNSUPPORTED, "x and W^T must be 16-byte aligned with ldw a multiple of %d elements, "
                                      "y and idx 4-byte aligned", ve);
    if (!rmm::select_gemv_fits(K, M, xt == RMM_BF16))
        return fail(RMM_EUNSUPPORTED, "no split of K = %lld over the fused launch (at most 1024 slices per split)",
                    (long long)K);
    const size_t need = rmm_select_linear_workspace_size(K, M, xt);
    if (!ws || ws_bytes < need)
        return fail(RMM_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    init_once();
    return launch_status(rmm::launch_select_gemv(x, xt == RMM_BF16, K, c, k, wt, ldw, M, idx, y, (char *)ws,
                                                 (char *)ws + RMM_WS_HEADER_BYTES, stream),
                         "select_linear");
}

// ------------------------------------------------------------------ block-granular selection
int64_t rmm_block_keep_count(int64_t nb, double keep)
{
    if (nb < 1 || !(keep > 0.0) || !(keep <= 1.0))
        return -1;
    int64_t kk = (int64_t)floor((double)nb * keep); // truncation of the double product
    if (kk < 1)
        kk = 1;
    if (kk > nb)
        kk = nb;
    return kk;
}

size_t rmm_select_blocks_workspace_size(int64_t T, int64_t K, int64_t tile, int64_t block, rmm_dtype_t xt)
{
    (void)xt;
    if (T < 1 || K < 1 || tile < 1 || block < 1)
        return 0;
    return RMM_WS_HEADER_BYTES + round256(rmm::select_ws_bytes(T, K, tile));
}

rmm_status_t rmm_select_blocks(const void *x, rmm_dtype_t xt, int64_t T, int64_t K, int64_t ldx, int64_t tile,
                               int64_t block, double keep, int32_t *idx, void *ws, size_t ws_bytes,
                               hipStream_t stream)
{
    if (!x || !idx)
        return fail(RMM_EINVAL, "null pointer (x=%p idx=%p)", x, (void *)idx);
    if (T < 1 || K < 1 || tile < 1 || block < 1)
        return fail(RMM_EINVAL, "sizes must be positive (T=%lld K=%lld tile=%lld block=%lld)", (long long)T,
                    (long long)K, (long long)tile, (long long)block);
    if (xt != RMM_F32 && xt != RMM_BF16)
        return fail(RMM_EINVAL, "unknown dtype %d", (int)xt);
    if (ldx < K)
        return fail(RMM_EINVAL, "ldx (%lld) < K (%lld)", (long long)ldx, (long long)K);
    if (K % block)
        return fail(RMM_EINVAL, "K = %lld is not a multiple of the block size %lld", (long long)K, (long long)block);
    const int64_t nb = K / block;
    const int64_t nk = rmm_block_keep_count(nb, keep);
    if (nk < 0)
        return fail(RMM_EINVAL, "keep ratio %g not in (0, 1]", keep);
    if (K > SELECT_MAX_K || nb > SELECT_BLOCKS_MAX_NB)
        return fail(RMM_EUNSUPPORTED, "K = %lld or %lld blocks above the limits %d / %d", (long long)K,
                    (long long)nb, SELECT_MAX_K, SELECT_BLOCKS_MAX_NB);
    if (T > INT32_MAX)
        return fail(RMM_EUNSUPPORTED, "T beyond 2^31");
    const int ve = vec_elems(xt);
    if (!aligned16(x) || ldx % ve)
        return fail(RMM_EUNSUPPORTED, "x must be 16-byte aligned with ldx a multiple of %d elements", ve);
    const size_t need = rmm_select_blocks_workspace_size(T, K, tile, block, xt);
    if (!ws || ws_bytes < need)
        return fail(RMM_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    init_once();
    float *pmax = (float *)((char *)ws + RMM_WS_HEADER_BYTES);
    return launch_status(
        rmm::launch_select_blocks(x, xt == RMM_BF16, T, K, ldx, tile, block, nk, idx, pmax, stream), "select_blocks");
}

// ------------------------------------------------------------------ linear
size_t rmm_linear_workspace_size(int64_t T, int64_t K, int64_t M, int64_t k, int64_t tile, rmm_dtype_t xt)
{
    if (T < 1 || K < 1 || M < 1 || k < 1 || k > K || tile < 1)
        return 0;
    return linear_ws(T, K, M, k, tile, xt, false);
}

static rmm_status_t linear_common(const void *x, rmm_dtype_t xt, int64_t T, int64_t K, int64_t ldx, const void *wt,
                                  int64_t M, int64_t ldw, const int32_t *idx, int64_t k, int64_t tile, bool dense,
                                  float *y, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t stream)
{
    const size_t need = linear_ws(T, K, M, k, dense ? T : tile, xt, dense);
    if (!ws || ws_bytes < need)
        return fail(RMM_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    init_once();
    char *scratch = (char *)ws + RMM_WS_HEADER_BYTES;
    const int64_t tl = dense ? T : tile;
    hipError_t e;
    if (use_mfma(T, tl, xt))
        e = rmm::launch_gemm(x, T, K, ldx, wt, ldw, M, idx, k, tl, dense, y, ldy, scratch, stream);
    else
        e = rmm::launch_gemv(x, xt == RMM_BF16, T, ldx, wt, ldw, M, idx, k, tl, dense, y, ldy, (float *)scratch,
                             stream);
    return launch_status(e, dense ? "linear_dense" : "linear");
}

rmm_status_t rmm_linear(const void *x, rmm_dtype_t xt, int64_t T, int64_t K, int64_t ldx, const void *wt,
                        rmm_dtype_t wt_t, int64_t M, int64_t ldw, const int32_t *idx, int64_t k, int64_t tile,
                        float *y, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t stream)
{
    rmm_status_t st = check_linear(x, xt, T, K, ldx, wt, wt_t, M, ldw, y, ldy);
    if (st != RMM_OK)
        return st;
    if (!idx)
        return fail(RMM_EINVAL, "null idx");
    if (k < 1 || k > K)
        return fail(RMM_EINVAL, "k = %lld not in [1, K=%lld]", (long long)k, (long long)K);
    if (tile < 1)
        return fail(RMM_EINVAL, "tile must be positive");
    return linear_common(x, xt, T, K, ldx, wt, M, ldw, idx, k, tile, false, y, ldy, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ linear without a caller workspace
// For callers that cannot allocate device memory: the split-K partials (or the
// packed activations of the MFMA path) live in a file-scope device array of
// RMM_NOALLOC_SCRATCH_BYTES, one copy per GPU, held until the process ends.
// Host code never passes the array's name to a kernel: each device's address
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is used.
static __device__ __align__(256) char scratch[RMM_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

rmm_status_t scratch_for_current_device(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(RMM_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(RMM_EUNSUPPORTED, "device %d beyond the %d devices the scratch table covers", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(RMM_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return RMM_OK;
}
} // namespace

rmm_status_t rmm_linear_noalloc(const void *x, rmm_dtype_t xt, int64_t T, int64_t K, int64_t ldx, const void *wt,
                                rmm_dtype_t wt_t, int64_t M, int64_t ldw, const int32_t *idx, int64_t k, int64_t tile,
                                float *y, int64_t ldy, hipStream_t stream)
{
    rmm_status_t st = check_linear(x, xt, T, K, ldx, wt, wt_t, M, ldw, y, ldy);
    if (st != RMM_OK)
        return st;
    if (!idx)
        return fail(RMM_EINVAL, "null idx");
    if (k < 1 || k > K)
        return fail(RMM_EINVAL, "k = %lld not in [1, K=%lld]", (long long)k, (long long)K);
    if (tile < 1)
        return fail(RMM_EINVAL, "tile must be positive");
    const size_t need = linear_ws(T, K, M, k, tile, xt, false);
    if (need > (size_t)RMM_NOALLOC_SCRATCH_BYTES)
        return fail(RMM_EUNSUPPORTED, "this product needs %zu bytes of scratch, above the %d-byte device array",
                    need, RMM_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if ((st = scratch_for_current_device(&ws)) != RMM_OK)
        return st;
    return linear_common(x, xt, T, K, ldx, wt, M, ldw, idx, k, tile, false, y, ldy, ws,
                         (size_t)RMM_NOALLOC_SCRATCH_BYTES, stream);
}

size_t rmm_linear_dense_workspace_size(int64_t T, int64_t K, int64_t M, rmm_dtype_t xt)
{
    if (T < 1 || K < 1 || M < 1)
        return 0;
    return linear_ws(T, K, M, K, T, xt, true);
}

rmm_status_t rmm_linear_dense(const void *x, rmm_dtype_t xt, int64_t T, int64_t K, int64_t ldx, const void *wt,
                              rmm_dtype_t wt_t, int64_t M, int64_t ldw, float *y, int64_t ldy, void *ws,
                              size_t ws_bytes, hipStream_t stream)
{
    rmm_status_t st = check_linear(x, xt, T, K, ldx, wt, wt_t, M, ldw, y, ldy);
    if (st != RMM_OK)
        return st;
    return linear_common(x, xt, T, K, ldx, wt, M, ldw, nullptr, K, T, true, y, ldy, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ gated FFN producer
size_t rmm_gate_up_workspace_size(int64_t T, int64_t H, int64_t Mi, int64_t tile)
{
    if (T < 1 || H < 1 || Mi < 1 || tile < 1 || T > INT32_MAX || H > INT32_MAX || Mi > INT32_MAX)
        return 0;
    return RMM_WS_HEADER_BYTES + round256(rmm::gateup_ws_bytes(T, H, Mi, tile < T ? tile : T));
}

rmm_status_t rmm_gate_up(const void *x, int64_t T, int64_t H, int64_t ldx, const void *wg, const void *wu,
                         int64_t ldw, int64_t Mi, int64_t tile, void *h, int64_t ldh, float *pmax, void *ws,
                         size_t ws_bytes, hipStream_t stream)
{
    if (!x || !wg || !wu || !h)
        return fail(RMM_EINVAL, "null pointer (x=%p wg=%p wu=%p h=%p)", x, wg, wu, h);
    if (T < 1 || H < 1 || Mi < 1 || tile < 1)
        return fail(RMM_EINVAL, "sizes must be positive (T=%lld H=%lld Mi=%lld tile=%lld)", (long long)T,
                    (long long)H, (long long)Mi, (long long)tile);
    if (ldx < H || ldw < Mi || ldh < Mi)
        return fail(RMM_EINVAL, "leading dimension too small (ldx=%lld H=%lld, ldw=%lld ldh=%lld Mi=%lld)",
                    (long long)ldx, (long long)H, (long long)ldw, (long long)ldh, (long long)Mi);
    if (T > INT32_MAX || H > INT32_MAX || Mi > INT32_MAX)
        return fail(RMM_EUNSUPPORTED, "sizes beyond 2^31");
    if (!aligned16(x) || !aligned16(wg) || !aligned16(wu) || ldx % 8 || ldw % 8 || ((uintptr_t)h & 1u) ||
        ((uintptr_t)pmax & 3u))
        return fail(RMM_EUNSUPPORTED, "x, wg and wu must be 16-byte aligned with ldx/ldw multiples of 8 elements, "
                                      "h 2-byte and pmax 4-byte aligned");
    const int64_t tl = tile < T ? tile : T;
    const size_t need = rmm_gate_up_workspace_size(T, H, Mi, tile);
    if (!ws || ws_bytes < need)
        return fail(RMM_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    if (rmm::gateup_grid(T, H, Mi, tl) > (int64_t)INT32_MAX)
        return fail(RMM_EUNSUPPORTED, "too many workgroups");
    init_once();
    float *part = (float *)((char *)ws + RMM_WS_HEADER_BYTES);
    return launch_status(rmm::launch_gateup((const uint16_t *)x, T, H, ldx, (const uint16_t *)wg,
                                            (const uint16_t *)wu, ldw, Mi, tl, (uint16_t *)h, ldh, pmax, part, stream),
                         "gate_up");
}

// ------------------------------------------------------------------ attention
static rmm_status_t attn_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t S, int64_t ldk, int64_t ldv,
                               float scale, double r_dim, double r_pos, int mode, rmm::AttnShape *s)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || S < 1)
        return fail(RMM_EINVAL, "sizes must be positive");
    if (Hq % Hkv)
        return fail(RMM_EINVAL, "Hq (%lld) not a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
    if (ldk < S || ldv < S)
        return fail(RMM_EINVAL, "ldk/ldv (%lld/%lld) < S (%lld)", (long long)ldk, (long long)ldv, (long long)S);
    if (mode != RMM_SEL_PER_KV_GROUP && mode != RMM_SEL_PER_Q_HEAD)
        return fail(RMM_EINVAL, "unknown selection mode %d", mode);
    if (!isfinite(scale))
        return fail(RMM_EINVAL, "scale must be finite");
    const int64_t kd = keep_count(D, r_dim), ks = keep_count(S, r_pos);
    if (kd < 0 || ks < 0)
        return fail(RMM_EINVAL, "ratios (%g, %g) not in (0, 1]", r_dim, r_pos);
    const int64_t G = Hq / Hkv;
    if (D != ATTN_D)
        return fail(RMM_EUNSUPPORTED, "head_dim %lld (kernels take %d)", (long long)D, ATTN_D);
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(RMM_EUNSUPPORTED, "Hq/Hkv = %lld not in {1,2,4,8}", (long long)G);
    if (S > (1 << 24))
        return fail(RMM_EUNSUPPORTED, "S above 2^24");
    if (ldk % 8)
        return fail(RMM_EUNSUPPORTED, "ldk must be a multiple of 8");
    const int64_t Hsel = mode == RMM_SEL_PER_KV_GROUP ? Hkv : Hq;
    if (B * Hsel > ATTN_MAX_GROUPS || B * Hkv > ATTN_MAX_GROUPS)
        return fail(RMM_EUNSUPPORTED, "B * selection groups = %lld above %d", (long long)(B * Hsel),
                    ATTN_MAX_GROUPS);
    s->B = B;
    s->Hq = Hq;
    s->Hkv = Hkv;
    s->S = S;
    s->ldk = ldk;
    s->ldv = ldv;
    s->G = (int)G;
    s->GS = mode == RMM_SEL_PER_KV_GROUP ? (int)G : 1;
    s->Hsel = (int)Hsel;
    s->kd = (int)kd;
    s->ks = (int)ks;
    s->scale = scale;
    return RMM_OK;
}

size_t rmm_attn_decode_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t S, double r_dim,
                                      double r_pos, rmm_sel_mode_t mode)
{
    rmm::AttnShape s;
    const int64_t S8 = (S + 7) / 8 * 8; // the size does not depend on the pitches
    if (attn_shape(B, Hq, Hkv, D, S, S8, S8, 1.0f, r_dim, r_pos, (int)mode, &s) != RMM_OK)
        return 0;
    return rmm::attn_ws_layout(s, nullptr, nullptr);
}

rmm_status_t rmm_attn_decode_ex(const void *q, const void *kt, const void *v, const float *kn, const float *vn,
                                int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t S, int64_t ldk, int64_t ldv,
                                float scale, double r_dim, double r_pos, rmm_sel_mode_t mode, float *out,
                                int32_t *dim_idx, int32_t *pos_idx, float *lse, void *ws, size_t ws_bytes,
                                hipStream_t stream)
{
    if (!q || !kt || !v || !kn || !out)
        return fail(RMM_EINVAL, "null required pointer");
    rmm::AttnShape s;
    rmm_status_t st = attn_shape(B, Hq, Hkv, D, S, ldk, ldv, scale, r_dim, r_pos, (int)mode, &s);
    if (st != RMM_OK)
        return st;
    if (!aligned16(q) || !aligned16(kt) || !aligned16(v) || ((uintptr_t)out & 3u))
        return fail(RMM_EUNSUPPORTED, "q, kt and v must be 16-byte aligned, out 4-byte aligned");
    if (vn && (!aligned16(vn) || ldv % 8))
        return fail(RMM_EUNSUPPORTED, "vn must be 16-byte aligned and ldv a multiple of 8");
    const size_t need = rmm::attn_ws_layout(s, nullptr, nullptr);
    if (!ws || ws_bytes < need)
        return fail(RMM_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    init_once();
    rmm::AttnWs w;
    rmm::attn_ws_layout(s, &w, (char *)ws);
    const rmm::KvMap m{nullptr, nullptr, 0, 0, r_pos};
    return launch_status(rmm::launch_attn(s, m, (const uint16_t *)q, (const uint16_t *)kt, (const uint16_t *)v, kn,
                                          vn, out, dim_idx, pos_idx, lse, w, stream),
                         "attn_decode");
}

// paged caches: shape checks shared by the reduced and the dense entry points
static rmm_status_t paged_map(const void *kp, const void *vp, const int32_t *block_table, int64_t max_pages,
                              int64_t page, const int32_t *seqlens, int64_t S, double r_pos, rmm::KvMap *m)
{
    if (!kp || !vp || !block_table || !seqlens)
        return fail(RMM_EINVAL, "null page pool, block table or sequence lengths");
    if (page < 8 || page % 8 || page > (1 << 24))
        return fail(RMM_EUNSUPPORTED, "page size %lld must be a multiple of 8 in [8, 2^24]", (long long)page);
    if (max_pages < 1 || S > max_pages * page)
        return fail(RMM_EINVAL, "S = %lld exceeds max_pages * page = %lld", (long long)S,
                    (long long)(max_pages * page));
    if (!aligned16(kp) || !aligned16(vp))
        return fail(RMM_EUNSUPPORTED, "page pools must be 16-byte aligned");
    *m = rmm::KvMap{block_table, seqlens, max_pages, (int)page, r_pos};
    return RMM_OK;
}

rmm_status_t rmm_attn_decode_paged(const void *q, const void *k_pages, const void *v_pages, const float *kn,
                                   const float *vn_pages, const int32_t *block_table, int64_t max_pages, int64_t page,
                                   const int32_t *seqlens, int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t S,
                                   float scale, double r_dim, double r_pos, rmm_sel_mode_t mode, float *out,
                                   int32_t *dim_idx, int32_t *pos_idx, float *lse, void *ws, size_t ws_bytes,
                                   hipStream_t stream)
{
    if (!q || !kn || !out)
        return fail(RMM_EINVAL, "null required pointer");
    rmm::AttnShape s;
    const int64_t S8 = (S + 7) / 8 * 8;
    rmm_status_t st = attn_shape(B, Hq, Hkv, D, S, S8, S8, scale, r_dim, r_pos, (int)mode, &s);
    if (st != RMM_OK)
        return st;
    rmm::KvMap m;
    if ((st = paged_map(k_pages, v_pages, block_table, max_pages, page, seqlens, S, r_pos, &m)) != RMM_OK)
        return st;
    if (!aligned16(q) || ((uintptr_t)out & 3u) || (vn_pages && !aligned16(vn_pages)))
        return fail(RMM_EUNSUPPORTED, "q and vn must be 16-byte aligned, out 4-byte aligned");
    const size_t need = rmm::attn_ws_layout(s, nullptr, nullptr);
    if (!ws || ws_bytes < need)
        return fail(RMM_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    init_once();
    rmm::AttnWs w;
    rmm::attn_ws_layout(s, &w, (char *)ws);
    return launch_status(rmm::launch_attn(s, m, (const uint16_t *)q, (const uint16_t *)k_pages,
                                          (const uint16_t *)v_pages, kn, vn_pages, out, dim_idx, pos_idx, lse, w,
                                          stream),
                         "attn_decode_paged");
}

rmm_status_t rmm_attn_decode(const void *q, const void *kt, const void *v, const float *kn, int64_t B, int64_t Hq,
                             int64_t Hkv, int64_t D, int64_t S, int64_t ldk, int64_t ldv, float scale, double r_dim,
                             double r_pos, rmm_sel_mode_t mode, float *out, int32_t *dim_idx, int32_t *pos_idx,
                             float *lse, void *ws, size_t ws_bytes, hipStream_t stream)
{
    return rmm_attn_decode_ex(q, kt, v, kn, nullptr, B, Hq, Hkv, D, S, ldk, ldv, scale, r_dim, r_pos, mode, out,
                              dim_idx, pos_idx, lse, ws, ws_bytes, stream);
}

size_t rmm_attn_decode_dense_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t S)
{
    rmm::AttnShape s;
    const int64_t S8 = (S + 7) / 8 * 8;
    if (attn_shape(B, Hq, Hkv, D, S, S8, S8, 1.0f, 1.0, 1.0, 0, &s) != RMM_OK)
        return 0;
    return rmm::attn_dense_ws_layout(B, Hq, S, nullptr, nullptr, nullptr);
}

rmm_status_t rmm_attn_decode_dense(const void *q, const void *kt, const void *v, int64_t B, int64_t Hq, int64_t Hkv,
                                   int64_t D, int64_t S, int64_t ldk, int64_t ldv, float scale, float *out,
                                   float *lse, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (!q || !kt || !v || !out)
        return fail(RMM_EINVAL, "null required pointer");
    rmm::AttnShape s;
    rmm_status_t st = attn_shape(B, Hq, Hkv, D, S, ldk, ldv, scale, 1.0, 1.0, 0, &s);
    if (st != RMM_OK)
        return st;
    if (!aligned16(q) || !aligned16(kt) || !aligned16(v) || ((uintptr_t)out & 3u))
        return fail(RMM_EUNSUPPORTED, "q, kt and v must be 16-byte aligned, out 4-byte aligned");
    const size_t need = rmm::attn_dense_ws_layout(B, Hq, S, nullptr, nullptr, nullptr);
    if (!ws || ws_bytes < need)
        return fail(RMM_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    init_once();
    float *part;
    float2 *stat;
    rmm::attn_dense_ws_layout(B, Hq, S, (char *)ws, &part, &stat);
    const rmm::KvMap m{nullptr, nullptr, 0, 0, 1.0};
    return launch_status(rmm::launch_attn_dense(s, m, (const uint16_t *)q, (const uint16_t *)kt, (const uint16_t *)v,
                                                out, lse, part, stat, stream),
                         "attn_decode_dense");
}

rmm_status_t rmm_attn_decode_dense_paged(const void *q, const void *k_pages, const void *v_pages,
                                         const int32_t *block_table, int64_t max_pages, int64_t page,
                                         const int32_t *seqlens, int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                                         int64_t S, float scale, float *out, float *lse, void *ws, size_t ws_bytes,
                                         hipStream_t stream)
{
    if (!q || !out)
        return fail(RMM_EINVAL, "null required pointer");
    rmm::AttnShape s;
    const int64_t S8 = (S + 7) / 8 * 8;
    rmm_status_t st = attn_shape(B, Hq, Hkv, D, S, S8, S8, scale, 1.0, 1.0, 0, &s);
    if (st != RMM_OK)
        return st;
    rmm::KvMap m;
    if ((st = paged_map(k_pages, v_pages, block_table, max_pages, page, seqlens, S, 1.0, &m)) != RMM_OK)
        return st;
    if (!aligned16(q) || ((uintptr_t)out & 3u))
        return fail(RMM_EUNSUPPORTED, "q must be 16-byte aligned, out 4-byte aligned");
    const size_t need = rmm::attn_dense_ws_layout(B, Hq, S, nullptr, nullptr, nullptr);
    if (!ws || ws_bytes < need)
        return fail(RMM_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    init_once();
    float *part;
    float2 *stat;
    rmm::attn_dense_ws_layout(B, Hq, S, (char *)ws, &part, &stat);
    return launch_status(rmm::launch_attn_dense(s, m, (const uint16_t *)q, (const uint16_t *)k_pages,
                                                (const uint16_t *)v_pages, out, lse, part, stat, stream),
                         "attn_decode_dense_paged");
}

} // extern "C"
