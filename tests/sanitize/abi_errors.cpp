// Sanitizer driver for the C ABI's host side (test infrastructure).  Every
// call below is refused by argument validation before anything touches a
// device, so it runs without a GPU; the pointers are stand-ins that are never
// dereferenced.  tests/test_sanitize.py links it with librmm's objects, api.hip
// rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer on its host
// code; a sanitizer report or a wrong status ends it with a non-zero status.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "rmm.h"

static int failures = 0;
#define EXPECT(call, want)                                                                             \
    do {                                                                                               \
        const int got = (int)(call);                                                                   \
        if (got != (want)) {                                                                           \
            std::fprintf(stderr, "line %d: %s gave %d, want %d (%s)\n", __LINE__, #call, got, (int)(want), \
                         rmm_last_error());                                                            \
            ++failures;                                                                                \
        }                                                                                              \
    } while (0)

int main()
{
    void *p = reinterpret_cast<void *>(256);
    float *pf = static_cast<float *>(p);
    int32_t *pi = static_cast<int32_t *>(p);
    const int32_t *cpi = pi;

    // keep counts (host only)
    EXPECT(rmm_keep_count(100, 0.07), 7);
    EXPECT(rmm_keep_count(0, 0.5), -1);
    EXPECT(rmm_keep_count(5, NAN), -1);
    EXPECT(rmm_block_keep_count(7, 0.5), 3);
    EXPECT(rmm_block_keep_count(7, 0.0), -1);

    // selector
    EXPECT(rmm_select(nullptr, RMM_BF16, 1, 64, 64, pf, 1, 0.5, pi, nullptr, 0, nullptr), RMM_EINVAL);
    EXPECT(rmm_select(p, RMM_BF16, 1, 64, 64, pf, 1, 0.0, pi, nullptr, 0, nullptr), RMM_EINVAL);
    EXPECT(rmm_select(p, RMM_BF16, 0, 64, 64, pf, 1, 0.5, pi, nullptr, 0, nullptr), RMM_EINVAL);
    EXPECT(rmm_select(p, RMM_BF16, 1, 64, 8, pf, 1, 0.5, pi, nullptr, 0, nullptr), RMM_EINVAL);
    EXPECT(rmm_select(p, (rmm_dtype_t)7, 1, 64, 64, pf, 1, 0.5, pi, nullptr, 0, nullptr), RMM_EINVAL);
    EXPECT(rmm_select(p, (rmm_dtype_t)-1, 1, 64, 64, pf, 1, 0.5, pi, nullptr, 0, nullptr), RMM_EINVAL);
    EXPECT(rmm_select(p, RMM_BF16, 1, 40000, 40000, pf, 1, 0.5, pi, nullptr, 0, nullptr), RMM_EUNSUPPORTED);
    EXPECT(rmm_select(reinterpret_cast<void *>(18), RMM_BF16, 1, 64, 64, pf, 1, 0.5, pi, nullptr, 0, nullptr),
           RMM_EUNSUPPORTED);
    EXPECT(rmm_select(p, RMM_BF16, 1, 64, 64, pf, 1, 0.5, pi, nullptr, 0, nullptr), RMM_EWORKSPACE);
    EXPECT(rmm_select(p, RMM_BF16, 1, 64, 64, pf, 1, 0.5, pi, p, 16, nullptr), RMM_EWORKSPACE);
    if (std::strstr(rmm_last_error(), "workspace") == nullptr) {
        std::fprintf(stderr, "the last error does not name the workspace: %s\n", rmm_last_error());
        ++failures;
    }
    if (rmm_select_workspace_size(1, 14336, 1, RMM_BF16) == 0)
        ++failures;

    // block selector
    EXPECT(rmm_select_blocks(p, RMM_BF16, 1, 4096, 4096, 1, 100, 0.5, pi, nullptr, 0, nullptr), RMM_EINVAL);
    EXPECT(rmm_select_blocks(p, RMM_BF16, 1, 4096, 4096, 1, 2, 0.5, pi, nullptr, 0, nullptr), RMM_EUNSUPPORTED);
    EXPECT(rmm_select_blocks(p, RMM_BF16, 1, 4096, 4096, 1, 64, 0.5, pi, nullptr, 0, nullptr), RMM_EWORKSPACE);

    // reduced and dense products
    EXPECT(rmm_linear(p, RMM_BF16, 1, 64, 64, p, RMM_F32, 64, 64, cpi, 8, 1, pf, 64, nullptr, 0, nullptr),
           RMM_EINVAL);
    EXPECT(rmm_linear(p, RMM_BF16, 1, 64, 64, p, RMM_BF16, 64, 64, cpi, 65, 1, pf, 64, nullptr, 0, nullptr),
           RMM_EINVAL);
    EXPECT(rmm_linear(p, RMM_BF16, 1, 64, 64, p, RMM_BF16, 60, 60, cpi, 8, 1, pf, 64, nullptr, 0, nullptr),
           RMM_EUNSUPPORTED);
    EXPECT(rmm_linear(p, RMM_BF16, 1, 64, 64, p, RMM_BF16, 64, 64, cpi, 8, 1, pf, 64, nullptr, 0, nullptr),
           RMM_EWORKSPACE);
    EXPECT(rmm_linear_noalloc(nullptr, RMM_BF16, 1, 64, 64, p, RMM_BF16, 64, 64, cpi, 8, 1, pf, 64, nullptr),
           RMM_EINVAL);
    EXPECT(rmm_linear_noalloc(p, RMM_BF16, 1, 64, 64, p, RMM_BF16, 64, 64, cpi, 65, 1, pf, 64, nullptr),
           RMM_EINVAL);
    EXPECT(rmm_linear_dense(p, RMM_BF16, 1, 64, 64, p, RMM_BF16, 64, 64, pf, 64, nullptr, 0, nullptr),
           RMM_EWORKSPACE);
    EXPECT(rmm_select_linear(nullptr, RMM_BF16, 14336, pf, 0.5, p, RMM_BF16, 4096, 4096, pi, pf, nullptr, 0,
                             nullptr),
           RMM_EINVAL);
    EXPECT(rmm_select_linear(p, RMM_BF16, 14336, pf, 1.5, p, RMM_BF16, 4096, 4096, pi, pf, nullptr, 0, nullptr),
           RMM_EINVAL);
    EXPECT(rmm_select_linear(p, RMM_BF16, 14336, pf, 0.5, p, RMM_BF16, 4096, 4096, pi, pf, nullptr, 0, nullptr),
           RMM_EWORKSPACE);
    if (rmm_select_linear_workspace_size(14336, 4096, RMM_BF16) == 0)
        ++failures;

    // gated FFN producer
    EXPECT(rmm_gate_up(nullptr, 1, 64, 64, p, p, 128, 128, 1, p, 128, nullptr, nullptr, 0, nullptr), RMM_EINVAL);
    EXPECT(rmm_gate_up(p, 1, 64, 32, p, p, 128, 128, 1, p, 128, nullptr, nullptr, 0, nullptr), RMM_EINVAL);
    EXPECT(rmm_gate_up(p, 1, 64, 64, p, p, 132, 128, 1, p, 128, nullptr, nullptr, 0, nullptr), RMM_EUNSUPPORTED);
    EXPECT(rmm_gate_up(p, 1, 64, 64, p, p, 128, 128, 1, p, 128, nullptr, nullptr, 0, nullptr), RMM_EWORKSPACE);

    // attention
    EXPECT(rmm_attn_decode(p, p, p, pf, 1, 30, 8, 128, 1000, 1000, 1000, 0.088f, 0.5, 0.5, RMM_SEL_PER_KV_GROUP, pf,
                           nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           RMM_EINVAL);
    EXPECT(rmm_attn_decode(p, p, p, pf, 1, 32, 8, 128, 1000, 1000, 1000, 0.088f, 0.5, 0.5, (rmm_sel_mode_t)5, pf,
                           nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           RMM_EINVAL);
    EXPECT(rmm_attn_decode(p, p, p, pf, 1, 32, 8, 64, 1000, 1000, 1000, 0.088f, 0.5, 0.5, RMM_SEL_PER_KV_GROUP, pf,
                           nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           RMM_EUNSUPPORTED);
    EXPECT(rmm_attn_decode(p, p, p, pf, 1, 32, 8, 128, 1000, 1000, 1000, 0.088f, 0.0, 0.5, RMM_SEL_PER_KV_GROUP, pf,
                           nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           RMM_EINVAL);
    EXPECT(rmm_attn_decode(p, p, p, pf, 65, 32, 8, 128, 1000, 1000, 1000, 0.088f, 0.5, 0.5, RMM_SEL_PER_KV_GROUP, pf,
                           nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           RMM_EUNSUPPORTED);
    EXPECT(rmm_attn_decode(p, p, p, pf, 1, 32, 8, 128, 1000, 1000, 1000, 0.088f, 0.5, 0.5, RMM_SEL_PER_KV_GROUP, pf,
                           nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           RMM_EWORKSPACE);
    EXPECT(rmm_attn_decode_ex(p, p, p, pf, reinterpret_cast<const float *>(260), 1, 32, 8, 128, 1000, 1000, 1000,
                              0.088f, 0.5, 0.5, RMM_SEL_PER_KV_GROUP, pf, nullptr, nullptr, nullptr, nullptr, 0,
                              nullptr),
           RMM_EUNSUPPORTED);
    EXPECT(rmm_attn_decode_paged(p, p, p, pf, nullptr, nullptr, 4, 256, cpi, 2, 32, 8, 128, 1000, 0.088f, 0.5, 0.5,
                                 RMM_SEL_PER_KV_GROUP, pf, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           RMM_EINVAL);
    EXPECT(rmm_attn_decode_paged(p, p, p, pf, nullptr, cpi, 4, 256, cpi, 2, 32, 8, 128, 1025, 0.088f, 0.5, 0.5,
                                 RMM_SEL_PER_KV_GROUP, pf, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           RMM_EINVAL);
    EXPECT(rmm_attn_decode_paged(p, p, p, pf, nullptr, cpi, 4, 12, cpi, 2, 32, 8, 128, 40, 0.088f, 0.5, 0.5,
                                 RMM_SEL_PER_KV_GROUP, pf, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           RMM_EUNSUPPORTED);
    EXPECT(rmm_attn_decode_paged(p, p, p, pf, nullptr, cpi, 4, 256, cpi, 2, 32, 8, 128, 1000, 0.088f, 0.5, 0.5,
                                 RMM_SEL_PER_KV_GROUP, pf, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
           RMM_EWORKSPACE);
    EXPECT(rmm_attn_decode_dense_paged(p, p, p, cpi, 3, 256, cpi, 2, 32, 8, 128, 1000, 0.088f, pf, nullptr, nullptr,
                                       0, nullptr),
           RMM_EINVAL);
    EXPECT(rmm_attn_decode_dense(p, p, p, 1, 32, 8, 128, 1000, 1000, 1000, 0.088f, pf, nullptr, nullptr, 0, nullptr),
           RMM_EWORKSPACE);
    if (rmm_attn_decode_workspace_size(4, 32, 8, 128, 131072, 0.5, 0.25, RMM_SEL_PER_KV_GROUP) == 0 ||
        rmm_attn_decode_workspace_size(2, 8, 2, 128, 2500, 0.5, 0.25, RMM_SEL_PER_Q_HEAD) == 0 ||
        rmm_attn_decode_dense_workspace_size(1, 8, 2, 128, 9999) == 0)
        ++failures;
    if (std::strncmp(rmm_status_string(RMM_EWORKSPACE), "RMM_EWORKSPACE", 14) != 0 ||
        rmm_status_string((rmm_status_t)99) == nullptr || rmm_status_string((rmm_status_t)-3) == nullptr)
        ++failures;

    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("abi checks passed\n");
    return 0;
}
