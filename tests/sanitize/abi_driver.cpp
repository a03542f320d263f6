// Drives every entry point of the C ABI (host code built with the address and undefined-behaviour
// sanitizers, kernel launchers stubbed) through its rejections and its launch path.  Pointers are fake:
// the host code never dereferences them.  Exit status 0 when every status is the expected one.
#include <cmath>
#include <cstdio>
#include <cstdlib>

#include "attn.h"

static int g_bad = 0;
#define EXPECT(call, want)                                                                                      \
    do {                                                                                                        \
        const attn_status_t s_ = (call);                                                                        \
        if (s_ != (want)) {                                                                                     \
            std::fprintf(stderr, "line %d: status %d, expected %d (%s)\n", __LINE__, (int)s_, (int)(want),      \
                         attn_last_error_message());                                                            \
            ++g_bad;                                                                                            \
        }                                                                                                       \
    } while (0)

int main()
{
    void *F = reinterpret_cast<void *>(0x1000);
    const int32_t *I = static_cast<const int32_t *>(F);
    float *Lf = static_cast<float *>(F);
    uint8_t *M = static_cast<uint8_t *>(F);
    const size_t big = (size_t)1 << 40;
    // prefill
    EXPECT(attn_prefill_varlen(ATTN_BF16, F, F, F, I, I, 4, 300, 300, 32, 8, 128, 0.088f, 1, 0.f, F, Lf, nullptr, 0,
                               nullptr), ATTN_OK);
    EXPECT(attn_prefill_varlen(ATTN_BF16, F, F, F, I, I, 4, 300, 300, 32, 8, 64, 0.1f, 0, 0.1f, F, nullptr, M, 10,
                               nullptr), ATTN_OK);
    EXPECT(attn_prefill_varlen(ATTN_F32, F, F, F, I, I, 2, 128, 128, 4, 2, 64, 0.125f, 1, 0.1f, F, Lf, M, 4, nullptr),
           ATTN_OK);
    EXPECT(attn_prefill_varlen(ATTN_BF16, F, F, F, I, I, 4, 300, 300, 32, 8, 128, 0.f, 1, 0.f, F, Lf, nullptr, 0,
                               nullptr), ATTN_ERR_INVALID);
    EXPECT(attn_prefill_varlen(ATTN_BF16, F, F, F, I, I, 4, 300, 300, 32, 8, 128, NAN, 1, 0.f, F, nullptr, nullptr, 0,
                               nullptr), ATTN_ERR_INVALID);
    EXPECT(attn_prefill_varlen(ATTN_BF16, F, F, F, I, I, 4, 300, 300, 32, 8, 96, 0.1f, 1, 0.f, F, nullptr, nullptr, 0,
                               nullptr), ATTN_ERR_UNSUPPORTED);
    EXPECT(attn_prefill_varlen((attn_dtype_t)9, F, F, F, I, I, 4, 3, 3, 8, 8, 128, 0.1f, 1, 0.f, F, nullptr, nullptr,
                               0, nullptr), ATTN_ERR_INVALID);
    EXPECT(attn_prefill_varlen(ATTN_BF16, F, F, F, I, I, 4, 300, 300, 32, 8, 128, 0.1f, 1, 0.f, F, nullptr, M, 1,
                               nullptr), ATTN_ERR_INVALID);
    EXPECT(attn_prefill_varlen(ATTN_BF16, F, F, F, I, I, 0, 0, 0, 32, 8, 128, 0.1f, 1, 0.f, nullptr, nullptr, nullptr,
                               0, nullptr), ATTN_OK);
    // decode (split-K and sequential), NVFP4, multi-token
    const size_t ws = attn_decode_paged_workspace_size(64, 32, 128, 32);
    EXPECT(attn_decode_paged(F, F, F, I, I, 64, 32, 8, 128, 16, 140000, 2048, 0.088f, 0.f, 32, F, ws, F, Lf, nullptr,
                             0, nullptr), ATTN_OK);
    EXPECT(attn_decode_paged(F, F, F, I, I, 64, 32, 8, 128, 16, 140000, 2048, 0.088f, 0.1f, 1, nullptr, 0, F, Lf, M,
                             1024, nullptr), ATTN_OK);
    EXPECT(attn_decode_paged(F, F, F, I, I, 64, 32, 8, 128, 16, 140000, 2048, 0.088f, 0.f, 32, F, ws - 1, F, Lf,
                             nullptr, 0, nullptr), ATTN_ERR_WORKSPACE);
    EXPECT(attn_decode_paged(F, F, F, I, I, 64, 32, 8, 128, 16, 140000, 2048, -1.f, 0.f, 32, F, ws, F, Lf, nullptr, 0,
                             nullptr), ATTN_ERR_INVALID);
    EXPECT(attn_decode_paged_noalloc(F, F, F, I, I, 1024, 32, 8, 128, 16, 140000, 2048, 0.088f, 0.f, 32, F, Lf,
                                     nullptr, 0, nullptr), ATTN_ERR_WORKSPACE);
    EXPECT(attn_decode_paged_noalloc(F, F, F, I, I, 64, 32, 8, 128, 16, 140000, 2048, 0.088f, 0.1f, 1, F, Lf, M, 1024,
                                     nullptr), ATTN_OK);
    EXPECT(attn_decode_paged_qdq(F, F, F, I, I, 64, 32, 8, 128, 16, 140000, 2048, 0.088f, 0.1f, 1.f, 1.f, F, Lf, M,
                                 1024, nullptr), ATTN_OK);
    EXPECT(attn_decode_paged_qdq(F, F, F, I, I, 64, 32, 8, 128, 16, 140000, 2048, 0.088f, 0.1f, 1e-30f, 0.f, F, Lf,
                                 nullptr, 0, nullptr), ATTN_ERR_INVALID);
    const size_t wm = attn_decode_paged_multi_workspace_size(166, 4, 32, 8, 128, 32);
    EXPECT(attn_decode_paged_multi(F, I, 166, 4, F, F, I, I, 64, 32, 8, 128, 16, 140000, 2048, 0.088f, 0.f, 32, F, wm,
                                   F, Lf, nullptr, 0, nullptr), ATTN_OK);
    EXPECT(attn_decode_paged_multi(F, I, 16384, 256, F, F, I, I, 64, 32, 8, 128, 16, 140000, 2048, 0.088f, 0.1f, 0,
                                   nullptr, 0, F, Lf, M, 1024, nullptr), ATTN_OK);
    EXPECT(attn_decode_paged_multi(F, I, 166, 4, F, F, I, I, 64, 32, 8, 128, 16, 140000, 2048, 0.088f, 0.f, 32, F,
                                   wm - 4, F, Lf, nullptr, 0, nullptr), ATTN_ERR_WORKSPACE);
    // small-seq forward and backward
    EXPECT(attn_smallseq_cross(F, F, F, I, 30720, 16, 128, 16, 0.088f, F, F, Lf, nullptr), ATTN_OK);
    EXPECT(attn_smallseq_cross(F, F, F, I, 30720, 16, 128, 17, 0.088f, F, F, Lf, nullptr), ATTN_ERR_INVALID);
    EXPECT(attn_smallseq_cross_backward(F, F, F, F, F, I, 30720, 16, 128, 16, 0.088f, F, F, F, nullptr), ATTN_OK);
    EXPECT(attn_smallseq_cross_backward(F, F, F, nullptr, F, I, 30720, 16, 128, 16, 0.088f, F, F, F, nullptr),
           ATTN_ERR_INVALID);
    // prefill backward
    const size_t wb = attn_prefill_varlen_backward_workspace_size(16, 4096, 32);
    EXPECT(attn_prefill_varlen_backward(ATTN_BF16, F, F, F, F, F, Lf, I, I, 16, 4096, 4096, 32, 8, 128, 0.088f, 1, F, F,
                                        F, F, wb, nullptr), ATTN_OK);
    EXPECT(attn_prefill_varlen_backward(ATTN_BF16, F, F, F, F, F, Lf, I, I, 16, 4096, 4096, 32, 8, 128, 0.088f, 1, F, F,
                                        F, F, wb - 1, nullptr), ATTN_ERR_WORKSPACE);
    EXPECT(attn_prefill_varlen_backward(ATTN_BF16, F, F, F, F, F, Lf, I, I, 1 << 20, 1 << 20, 4096, 32, 8, 128, 0.088f,
                                        1, F, F, F, F, big, nullptr), ATTN_ERR_UNSUPPORTED);
    for (int s = 0; s < 6; ++s)
        if (!attn_status_string((attn_status_t)s)[0])
            ++g_bad;
    std::printf("abi driver: %d unexpected statuses\n", g_bad);
    return g_bad ? 1 : 0;
}
