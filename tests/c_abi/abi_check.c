/* Plain C consumer of the library's public headers: compiled with gcc by
 * tests/test_c_abi.py and run on the CPU.  Every call here is rejected by the
 * library's argument checks before any HIP call (or is a zero-size no-op),
 * so no GPU is needed.  Prints "ok" and exits 0 when every code matches. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fuse_scale_shift.h"
#include "group_norm_silu.h"
#include "qknorm_rope.h"

#define EXPECT(call, code)                                                          \
    do {                                                                            \
        int got_ = (call);                                                          \
        if (got_ != (code)) {                                                       \
            printf("FAIL line %d: got %d (%s), want %d\n", __LINE__, got_,          \
                   qknorm_rope_strerror(got_), (code));                             \
            return 1;                                                               \
        }                                                                           \
    } while (0)

int main(void)
{
    void* a = (void*)(uintptr_t)0x10000;      /* aligned fake device addresses */
    void* b = (void*)(uintptr_t)0x90000;
    void* far = (void*)(uintptr_t)0x40000000;  /* beyond any x range used below */
    void* mis = (void*)(uintptr_t)0x10004;
    const float* g = (const float*)a;

    if (qknorm_rope_version() != QKNORM_ROPE_VERSION) {
        printf("FAIL version\n");
        return 1;
    }
    if (strcmp(qknorm_rope_strerror(QKR_OK), "ok") != 0) {
        printf("FAIL strerror\n");
        return 1;
    }
    EXPECT(qknorm_rope_fused(a, NULL, NULL, 0, 40, 128, g, g, 1e-6f, a, a, QKR_COS_SHARED,
                             QKR_FP32, QKR_ROPE_INTERLEAVED, QKR_BF16, NULL), QKR_OK);
    EXPECT(qknorm_rope_fused(a, NULL, NULL, 8, 40, 96, g, g, 1e-6f, a, a, QKR_COS_SHARED,
                             QKR_FP32, QKR_ROPE_INTERLEAVED, QKR_BF16, NULL), QKR_ERR_UNSUPPORTED);
    EXPECT(qknorm_rope_fused(a, a, NULL, 8, 40, 128, g, g, 1e-6f, a, a, QKR_COS_SHARED,
                             QKR_FP32, QKR_ROPE_INTERLEAVED, QKR_BF16, NULL), QKR_ERR_MODE);
    EXPECT(qknorm_rope_fused(mis, NULL, NULL, 8, 40, 128, g, g, 1e-6f, a, a, QKR_COS_SHARED,
                             QKR_FP32, QKR_ROPE_INTERLEAVED, QKR_BF16, NULL), QKR_ERR_ALIGN);
    EXPECT(qknorm_rope_fused(NULL, a, NULL, 8, 40, 128, NULL, g, 1e-6f, a, a, QKR_COS_PER_HEAD,
                             QKR_BF16, QKR_ROPE_ROTATE_HALF, QKR_FP16, NULL), QKR_ERR_NULL);
    EXPECT(qknorm_rope_fused(a, NULL, NULL, 8, 40, 128, g, g, -1.0f, a, a, QKR_COS_SHARED,
                             QKR_FP32, QKR_ROPE_INTERLEAVED, QKR_BF16, NULL), QKR_ERR_ARG);
    EXPECT(qknorm_rope_fused(a, NULL, NULL, -5, 40, 128, g, g, 1e-6f, a, a, QKR_COS_SHARED,
                             QKR_FP32, QKR_ROPE_INTERLEAVED, QKR_BF16, NULL), QKR_ERR_SHAPE);

    EXPECT(dit_fuse_scale_shift(a, b, 0, 6144, 1, a, a, QKR_FP32, 1e-6f, QKR_BF16, NULL), QKR_OK);
    EXPECT(dit_fuse_scale_shift(a, b, 4, 6145, 1, a, a, QKR_FP32, 1e-6f, QKR_BF16, NULL),
           QKR_ERR_UNSUPPORTED);
    EXPECT(dit_fuse_scale_shift(a, b, 4, FSS_MAX_HIDDEN + 8, 1, a, a, QKR_FP32, 1e-6f, QKR_BF16,
                                NULL), QKR_ERR_UNSUPPORTED);
    EXPECT(dit_fuse_scale_shift(a, (char*)a + 64, 4, 6144, 1, a, a, QKR_FP32, 1e-6f, QKR_BF16,
                                NULL), QKR_ERR_ARG);
    EXPECT(dit_fuse_scale_shift(a, b, 4, 6144, 0, a, a, QKR_FP32, 1e-6f, QKR_BF16, NULL),
           QKR_ERR_SHAPE);
    EXPECT(dit_fuse_scale_shift(a, b, 4, 6144, 1, NULL, a, QKR_FP32, 1e-6f, QKR_BF16, NULL),
           QKR_ERR_NULL);
    if (dit_group_norm_silu_workspace_size(1, 512, 128 * 128, 32) != 32 * 64 * 8) {
        printf("FAIL workspace size\n");
        return 1;
    }
    {
        int64_t chunk = 0;
        EXPECT(dit_group_norm_silu_schedule(1, 512, 128 * 128, 32, &chunk), 2);
        if (chunk != 4096) {
            printf("FAIL schedule chunk %lld\n", (long long)chunk);
            return 1;
        }
        EXPECT(dit_group_norm_silu_schedule(1, 128, 1024 * 1024, 32, NULL), 1);
        EXPECT(dit_group_norm_silu_schedule(2, 64, 512, 32, NULL), 0);
        EXPECT(dit_group_norm_silu_schedule(1, 30, 64, 4, NULL), QKR_ERR_SHAPE);
    }
    EXPECT(dit_group_norm_silu(a, b, 1, 512, 128 * 128, 32, a, a, QKR_FP32, 1e-6f, QKR_BF16, NULL,
                               0, NULL), QKR_ERR_ARG);          /* y inside x's 16 MB */
    EXPECT(dit_group_norm_silu(a, far, 1, 512, 128 * 128, 32, a, a, QKR_FP32, 1e-6f, QKR_BF16,
                               NULL, 0, NULL), QKR_ERR_WORKSPACE);
    EXPECT(dit_group_norm_silu(a, b, 1, 512, 100, 32, a, a, QKR_FP32, 1e-6f, QKR_BF16, NULL, 0,
                               NULL), QKR_ERR_UNSUPPORTED);
    EXPECT(dit_group_norm_silu(a, b, 0, 512, 64, 32, a, a, QKR_FP32, 1e-6f, QKR_BF16, NULL, 0,
                               NULL), QKR_OK);
    /* the entry point without workspace: a call beyond its fixed scratch is
     * refused before any HIP call; n == 0 is a no-op */
    EXPECT(dit_group_norm_silu_noalloc(a, (void*)(uintptr_t)0x1000000000ull, 65, 512, 65536, 32, a,
                                       a, QKR_FP32, 1e-6f, QKR_BF16, NULL), QKR_ERR_SCRATCH);
    EXPECT(dit_group_norm_silu_noalloc(a, b, 0, 64, 64, 8, a, a, QKR_FP32, 1e-6f, QKR_BF16, NULL),
           QKR_OK);
    printf("ok\n");
    return 0;
}
