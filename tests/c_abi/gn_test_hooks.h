/*
 * gn_test_hooks.h -- test-only entry point of libqknorm_rope.so (not part of
 * the library's public headers under include/).
 *
 * dit_group_norm_silu_polls is dit_group_norm_silu (include/group_norm_silu.h)
 * with the lagged schedule's polls of an unpublished chunk word set by the
 * caller instead of the library's fixed 4096.  With 0, every workgroup whose
 * output group is incomplete at its first look reduces the missing chunks
 * itself, which lets a test drive that rarely taken path on purpose.  Every
 * other argument, check and status is that of dit_group_norm_silu; a
 * wait_polls outside 0..4096 returns QKR_ERR_ARG before any HIP call.
 */
#ifndef GN_TEST_HOOKS_H
#define GN_TEST_HOOKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int dit_group_norm_silu_polls(const void* x, void* y, int64_t n, int32_t channels,
                              int64_t spatial, int32_t groups, const void* gamma, const void* beta,
                              int32_t param_dtype, float eps, int32_t dtype, void* workspace,
                              int64_t workspace_bytes, void* stream, int32_t wait_polls);

#ifdef __cplusplus
}
#endif

#endif /* GN_TEST_HOOKS_H */
