/*
 * group_norm_silu.h -- C ABI of the fused group norm + SiLU step (VAE) for AMD
 * Instinct MI355X (gfx950), built into the same library as qknorm_rope.h
 * (libqknorm_rope.so).
 *
 * The operation is the "group_norm_silu" (VAE) follow-up that
 * TensorRT-Model-Connect PR "perf(diffusion): fused qknorm rope Flux 2.0"
 * names (section "Not in this PR - follow-ups").  The page gives only the
 * name; this library implements the plain definition, a group normalisation
 * with a per-channel affine followed by SiLU:
 *
 *   x, y [n, channels, spatial] contiguous (spatial = H*W, or T*H*W);
 *   G = groups, Cg = channels / G; for sample i and group g, over the
 *   Cg * spatial elements of channels g*Cg .. g*Cg + Cg - 1:
 *     mean = average;  var = average squared deviation (biased)
 *     t    = (x - mean) / sqrt(var + eps) * gamma[c] + beta[c]
 *     y    = t / (1 + exp(-t))
 *
 * Math is fp32; y is rounded once, to nearest even, to x's dtype.  Large
 * groups are reduced in chunks whose partial statistics (mean and sum of
 * squared deviations per chunk) go to a caller-owned workspace; the chunks
 * are then combined exactly as a two-level reduction (Chan et al.).  Every
 * schedule combines them in the same order, so a shape's output bits do not
 * depend on which schedule runs it (dit_group_norm_silu_schedule).  Any
 * finite input is normalised correctly: a chunk or group whose plain fp32
 * sums would overflow (bf16 values beyond about 1e17) or sink into the
 * subnormal range while eps is below 2^-100 is reduced again on x * 2^-e,
 * e the binary exponent of its largest magnitude (an exact rescaling).
 *
 * Pointers are DEVICE pointers owned by the caller; the library allocates,
 * frees and synchronises nothing.  y may be x itself or a buffer that does
 * not overlap it.  Calls that share a workspace must not run concurrently.
 */
#ifndef GROUP_NORM_SILU_H
#define GROUP_NORM_SILU_H

#include <stdint.h>

#include "qknorm_rope.h" /* status codes and dtype constants */

#ifdef __cplusplus
extern "C" {
#endif

/*
 * dit_group_norm_silu_workspace_size -- bytes of workspace a call with these
 * sizes needs (0 when every group fits one chunk), or a negative QKR_ERR_*
 * code for sizes dit_group_norm_silu would reject.
 */
int64_t dit_group_norm_silu_workspace_size(int64_t n, int32_t channels, int64_t spatial,
                                           int32_t groups);

/*
 * dit_group_norm_silu_schedule -- how dit_group_norm_silu runs a call with
 * these sizes, or a negative QKR_ERR_* code for sizes it would reject.  If
 * chunk_elems is not NULL it receives the elements per chunk (16384, 8192 or
 * 4096; a group of one chunk may be shorter).  Returns
 *   0  one chunk per group: one kernel reads each group once;
 *   1  lagged single read: one kernel in which workgroup b publishes chunk
 *      b's statistics to the workspace and then writes chunk b - lag, after
 *      waiting for every chunk of that chunk's group (all held by lower
 *      workgroups); x comes from HBM once, the second read of a chunk from
 *      the L2 of the die that first read it.  Taken from 4096 chunks of 16384
 *      elements per call, for groups of at most 256 chunks.  A workgroup
 *      that finds a word still unpublished after a few ms of polling reduces
 *      that chunk itself; the first word published for a chunk stands
 *      (compare-and-swap), so the call ends whatever order its workgroups
 *      start in, also beside other work.  A small kernel first marks the
 *      workspace's words unpublished;
 *   2  two passes: a statistics kernel, then an apply kernel that re-reads x.
 */
int32_t dit_group_norm_silu_schedule(int64_t n, int32_t channels, int64_t spatial, int32_t groups,
                                     int64_t* chunk_elems);

/*
 * dit_group_norm_silu -- group norm + SiLU of an [n, channels, spatial] tensor.
 *
 * n                >= 0 (0 is a no-op returning QKR_OK once scalars are valid).
 * channels, groups >= 1, groups divides channels.
 * spatial          >= 8, a multiple of 8; channels/groups * spatial < 2^31.
 *                  The call takes one 256-thread workgroup per chunk of a
 *                  group (up to 16,384 elements; one chunk for a group that
 *                  fits); more than 2^24 - 1 workgroups (a launch grid holds
 *                  fewer than 2^32 work-items) is QKR_ERR_SHAPE, which in
 *                  practice only n * groups >= 2^24 small groups reach.
 * gamma, beta      [channels] of param_dtype (QKR_BF16, QKR_FP16, QKR_FP32).
 * eps              finite and > 0, added to the variance inside the root.
 * dtype            QKR_BF16 or QKR_FP16 (x and y).
 * workspace        device buffer of at least
 *                  dit_group_norm_silu_workspace_size(...) bytes (may be NULL
 *                  when that size is 0), 16-byte aligned; its contents on
 *                  entry do not matter and are left undefined.
 * stream           a hipStream_t (NULL = the default stream).
 *
 * x, y, gamma and beta must be 16-byte aligned.  Returns QKR_OK or a negative
 * QKR_ERR_* code (QKR_ERR_WORKSPACE for a missing or short workspace,
 * QKR_ERR_ARG also when y partly overlaps x, y overlaps gamma or beta, or the
 * workspace overlaps any other buffer); all checks happen before any HIP call
 * and nothing is enqueued on error.
 */
int dit_group_norm_silu(const void* x, void* y, int64_t n, int32_t channels, int64_t spatial,
                        int32_t groups, const void* gamma, const void* beta, int32_t param_dtype,
                        float eps, int32_t dtype, void* workspace, int64_t workspace_bytes,
                        void* stream);

/* Largest workspace dit_group_norm_silu_noalloc can use (1 MiB per GPU). */
#define QKR_GN_NOALLOC_WORKSPACE_MAX ((int64_t)1 << 20)

/*
 * dit_group_norm_silu_noalloc -- dit_group_norm_silu for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, kernels and output
 * bits, with the workspace taken from a fixed array inside the library
 * instead of a caller's buffer.
 *
 * The array is QKR_GN_NOALLOC_WORKSPACE_MAX bytes, one copy per GPU the
 * library runs on, held until the process ends; its device address is
 * looked up once per device, on the first call that needs it.  The call
 * allocates and frees nothing.  A call whose workspace size
 * (dit_group_norm_silu_workspace_size) exceeds the maximum returns
 * QKR_ERR_SCRATCH with nothing enqueued (for example more than 131,072
 * chunks of 16,384 elements; groups of one chunk need no workspace at all).
 *
 * Every call on one GPU shares that GPU's array, and each call starts by
 * initialising what it reads (the lagged schedule marks its words
 * unpublished; the two-pass schedule writes every partial before reading
 * it).  Calls that overlap in time on one GPU -- on different streams, or
 * from different threads without ordering -- race on the array and must not
 * be issued.
 *
 * Arguments, checks and the other status codes are those of
 * dit_group_norm_silu without workspace and workspace_bytes.  QKR_ERR_HIP
 * is also returned when the array's address cannot be looked up.
 */
int dit_group_norm_silu_noalloc(const void* x, void* y, int64_t n, int32_t channels,
                                int64_t spatial, int32_t groups, const void* gamma,
                                const void* beta, int32_t param_dtype, float eps, int32_t dtype,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GROUP_NORM_SILU_H */
