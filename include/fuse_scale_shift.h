/*
 * fuse_scale_shift.h -- C ABI of the fused adaptive layer norm with scale and
 * shift (AdaLN modulation) for AMD Instinct MI355X (gfx950), built into the
 * same library as qknorm_rope.h (libqknorm_rope.so).
 *
 * The operation is the "fuse_scale_shift" (AdaLN) step that
 * TensorRT-Model-Connect PR "perf(diffusion): fused qknorm rope Flux 2.0"
 * lists as its largest follow-up (section "Not in this PR - follow-ups").  The
 * page names it only; this library implements the plain AdaLN definition,
 * a layer norm without learned affine followed by the per-sample modulation:
 *
 *   for row r of x [rows, hidden], batch b = r / rows_per_batch:
 *     mean = (1/hidden) sum_c x[c]
 *     var  = (1/hidden) sum_c (x[c] - mean)^2             (biased)
 *     y[c] = (x[c] - mean) / sqrt(var + eps) * (1 + scale[b, c]) + shift[b, c]
 *
 * Math is fp32 (two passes over the row held in registers); y is rounded
 * once, to nearest even, to x's dtype.  Any finite input is normalised
 * correctly: a row whose plain fp32 sums would overflow (bf16 values beyond
 * about 1e17) or sink into the subnormal range while eps is below 2^-100 is
 * reduced again on x * 2^-e, e the binary exponent of its largest magnitude
 * (an exact rescaling), and normalised in that scale.
 *
 * Pointers are DEVICE pointers owned by the caller; the library allocates,
 * frees and synchronises nothing.  y may be x itself (in place) or a buffer
 * that does not overlap it.  Work is only enqueued on `stream`.
 */
#ifndef FUSE_SCALE_SHIFT_H
#define FUSE_SCALE_SHIFT_H

#include <stdint.h>

#include "qknorm_rope.h" /* status codes and dtype constants */

#ifdef __cplusplus
extern "C" {
#endif

#define FSS_MAX_HIDDEN 8192   /* hidden must be a multiple of 8 in [8, 8192] */

/*
 * dit_fuse_scale_shift -- AdaLN modulation of `rows` rows.
 *
 * x, y            [rows, hidden] contiguous, dtype QKR_BF16 or QKR_FP16.
 * rows            >= 0 (0 is a no-op returning QKR_OK once scalars are valid),
 *                 below QKR_MAX_TOKENS.
 * hidden          multiple of 8, 8 .. FSS_MAX_HIDDEN.
 * rows_per_batch  >= 1; row r reads modulation row r / rows_per_batch.
 * scale, shift    [ceil(rows / rows_per_batch), hidden] contiguous, mod_dtype
 *                 QKR_BF16, QKR_FP16 or QKR_FP32.
 * eps             finite and > 0, added to the variance inside the root.
 * stream          a hipStream_t (NULL = the default stream).
 *
 * Every pointer must be 16-byte aligned.  Returns QKR_OK or a negative
 * QKR_ERR_* code (QKR_ERR_ARG also when y partly overlaps x, or overlaps scale
 * or shift); all checks happen before any HIP call and nothing is enqueued on
 * error.
 */
int dit_fuse_scale_shift(const void* x, void* y, int64_t rows, int32_t hidden,
                         int64_t rows_per_batch, const void* scale, const void* shift,
                         int32_t mod_dtype, float eps, int32_t dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FUSE_SCALE_SHIFT_H */
