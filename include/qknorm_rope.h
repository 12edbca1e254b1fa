/*
 * qknorm_rope.h -- C ABI of the fused diffusion-transformer QK-norm + RoPE
 * pass for AMD Instinct MI355X (gfx950).
 *
 * The operation (TensorRT-LLM PR "VisualGen Wan: deduplicate shared RoPE SMEM
 * staging", Description; TensorRT-Model-Connect PR "perf(diffusion): fused
 * qknorm rope Flux 2.0", intro): for every token and every Q and K head,
 *
 *   r      = 1 / sqrt(mean_d x[d]^2 + eps)          per-head RMSNorm over head_dim
 *   n[d]   = x[d] * r * gamma[d]                     gamma: q_gamma for Q, k_gamma for K
 *   o[a]   = n[a] * cos[a] - n[b] * sin[a]           for each rotary pair (a, b):
 *   o[b]   = n[b] * cos[b] + n[a] * sin[b]             interleaved (2i, 2i+1) or
 *                                                      rotate-half (i, i + head_dim/2)
 *
 * written back in place over Q and K, rounded once (round to nearest even) to
 * the tensor's dtype; math is fp32 inside.  Any finite input is normalised
 * correctly: a head whose fp32 sum of squares would overflow (bf16 values
 * with an RMS beyond about 1.6e18) or sink into the subnormal range while
 * eps is below 2^-100 is summed again on x * 2^-e, e the binary exponent of
 * its largest |x| (an exact rescaling).  The cos/sin row of token t is
 * either shared by all heads ([tokens, head_dim], "shared") or given per head
 * ([tokens, heads, head_dim], "per-head"); row (t, h) serves Q head h and K
 * head h.  The V slice of a fused buffer is never read or written.
 *
 * All pointers are DEVICE pointers owned by the caller; the library never
 * allocates, frees or synchronises and keeps no state between calls (calls
 * are thread-safe).  Q and K are modified in place; every other buffer is
 * read-only.  Buffers must stay valid until the work queued on `stream`
 * completes.  Work is only enqueued: the call returns before it runs.
 */
#ifndef QKNORM_ROPE_H
#define QKNORM_ROPE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKNORM_ROPE_VERSION 2

/* Return codes.  On any error nothing is enqueued and no buffer is touched. */
enum {
    QKR_OK = 0,
    QKR_ERR_NULL = -1,        /* a required pointer is NULL                          */
    QKR_ERR_SHAPE = -2,       /* tokens < 0, heads < 1, or a size over the limits    */
    QKR_ERR_ALIGN = -3,       /* a pointer is not 16-byte aligned                    */
    QKR_ERR_UNSUPPORTED = -4, /* head_dim not 64/128/256, or an unsupported dtype    */
    QKR_ERR_MODE = -5,        /* not exactly one of {qkv} / {q and/or k}             */
    QKR_ERR_HIP = -6,         /* the kernel launch (or an attribute query) failed     */
    QKR_ERR_ARG = -7,         /* eps not finite and > 0, an enum out of range, or a   */
                              /* buffer the call writes overlapping another buffer    */
    QKR_ERR_WORKSPACE = -8,   /* workspace missing or smaller than required           */
    QKR_ERR_SCRATCH = -9      /* the call needs more than the library's fixed scratch  */
};

/* Element types. */
enum { QKR_BF16 = 0, QKR_FP16 = 1, QKR_FP32 = 2 };
/* cos/sin layouts. */
enum { QKR_COS_SHARED = 0, QKR_COS_PER_HEAD = 1 };
/* RoPE pairing styles. */
enum { QKR_ROPE_INTERLEAVED = 0, QKR_ROPE_ROTATE_HALF = 1 };

/* Limits checked by qknorm_rope_fused (and, for rows, dit_fuse_scale_shift).
 * A launch grid holds fewer than 2^32 work-items; with 256-thread workgroups
 * of two tokens (one row for short AdaLN calls: 64 threads) 2^24 tokens stay
 * far inside it. */
#define QKR_MAX_TOKENS ((int64_t)1 << 24)   /* tokens must be below this     */
#define QKR_MAX_HEADS 65536                 /* heads must not exceed this    */

/*
 * qknorm_rope_fused -- the pass, in place, on one stream.
 *
 * Modes (exactly one):
 *   fused:    qkv != NULL, q == k == NULL.  qkv is [tokens, 3*heads*head_dim],
 *             row-major, Q columns [0, H*D), K [H*D, 2*H*D), V [2*H*D, 3*H*D)
 *             (V untouched).  q_gamma and k_gamma are both required.
 *   separate: qkv == NULL and at least one of q, k != NULL.  Each given
 *             tensor is [tokens, heads, head_dim] contiguous; a tensor that is
 *             NULL is skipped and its gamma may be NULL.
 *
 * tokens      number of rows (batch folded in); 0 is a no-op that returns
 *             QKR_OK once the scalar arguments are valid (pointers unchecked).
 * heads       heads per tensor (Q, K and V have the same count), 1..65536.
 * head_dim    64, 128 or 256.
 * q_gamma, k_gamma  fp32 [head_dim] norm weights.
 * eps         added to the mean square inside the root; finite and > 0.
 * cos, sin    cos_dtype (QKR_FP32 or QKR_BF16) tables, contiguous:
 *             QKR_COS_SHARED [tokens, head_dim] or QKR_COS_PER_HEAD
 *             [tokens, heads, head_dim]; indexed by dimension (no assumption
 *             that paired dimensions hold equal values).
 * style       QKR_ROPE_INTERLEAVED or QKR_ROPE_ROTATE_HALF.
 * dtype       QKR_BF16 or QKR_FP16: element type of qkv / q / k.
 * stream      a hipStream_t (NULL = the default stream).
 *
 * Long calls of the shared layout (at least 4096 workgroups, each wave
 * keeping at least 6 KB of Q/K loads in flight) reserve 56 KB of LDS per
 * workgroup at launch, which holds a CU to 2 of the pass's workgroups: the
 * HBM stream runs faster with fewer waves resident (qknorm_rope_kernel_info
 * reports it).  Kernels of other streams share what the pass leaves free.
 *
 * Every data pointer must be 16-byte aligned.  The tensors written (qkv, or q
 * and k) must not overlap each other, gamma, cos or sin (QKR_ERR_ARG).
 * Returns QKR_OK or a negative QKR_ERR_* code; all checks happen before any
 * HIP call.
 */
int qknorm_rope_fused(void* qkv, void* q, void* k, int64_t tokens, int32_t heads,
                      int32_t head_dim, const float* q_gamma, const float* k_gamma, float eps,
                      const void* cos, const void* sin, int32_t cos_layout, int32_t cos_dtype,
                      int32_t style, int32_t dtype, void* stream);

/* Static description of a status code (never NULL). */
const char* qknorm_rope_strerror(int status);

/* QKNORM_ROPE_VERSION of the built library. */
int qknorm_rope_version(void);

/* Resources of the kernel one configuration launches (from the code object). */
typedef struct {
    int32_t num_vgprs;        /* registers per lane                               */
    int32_t lds_bytes;        /* static LDS per workgroup                         */
    int32_t scratch_bytes;    /* private (spill) memory per lane; 0 expected       */
    int32_t block_threads;    /* workgroup size the library launches              */
    int32_t tokens_per_block; /* tokens one workgroup covers                      */
    int32_t heads_in_flight;  /* head iterations whose loads a lane keeps in flight */
    int32_t die_runs;         /* 1: each die processes one contiguous token run   */
    int32_t dynamic_lds_bytes; /* LDS reserved per workgroup at launch (unused by  */
                              /* the kernel) to cap residency; 0 for none          */
    int32_t workgroups_per_cu; /* the residency that reservation allows on a      */
                              /* 160 KB-LDS CU; 0 when not capped                  */
} qkr_kernel_info;

/* Which tensors a call passes, for qknorm_rope_kernel_info. */
enum {
    QKR_TENSORS_FUSED = 0,    /* qkv: one fused [tokens, 3*heads*head_dim] buffer */
    QKR_TENSORS_PAIR = 1,     /* q and k, two separate buffers                     */
    QKR_TENSORS_ONE = 2       /* q or k alone                                      */
};

/*
 * qknorm_rope_kernel_info -- fill *out for the kernel that qknorm_rope_fused
 * launches for `tokens` tokens of `heads` heads of `head_dim`, with the
 * tensors given as `tensors` (QKR_TENSORS_*) and the given layout and dtypes
 * (the unroll depth and block order depend on heads, tokens and tensors).
 * Needs a HIP device (queries the loaded code object).  Returns QKR_OK,
 * QKR_ERR_NULL, QKR_ERR_ARG / QKR_ERR_UNSUPPORTED / QKR_ERR_SHAPE for a bad
 * configuration (checked before any HIP call), or QKR_ERR_HIP.
 */
int qknorm_rope_kernel_info(int32_t head_dim, int32_t heads, int64_t tokens, int32_t tensors,
                            int32_t cos_layout, int32_t cos_dtype, int32_t style, int32_t dtype,
                            qkr_kernel_info* out);

#ifdef __cplusplus
}
#endif

#endif /* QKNORM_ROPE_H */
