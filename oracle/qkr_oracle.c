/*
 * CPU oracle for the fused diffusion-transformer QK-norm + RoPE pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Tests, the smoke check and the bench's CPU
 * baseline call this file; the product path (the HIP library) never does and
 * shares no code, header or table with it.
 *
 * What it computes (plain definition, fp64, no blocking or fusion):
 *   The pages describe one kernel that replaces a chain of per-head RMSNorms
 *   followed by RoPEs on Q and K (FLUX.2 PR "perf(diffusion): fused qknorm
 *   rope Flux 2.0", intro), working in place on a fused QKV buffer with the V
 *   slice untouched (TensorRT-LLM PR "VisualGen Wan: deduplicate shared RoPE
 *   SMEM staging", Description and Test Coverage).  The cos/sin row is
 *   indexed by dimension for every head (same PR, Description), either one
 *   row per token shared by all heads or one materialised row per head (Test
 *   Coverage), in interleaved or rotate-half style (Test Coverage).
 *
 *   For each token t and head h of the tensor:
 *     v[d]  = decode(x[t, h, d])                 exact widening to fp64
 *     ms    = (sum_d v[d]^2) / D                 mean over head_dim
 *     r     = 1 / sqrt(ms + eps)                 eps inside the root
 *     n[d]  = v[d] * r * gamma[d]                learned head_dim-wide weight
 *     pair (a, b) = (d, partner(d)):
 *       interleaved  a = 2i, b = 2i+1;  rotate-half  a = i, b = i + D/2
 *       o[a] = n[a] * c[a] - n[b] * s[a]
 *       o[b] = n[b] * c[b] + n[a] * s[b]         (rotation by +angle)
 *   with c, s the cos/sin row of token t (shared layout) or of (t, h)
 *   (per-head layout).  Output is the unrounded fp64 o.
 *
 * Readings where the pages are silent (eps inside the root, mean over D,
 * gamma multiplied directly and before RoPE, the +angle sign, no intermediate
 * rounding) are the plain RMSNorm / RoPE definitions.
 *
 * The file also holds the oracles of the adaptive layer norm with scale and
 * shift (qkr_oracle_adaln) and of the group norm followed by SiLU
 * (qkr_oracle_group_norm_silu), below.
 *
 * Every function here is pinned by CPU tests against brute force in exact
 * arithmetic, closed forms, invariants and library routines.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define QKR_O_BF16 0
#define QKR_O_FP16 1
#define QKR_O_FP32 2
#define QKR_O_SHARED 0
#define QKR_O_PER_HEAD 1
#define QKR_O_INTERLEAVED 0
#define QKR_O_ROTATE_HALF 1

/* bf16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
static double decode_bf16(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xff;
    int m = bits & 0x7f;
    double mag;
    if (e == 0xff)
        mag = m ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)m / 128.0, -126);
    else
        mag = ldexp(1.0 + (double)m / 128.0, e - 127);
    return sign ? -mag : mag;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double decode_fp16(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1f;
    int m = bits & 0x3ff;
    double mag;
    if (e == 0x1f)
        mag = m ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)m / 1024.0, -14);
    else
        mag = ldexp(1.0 + (double)m / 1024.0, e - 15);
    return sign ? -mag : mag;
}

static double decode16(uint16_t bits, int dtype)
{
    return dtype == QKR_O_FP16 ? decode_fp16(bits) : decode_bf16(bits);
}

static double table_value(const void* table, int dtype, int64_t index)
{
    if (dtype == QKR_O_FP32)
        return (double)((const float*)table)[index];
    return decode_bf16(((const uint16_t*)table)[index]);
}

/* Exact decode of n 16-bit values (bf16 or fp16) to fp64. */
void qkr_oracle_decode(const uint16_t* in, int64_t n, int dtype, double* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = decode16(in[i], dtype);
}

/*
 * Round each value to the nearest bf16 / fp16 number, ties to even, in place
 * (the rounded image of the output, for diagnostics).  Works on the real
 * line: the quantum is 2^(e - p + 1) with p the significand precision (8 for
 * bf16, 11 for fp16) and e the binade, floored at the least normal exponent
 * so subnormals get the fixed subnormal quantum; rint() rounds to nearest,
 * ties to even, in the default mode.  Results beyond the largest finite
 * value become infinities.
 */
void qkr_oracle_round(double* v, int64_t n, int dtype)
{
    const int p = dtype == QKR_O_FP16 ? 11 : 8;
    const int emin = dtype == QKR_O_FP16 ? -14 : -126;
    const int emax = dtype == QKR_O_FP16 ? 15 : 127;
    const double maxfin = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    for (int64_t i = 0; i < n; ++i) {
        double x = v[i];
        if (!isfinite(x) || x == 0.0)
            continue;
        double a = fabs(x);
        int e;
        frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1) -> binade e-1 */
        int binade = e - 1;
        if (binade < emin)
            binade = emin;
        double q = ldexp(1.0, binade - p + 1);
        double r = rint(a / q) * q;
        /* overflow: at or beyond the midpoint above maxfin rounds to infinity */
        if (r > maxfin)
            r = INFINITY;
        v[i] = x < 0 ? -r : r;
    }
}

/*
 * The pass on one tensor, tokens [t_begin, t_end).
 *
 *   x          16-bit elements; head h of token t starts at
 *              x + t*row_stride + col0 + h*head_dim (element offsets), so a
 *              fused QKV buffer uses row_stride = 3*heads*head_dim with
 *              col0 = 0 for Q and heads*head_dim for K, and a separate
 *              [T, heads, head_dim] tensor uses row_stride = heads*head_dim.
 *   x_dtype    0 bf16, 1 fp16
 *   gamma      fp32 [head_dim]
 *   cos, sin   [T, head_dim] (shared) or [T, heads, head_dim] (per-head),
 *              fp32 (cos_dtype 2) or bf16 (cos_dtype 0)
 *   out        fp64 [t_end - t_begin, heads, head_dim]
 * Returns 0, or -1 on an argument it cannot handle.
 */
int qkr_oracle_qknorm_rope(const uint16_t* x, int x_dtype, int64_t row_stride, int64_t col0,
                           int64_t t_begin, int64_t t_end, int32_t heads, int32_t head_dim,
                           const float* gamma, float eps, const void* cos, const void* sin,
                           int cos_dtype, int cos_layout, int style, double* out)
{
    if (head_dim <= 0 || head_dim > 512 || head_dim % 2 || heads <= 0 || t_end < t_begin)
        return -1;
    if (style != QKR_O_INTERLEAVED && style != QKR_O_ROTATE_HALF)
        return -1;
    if (cos_layout != QKR_O_SHARED && cos_layout != QKR_O_PER_HEAD)
        return -1;
    const int64_t D = head_dim;
    const int64_t half = D / 2;
    const double eps64 = (double)eps;

#pragma omp parallel for schedule(static)
    for (int64_t t = t_begin; t < t_end; ++t) {
        double v[512], nrm[512];
        for (int64_t h = 0; h < heads; ++h) {
            const uint16_t* xh = x + t * row_stride + col0 + h * D;
            double* oh = out + ((t - t_begin) * heads + h) * D;

            double sum_sq = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                v[d] = decode16(xh[d], x_dtype);
                sum_sq += v[d] * v[d];
            }
            const double ms = sum_sq / (double)D;
            const double r = 1.0 / sqrt(ms + eps64);
            for (int64_t d = 0; d < D; ++d)
                nrm[d] = v[d] * r * (double)gamma[d];

            const int64_t row = cos_layout == QKR_O_SHARED ? t : t * heads + h;
            for (int64_t i = 0; i < half; ++i) {
                int64_t a, b;
                if (style == QKR_O_INTERLEAVED) {
                    a = 2 * i;
                    b = 2 * i + 1;
                } else {
                    a = i;
                    b = i + half;
                }
                const double ca = table_value(cos, cos_dtype, row * D + a);
                const double sa = table_value(sin, cos_dtype, row * D + a);
                const double cb = table_value(cos, cos_dtype, row * D + b);
                const double sb = table_value(sin, cos_dtype, row * D + b);
                oh[a] = nrm[a] * ca - nrm[b] * sa;
                oh[b] = nrm[b] * cb + nrm[a] * sb;
            }
        }
    }
    return 0;
}

/* One element of a modulation table: bf16 (0), fp16 (1) or fp32 (2). */
static double mod_value(const void* table, int dtype, int64_t index)
{
    if (dtype == QKR_O_FP32)
        return (double)((const float*)table)[index];
    return decode16(((const uint16_t*)table)[index], dtype);
}

/*
 * Adaptive layer norm with a per-sample scale and shift: the "fuse_scale_shift"
 * (AdaLN) step that TensorRT-Model-Connect PR "perf(diffusion): fused qknorm
 * rope Flux 2.0" lists as its largest follow-up.  The page gives only the
 * name; this is the plain definition of an AdaLN modulation (layer norm
 * without learned affine, then (1 + scale) and shift):
 *
 *   for row r of x [rows, hidden] (C = hidden), batch b = r / rows_per_batch:
 *     mean = (sum_c x[c]) / C
 *     var  = (sum_c (x[c] - mean)^2) / C          biased variance
 *     n[c] = (x[c] - mean) / sqrt(var + eps)
 *     y[c] = n[c] * (1 + scale[b, c]) + shift[b, c]
 *
 * x: 16-bit (x_dtype 0 bf16, 1 fp16); scale, shift: [batches, C] of
 * mod_dtype (0 bf16, 1 fp16, 2 fp32).  out: fp64 [row_end - row_begin, C].
 */
int qkr_oracle_adaln(const uint16_t* x, int x_dtype, int64_t row_begin, int64_t row_end,
                     int64_t hidden, int64_t rows_per_batch, const void* scale, const void* shift,
                     int mod_dtype, float eps, double* out)
{
    if (hidden <= 0 || rows_per_batch <= 0 || row_end < row_begin || row_begin < 0)
        return -1;
    if (mod_dtype != QKR_O_BF16 && mod_dtype != QKR_O_FP16 && mod_dtype != QKR_O_FP32)
        return -1;
    const int64_t C = hidden;
    const double eps64 = (double)eps;

#pragma omp parallel for schedule(static)
    for (int64_t r = row_begin; r < row_end; ++r) {
        const uint16_t* xr = x + r * C;
        double* yr = out + (r - row_begin) * C;
        const int64_t b = r / rows_per_batch;

        double sum = 0.0;
        for (int64_t c = 0; c < C; ++c)
            sum += decode16(xr[c], x_dtype);
        const double mean = sum / (double)C;
        double sum_dev = 0.0;
        for (int64_t c = 0; c < C; ++c) {
            const double dev = decode16(xr[c], x_dtype) - mean;
            sum_dev += dev * dev;
        }
        const double var = sum_dev / (double)C;
        const double inv = 1.0 / sqrt(var + eps64);
        for (int64_t c = 0; c < C; ++c) {
            const double n = (decode16(xr[c], x_dtype) - mean) * inv;
            yr[c] = n * (1.0 + mod_value(scale, mod_dtype, b * C + c))
                    + mod_value(shift, mod_dtype, b * C + c);
        }
    }
    return 0;
}

/*
 * Group norm followed by SiLU: the "group_norm_silu" (VAE) step that
 * TensorRT-Model-Connect PR "perf(diffusion): fused qknorm rope Flux 2.0"
 * lists among its follow-ups.  The page gives only the name; this is the
 * plain definition (group normalisation with a per-channel affine, then
 * SiLU(y) = y / (1 + exp(-y))):
 *
 *   x [n, C, S] contiguous, G groups of Cg = C / G channels; for sample i
 *   and group g, over the Cg * S elements of channels g*Cg .. g*Cg + Cg - 1:
 *     mean = (1/(Cg S)) sum x;  var = (1/(Cg S)) sum (x - mean)^2   (biased)
 *     y    = (x - mean) / sqrt(var + eps) * gamma[c] + beta[c]
 *     out  = y / (1 + exp(-y))
 *
 * x: 16-bit (x_dtype 0 bf16, 1 fp16); gamma, beta: [C] of param_dtype
 * (0 bf16, 1 fp16, 2 fp32).  out: fp64 [n, C, S] for the groups
 * [group_begin, group_end) of the n*G (sample, group) pairs, in order.
 */
int qkr_oracle_group_norm_silu(const uint16_t* x, int x_dtype, int64_t channels, int64_t spatial,
                               int64_t groups, int64_t group_begin, int64_t group_end,
                               const void* gamma, const void* beta, int param_dtype, float eps,
                               double* out)
{
    if (channels <= 0 || spatial <= 0 || groups <= 0 || channels % groups)
        return -1;
    if (group_begin < 0 || group_end < group_begin)
        return -1;
    if (param_dtype != QKR_O_BF16 && param_dtype != QKR_O_FP16 && param_dtype != QKR_O_FP32)
        return -1;
    const int64_t cg = channels / groups;
    const int64_t gsize = cg * spatial;
    const double eps64 = (double)eps;

#pragma omp parallel for schedule(dynamic)
    for (int64_t q = group_begin; q < group_end; ++q) {
        /* (sample, group) pair q covers one contiguous run of gsize elements */
        const uint16_t* xq = x + q * gsize;
        double* oq = out + (q - group_begin) * gsize;
        const int64_t c0 = (q % groups) * cg;

        double sum = 0.0;
        for (int64_t e = 0; e < gsize; ++e)
            sum += decode16(xq[e], x_dtype);
        const double mean = sum / (double)gsize;
        double sum_dev = 0.0;
        for (int64_t e = 0; e < gsize; ++e) {
            const double dev = decode16(xq[e], x_dtype) - mean;
            sum_dev += dev * dev;
        }
        const double inv = 1.0 / sqrt(sum_dev / (double)gsize + eps64);
        for (int64_t e = 0; e < gsize; ++e) {
            const int64_t c = c0 + e / spatial;
            const double y = (decode16(xq[e], x_dtype) - mean) * inv * mod_value(gamma, param_dtype, c)
                             + mod_value(beta, param_dtype, c);
            oq[e] = y / (1.0 + exp(-y));
        }
    }
    return 0;
}

int qkr_oracle_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the next oracle calls use (n >= 1); for timing the oracle on one
 * core beside all cores. */
void qkr_oracle_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
