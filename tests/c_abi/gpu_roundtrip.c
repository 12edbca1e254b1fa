/* Plain C use of the library on the GPU, with no Python and no torch: HIP's C
 * runtime API for memory, the public header for the call, and the CPU oracle
 * (test infrastructure) for the check.  Built with gcc and run by
 * tests/test_gpu_c_roundtrip.py.
 *
 * A fused QKV bf16 buffer of 37 tokens x 3 x 3 heads x 128 goes to the GPU;
 * qknorm_rope_fused runs in place with one shared fp32 cos/sin row per token
 * (interleaved pairs); the result comes back and every Q and K element is
 * compared with the fp64 oracle (max_abs <= 1.6e-2, bf16), and every V element
 * bit for bit with the input.  Then the AdaLN modulation (two batches) and
 * group norm + SiLU in its two-pass and lagged schedules, with the workspace
 * sized by its query, each against the oracle (within (max |ref| + 1) / 256).
 * Prints each step's max_abs, then "ok", and exits 0. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fuse_scale_shift.h"
#include "group_norm_silu.h"
#include "qknorm_rope.h"

/* the oracle's entry points (libqkr_oracle.so; dtype codes bf16 0, fp32 2) */
int qkr_oracle_qknorm_rope(const uint16_t* x, int x_dtype, int64_t row_stride, int64_t col0,
                           int64_t t_begin, int64_t t_end, int32_t heads, int32_t head_dim,
                           const float* gamma, float eps, const void* cos, const void* sin,
                           int cos_dtype, int cos_layout, int style, double* out);
int qkr_oracle_adaln(const uint16_t* x, int x_dtype, int64_t row_begin, int64_t row_end,
                     int64_t hidden, int64_t rows_per_batch, const void* scale, const void* shift,
                     int mod_dtype, float eps, double* out);
int qkr_oracle_group_norm_silu(const uint16_t* x, int x_dtype, int64_t channels, int64_t spatial,
                               int64_t groups, int64_t group_begin, int64_t group_end,
                               const void* gamma, const void* beta, int param_dtype, float eps,
                               double* out);

static uint32_t next_u32(uint32_t* s)
{
    *s = *s * 1664525u + 1013904223u;
    return *s;
}

static float uniform(uint32_t* s) /* [0, 1) */
{
    return (float)(next_u32(s) >> 8) * (1.0f / 16777216.0f);
}

static uint16_t bf16_of(float f) /* round to nearest even; inputs are finite */
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static double double_of_bf16(uint16_t b)
{
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

#define CHECK_HIP(call)                                                         \
    do {                                                                        \
        hipError_t e_ = (call);                                                 \
        if (e_ != hipSuccess) {                                                 \
            printf("FAIL %s: %s\n", #call, hipGetErrorString(e_));              \
            return 1;                                                           \
        }                                                                       \
    } while (0)

/* max |got - ref| over n outputs, or -1 if one exceeds (max |ref| + 1) / 256
 * (half a bf16 ulp at the largest output, with margin, as in the smoke check) */
static double check_bf16(const uint16_t* got, const double* ref, int64_t n)
{
    double big = 0.0, worst = 0.0;
    for (int64_t i = 0; i < n; ++i)
        if (fabs(ref[i]) > big)
            big = fabs(ref[i]);
    for (int64_t i = 0; i < n; ++i) {
        const double err = fabs(double_of_bf16(got[i]) - ref[i]);
        if (!(err <= (big + 1.0) / 256.0))
            return -1.0;
        if (err > worst)
            worst = err;
    }
    return worst;
}

/* AdaLN modulation: 37 rows of 1000 in 2 batches (19 rows each), fp32 scale/shift */
static int adaln(uint32_t* seed)
{
    enum { R = 37, C = 1000, RPB = 19, B = 2 };
    uint16_t* x = malloc((size_t)R * C * 2);
    uint16_t* y = malloc((size_t)R * C * 2);
    float* sc = malloc((size_t)B * C * 4);
    float* sh = malloc((size_t)B * C * 4);
    double* ref = malloc((size_t)R * C * sizeof(double));
    if (!x || !y || !sc || !sh || !ref)
        return printf("FAIL host allocation\n"), 1;
    for (int i = 0; i < R * C; ++i)
        x[i] = bf16_of((uniform(seed) * 2.0f - 1.0f) * 2.0f + 0.5f);
    for (int i = 0; i < B * C; ++i) {
        sc[i] = (uniform(seed) * 2.0f - 1.0f) * 0.5f;
        sh[i] = (uniform(seed) * 2.0f - 1.0f) * 0.5f;
    }
    void *dx, *dy, *dsc, *dsh;
    CHECK_HIP(hipMalloc(&dx, (size_t)R * C * 2));
    CHECK_HIP(hipMalloc(&dy, (size_t)R * C * 2));
    CHECK_HIP(hipMalloc(&dsc, (size_t)B * C * 4));
    CHECK_HIP(hipMalloc(&dsh, (size_t)B * C * 4));
    CHECK_HIP(hipMemcpy(dx, x, (size_t)R * C * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dsc, sc, (size_t)B * C * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dsh, sh, (size_t)B * C * 4, hipMemcpyHostToDevice));
    const int rc = dit_fuse_scale_shift(dx, dy, R, C, RPB, dsc, dsh, QKR_FP32, 1e-6f, QKR_BF16, NULL);
    if (rc != QKR_OK)
        return printf("FAIL dit_fuse_scale_shift: %s\n", qknorm_rope_strerror(rc)), 1;
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(y, dy, (size_t)R * C * 2, hipMemcpyDeviceToHost));
    if (qkr_oracle_adaln(x, 0, 0, R, C, RPB, sc, sh, 2, 1e-6f, ref) != 0)
        return printf("FAIL adaln oracle\n"), 1;
    const double worst = check_bf16(y, ref, (int64_t)R * C);
    if (worst < 0)
        return printf("FAIL adaln output outside the bound\n"), 1;
    printf("adaln max_abs %.4g\n", worst);
    CHECK_HIP(hipFree(dx));
    CHECK_HIP(hipFree(dy));
    CHECK_HIP(hipFree(dsc));
    CHECK_HIP(hipFree(dsh));
    free(x), free(y), free(sc), free(sh), free(ref);
    return 0;
}

/* group norm + SiLU on [n, channels, spatial] with `groups` groups, fp32
 * affine, workspace from the size query; the oracle checks the first and
 * last group */
static int group_norm(uint32_t* seed, int64_t n, int32_t channels, int64_t spatial,
                      int32_t groups, int32_t want_schedule)
{
    const int64_t count = n * channels * spatial, gsize = channels / groups * spatial;
    const int64_t pairs = n * groups;
    uint16_t* x = malloc((size_t)count * 2);
    uint16_t* y = malloc((size_t)count * 2);
    float* g = malloc((size_t)channels * 4);
    float* b = malloc((size_t)channels * 4);
    double* ref = malloc((size_t)gsize * sizeof(double));
    if (!x || !y || !g || !b || !ref)
        return printf("FAIL host allocation\n"), 1;
    for (int64_t i = 0; i < count; ++i)
        x[i] = bf16_of((uniform(seed) * 2.0f - 1.0f) * 3.0f + 1.0f);
    for (int c = 0; c < channels; ++c) {
        g[c] = 1.0f + 0.2f * (uniform(seed) * 2.0f - 1.0f);
        b[c] = 0.3f * (uniform(seed) * 2.0f - 1.0f);
    }
    int64_t chunk = 0;
    const int32_t schedule = dit_group_norm_silu_schedule(n, channels, spatial, groups, &chunk);
    if (schedule != want_schedule)
        return printf("FAIL schedule %d, want %d\n", schedule, want_schedule), 1;
    const int64_t ws_bytes = dit_group_norm_silu_workspace_size(n, channels, spatial, groups);
    if (ws_bytes < 0)
        return printf("FAIL workspace size %lld\n", (long long)ws_bytes), 1;
    void *dx, *dy, *dg, *db, *ws = NULL;
    CHECK_HIP(hipMalloc(&dx, (size_t)count * 2));
    CHECK_HIP(hipMalloc(&dy, (size_t)count * 2));
    CHECK_HIP(hipMalloc(&dg, (size_t)channels * 4));
    CHECK_HIP(hipMalloc(&db, (size_t)channels * 4));
    if (ws_bytes > 0)
        CHECK_HIP(hipMalloc(&ws, (size_t)ws_bytes));
    CHECK_HIP(hipMemcpy(dx, x, (size_t)count * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dg, g, (size_t)channels * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(db, b, (size_t)channels * 4, hipMemcpyHostToDevice));
    const int rc = dit_group_norm_silu(dx, dy, n, channels, spatial, groups, dg, db, QKR_FP32,
                                       1e-6f, QKR_BF16, ws, ws_bytes, NULL);
    if (rc != QKR_OK)
        return printf("FAIL dit_group_norm_silu: %s\n", qknorm_rope_strerror(rc)), 1;
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(y, dy, (size_t)count * 2, hipMemcpyDeviceToHost));
    double worst = 0.0;
    const int64_t check[2] = {0, pairs - 1};
    for (int i = 0; i < 2; ++i) {
        const int64_t q = check[i];
        if (qkr_oracle_group_norm_silu(x, 0, channels, spatial, groups, q, q + 1, g, b, 2, 1e-6f,
                                       ref) != 0)
            return printf("FAIL group-norm oracle\n"), 1;
        const double w = check_bf16(y + q * gsize, ref, gsize);
        if (w < 0)
            return printf("FAIL group %lld outside the bound\n", (long long)q), 1;
        if (w > worst)
            worst = w;
    }
    printf("group_norm_silu schedule %d chunk %lld max_abs %.4g\n", schedule, (long long)chunk,
           worst);
    CHECK_HIP(hipFree(dx));
    CHECK_HIP(hipFree(dy));
    CHECK_HIP(hipFree(dg));
    CHECK_HIP(hipFree(db));
    if (ws)
        CHECK_HIP(hipFree(ws));
    free(x), free(y), free(g), free(b), free(ref);
    return 0;
}

static int qk_pass(uint32_t* seed_in);

int main(void)
{
    uint32_t seed = 20251202u;
    if (qk_pass(&seed) || adaln(&seed) || group_norm(&seed, 2, 8, 8192, 2, 2) ||
        group_norm(&seed, 8, 512, 16384, 32, 1))
        return 1;
    printf("ok\n");
    return 0;
}

/* the fused pass on a fused QKV buffer; returns 0 and prints max_abs */
static int qk_pass(uint32_t* seed_in)
{
    enum { T = 37, H = 3, D = 128 };
    const int64_t width = 3 * H * D;
    const size_t x_bytes = (size_t)T * width * 2, table_bytes = (size_t)T * D * 4;
    uint16_t* x = malloc(x_bytes);
    uint16_t* back = malloc(x_bytes);
    float* qg = malloc(D * 4);
    float* kg = malloc(D * 4);
    float* cs = malloc(table_bytes);
    float* sn = malloc(table_bytes);
    double* ref = malloc((size_t)T * H * D * sizeof(double));
    if (!x || !back || !qg || !kg || !cs || !sn || !ref) {
        printf("FAIL host allocation\n");
        return 1;
    }
    uint32_t seed = *seed_in;
    for (int64_t i = 0; i < T * width; ++i)
        x[i] = bf16_of((uniform(&seed) * 2.0f - 1.0f) * 3.0f);
    for (int d = 0; d < D; ++d) {
        qg[d] = 1.0f + 0.1f * (uniform(&seed) * 2.0f - 1.0f);
        kg[d] = 1.0f + 0.1f * (uniform(&seed) * 2.0f - 1.0f);
    }
    for (int t = 0; t < T; ++t)
        for (int i = 0; i < D / 2; ++i) {   /* interleaved: pair (2i, 2i+1) shares an angle */
            const double angle = (double)t * pow(10000.0, -2.0 * i / D);
            cs[t * D + 2 * i] = cs[t * D + 2 * i + 1] = (float)cos(angle);
            sn[t * D + 2 * i] = sn[t * D + 2 * i + 1] = (float)sin(angle);
        }

    void *dx, *dqg, *dkg, *dc, *ds;
    CHECK_HIP(hipMalloc(&dx, x_bytes));
    CHECK_HIP(hipMalloc(&dqg, D * 4));
    CHECK_HIP(hipMalloc(&dkg, D * 4));
    CHECK_HIP(hipMalloc(&dc, table_bytes));
    CHECK_HIP(hipMalloc(&ds, table_bytes));
    CHECK_HIP(hipMemcpy(dx, x, x_bytes, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dqg, qg, D * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dkg, kg, D * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dc, cs, table_bytes, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(ds, sn, table_bytes, hipMemcpyHostToDevice));

    const int rc = qknorm_rope_fused(dx, NULL, NULL, T, H, D, (const float*)dqg,
                                     (const float*)dkg, 1e-6f, dc, ds, QKR_COS_SHARED, QKR_FP32,
                                     QKR_ROPE_INTERLEAVED, QKR_BF16, NULL);
    if (rc != QKR_OK) {
        printf("FAIL qknorm_rope_fused: %s\n", qknorm_rope_strerror(rc));
        return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(back, dx, x_bytes, hipMemcpyDeviceToHost));

    double max_abs = 0.0;
    for (int s = 0; s < 2; ++s) {
        if (qkr_oracle_qknorm_rope(x, 0, width, (int64_t)s * H * D, 0, T, H, D, s ? kg : qg,
                                   1e-6f, cs, sn, 2, 0, 0, ref) != 0) {
            printf("FAIL oracle\n");
            return 1;
        }
        for (int t = 0; t < T; ++t)
            for (int i = 0; i < H * D; ++i) {
                const double got = double_of_bf16(back[t * width + s * H * D + i]);
                const double err = fabs(got - ref[t * H * D + i]);
                if (!(err <= 1.6e-2)) {
                    printf("FAIL token %d tensor %d element %d: %g vs %g\n", t, s, i, got,
                           ref[t * H * D + i]);
                    return 1;
                }
                if (err > max_abs)
                    max_abs = err;
            }
    }
    for (int t = 0; t < T; ++t)
        if (memcmp(back + t * width + 2 * H * D, x + t * width + 2 * H * D, (size_t)H * D * 2)) {
            printf("FAIL V of token %d changed\n", t);
            return 1;
        }
    CHECK_HIP(hipFree(dx));
    CHECK_HIP(hipFree(dqg));
    CHECK_HIP(hipFree(dkg));
    CHECK_HIP(hipFree(dc));
    CHECK_HIP(hipFree(ds));
    free(x), free(back), free(qg), free(kg), free(cs), free(sn), free(ref);
    *seed_in = seed;
    printf("qknorm_rope max_abs %.4g\n", max_abs);
    return 0;
}
