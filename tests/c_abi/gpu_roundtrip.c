/* Plain C use of the library on the GPU, with no Python and no torch: HIP's C
 * runtime API for memory, the public header for the call, and the CPU oracle
 * (test infrastructure) for the check.  Built with gcc and run by
 * tests/test_gpu_c_roundtrip.py.
 *
 * A fused QKV bf16 buffer of 37 tokens x 3 x 3 heads x 128 goes to the GPU;
 * qknorm_rope_fused runs in place with one shared fp32 cos/sin row per token
 * (interleaved pairs); the result comes back and every Q and K element is
 * compared with the fp64 oracle (max_abs <= 1.6e-2, bf16), and every V element
 * bit for bit with the input.  Prints "ok max_abs <value>" and exits 0. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "qknorm_rope.h"

/* the oracle's entry point (libqkr_oracle.so; dtype codes bf16 0, fp32 2) */
int qkr_oracle_qknorm_rope(const uint16_t* x, int x_dtype, int64_t row_stride, int64_t col0,
                           int64_t t_begin, int64_t t_end, int32_t heads, int32_t head_dim,
                           const float* gamma, float eps, const void* cos, const void* sin,
                           int cos_dtype, int cos_layout, int style, double* out);

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

int main(void)
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
    uint32_t seed = 20251202u;
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
    printf("ok max_abs %.4g\n", max_abs);
    return 0;
}
