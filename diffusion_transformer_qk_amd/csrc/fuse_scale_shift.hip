// fuse_scale_shift.hip -- fused AdaLN modulation (layer norm without affine,
// then (1 + scale) and shift per sample) for gfx950.
//
// The step is the "fuse_scale_shift" (AdaLN) follow-up of TensorRT-Model-
// Connect PR "perf(diffusion): fused qknorm rope Flux 2.0"; the definition
// implemented is the plain AdaLN one (see include/fuse_scale_shift.h).
//
// Work mapping (memory-bound, no matrix cores):
//   * a 256-thread workgroup owns a contiguous run of rows and handles them
//     one at a time: thread j holds vectors j, j+256, ... of the row (8
//     elements each, 16-byte non-temporal loads), VPT vectors per thread, so
//     each load instruction of the workgroup reads one contiguous 4 KB and the
//     whole row sits in registers; the loads of the next two rows are in
//     flight while the current row is reduced;
//   * the modulation vectors (scale and shift, the same channels as the
//     thread's row vectors) stay in registers across the run and are reloaded
//     only when the batch changes, so they cost L2 traffic once per run, not
//     once per row.  Spreading a row over a workgroup rather than a wave keeps
//     these registers small (hidden * 2 tables * bytes / 256 threads);
//   * two passes over the registers: the sum (mean), then the sum of squared
//     deviations (biased variance).  Each is reduced in the wave with DPP
//     inside 16-lane rows and two lane swaps, then across the 4 waves through
//     LDS in a fixed order, so every thread holds the same bits;
//   * y = fma((x - mean) * rsqrt(var + eps), 1 + scale, shift), packed with
//     the round-to-nearest-even converts and stored non-temporally.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "device_common.h"
#include "host_common.h"
#include "fuse_scale_shift.h"

namespace {

using namespace qkr_dev;
using qkr_host::aligned16;
using qkr_host::overlaps;

constexpr int kWaves = 4;
constexpr int kBlock = kWaves * kWave;   // one row per workgroup

struct FssParams {
    const uint16_t* x;
    uint16_t* y;
    const void* scale;
    const void* shift;
    int64_t rows;
    int64_t rows_per_batch;
    int64_t rows_per_block;    // length of each workgroup's run of rows
    int32_t hidden;
    float eps;
};

template <int MOD>
constexpr int mod_vecs() { return MOD == QKR_FP32 ? 2 : 1; }   // 16-byte vectors per 8 entries

template <int MOD>
__device__ __forceinline__ void widen_mod(const u32x4* w, float f[8])
{
    if constexpr (MOD == QKR_FP32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[i] = __uint_as_float(w[0][i]);
            f[4 + i] = __uint_as_float(w[1][i]);
        }
    } else {
        unpack8<MOD == QKR_FP16>(w[0], f);
    }
}

// Issue the row's VPT vector loads; vectors past the row end load the last
// vector again (clamped index, so every load is valid and unconditional) and
// are zeroed by the caller's mask.
template <int VPT>
__device__ __forceinline__ void load_row(const uint16_t* xr, int nvec, u32x4 (&v)[VPT])
{
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        const int i = u * kBlock + threadIdx.x;
        v[u] = load16<true>(xr + (i < nvec ? i : nvec - 1) * kVec);
    }
}

template <int VPT, int MOD, int NV>
__device__ __forceinline__ void load_mods(const FssParams& p, int64_t mrow, int nvec,
                                          u32x4 (&sc)[VPT * NV], u32x4 (&sh)[VPT * NV])
{
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        const int i = u * kBlock + threadIdx.x;
        const int ic = i < nvec ? i : nvec - 1;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int64_t e = mrow + ic * kVec + k * 4;
            if constexpr (MOD == QKR_FP32) {
                sc[u * NV + k] = load16<false>(static_cast<const float*>(p.scale) + e);
                sh[u * NV + k] = load16<false>(static_cast<const float*>(p.shift) + e);
            } else {
                sc[u * NV + k] = load16<false>(static_cast<const uint16_t*>(p.scale) + e);
                sh[u * NV + k] = load16<false>(static_cast<const uint16_t*>(p.shift) + e);
            }
        }
    }
}

// AHEAD: rows whose loads are in flight beyond the one being reduced (1 or 2).
template <int VPT, bool X_FP16, int MOD, int AHEAD>
__global__ __launch_bounds__(kBlock) void fuse_scale_shift_kernel(const FssParams p)
{
    constexpr int NV = mod_vecs<MOD>();
    __shared__ float red[2][kWaves];
    const int tid = threadIdx.x;
    const int C = p.hidden;
    const int nvec = C / kVec;
    const int64_t r0 = (int64_t)blockIdx.x * p.rows_per_block;
    const int64_t r1 = r0 + p.rows_per_block < p.rows ? r0 + p.rows_per_block : p.rows;

    u32x4 v[VPT], vn[VPT], vnn[VPT], sc[VPT * NV], sh[VPT * NV];
    load_row<VPT>(p.x + r0 * C, nvec, v);
    if (AHEAD > 1 && r0 + 1 < r1)
        load_row<VPT>(p.x + (r0 + 1) * C, nvec, vn);
    int64_t batch = r0 / p.rows_per_batch;
    load_mods<VPT, MOD, NV>(p, batch * C, nvec, sc, sh);

    for (int64_t r = r0; r < r1; ++r) {
        if (AHEAD > 1) {
            if (r + 2 < r1)
                load_row<VPT>(p.x + (r + 2) * C, nvec, vnn);
        } else if (r + 1 < r1) {
            load_row<VPT>(p.x + (r + 1) * C, nvec, vn);
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u)
            if (u * kBlock + tid >= nvec)
                v[u] = u32x4{0, 0, 0, 0};

        // pass 1: mean (vectors past the row end hold zeros and add nothing)
        float sum = 0.0f;
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            float f[8];
            unpack8<X_FP16>(v[u], f);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                sum += f[k];
        }
        const float mean = block_sum<kWaves>(sum, red[0]) / (float)C;

        // pass 2: biased variance from the deviations
        float ss = 0.0f;
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            if (u * kBlock + tid < nvec) {
                float f[8];
                unpack8<X_FP16>(v[u], f);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float d = f[k] - mean;
                    ss = __builtin_fmaf(d, d, ss);
                }
            }
        }
        const float rstd = __builtin_amdgcn_rsqf(block_sum<kWaves>(ss, red[1]) / (float)C + p.eps);

        // the row's batch (uniform over the workgroup): reload its modulation
        const int64_t b = r / p.rows_per_batch;
        if (b != batch) {
            batch = b;
            load_mods<VPT, MOD, NV>(p, batch * C, nvec, sc, sh);
        }

        // pass 3: normalise, modulate, round, store
        uint16_t* yr = p.y + r * C;
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int i = u * kBlock + tid;
            if (i < nvec) {
                float f[8], s[8], h[8], o[8];
                unpack8<X_FP16>(v[u], f);
                widen_mod<MOD>(&sc[u * NV], s);
                widen_mod<MOD>(&sh[u * NV], h);
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    o[k] = __builtin_fmaf((f[k] - mean) * rstd, 1.0f + s[k], h[k]);
                store16<true>(yr + i * kVec, pack8<X_FP16>(o));
            }
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            v[u] = vn[u];
            if (AHEAD > 1)
                vn[u] = vnn[u];
        }
    }
}

using FssFn = void (*)(FssParams);

constexpr int kRowsAhead = 2;

template <int VPT, bool XF>
FssFn select_mod(int mod)
{
    if (mod == QKR_FP32)
        return fuse_scale_shift_kernel<VPT, XF, QKR_FP32, kRowsAhead>;
    if (mod == QKR_FP16)
        return fuse_scale_shift_kernel<VPT, XF, QKR_FP16, kRowsAhead>;
    return fuse_scale_shift_kernel<VPT, XF, QKR_BF16, kRowsAhead>;
}

template <int VPT>
FssFn select_x(bool xf, int mod) { return xf ? select_mod<VPT, true>(mod) : select_mod<VPT, false>(mod); }

// Row vectors per thread: ceil(hidden / 8 / 256), 1..4 for hidden <= 8192.
int vectors_per_thread(int hidden) { return (hidden / kVec + kBlock - 1) / kBlock; }

FssFn select_kernel(int vpt, bool xf, int mod)
{
    switch (vpt) {
    case 1: return select_x<1>(xf, mod);
    case 2: return select_x<2>(xf, mod);
    case 3: return select_x<3>(xf, mod);
    default: return select_x<4>(xf, mod);
    }
}

// Rows per workgroup: runs of 3 rows (loads two rows ahead) amortise the
// modulation loads and still leave about 11000 workgroups on a 32K-row call;
// shorter runs for small calls keep the grid large enough to fill the chip
// (measured over 1..32 rows per workgroup and 1..2 rows ahead on 32760 x 5120
// and 4608 x 6144).
int64_t rows_per_block(int64_t rows) { return rows >= 16384 ? 3 : rows >= 4096 ? 2 : 1; }


}  // namespace

extern "C" int dit_fuse_scale_shift(const void* x, void* y, int64_t rows, int32_t hidden,
                                    int64_t rows_per_batch, const void* scale, const void* shift,
                                    int32_t mod_dtype, float eps, int32_t dtype, void* stream)
{
    if (dtype < QKR_BF16 || dtype > QKR_FP32 || mod_dtype < QKR_BF16 || mod_dtype > QKR_FP32)
        return QKR_ERR_ARG;
    if (dtype == QKR_FP32)
        return QKR_ERR_UNSUPPORTED;
    if (hidden < kVec || hidden > FSS_MAX_HIDDEN || hidden % kVec)
        return QKR_ERR_UNSUPPORTED;
    if (!(eps > 0.0f) || !isfinite(eps))
        return QKR_ERR_ARG;
    if (rows < 0 || rows >= QKR_MAX_TOKENS || rows_per_batch < 1)
        return QKR_ERR_SHAPE;
    if (rows == 0)
        return QKR_OK;
    if (!x || !y || !scale || !shift)
        return QKR_ERR_NULL;
    if (!aligned16(x) || !aligned16(y) || !aligned16(scale) || !aligned16(shift))
        return QKR_ERR_ALIGN;
    // y is x itself or disjoint from it, and never overlaps the modulation
    const uint64_t bytes = (uint64_t)rows * (uint64_t)hidden * 2u;
    const uint64_t mod_bytes = (uint64_t)((rows + rows_per_batch - 1) / rows_per_batch) *
                               (uint64_t)hidden * (mod_dtype == QKR_FP32 ? 4u : 2u);
    if ((x != y && overlaps(x, bytes, y, bytes)) || overlaps(y, bytes, scale, mod_bytes) ||
        overlaps(y, bytes, shift, mod_bytes))
        return QKR_ERR_ARG;

    FssParams p;
    p.x = static_cast<const uint16_t*>(x);
    p.y = static_cast<uint16_t*>(y);
    p.scale = scale;
    p.shift = shift;
    p.rows = rows;
    p.rows_per_batch = rows_per_batch;
    p.rows_per_block = rows_per_block(rows);
    p.hidden = hidden;
    p.eps = eps;
    FssFn fn = select_kernel(vectors_per_thread(hidden), dtype == QKR_FP16, mod_dtype);
    void* args[] = {&p};
    const int64_t blocks = (rows + p.rows_per_block - 1) / p.rows_per_block;
    hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)blocks),
                                     dim3(kBlock), args, 0, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? QKR_OK : QKR_ERR_HIP;
}
