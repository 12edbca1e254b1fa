// fuse_scale_shift.hip -- fused AdaLN modulation (layer norm without affine,
// then (1 + scale) and shift per sample) for gfx950.
//
// The step is the "fuse_scale_shift" (AdaLN) follow-up of TensorRT-Model-
// Connect PR "perf(diffusion): fused qknorm rope Flux 2.0"; the definition
// implemented is the plain AdaLN one (see include/fuse_scale_shift.h).
//
// Work mapping (memory-bound, no matrix cores):
//   * one wave per row: lane j holds the row's 16-byte vectors j, j+64, ...
//     (VPT of them, 8 elements each), loaded non-temporally with buffer
//     loads whose range is the row, so vectors past the row end read as zero
//     and their stores are dropped (no clamped addressing); each load
//     instruction of the wave reads one contiguous 1 KB;
//   * two passes over the registers: the sum (mean), then the sum of squared
//     deviations (biased variance); each is reduced inside the wave only
//     (DPP within 16-lane rows, then the four row totals read as scalars and
//     added as (r0 + r1) + (r2 + r3)), so no workgroup barrier sits between a
//     row's loads and its stores;
//   * modulation: for large calls a workgroup of 4 waves (4 consecutive rows)
//     first stages the scale and shift rows of its first row's batch in LDS
//     (the rows' loads are already in flight) and every wave whose row is in
//     that batch reads them from there; for small calls (a grid that fits
//     the chip at once) each wave is its own workgroup and reads them from
//     L2, which keeps every row's loads in flight without a staging step;
//   * y = fma((x - mean) * rsqrt(var + eps), 1 + scale, shift), packed with
//     the round-to-nearest-even converts, stored non-temporally.
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

constexpr int kBufferNT = 2;                     // buffer cache policy bits: non-temporal
constexpr uint32_t kBufferFlags = 0x00020000u;   // raw buffer resource, 32-bit data

struct FssParams {
    const uint16_t* x;
    uint16_t* y;
    const void* scale;
    const void* shift;
    int64_t rows;
    uint32_t rows_per_batch;   // clamped to rows (same batch of every row), so 32-bit math
    int32_t hidden;
    float eps;
};

template <int MOD>
constexpr int mod_vecs() { return MOD == QKR_FP32 ? 2 : 1; }   // 16-byte vectors per 8 entries

template <int MOD>
constexpr int mod_bytes() { return MOD == QKR_FP32 ? 4 : 2; }

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

// Sum over the wave; every lane gets the same bits.
__device__ __forceinline__ float wave_total(float v)
{
    v += dpp<0xB1>(v);      // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);      // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);     // row_half_mirror
    v += dpp<0x140>(v);     // row_mirror: each 16-lane row's total in all its lanes
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
}

// Sums of squared deviations at or above this keep full fp32 precision;
// below it subnormal squares lose bits, which only matters when eps is below
// it too.
constexpr float kTinySum = 0x1p-100f;

// Whether the plain fp32 statistics of a row are usable: q = var + eps finite
// (false when the sum or the squared deviations overflowed: 16-bit rows with
// values beyond about 1e17, or NaN), and the sum of squared deviations ss
// clear of the subnormal range or swamped by eps.  When true, q is at least
// 2^-113, a normal number, as the hardware reciprocal square root needs.
__device__ __forceinline__ bool stats_in_range(float ss, float q, float eps)
{
    return q <= 0x1.fffffep127f && (ss >= kTinySum || eps >= kTinySum);
}

// Make the compiler forget what v holds, so the fp32 values unpacked from it
// are unpacked again for each pass instead of being kept alive across them.
template <int VPT>
__device__ __forceinline__ void forget_unpacked(u32x4 (&v)[VPT])
{
#pragma unroll
    for (int u = 0; u < VPT; ++u)
        __asm__ volatile("" : "+v"(v[u]));
}

// Vector i (8 entries) of a modulation row, from LDS (staged as 16-byte
// vectors: scale at [0, nvec * NV), shift after it) or from global memory.
template <int MOD, bool FROM_LDS>
__device__ __forceinline__ void mod_entries(const FssParams& p, const u32x4* staged, int nvec,
                                            int64_t mrow, int i, float s[8], float h[8])
{
    constexpr int NV = mod_vecs<MOD>();
    u32x4 ws[NV], wh[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        if constexpr (FROM_LDS) {
            ws[k] = staged[i * NV + k];
            wh[k] = staged[nvec * NV + i * NV + k];
        } else {
            const int64_t e = mrow + (int64_t)i * kVec + k * 4;   // entries
            if constexpr (MOD == QKR_FP32) {
                ws[k] = load16<false>(static_cast<const float*>(p.scale) + e);
                wh[k] = load16<false>(static_cast<const float*>(p.shift) + e);
            } else {
                ws[k] = load16<false>(static_cast<const uint16_t*>(p.scale) + e);
                wh[k] = load16<false>(static_cast<const uint16_t*>(p.shift) + e);
            }
        }
    }
    widen_mod<MOD>(ws, s);
    widen_mod<MOD>(wh, h);
}

template <int VPT, bool X_FP16, int MOD, bool FROM_LDS, bool FULL>
__device__ __forceinline__ void modulate_store(const FssParams& p, __amdgpu_buffer_rsrc_t yr,
                                               const u32x4 (&v)[VPT], const u32x4* staged, int nvec,
                                               int64_t mrow, float mean, float rstd)
{
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        const int i = u * kWave + lane;
        if (FULL || i < nvec) {
            float f[8], s[8], h[8], o[8];
            unpack8<X_FP16>(v[u], f);
            mod_entries<MOD, FROM_LDS>(p, staged, nvec, mrow, i, s, h);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                o[k] = __builtin_fmaf((f[k] - mean) * rstd, 1.0f + s[k], h[k]);
            __builtin_amdgcn_raw_buffer_store_b128(pack8<X_FP16>(o), yr, i * 16, 0, kBufferNT);
        }
    }
}

// A row whose plain fp32 statistics are out of range (stats_in_range; the
// branch is wave-uniform): with e the binary exponent of the row's largest
// |x|, recompute mean and variance on x * 2^-e (an exact power-of-two
// scaling, every term <= 1 in magnitude) and normalise x * 2^-e with them,
// since (x - mean) / sqrt(var + eps) equals (x 2^-e - mean_e) / sqrt(var_e +
// eps 2^-2e).  If eps 2^-2e overflows, the variance is below eps by more than
// 2^128 and the plain mean with 1 / sqrt(eps) is exact to fp32.  Nothing of
// the row is written yet, so this path reads it again from memory (a vector
// at a time, the same vectors and order as the register passes) and leaves
// the registers of the common path free.
template <int VPT, bool X_FP16, int MOD>
__device__ __forceinline__ void rescaled_row(const FssParams& p, int64_t r, const u32x4* staged,
                                             bool from_lds, int64_t mrow, float mean)
{
    const int lane = threadIdx.x % kWave;
    const int C = p.hidden;
    const int nvec = C / kVec;
    const int row_bytes = C * 2;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.x + r * C), 0, row_bytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t yr =
        __builtin_amdgcn_make_buffer_rsrc(p.y + r * C, 0, row_bytes, kBufferFlags);
    // vectors past the row end read as zero (buffer range), like the loads
    // of the register passes
    float m = 0.0f;
#pragma unroll 1
    for (int u = 0; u < VPT; ++u) {
        float f[8];
        unpack8<X_FP16>(__builtin_amdgcn_raw_buffer_load_b128(xr, (u * kWave + lane) * 16, 0, 0), f);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            m = fmaxf(m, fabsf(f[k]));
    }
    const int e = __builtin_amdgcn_frexp_expf(wave_max(m));
    const float eps_s = __builtin_amdgcn_ldexpf(p.eps, -2 * e);
    float mean_s = mean, rstd = rsqrt_full_range(p.eps);
    int shift = 0;
    if (eps_s <= 0x1.fffffep127f) {
        shift = e;
        float sum = 0.0f;
#pragma unroll 1
        for (int u = 0; u < VPT; ++u) {
            float f[8];
            unpack8<X_FP16>(__builtin_amdgcn_raw_buffer_load_b128(xr, (u * kWave + lane) * 16, 0, 0), f);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                sum += __builtin_amdgcn_ldexpf(f[k], -shift);
        }
        mean_s = wave_total(sum) / (float)C;
        float ss = 0.0f;
#pragma unroll 1
        for (int u = 0; u < VPT; ++u) {
            if (u * kWave + lane < nvec) {
                float f[8];
                unpack8<X_FP16>(__builtin_amdgcn_raw_buffer_load_b128(xr, (u * kWave + lane) * 16, 0, 0), f);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float d = __builtin_amdgcn_ldexpf(f[k], -shift) - mean_s;
                    ss = __builtin_fmaf(d, d, ss);
                }
            }
        }
        // a constant row of large values has var_e = 0 and eps 2^-2e may
        // underflow to 0: the floor keeps rstd finite for its zero deviations
        rstd = __builtin_amdgcn_rsqf(fmaxf(wave_total(ss) / (float)C + eps_s, 0x1p-126f));
    }
#pragma unroll 1
    for (int u = 0; u < VPT; ++u) {
        const int i = u * kWave + lane;
        if (i < nvec) {
            float f[8], sc[8], sh[8], o[8];
            unpack8<X_FP16>(__builtin_amdgcn_raw_buffer_load_b128(xr, i * 16, 0, 0), f);
            if (from_lds)
                mod_entries<MOD, true>(p, staged, nvec, 0, i, sc, sh);
            else
                mod_entries<MOD, false>(p, staged, nvec, mrow, i, sc, sh);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                o[k] = __builtin_fmaf((__builtin_amdgcn_ldexpf(f[k], -shift) - mean_s) * rstd,
                                      1.0f + sc[k], sh[k]);
            __builtin_amdgcn_raw_buffer_store_b128(pack8<X_FP16>(o), yr, i * 16, 0, 0);
        }
    }
}

// WAVES == 1: one row per workgroup, modulation from L2.  WAVES > 1: WAVES
// consecutive rows per workgroup, the first row's batch staged in LDS.
// FULL: the row is exactly VPT vectors per lane (hidden = 512 * VPT), so no
// lane needs the row-end masks (a masked store costs an exec-mask branch per
// vector, measured at 3% on 32760 x 5120).
// Occupancy the register allocation must keep (waves per SIMD).  Staging
// kernels: what their LDS allows (4 workgroups per CU up to 40 KB of staged
// modulation, 2 above 48 KB); one-row kernels: as many as the row's registers
// leave room for without spilling.
template <int VPT, int WAVES>
constexpr int min_waves_per_simd()
{
    if constexpr (WAVES > 1)
        return VPT <= 12 ? 4 : 2;
    else
        return VPT <= 10 ? 7 : VPT <= 12 ? 6 : 5;
}

template <int VPT, bool X_FP16, int MOD, int WAVES, bool FULL>
__global__ __launch_bounds__(WAVES * kWave, (min_waves_per_simd<VPT, WAVES>()))
void fuse_scale_shift_kernel(const FssParams p)
{
    constexpr int NV = mod_vecs<MOD>();
    extern __shared__ u32x4 staged[];        // WAVES > 1: [2][nvec * NV]
    const int lane = threadIdx.x % kWave;
    const int C = p.hidden;
    const int nvec = C / kVec;
    const int64_t first = (int64_t)blockIdx.x * WAVES;
    // the wave's row, made visibly wave-uniform so the buffer resources built
    // from it live in scalar registers
    const int64_t r = first + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const bool active = r < p.rows;
    const int row_bytes = C * 2;

    // the row's loads first: nothing they need waits on the staging below
    u32x4 v[VPT];
    if (active) {
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(p.x + r * C), 0, row_bytes, kBufferFlags);
#pragma unroll
        for (int u = 0; u < VPT; ++u)
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(xr, (u * kWave + lane) * 16, 0, kBufferNT);
    }
    const uint32_t staged_batch = (uint32_t)first / p.rows_per_batch;
    if constexpr (WAVES > 1) {
        const int64_t off = (int64_t)staged_batch * C * mod_bytes<MOD>();
        const char* sc = static_cast<const char*>(p.scale) + off;
        const char* sh = static_cast<const char*>(p.shift) + off;
        // the staging loads are issued in groups of up to 4 per table before
        // their writes, so the workgroup waits for one or two L2 round trips
        // rather than one per vector (measured: 125 -> 116 us on 32760 x 5120)
        constexpr int kPer = (VPT * kWave * NV + WAVES * kWave - 1) / (WAVES * kWave);
        constexpr int kGroup = kPer < 4 ? kPer : 4;
#pragma unroll
        for (int j0 = 0; j0 < kPer; j0 += kGroup) {
            u32x4 ws[kGroup], wh[kGroup];
#pragma unroll
            for (int j = 0; j < kGroup; ++j) {
                const int i = threadIdx.x + (j0 + j) * WAVES * kWave;
                if (j0 + j < kPer && i < nvec * NV) {
                    ws[j] = load16<false>(sc + i * 16);
                    wh[j] = load16<false>(sh + i * 16);
                }
            }
#pragma unroll
            for (int j = 0; j < kGroup; ++j) {
                const int i = threadIdx.x + (j0 + j) * WAVES * kWave;
                if (j0 + j < kPer && i < nvec * NV) {
                    staged[i] = ws[j];
                    staged[nvec * NV + i] = wh[j];
                }
            }
        }
        __syncthreads();
    }
    if (!active)
        return;

    // pass 1: mean (vectors past the row end read as zero and add nothing)
    float sum = 0.0f;
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        float f[8];
        unpack8<X_FP16>(v[u], f);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            sum += f[k];
    }
    const float mean = wave_total(sum) / (float)C;
    forget_unpacked(v);

    // pass 2: biased variance from the deviations (row vectors only)
    float ss = 0.0f;
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        if (FULL || u * kWave + lane < nvec) {
            float f[8];
            unpack8<X_FP16>(v[u], f);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float d = f[k] - mean;
                ss = __builtin_fmaf(d, d, ss);
            }
        }
    }
    const float ss_row = wave_total(ss);
    const float q = ss_row / (float)C + p.eps;
    forget_unpacked(v);

    // pass 3: normalise, modulate, round, store
    const __amdgpu_buffer_rsrc_t yr =
        __builtin_amdgcn_make_buffer_rsrc(p.y + r * C, 0, row_bytes, kBufferFlags);
    const uint32_t batch = (uint32_t)r / p.rows_per_batch;
    const bool from_lds = WAVES > 1 && batch == staged_batch;
    const int64_t mrow = (int64_t)batch * C;
    if (__builtin_expect(stats_in_range(ss_row, q, p.eps), 1)) {
        const float rstd = __builtin_amdgcn_rsqf(q);
        if (from_lds)
            modulate_store<VPT, X_FP16, MOD, true, FULL>(p, yr, v, staged, nvec, 0, mean, rstd);
        else
            modulate_store<VPT, X_FP16, MOD, false, FULL>(p, yr, v, staged, nvec, mrow, mean, rstd);
    } else {
        rescaled_row<VPT, X_FP16, MOD>(p, r, staged, from_lds, mrow, mean);
    }
}

using FssFn = void (*)(FssParams);

// Rows from which workgroups of 4 rows stage the modulation in LDS; below it
// one-row workgroups read it from L2.  Measured at widths 5120 and 6144: the
// one-row schedule wins up to about 6000 rows (23.0 vs 26.0 us at 6144 x 5120,
// 17.5 vs 26 us at 4608 x 6144), staging wins from 8192 rows on (33.7 vs
// 41.1 us at 8192 x 5120, 116 vs 143 us at 32760 x 5120).
constexpr int64_t kStageFromRows = 8192;
constexpr int kStageWaves = 4;

template <int VPT, bool XF, int WAVES, bool FULL>
FssFn select_mod(int mod)
{
    if (mod == QKR_FP32)
        return fuse_scale_shift_kernel<VPT, XF, QKR_FP32, WAVES, FULL>;
    if (mod == QKR_FP16)
        return fuse_scale_shift_kernel<VPT, XF, QKR_FP16, WAVES, FULL>;
    return fuse_scale_shift_kernel<VPT, XF, QKR_BF16, WAVES, FULL>;
}

template <int VPT, bool XF, bool FULL>
FssFn select_waves(int waves, int mod)
{
    return waves > 1 ? select_mod<VPT, XF, kStageWaves, FULL>(mod) : select_mod<VPT, XF, 1, FULL>(mod);
}

template <int VPT>
FssFn select_x(bool xf, bool full, int waves, int mod)
{
    if (full)
        return xf ? select_waves<VPT, true, true>(waves, mod) : select_waves<VPT, false, true>(waves, mod);
    return xf ? select_waves<VPT, true, false>(waves, mod) : select_waves<VPT, false, false>(waves, mod);
}

// Row vectors per lane: ceil(hidden / 8 / 64) rounded up to an even count,
// 2..16 for hidden <= 8192 (the extra vectors of a rounded-up count read as
// zero and store nothing).
int vectors_per_lane(int hidden)
{
    const int v = (hidden / kVec + kWave - 1) / kWave;
    return v + (v & 1);
}

FssFn select_kernel(int hidden, bool xf, int waves, int mod)
{
    const int vpl = vectors_per_lane(hidden);
    const bool full = hidden == vpl * kWave * kVec;
    switch (vpl) {
    case 2: return select_x<2>(xf, full, waves, mod);
    case 4: return select_x<4>(xf, full, waves, mod);
    case 6: return select_x<6>(xf, full, waves, mod);
    case 8: return select_x<8>(xf, full, waves, mod);
    case 10: return select_x<10>(xf, full, waves, mod);
    case 12: return select_x<12>(xf, full, waves, mod);
    case 14: return select_x<14>(xf, full, waves, mod);
    default: return select_x<16>(xf, full, waves, mod);
    }
}

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
    p.rows_per_batch = (uint32_t)(rows_per_batch < rows ? rows_per_batch : rows);
    p.hidden = hidden;
    p.eps = eps;
    const int waves = rows >= kStageFromRows ? kStageWaves : 1;
    FssFn fn = select_kernel(hidden, dtype == QKR_FP16, waves, mod_dtype);
    // staged scale and shift rows: 2 * hidden * 4 bytes at most (64 KB at 8192)
    const size_t lds = waves > 1 ? (size_t)2 * hidden * (mod_dtype == QKR_FP32 ? 4 : 2) : 0;
    void* args[] = {&p};
    const int64_t blocks = (rows + waves - 1) / waves;
    hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)blocks),
                                     dim3(waves * kWave), args, lds,
                                     static_cast<hipStream_t>(stream));
    return err == hipSuccess ? QKR_OK : QKR_ERR_HIP;
}
