// group_norm_silu.hip -- fused group norm + per-channel affine + SiLU for
// gfx950 (the VAE step; definition in include/group_norm_silu.h).
//
// A group (Cg channels x spatial elements of one sample) is one contiguous
// run of memory.  Work is cut into chunks, one 256-thread workgroup per
// (group, chunk), each thread holding VPT 16-byte vectors (chunks of 16384
// elements, or 8192 / 4096 when that is needed to give a small call enough
// workgroups):
//   * one chunk per group: a single kernel keeps the chunk in registers,
//     reduces mean and biased variance in two passes and writes y (one read,
//     one write);
//   * several chunks, large calls (gn_lagged_kernel): workgroup b reduces
//     chunk b to (mean, sum of squared deviations) and publishes it as one
//     64-bit word, then writes the output of chunk b - lag.  It waits until
//     every word of that chunk's group is published (all belong to lower
//     workgroups; one still missing after a short wait is reduced by the
//     waiter itself), combines them and re-reads the chunk.  Workgroups are
//     dealt to the dies in turn and lag is a multiple of 8, so the re-read
//     runs on the die that read the chunk a few MB earlier and comes from its
//     L2: HBM sees x once;
//   * several chunks, small calls: gn_stats_kernel writes every chunk's
//     partial statistics to the workspace, then gn_apply_kernel re-reads
//     each chunk (two launches; x is read twice).
//   Both combine a group's partials with the pairwise update (sum n_i m_i / N,
//   then sum M2_i + n_i (m_i - m)^2) in the same fixed order, so every
//   workgroup of a group gets the same statistics and both schedules give
//   identical bits.
// Per vector of 8 elements (spatial is a multiple of 8, so a vector never
// straddles channels): t = fma(x - mean, rstd * gamma[c], beta[c]),
// y = t * rcp(1 + exp(-t)), packed with round-to-nearest-even.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "device_common.h"
#include "host_common.h"
#include "group_norm_silu.h"

namespace {

using namespace qkr_dev;
using qkr_host::aligned16;
using qkr_host::overlaps;

constexpr int kWaves = 4;
constexpr int kBlock = kWaves * kWave;
constexpr int kVptMax = 8;                                      // vectors per thread, largest chunk
constexpr int64_t kChunkMax = (int64_t)kBlock * kVptMax * kVec; // 16384 elements

// Elements in a chunk of VPT vectors per thread.
template <int VPT>
constexpr int64_t chunk_elems() { return (int64_t)kBlock * VPT * kVec; }

struct GnParams {
    const uint16_t* x;
    uint16_t* y;
    const void* gamma;
    const void* beta;
    float* partial;          // [pairs][chunks][2]: chunk mean, sum of squared deviations
    int64_t group_size;      // Cg * spatial elements, a multiple of 8, < 2^31
    int32_t spatial;
    int32_t cg;
    int32_t groups;
    int32_t chunks;          // chunks per group
    float eps;
    int64_t total;           // chunks of the call (pairs * chunks)
    int64_t lag;             // lagged schedule: chunks between a reduction and an output
    int32_t wait_polls;      // lagged schedule: polls of a word before reducing it here
};

// Vectors valid in chunk k of a group.
template <int VPT>
__device__ __forceinline__ int chunk_vectors(const GnParams& p, int k)
{
    constexpr int64_t kChunk = chunk_elems<VPT>();
    const int64_t left = p.group_size - (int64_t)k * kChunk;
    return (int)((left < kChunk ? left : kChunk) / kVec);
}

// Load the chunk's vectors; thread vectors past `nv` reload the last valid
// vector (clamped, so every load is unconditional) and are zeroed.
template <bool NT, int VPT>
__device__ __forceinline__ void load_chunk(const uint16_t* base, int nv, u32x4 (&v)[VPT])
{
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        const int i = u * kBlock + threadIdx.x;
        const u32x4 t = load16<NT>(base + (int64_t)(i < nv ? i : nv - 1) * kVec);
        v[u] = i < nv ? t : u32x4{0, 0, 0, 0};
    }
}

// Make the compiler forget what v holds, so the fp32 values unpacked from it
// are not kept alive (64 registers) from one pass over the chunk to the next
// but unpacked again from the 32 packed registers.
template <int VPT>
__device__ __forceinline__ void forget_unpacked(u32x4 (&v)[VPT])
{
#pragma unroll
    for (int u = 0; u < VPT; ++u)
        __asm__ volatile("" : "+v"(v[u]));
}

// Mean and sum of squared deviations of the chunk held in v (nv valid vectors).
template <bool X_FP16, int VPT>
__device__ __forceinline__ void chunk_moments(u32x4 (&v)[VPT], int nv, float* red0,
                                              float* red1, float& mean, float& m2)
{
    float sum = 0.0f;
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        float f[8];
        unpack8<X_FP16>(v[u], f);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            sum += f[k];
    }
    mean = block_sum<kWaves>(sum, red0) / (float)(nv * kVec);
    forget_unpacked(v);
    float ss = 0.0f;
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        if (u * kBlock + (int)threadIdx.x < nv) {
            float f[8];
            unpack8<X_FP16>(v[u], f);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float d = f[k] - mean;
                ss = __builtin_fmaf(d, d, ss);
            }
        }
    }
    m2 = block_sum<kWaves>(ss, red1);
    forget_unpacked(v);
}

// chunk_moments over a chunk read from memory one vector at a time (the same
// vectors, sums and order, so the same bits), for callers that cannot spare
// registers for the whole chunk.
template <bool X_FP16, int VPT>
__device__ __forceinline__ void chunk_moments_streamed(const uint16_t* base, int nv, float* red0,
                                                       float* red1, float& mean, float& m2)
{
    float sum = 0.0f;
#pragma unroll 1
    for (int u = 0; u < VPT; ++u) {
        const int i = u * kBlock + threadIdx.x;
        const u32x4 t = load16<false>(base + (int64_t)(i < nv ? i : nv - 1) * kVec);
        float f[8];
        unpack8<X_FP16>(i < nv ? t : u32x4{0, 0, 0, 0}, f);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            sum += f[k];
    }
    mean = block_sum<kWaves>(sum, red0) / (float)(nv * kVec);
    float ss = 0.0f;
#pragma unroll 1
    for (int u = 0; u < VPT; ++u) {
        const int i = u * kBlock + threadIdx.x;
        if (i < nv) {
            float f[8];
            unpack8<X_FP16>(load16<false>(base + (int64_t)i * kVec), f);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float d = f[k] - mean;
                ss = __builtin_fmaf(d, d, ss);
            }
        }
    }
    m2 = block_sum<kWaves>(ss, red1);
}

// ------------------------------------------------------------ out-of-range statistics
//
// The plain fp32 statistics overflow for 16-bit groups whose values exceed
// about 1e17 (squared deviations) or 1e34 (sums), and lose bits to subnormal
// squares when the sums fall below kTinySum while eps is below it too.  Such
// chunks and groups are recomputed on x * 2^-e, e the binary exponent of the
// largest magnitude involved (an exact power-of-two scaling that brings every
// term to at most 1), and normalised in that scale: (x - mean) / sqrt(var +
// eps) equals (x 2^-e - mean_e) / sqrt(var_e + eps 2^-2e).  If eps 2^-2e
// overflows, the variance is below eps by more than 2^128 and the plain mean
// with 1 / sqrt(eps) is exact to fp32.
constexpr float kTinySum = 0x1p-100f;
constexpr float kFltMax = 0x1.fffffep127f;

__device__ __forceinline__ bool moments_in_range(float m2, float eps)
{
    // false for an overflowed (inf) or NaN sum of squared deviations too
    return m2 <= kFltMax && (m2 >= kTinySum || eps >= kTinySum);
}

// A group's normalisation: t = (x 2^-shift - mean) * rstd * gamma + beta.
struct GroupStats {
    float mean;
    float rstd;
    int shift;
};

// Statistics of a chunk (nv valid vectors at base) on x * 2^-e, read from
// memory a vector at a time: e the exponent of the chunk's largest |x|,
// mean_s and m2_s (sum of squared deviations) of the rescaled values.  Uses
// three slots (red[0..2]); every thread gets the same bits.
template <bool X_FP16, int VPT>
__device__ __forceinline__ void chunk_moments_rescaled(const uint16_t* base, int nv, float (*red)[kWaves],
                                                    int& e, float& mean_s, float& m2_s)
{
    float m = 0.0f;
#pragma unroll 1
    for (int u = 0; u < VPT; ++u) {
        const int i = u * kBlock + threadIdx.x;
        if (i < nv) {
            float f[8];
            unpack8<X_FP16>(load16<false>(base + (int64_t)i * kVec), f);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                m = fmaxf(m, fabsf(f[k]));
        }
    }
    e = __builtin_amdgcn_frexp_expf(block_max<kWaves>(m, red[0]));
    float sum = 0.0f;
#pragma unroll 1
    for (int u = 0; u < VPT; ++u) {
        const int i = u * kBlock + threadIdx.x;
        if (i < nv) {
            float f[8];
            unpack8<X_FP16>(load16<false>(base + (int64_t)i * kVec), f);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                sum += __builtin_amdgcn_ldexpf(f[k], -e);
        }
    }
    mean_s = block_sum<kWaves>(sum, red[1]) / (float)(nv * kVec);
    float ss = 0.0f;
#pragma unroll 1
    for (int u = 0; u < VPT; ++u) {
        const int i = u * kBlock + threadIdx.x;
        if (i < nv) {
            float f[8];
            unpack8<X_FP16>(load16<false>(base + (int64_t)i * kVec), f);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float d = __builtin_amdgcn_ldexpf(f[k], -e) - mean_s;
                ss = __builtin_fmaf(d, d, ss);
            }
        }
    }
    m2_s = block_sum<kWaves>(ss, red[2]);
}

// A chunk's published partial: (mean, sum of squared deviations) as two fp32
// words, or, for a chunk whose plain sum is out of range, (mean, -sd) with sd
// the chunk's standard deviation (always a finite fp32 for finite data; the
// sign bit of the second word marks this form).  `mean` and `m2` are the
// plain statistics already computed; the chunk is read again only when they
// are out of range.
template <bool X_FP16, int VPT>
__device__ __forceinline__ f32x2 chunk_partial(const GnParams& p, const uint16_t* base, int nv,
                                               float mean, float m2, float (*red)[kWaves])
{
    if (__builtin_expect(moments_in_range(m2, p.eps), 1))
        return f32x2{mean, m2};
    int e;
    float mean_s, m2_s;
    chunk_moments_rescaled<X_FP16, VPT>(base, nv, red, e, mean_s, m2_s);
    if (!(__builtin_amdgcn_ldexpf(p.eps, -2 * e) <= kFltMax))
        return f32x2{mean, m2};     // the chunk's variance is nothing next to eps
    const float sd = __builtin_amdgcn_ldexpf(__builtin_sqrtf(m2_s / (float)(nv * kVec)), e);
    return f32x2{__builtin_amdgcn_ldexpf(mean_s, e), -sd};
}

template <int PARAM>
__device__ __forceinline__ float param(const void* table, int c)
{
    if constexpr (PARAM == QKR_FP32) {
        return static_cast<const float*>(table)[c];
    } else {
        const uint16_t h = static_cast<const uint16_t*>(table)[c];
        if constexpr (PARAM == QKR_FP16)
            return (float)__builtin_bit_cast(_Float16, h);
        else
            return __uint_as_float((uint32_t)h << 16);
    }
}

// Normalise, apply the channel affine and SiLU to the chunk, store it:
// t = fma(x 2^-shift - mean, a[c], beta[c]) with a[c] = rstd * gamma[c]
// formed once per channel, then y = t * rcp(1 + exp(-t)).  When a channel
// holds at least a chunk, the chunk covers at most two channels: their
// coefficients come from uniform addresses once, and each vector picks one by
// comparing its offset with the channel boundary.  Otherwise each vector
// divides its offset by spatial to find its channel.  The chunk comes from
// the registers v (st.shift == 0) or, for statistics taken in a rescaled
// form (RESCALED), from memory a vector at a time: it is not written yet, and
// each thread reads a vector before it writes it.
template <bool X_FP16, int PARAM, int VPT, bool RESCALED>
__device__ __forceinline__ void chunk_apply_as(const GnParams& p, int64_t q, int k, int nv,
                                               const u32x4 (&v)[VPT], const GroupStats& st)
{
    constexpr int64_t kChunk = chunk_elems<VPT>();
    const float mean = st.mean, rstd = st.rstd;
    uint16_t* yq = p.y + q * p.group_size + (int64_t)k * kChunk;
    const uint16_t* xq = p.x + q * p.group_size + (int64_t)k * kChunk;
    const int c0 = (int)(q % p.groups) * p.cg;
    const uint32_t e0 = (uint32_t)(k * kChunk);           // chunk offset in the group, < 2^31
    const uint32_t sp = (uint32_t)p.spatial;
    const bool two = sp >= (uint32_t)kChunk;
    float a0 = 0.0f, b0 = 0.0f, a1 = 0.0f, b1 = 0.0f;
    uint32_t boundary = 0;
    if (two) {
        const uint32_t ci = e0 / sp;                       // the chunk's first channel in the group
        boundary = (ci + 1) * sp;                          // where the next channel starts (<= group size)
        const int c = c0 + (int)ci;
        const int cn = ci + 1 < (uint32_t)p.cg ? c + 1 : c;
        a0 = rstd * param<PARAM>(p.gamma, c);
        b0 = param<PARAM>(p.beta, c);
        a1 = rstd * param<PARAM>(p.gamma, cn);
        b1 = param<PARAM>(p.beta, cn);
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        const int i = u * kBlock + threadIdx.x;
        if (i < nv) {
            const uint32_t e = e0 + (uint32_t)i * kVec;
            float a, b;
            if (two) {
                const bool next = e >= boundary;
                a = next ? a1 : a0;
                b = next ? b1 : b0;
            } else {
                const int c = c0 + (int)(e / sp);
                a = rstd * param<PARAM>(p.gamma, c);
                b = param<PARAM>(p.beta, c);
            }
            float f[8], o[8];
            if constexpr (RESCALED) {
                unpack8<X_FP16>(load16<false>(xq + (int64_t)i * kVec), f);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    f[j] = __builtin_amdgcn_ldexpf(f[j], -st.shift);
            } else {
                unpack8<X_FP16>(v[u], f);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float t = __builtin_fmaf(f[j] - mean, a, b);
                o[j] = t * __builtin_amdgcn_rcpf(1.0f + __expf(-t));
            }
            store16<true>(yq + (int64_t)i * kVec, pack8<X_FP16>(o));
        }
    }
}

template <bool X_FP16, int PARAM, int VPT>
__device__ __forceinline__ void chunk_apply(const GnParams& p, int64_t q, int k, int nv,
                                            const u32x4 (&v)[VPT], const GroupStats& st)
{
    if (__builtin_expect(st.shift == 0, 1))
        chunk_apply_as<X_FP16, PARAM, VPT, false>(p, q, k, nv, v, st);
    else
        chunk_apply_as<X_FP16, PARAM, VPT, true>(p, q, k, nv, v, st);
}

// 1 / sqrt(var + eps) in the rescaled form, with the same floor: a group of
// equal values has var_e = 0, and eps 2^-2e can underflow to 0 when e is
// large; the floor keeps rstd finite for the group's zero deviations.
__device__ __forceinline__ float rescaled_rstd(float var_s, float eps_s)
{
    return __builtin_amdgcn_rsqf(fmaxf(var_s + eps_s, 0x1p-126f));
}

// One chunk per group: statistics and output from one read.
template <bool X_FP16, int PARAM>
__global__ __launch_bounds__(kBlock) void gn_single_kernel(const GnParams p)
{
    __shared__ float red[5][kWaves];
    const int64_t q = blockIdx.x;
    const int nv = chunk_vectors<kVptMax>(p, 0);
    u32x4 v[kVptMax];
    const uint16_t* const base = p.x + q * p.group_size;
    load_chunk<true>(base, nv, v);
    float mean, m2;
    chunk_moments<X_FP16>(v, nv, red[0], red[1], mean, m2);
    // in range, m2 / group_size + eps >= 2^-114: normal, as the hardware
    // reciprocal square root needs
    GroupStats st = {mean, __builtin_amdgcn_rsqf(m2 / (float)p.group_size + p.eps), 0};
    if (__builtin_expect(!moments_in_range(m2, p.eps), 0)) {
        int e;
        float mean_s, m2_s;
        chunk_moments_rescaled<X_FP16, kVptMax>(base, nv, red + 2, e, mean_s, m2_s);
        const float eps_s = __builtin_amdgcn_ldexpf(p.eps, -2 * e);
        if (eps_s <= kFltMax)
            st = GroupStats{mean_s, rescaled_rstd(m2_s / (float)p.group_size, eps_s), e};
        else    // the plain mean stands; the variance is nothing next to eps
            st.rstd = rsqrt_full_range(m2 / (float)p.group_size + p.eps);
    }
    chunk_apply<X_FP16, PARAM>(p, q, 0, nv, v, st);
}

// Several chunks, pass 1: per-chunk mean and sum of squared deviations.
template <bool X_FP16, int VPT>
__global__ __launch_bounds__(kBlock) void gn_stats_kernel(const GnParams p)
{
    __shared__ float red[5][kWaves];
    const int64_t q = blockIdx.x / p.chunks;
    const int k = (int)(blockIdx.x % p.chunks);
    const int nv = chunk_vectors<VPT>(p, k);
    u32x4 v[VPT];
    const uint16_t* const base = p.x + q * p.group_size + (int64_t)k * chunk_elems<VPT>();
    load_chunk<false>(base, nv, v);
    float mean, m2;
    chunk_moments<X_FP16>(v, nv, red[0], red[1], mean, m2);
    const f32x2 part = chunk_partial<X_FP16, VPT>(p, base, nv, mean, m2, red + 2);
    if (threadIdx.x == 0)
        *reinterpret_cast<f32x2*>(p.partial + 2 * (q * p.chunks + k)) = part;
}

// True when a partial is in the (mean, -sd) form of chunk_partial.
__device__ __forceinline__ bool rescaled_form(float second) { return (__float_as_uint(second) >> 31) != 0; }

// Partial (mean, m2 or -sd) of n elements as (mean, sd).
__device__ __forceinline__ f32x2 mean_sd(f32x2 w, float n)
{
    return rescaled_form(w[1]) ? f32x2{w[0], -w[1]} : f32x2{w[0], __builtin_sqrtf(w[1] / n)};
}

// combine_partials for a group whose plain combine is out of range, or that
// holds a partial in the (mean, -sd) form: with e the exponent of the largest
// |mean_i| or sd_i, the group mean and variance of x * 2^-e from
// sum n_i m_i 2^-e / N and sum n_i ((sd_i 2^-e)^2 + (m_i 2^-e - mean)^2) / N,
// every term at most 1 in magnitude.  Three slots (red[0..2]).
template <int VPT>
__device__ __forceinline__ GroupStats combine_rescaled(const GnParams& p, const float* part,
                                                       f32x2 first, float (*red)[kWaves])
{
    constexpr int64_t kChunk = chunk_elems<VPT>();
    const float last_n = (float)(p.group_size - (int64_t)(p.chunks - 1) * kChunk);
    const int i0 = threadIdx.x;
    const bool has0 = i0 < p.chunks;
    const float n0 = i0 == p.chunks - 1 ? last_n : (float)kChunk;
    const f32x2 a0 = mean_sd(first, n0);
    float mx = has0 ? fmaxf(fabsf(a0[0]), a0[1]) : 0.0f;
    for (int i = i0 + kBlock; i < p.chunks; i += kBlock) {
        const float n_i = i == p.chunks - 1 ? last_n : (float)kChunk;
        const f32x2 a = mean_sd(f32x2{part[2 * i], part[2 * i + 1]}, n_i);
        mx = fmaxf(mx, fmaxf(fabsf(a[0]), a[1]));
    }
    const int e = __builtin_amdgcn_frexp_expf(block_max<kWaves>(mx, red[0]));
    float s = has0 ? n0 * __builtin_amdgcn_ldexpf(a0[0], -e) : 0.0f;
    for (int i = i0 + kBlock; i < p.chunks; i += kBlock) {
        const float n_i = i == p.chunks - 1 ? last_n : (float)kChunk;
        s = __builtin_fmaf(n_i, __builtin_amdgcn_ldexpf(part[2 * i], -e), s);
    }
    const float mean_s = block_sum<kWaves>(s, red[1]) / (float)p.group_size;
    float v = 0.0f;
    if (has0) {
        const float sd = __builtin_amdgcn_ldexpf(a0[1], -e);
        const float d = __builtin_amdgcn_ldexpf(a0[0], -e) - mean_s;
        v = n0 * __builtin_fmaf(sd, sd, d * d);
    }
    for (int i = i0 + kBlock; i < p.chunks; i += kBlock) {
        const float n_i = i == p.chunks - 1 ? last_n : (float)kChunk;
        const f32x2 a = mean_sd(f32x2{part[2 * i], part[2 * i + 1]}, n_i);
        const float sd = __builtin_amdgcn_ldexpf(a[1], -e);
        const float d = __builtin_amdgcn_ldexpf(a[0], -e) - mean_s;
        v = __builtin_fmaf(n_i, __builtin_fmaf(sd, sd, d * d), v);
    }
    const float var_s = block_sum<kWaves>(v, red[2]) / (float)p.group_size;
    const float eps_s = __builtin_amdgcn_ldexpf(p.eps, -2 * e);
    if (eps_s <= kFltMax)
        return GroupStats{mean_s, rescaled_rstd(var_s, eps_s), e};
    return GroupStats{__builtin_amdgcn_ldexpf(mean_s, e), rsqrt_full_range(p.eps), 0};
}

// Group statistics from the group's chunk partials `part` ([chunks][2]),
// given this thread's first partial `first` (of chunk threadIdx.x, if there
// is one).  Same order in every workgroup of the group: thread sums over
// i = tid, tid + 256, ..., then the fixed-order workgroup reduction through
// red[0] and red[1].  A partial in the (mean, -sd) form turns the plain sum
// into NaN, so that such a group, like one whose plain combine overflows,
// takes combine_rescaled (slots red[2..4]).
template <int VPT>
__device__ __forceinline__ GroupStats combine_partials(const GnParams& p, const float* part,
                                                       f32x2 first, float (*red)[kWaves])
{
    constexpr int64_t kChunk = chunk_elems<VPT>();
    const float last_n = (float)(p.group_size - (int64_t)(p.chunks - 1) * kChunk);
    const float nan = __builtin_nanf("");
    const int i0 = threadIdx.x;
    const bool has0 = i0 < p.chunks;
    const float n0 = i0 == p.chunks - 1 ? last_n : (float)kChunk;
    float s = has0 ? n0 * (rescaled_form(first[1]) ? nan : first[0]) : 0.0f;
    for (int i = i0 + kBlock; i < p.chunks; i += kBlock) {
        const float n_i = i == p.chunks - 1 ? last_n : (float)kChunk;
        s = __builtin_fmaf(n_i, rescaled_form(part[2 * i + 1]) ? nan : part[2 * i], s);
    }
    const float mean = block_sum<kWaves>(s, red[0]) / (float)p.group_size;
    float m2 = 0.0f;
    if (has0) {
        const float d = first[0] - mean;
        m2 = __builtin_fmaf(n0 * d, d, first[1]);
    }
    for (int i = i0 + kBlock; i < p.chunks; i += kBlock) {
        const float n_i = i == p.chunks - 1 ? last_n : (float)kChunk;
        const float d = part[2 * i] - mean;
        m2 += __builtin_fmaf(n_i * d, d, part[2 * i + 1]);
    }
    const float m2t = block_sum<kWaves>(m2, red[1]);
    const float qv = m2t / (float)p.group_size + p.eps;
    // a NaN mean makes m2t NaN too; a group of up to 2^31 elements can bring
    // m2t / N below the normal range, which the hardware reciprocal square
    // root does not take
    if (__builtin_expect(moments_in_range(m2t, p.eps) && qv <= kFltMax && qv >= 0x1p-126f, 1))
        return GroupStats{mean, __builtin_amdgcn_rsqf(qv), 0};
    return combine_rescaled<VPT>(p, part, first, red + 2);
}

// Several chunks, pass 2: combine the group's partials, write the chunk.
template <bool X_FP16, int PARAM, int VPT>
__global__ __launch_bounds__(kBlock) void gn_apply_kernel(const GnParams p)
{
    constexpr int64_t kChunk = chunk_elems<VPT>();
    __shared__ float red[5][kWaves];
    const int64_t q = blockIdx.x / p.chunks;
    const int k = (int)(blockIdx.x % p.chunks);
    const int nv = chunk_vectors<VPT>(p, k);
    const float* part = p.partial + 2 * q * p.chunks;
    // This thread's first partial is read before the chunk, so that the
    // combine (two workgroup reductions) runs while the chunk is in flight.
    f32x2 first = {0.0f, 0.0f};
    if ((int)threadIdx.x < p.chunks)
        first = *reinterpret_cast<const f32x2*>(part + 2 * threadIdx.x);
    u32x4 v[VPT];
    load_chunk<true>(p.x + q * p.group_size + (int64_t)k * kChunk, nv, v);
    const GroupStats st = combine_partials<VPT>(p, part, first, red);
    chunk_apply<X_FP16, PARAM>(p, q, k, nv, v, st);
}

// Lagged schedule.  A chunk's word in the workspace holds its mean (low 32
// bits) and sum of squared deviations (high 32 bits), the layout of the
// two-pass partials; kEmpty (two all-ones NaNs, which no reduction of 16-bit
// data produces) marks a word not yet published.
constexpr uint64_t kEmpty = ~0ull;
// Polls of an unpublished word (a few ms) before a workgroup reduces that
// chunk itself.  Never reached in a lone call, where the chunks an output
// waits for were reduced several hundred workgroups earlier.  The library's
// calls always use it; only the test entry point dit_group_norm_silu_polls
// takes another count (0: reduce at once, which makes every waiter take the
// reduce-it-here path).
constexpr int kWaitPolls = 1 << 12;

// Mark every chunk word of the call as not yet published.
__global__ __launch_bounds__(kBlock) void gn_clear_kernel(const GnParams p)
{
    uint64_t* word = reinterpret_cast<uint64_t*>(p.partial);
    for (int64_t i = blockIdx.x * (int64_t)kBlock + threadIdx.x; i < p.total;
         i += (int64_t)gridDim.x * kBlock)
        word[i] = kEmpty;
}

// Reduce chunk k of group q and publish its word if none is published yet.
// The first word published for a chunk stands (compare-and-swap from
// kEmpty): every workgroup of the group then combines the same statistics,
// and in place, a reduction that read data the chunk's output had already
// replaced never stands, since that output was written only after a word
// was published.  Returns, in thread 0, the word that stands.
// Slots: red[0..1] for the plain moments, red[2..4] for a rescaled chunk.
template <bool X_FP16, bool STREAMED>
__device__ __forceinline__ uint64_t reduce_and_publish(const GnParams& p, int64_t q, int k,
                                                       float (*red)[kWaves])
{
    constexpr int VPT = kVptMax;
    const int nv = chunk_vectors<VPT>(p, k);
    const uint16_t* const base = p.x + q * p.group_size + (int64_t)k * chunk_elems<VPT>();
    float mean, m2;
    if constexpr (STREAMED) {
        chunk_moments_streamed<X_FP16, VPT>(base, nv, red[0], red[1], mean, m2);
    } else {
        u32x4 v[VPT];
        load_chunk<false>(base, nv, v);
        chunk_moments<X_FP16>(v, nv, red[0], red[1], mean, m2);
    }
    const f32x2 part = chunk_partial<X_FP16, VPT>(p, base, nv, mean, m2, red + 2);
    uint64_t stands = 0;
    if (threadIdx.x == 0) {
        uint64_t* const w = reinterpret_cast<uint64_t*>(p.partial) + q * p.chunks + k;
        const uint64_t mine =
            (uint64_t)__float_as_uint(part[0]) | ((uint64_t)__float_as_uint(part[1]) << 32);
        uint64_t expected = kEmpty;
        stands = __hip_atomic_compare_exchange_strong(w, &expected, mine, __ATOMIC_RELAXED,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                     ? mine : expected;
    }
    return stands;
}

// Workgroup b: statistics of chunk b (b < total), then the output of chunk
// j = b - lag (0 <= j < total).  lag >= chunks, so every chunk of j's group
// belongs to a lower workgroup, normally finished long before.  A word still
// unpublished after p.wait_polls polls (its workgroup has not run yet: other
// work may hold the die) is reduced here instead, so every workgroup ends
// whatever order the workgroups start in.
template <bool X_FP16, int PARAM>
__global__ __launch_bounds__(kBlock) void gn_lagged_kernel(const GnParams p)
{
    constexpr int VPT = kVptMax;
    constexpr int64_t kChunk = chunk_elems<VPT>();
    __shared__ float red[10][kWaves];     // [0..4] chunk reductions, [5..9] the combine
    __shared__ int missing;
    __shared__ uint64_t helped;
    const int64_t b = blockIdx.x;
    const int64_t j = b - p.lag;
    const bool out = j >= 0 && j < p.total;
    int64_t qo = 0;
    int ko = 0, nvo = 0;
    u32x4 w[VPT];
    if (out) {      // the output chunk's loads depend on nothing: issue them first
        qo = j / p.chunks;
        ko = (int)(j % p.chunks);
        nvo = chunk_vectors<VPT>(p, ko);
        load_chunk<true>(p.x + qo * p.group_size + (int64_t)ko * kChunk, nvo, w);
    }
    if (b < p.total)
        reduce_and_publish<X_FP16, false>(p, b / p.chunks, (int)(b % p.chunks), red);
    if (!out)
        return;

    // chunks <= 256: thread i watches the word of chunk i of the output's group
    const int i = threadIdx.x;
    const bool watch = i < p.chunks;
    uint64_t* const grp = reinterpret_cast<uint64_t*>(p.partial) + qo * p.chunks;
    uint64_t bits = 0;
    if (watch) {
        bits = __hip_atomic_load(grp + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int spin = 0; bits == kEmpty && spin < p.wait_polls; ++spin) {
            __builtin_amdgcn_s_sleep(1);
            bits = __hip_atomic_load(grp + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (__syncthreads_or(watch && bits == kEmpty)) {
        // Rare: reduce the chunks still unpublished here, lowest first, one
        // vector at a time (the output chunk stays loaded in registers).
        for (;;) {
            if (i == 0)
                missing = kBlock;
            __syncthreads();
            if (watch && bits == kEmpty)
                atomicMin(&missing, i);
            __syncthreads();
            const int m = missing;
            if (m == kBlock)
                break;
            const uint64_t stands = reduce_and_publish<X_FP16, true>(p, qo, m, red);
            if (i == 0)
                helped = stands;
            __syncthreads();
            if (i == m)
                bits = helped;
            __syncthreads();        // every thread has read `missing` and `helped`
        }
    }
    const f32x2 first = watch ? f32x2{__uint_as_float((uint32_t)bits),
                                      __uint_as_float((uint32_t)(bits >> 32))}
                              : f32x2{0.0f, 0.0f};
    const GroupStats st = combine_partials<VPT>(p, p.partial + 2 * qo * p.chunks, first, red + 5);
    chunk_apply<X_FP16, PARAM>(p, qo, ko, nvo, w, st);
}

using GnFn = void (*)(GnParams);

template <bool XF>
GnFn pick_single(int prm)
{
    return prm == QKR_FP32 ? gn_single_kernel<XF, QKR_FP32>
         : prm == QKR_FP16 ? gn_single_kernel<XF, QKR_FP16> : gn_single_kernel<XF, QKR_BF16>;
}

template <bool XF, int VPT>
GnFn pick_apply(int prm)
{
    return prm == QKR_FP32 ? gn_apply_kernel<XF, QKR_FP32, VPT>
         : prm == QKR_FP16 ? gn_apply_kernel<XF, QKR_FP16, VPT> : gn_apply_kernel<XF, QKR_BF16, VPT>;
}

template <bool XF>
GnFn pick_lagged(int prm)
{
    return prm == QKR_FP32 ? gn_lagged_kernel<XF, QKR_FP32>
         : prm == QKR_FP16 ? gn_lagged_kernel<XF, QKR_FP16> : gn_lagged_kernel<XF, QKR_BF16>;
}

template <int VPT>
void pick_pair(bool xf, int prm, GnFn* stats, GnFn* apply)
{
    *stats = xf ? gn_stats_kernel<true, VPT> : gn_stats_kernel<false, VPT>;
    *apply = xf ? pick_apply<true, VPT>(prm) : pick_apply<false, VPT>(prm);
}

int launch(GnFn fn, int64_t blocks, const GnParams& p, hipStream_t stream)
{
    GnParams copy = p;
    void* args[] = {&copy};
    if (hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)blocks), dim3(kBlock),
                        args, 0, stream) != hipSuccess)
        return QKR_ERR_HIP;
    return QKR_OK;
}

// Workgroups per pass below which groups are cut into smaller chunks: with
// 16K-element chunks a small call leaves most of the chip idle (the VAE mid
// stage, 32 groups of 262,144, runs 512 workgroups).
constexpr int64_t kFillBlocks = 2048;
// A launch grid holds fewer than 2^32 work-items.
constexpr int64_t kMaxBlocks = 0xFFFFFFFFll / kBlock;
// The lagged schedule: used from this many 16K-element chunks per call (below
// it the two launches are as fast: the whole input stays in the Infinity
// Cache), for groups of at most one chunk per thread of a workgroup.  Its
// lag is the group's chunks plus kLagExtra, rounded up to a multiple of the
// dies, so that a chunk is re-read about 3 MB later on the die that read it.
constexpr int64_t kLaggedFromChunks = 4096;
constexpr int kLaggedMaxChunks = kBlock;
constexpr int64_t kLagExtra = 512;

enum Schedule { kOneRead = 0, kLagged = 1, kTwoPass = 2 };

// How a call of this shape runs (chunks and vpt from check_shape).
Schedule schedule_for(int64_t pairs, int64_t chunks, int vpt, int64_t* lag)
{
    *lag = 0;
    if (chunks == 1)
        return kOneRead;
    const int64_t total = pairs * chunks;
    const int64_t l = (chunks + kLagExtra + kXcds - 1) / kXcds * kXcds;
    if (vpt == kVptMax && chunks <= kLaggedMaxChunks && total >= kLaggedFromChunks &&
        total + l <= kMaxBlocks) {
        *lag = l;
        return kLagged;
    }
    return kTwoPass;
}

// Shape checks shared by the size query and the call.  Sets pairs (samples x
// groups), the vectors per thread of a chunk (8, 4 or 2: the largest that
// still gives kFillBlocks workgroups, 8 for a group of one chunk) and the
// chunks per group.
int check_shape(int64_t n, int32_t channels, int64_t spatial, int32_t groups, int64_t* chunks,
                int64_t* pairs, int* vpt)
{
    if (n < 0 || channels < 1 || groups < 1 || channels % groups)
        return QKR_ERR_SHAPE;
    if (spatial < kVec || spatial % kVec || spatial >= (1ll << 31))
        return QKR_ERR_UNSUPPORTED;
    const int64_t gsize = (int64_t)(channels / groups) * spatial;
    if (gsize >= (1ll << 31))
        return QKR_ERR_SHAPE;
    if (n > ((1ll << 31) - 1) / groups)
        return QKR_ERR_SHAPE;
    *pairs = n * groups;
    *vpt = kVptMax;
    if (gsize > kChunkMax) {
        for (int v = kVptMax; v >= 2; v /= 2) {
            *vpt = v;
            const int64_t elems = (int64_t)kBlock * v * kVec;
            if (*pairs * ((gsize + elems - 1) / elems) >= kFillBlocks)
                break;
        }
    }
    const int64_t elems = (int64_t)kBlock * *vpt * kVec;
    *chunks = (gsize + elems - 1) / elems;
    if (*pairs * *chunks > kMaxBlocks)
        return QKR_ERR_SHAPE;
    return QKR_OK;
}

}  // namespace

extern "C" int64_t dit_group_norm_silu_workspace_size(int64_t n, int32_t channels, int64_t spatial,
                                                      int32_t groups)
{
    int64_t chunks = 0, pairs = 0;
    int vpt = 0;
    const int rc = check_shape(n, channels, spatial, groups, &chunks, &pairs, &vpt);
    if (rc != QKR_OK)
        return rc;
    return chunks > 1 ? pairs * chunks * 2 * (int64_t)sizeof(float) : 0;
}

extern "C" int32_t dit_group_norm_silu_schedule(int64_t n, int32_t channels, int64_t spatial,
                                                int32_t groups, int64_t* chunk_elems_out)
{
    int64_t chunks = 0, pairs = 0, lag = 0;
    int vpt = 0;
    const int rc = check_shape(n, channels, spatial, groups, &chunks, &pairs, &vpt);
    if (rc != QKR_OK)
        return rc;
    if (chunk_elems_out)
        *chunk_elems_out = (int64_t)kBlock * vpt * kVec;
    return schedule_for(pairs, chunks, vpt, &lag);
}

namespace {

// The call, with the lagged schedule's polls per unpublished word.
// Every check of a call's arguments but the workspace's (no HIP call).  On
// QKR_OK, *need holds the workspace bytes the call takes (0 for n == 0).
int check_call(const void* x, const void* y, int64_t n, int32_t channels, int64_t spatial,
               int32_t groups, const void* gamma, const void* beta, int32_t param_dtype,
               float eps, int32_t dtype, int64_t* need)
{
    *need = 0;
    if (dtype < QKR_BF16 || dtype > QKR_FP32 || param_dtype < QKR_BF16 || param_dtype > QKR_FP32)
        return QKR_ERR_ARG;
    if (dtype == QKR_FP32)
        return QKR_ERR_UNSUPPORTED;
    if (!(eps > 0.0f) || !isfinite(eps))
        return QKR_ERR_ARG;
    int64_t chunks = 0, pairs = 0;
    int vpt = 0;
    const int rc = check_shape(n, channels, spatial, groups, &chunks, &pairs, &vpt);
    if (rc != QKR_OK)
        return rc;
    if (n == 0)
        return QKR_OK;
    if (!x || !y || !gamma || !beta)
        return QKR_ERR_NULL;
    if (!aligned16(x) || !aligned16(y) || !aligned16(gamma) || !aligned16(beta))
        return QKR_ERR_ALIGN;
    const int64_t gsize = (int64_t)(channels / groups) * spatial;
    const uint64_t bytes = (uint64_t)(pairs * gsize) * 2u;
    const uint64_t param_bytes = (uint64_t)channels * (param_dtype == QKR_FP32 ? 4u : 2u);
    // y is x itself or disjoint from it, and never overlaps gamma or beta
    if ((x != y && overlaps(x, bytes, y, bytes)) || overlaps(y, bytes, gamma, param_bytes) ||
        overlaps(y, bytes, beta, param_bytes))
        return QKR_ERR_ARG;
    *need = chunks > 1 ? pairs * chunks * 2 * (int64_t)sizeof(float) : 0;
    return QKR_OK;
}

int run_group_norm_silu(const void* x, void* y, int64_t n, int32_t channels, int64_t spatial,
                        int32_t groups, const void* gamma, const void* beta, int32_t param_dtype,
                        float eps, int32_t dtype, void* workspace, int64_t workspace_bytes,
                        void* stream, int32_t wait_polls)
{
    int64_t need = 0;
    const int rc = check_call(x, y, n, channels, spatial, groups, gamma, beta, param_dtype, eps,
                              dtype, &need);
    if (rc != QKR_OK || n == 0)
        return rc;
    int64_t chunks = 0, pairs = 0;
    int vpt = 0;
    check_shape(n, channels, spatial, groups, &chunks, &pairs, &vpt);
    const int64_t gsize = (int64_t)(channels / groups) * spatial;
    const uint64_t bytes = (uint64_t)(pairs * gsize) * 2u;
    const uint64_t param_bytes = (uint64_t)channels * (param_dtype == QKR_FP32 ? 4u : 2u);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
        return QKR_ERR_WORKSPACE;
    // the workspace is written too: apart from every other buffer
    if (need > 0 && (overlaps(workspace, need, x, bytes) || overlaps(workspace, need, y, bytes) ||
                     overlaps(workspace, need, gamma, param_bytes) ||
                     overlaps(workspace, need, beta, param_bytes)))
        return QKR_ERR_ARG;

    GnParams p;
    p.x = static_cast<const uint16_t*>(x);
    p.y = static_cast<uint16_t*>(y);
    p.gamma = gamma;
    p.beta = beta;
    p.partial = static_cast<float*>(workspace);
    p.group_size = gsize;
    p.spatial = (int32_t)spatial;
    p.cg = channels / groups;
    p.groups = groups;
    p.chunks = (int32_t)chunks;
    p.eps = eps;
    p.total = pairs * chunks;
    p.wait_polls = wait_polls;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool xf = dtype == QKR_FP16;

    const Schedule sched = schedule_for(pairs, chunks, vpt, &p.lag);
    if (sched == kOneRead)
        return launch(xf ? pick_single<true>(param_dtype) : pick_single<false>(param_dtype), pairs,
                      p, s);
    if (sched == kLagged) {
        const int64_t clear_blocks = (p.total + kBlock - 1) / kBlock;
        const int r = launch(gn_clear_kernel, clear_blocks < 1024 ? clear_blocks : 1024, p, s);
        return r == QKR_OK ? launch(xf ? pick_lagged<true>(param_dtype)
                                       : pick_lagged<false>(param_dtype),
                                    p.total + p.lag, p, s)
                           : r;
    }

    GnFn stats, apply;
    if (vpt == 8)
        pick_pair<8>(xf, param_dtype, &stats, &apply);
    else if (vpt == 4)
        pick_pair<4>(xf, param_dtype, &stats, &apply);
    else
        pick_pair<2>(xf, param_dtype, &stats, &apply);
    const int r = launch(stats, pairs * chunks, p, s);
    return r == QKR_OK ? launch(apply, pairs * chunks, p, s) : r;
}

}  // namespace

// ---------------------------------------------------------------- fixed scratch
//
// The workspace of dit_group_norm_silu_noalloc: one copy of this array per
// GPU, held until the process ends.  Host code never passes `scratch` itself
// (in host code the name is a host-side stand-in, not a device address): it
// passes the device address hipGetSymbolAddress gives for the current device,
// looked up once per device.
static __device__ __align__(256) uint8_t scratch[QKR_GN_NOALLOC_WORKSPACE_MAX];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_status[kMaxDevices];

// The device address of `scratch` on the current device.
int scratch_address(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return QKR_ERR_HIP;
    std::call_once(g_scratch_once[dev], [dev] {
        void* ptr = nullptr;
        g_scratch_status[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = ptr;
    });
    if (g_scratch_status[dev] != hipSuccess || !g_scratch_ptr[dev])
        return QKR_ERR_HIP;
    *out = g_scratch_ptr[dev];
    return QKR_OK;
}

}  // namespace

extern "C" int dit_group_norm_silu_noalloc(const void* x, void* y, int64_t n, int32_t channels,
                                           int64_t spatial, int32_t groups, const void* gamma,
                                           const void* beta, int32_t param_dtype, float eps,
                                           int32_t dtype, void* stream)
{
    int64_t need = 0;
    const int rc = check_call(x, y, n, channels, spatial, groups, gamma, beta, param_dtype, eps,
                              dtype, &need);
    if (rc != QKR_OK || n == 0)
        return rc;
    if (need > QKR_GN_NOALLOC_WORKSPACE_MAX)
        return QKR_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        const int r = scratch_address(&ws);
        if (r != QKR_OK)
            return r;
    }
    return run_group_norm_silu(x, y, n, channels, spatial, groups, gamma, beta, param_dtype, eps,
                               dtype, ws, need, stream, kWaitPolls);
}

extern "C" int dit_group_norm_silu(const void* x, void* y, int64_t n, int32_t channels,
                                   int64_t spatial, int32_t groups, const void* gamma,
                                   const void* beta, int32_t param_dtype, float eps, int32_t dtype,
                                   void* workspace, int64_t workspace_bytes, void* stream)
{
    return run_group_norm_silu(x, y, n, channels, spatial, groups, gamma, beta, param_dtype, eps,
                               dtype, workspace, workspace_bytes, stream, kWaitPolls);
}

// Test entry point (declared in the tests' own header, not the library's):
// dit_group_norm_silu with the lagged schedule's polls per unpublished word
// set by the caller, 0 .. 4096 (QKR_ERR_ARG otherwise).
extern "C" int dit_group_norm_silu_polls(const void* x, void* y, int64_t n, int32_t channels,
                                         int64_t spatial, int32_t groups, const void* gamma,
                                         const void* beta, int32_t param_dtype, float eps,
                                         int32_t dtype, void* workspace, int64_t workspace_bytes,
                                         void* stream, int32_t wait_polls)
{
    if (wait_polls < 0 || wait_polls > kWaitPolls)
        return QKR_ERR_ARG;
    return run_group_norm_silu(x, y, n, channels, spatial, groups, gamma, beta, param_dtype, eps,
                               dtype, workspace, workspace_bytes, stream, wait_polls);
}
