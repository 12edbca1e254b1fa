// qknorm_rope.hip -- fused diffusion-transformer QK-norm + RoPE for gfx950.
//
// The pass (TensorRT-LLM PR "VisualGen Wan: deduplicate shared RoPE SMEM
// staging", Description; TensorRT-Model-Connect PR "perf(diffusion): fused
// qknorm rope Flux 2.0", intro): per token and per Q/K head, RMSNorm over
// head_dim with a learned weight, then RoPE with a cos/sin row indexed by
// dimension, in place; V untouched.  Math in fp32, one RNE rounding at the end.
//
// Work mapping (memory-bound: no matrix cores):
//   * a head of D elements is D/8 lanes, each holding 8 consecutive elements
//     in one 16-byte access; a wave covers 64/(D/8) heads per iteration;
//   * one wave owns one (token, tensor) slice: all H heads of Q, or of K, for
//     one token, with U iterations of loads in flight before any math;
//   * a 256-thread workgroup holds 4 waves = 2 tokens x {Q, K} (fused or two
//     separate tensors) or 4 tokens of a single tensor;
//   * shared layout: the workgroup stages each token's cos and sin rows once
//     in LDS as fp32 and every head indexes them by dimension (the row is
//     read from HBM once per token, not once per head);
//   * per-lane rotation coefficients A = gamma*cos and B = +/-gamma_partner*sin
//     are formed once per token (shared) or per head (per-head layout) with
//     the same instructions, so both layouts give bit-identical output;
//   * sum of squares: in-lane fma chain, then a DPP butterfly across the
//     head's lanes (quad_perm xor1 / xor2, row_half_mirror, row_mirror, and
//     for D = 256 a ds_swizzle xor 16 across the two 16-lane rows) that
//     leaves the identical sum in every lane of the head;
//   * rotate-half partners sit D/2 elements away = half the head's lanes:
//     exchanged with DPP row_ror:8 (D = 128) or ds_swizzle xor 4 / xor 16
//     (D = 64 / 256);
//   * fp32 -> bf16/fp16 with the packed round-to-nearest-even converts.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "device_common.h"
#include "host_common.h"
#include "qknorm_rope.h"

namespace {

using namespace qkr_dev;
using qkr_host::aligned16;
using qkr_host::overlaps;

constexpr int kInterleaved = QKR_ROPE_INTERLEAVED;
constexpr int kRotateHalf = QKR_ROPE_ROTATE_HALF;

struct Params {
    uint16_t* x[2];            // tensor s: element (t, h, d) at x[s] + t*row_stride + h*D + d
    const float* gamma[2];     // weight of tensor s
    const void* cos;
    const void* sin;
    int64_t row_stride;        // elements between consecutive tokens
    int64_t tokens;
    int32_t heads;
    int32_t n_tensors;         // 1 or 2
    float eps;
};

// ---------------------------------------------------------------- lane helpers

// Value of lane ^ 16 (within each 32-lane half of the wave): ds_swizzle in
// bit mode with and-mask 0x1F and xor-mask 0x10.
__device__ __forceinline__ float lane_xor16(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                 0x401F));
}

// Sum over the L lanes of one head (L = 8, 16 or 32, aligned groups).  Each
// step adds the same two partial sums in every lane, so all lanes end
// bit-equal.
template <int L>
__device__ __forceinline__ float head_sum(float v)
{
    v += dpp<0xB1>(v);       // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);       // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);      // row_half_mirror: the other quad of the 8-lane half
    if constexpr (L >= 16)
        v += dpp<0x140>(v);  // row_mirror: the other half of the 16-lane row
    if constexpr (L == 32)
        v += lane_xor16(v);  // the other 16-lane row of the head
    return v;
}

// Largest value over the L lanes of one head (the butterfly of head_sum).
template <int L>
__device__ __forceinline__ float head_max(float v)
{
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    if constexpr (L >= 16)
        v = fmaxf(v, dpp<0x140>(v));
    if constexpr (L == 32)
        v = fmaxf(v, lane_xor16(v));
    return v;
}

// Value held by the lane L/2 positions away within the head (the lane whose
// dimensions are D/2 away).
template <int L>
__device__ __forceinline__ float half_head_partner(float v)
{
    if constexpr (L == 32)
        return lane_xor16(v);
    else if constexpr (L == 16)
        return dpp_in_row<0x128>(v);  // row_ror:8 == lane ^ 8 inside a 16-lane row
    else
        return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                     0x101F));  // lane ^ 4
}

// 16-byte vectors holding eight table entries: one for bf16, two for fp32.
template <bool BF16_TABLE>
constexpr int table_vecs() { return BF16_TABLE ? 1 : 2; }

// Widen eight table entries held in table_vecs() raw vectors starting at w[0].
template <bool BF16_TABLE>
__device__ __forceinline__ void widen_table(const u32x4* w, float f[8])
{
    if constexpr (BF16_TABLE) {
        unpack8<false>(w[0], f);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[i] = __uint_as_float(w[0][i]);
            f[4 + i] = __uint_as_float(w[1][i]);
        }
    }
}

// Eight consecutive table entries starting at element `index`, widened to fp32.
template <bool BF16_TABLE>
__device__ __forceinline__ void load_table8(const void* table, int64_t index, float f[8])
{
    if constexpr (BF16_TABLE)
        unpack8<false>(load16<false>(static_cast<const uint16_t*>(table) + index), f);
    else
        load_f32x8(static_cast<const float*>(table) + index, f);
}

// o[d] = n[d] c[d] + sign(d) n[partner(d)] s[d] with n = y * gamma, folded
// into A[d] = gamma[d] c[d] and B[d] = sign(d) gamma[partner(d)] s[d].
template <int D, int STYLE>
__device__ __forceinline__ void rotation_coeffs(const float g[8], const float gp[8], const float c[8],
                                                const float s[8], int d0, float A[8], float B[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        A[i] = g[i] * c[i];
        const float b = gp[i] * s[i];
        const bool first_of_pair = STYLE == kInterleaved ? (i % 2 == 0) : (d0 < D / 2);
        B[i] = first_of_pair ? -b : b;
    }
}

// Sums of squares at or above this keep full fp32 precision (their largest
// terms are normal numbers); below it, subnormal squares lose bits, which
// only matters when eps is below it too.
constexpr float kTinySum = 0x1p-100f;

// Whether the fp32 sum of squares ss (of q = ss / D + eps) gives the head's
// scale exactly enough: q finite, and ss either clear of the subnormal range
// or swamped by eps.  False for a sum that overflowed (a head of 16-bit
// values whose RMS exceeds about 1.6e18) and for NaN.  When true, q is at
// least 2^-108, a normal number, as the hardware reciprocal square root needs.
__device__ __forceinline__ bool sum_in_range(float ss, float q, float eps)
{
    return q <= 0x1.fffffep127f && (ss >= kTinySum || eps >= kTinySum);
}

// The head's 1 / sqrt(mean(x^2) + eps) when the plain fp32 sum is out of
// range: with e the binary exponent of the head's largest |x|, sum the
// squares of x * 2^-e (an exact power-of-two scaling, all terms <= 1) and use
// 1 / sqrt(mean((x 2^-e)^2) + eps 2^-2e), which multiplies x * 2^-e: f is
// rescaled in place.  If eps 2^-2e overflows, mean(x^2) is below eps by more
// than 2^128 and 1 / sqrt(eps) is the answer, for f as it is.
template <int L, int D>
__device__ __forceinline__ float rescaled_rsqrt(float f[8], float eps)
{
    float m = fabsf(f[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i)
        m = fmaxf(m, fabsf(f[i]));
    const int e = __builtin_amdgcn_frexp_expf(head_max<L>(m));
    const float eps_s = __builtin_amdgcn_ldexpf(eps, -2 * e);
    if (!(eps_s <= 0x1.fffffep127f))
        return rsqrt_full_range(eps);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        f[i] = __builtin_amdgcn_ldexpf(f[i], -e);
    float ss = f[0] * f[0];
#pragma unroll
    for (int i = 1; i < 8; ++i)
        ss = __builtin_fmaf(f[i], f[i], ss);
    // the sum is at least 1/4 unless the head is all zeros; then it is eps,
    // which may be subnormal
    return rsqrt_full_range(__builtin_fmaf(head_sum<L>(ss), 1.0f / D, eps_s));
}

// Rotated, normalised output of one head's slice in this lane: y = f * r,
// then o = y A + y_partner B, rounded to the data type.
template <int D, int STYLE, bool X_FP16>
__device__ __forceinline__ u32x4 head_out(const float f[8], float r, const float A[8], const float B[8])
{
    constexpr int L = D / kVec;
    float y[8], yp[8], o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        y[i] = f[i] * r;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        yp[i] = STYLE == kInterleaved ? y[i ^ 1] : half_head_partner<L>(y[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        o[i] = __builtin_fmaf(y[i], A[i], yp[i] * B[i]);
    return pack8<X_FP16>(o);
}

// One head's slice in this lane: 8 elements in, 8 rotated, normalised out.
// `in_range` (the same in every lane of a head) is false when the head's
// plain fp32 sum of squares is out of range; its output is then not valid
// and the head goes through fix_heads instead.
template <int D, int STYLE, bool X_FP16>
__device__ __forceinline__ u32x4 head_math(const u32x4 v, const float A[8], const float B[8], float eps,
                                           bool& in_range)
{
    constexpr int L = D / kVec;
    float f[8];
    unpack8<X_FP16>(v, f);
    float ss = f[0] * f[0];
#pragma unroll
    for (int i = 1; i < 8; ++i)
        ss = __builtin_fmaf(f[i], f[i], ss);
    ss = head_sum<L>(ss);
    const float q = __builtin_fmaf(ss, 1.0f / D, eps);
    in_range = sum_in_range(ss, q, eps);
    return head_out<D, STYLE, X_FP16>(f, __builtin_amdgcn_rsqf(q), A, B);
}

// The heads of iterations `redo` (a bit per iteration u of the chunk at h0)
// whose plain sum of squares was out of range: they were not written, so
// each is read again and normalised through rescaled_rsqrt.  Kept out of the
// unrolled loop so that the registers of the in-flight loads are not charged
// for this rarely taken path.  Every lane of a head has the same bits.
template <int D, int STYLE, bool PER_HEAD, bool COS_BF16, bool X_FP16, int U>
__device__ __forceinline__ void fix_heads(const Params& p, uint16_t* row, int64_t t, int h0, int hs,
                                          int d0, uint32_t redo, const float g[8], const float gp[8],
                                          const float A[8], const float B[8])
{
    constexpr int L = D / kVec;
    constexpr int HPI = kWave / L;
#pragma unroll 1
    for (int u = 0; u < U; ++u) {
        if ((redo >> u) & 1u) {
            const int h = h0 + u * HPI + hs;
            float f[8];
            unpack8<X_FP16>(load16<false>(row + h * D + d0), f);
            float Ah[8], Bh[8];
            if constexpr (PER_HEAD) {
                const int64_t idx = (t * p.heads + h) * D + d0;
                float c[8], sn[8];
                load_table8<COS_BF16>(p.cos, idx, c);
                load_table8<COS_BF16>(p.sin, idx, sn);
                rotation_coeffs<D, STYLE>(g, gp, c, sn, d0, Ah, Bh);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    Ah[i] = A[i];
                    Bh[i] = B[i];
                }
            }
            const float r = rescaled_rsqrt<L, D>(f, p.eps);
            store16<false>(row + h * D + d0, head_out<D, STYLE, X_FP16>(f, r, Ah, Bh));
        }
    }
}

// Issue the loads of U head iterations starting at head h0 (plus, for the
// per-head layout, their cos/sin rows); heads past the end read as zero.
// tw holds, per head iteration u, the cos vectors then the sin vectors.
template <int D, bool PER_HEAD, bool COS_BF16, int U, int NT, int TW>
__device__ __forceinline__ void load_chunk(const Params& p, const uint16_t* row, int64_t t, int h0,
                                           int hs, int d0, u32x4 (&v)[U], u32x4 (&tw)[TW])
{
    constexpr int HPI = kWave / (D / kVec);
    const int H = p.heads;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int h = h0 + u * HPI + hs;
        if (h < H) {
            v[u] = load16<(NT & 1) != 0>(row + h * D + d0);
            if constexpr (PER_HEAD) {
                constexpr int NV = table_vecs<COS_BF16>();
                const int64_t idx = (t * H + h) * D + d0;
                const int per = COS_BF16 ? 8 : 4;          // entries per vector
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    tw[(2 * u) * NV + i] = COS_BF16
                        ? load16<false>(static_cast<const uint16_t*>(p.cos) + idx + i * per)
                        : load16<false>(static_cast<const float*>(p.cos) + idx + i * per);
                    tw[(2 * u + 1) * NV + i] = COS_BF16
                        ? load16<false>(static_cast<const uint16_t*>(p.sin) + idx + i * per)
                        : load16<false>(static_cast<const float*>(p.sin) + idx + i * per);
                }
            }
        } else {
            v[u] = u32x4{0, 0, 0, 0};
            if constexpr (PER_HEAD) {
                constexpr int NV = table_vecs<COS_BF16>();
#pragma unroll
                for (int i = 0; i < 2 * NV; ++i)
                    tw[2 * u * NV + i] = u32x4{0, 0, 0, 0};
            }
        }
    }
}

// ---------------------------------------------------------------- the kernel
//
// Waves per SIMD the register allocation must allow: 8 (64 VGPRs) for the
// shared-row kernels with at most 6 head iterations in flight, so that a
// grid of up to 2,048 workgroups (4,096 fused tokens) is resident at once
// instead of leaving a second, mostly idle round (measured: the mid-size
// 4096 x 3*24*128 call 19.0 -> 18.1 us back to back, the 5-head shard
// 42.6 -> 39.8 us; no spills).  Otherwise the register count the code needs.
template <bool PER_HEAD, int U>
constexpr int min_waves_per_simd() { return (!PER_HEAD && U <= 6) ? 8 : 1; }

// U      head iterations (of 64/L heads per wave) whose loads are in flight
//        before any arithmetic;
// WAVES  waves per workgroup (WAVES/2 tokens of Q and K per workgroup);
// NT     non-temporal Q/K accesses: bit 0 loads, bit 1 stores;
// ORDER  block order across dies (logical_block): 0 hardware, -1 die runs.

template <int D, int STYLE, bool PER_HEAD, bool COS_BF16, bool X_FP16, int U, int WAVES, int NT,
          int ORDER>
__global__ __launch_bounds__(WAVES * kWave, (min_waves_per_simd<PER_HEAD, U>()))
void qknorm_rope_kernel(const Params p)
{
    constexpr int L = D / kVec;        // lanes per head
    constexpr int HPI = kWave / L;     // heads per wave iteration
    constexpr int kThreads = WAVES * kWave;
    constexpr int TU = PER_HEAD ? U : 1;
    __shared__ float stage[PER_HEAD ? 4 : WAVES * 2 * D];   // [token][cos | sin][D]

    const int tid = threadIdx.x;
    // The wave index is uniform across the wave; saying so keeps the token,
    // the tensor and its row and weight pointers in scalar registers (a
    // per-lane index into the kernel arguments would be a memory load).
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int two = p.n_tensors == 2 ? 1 : 0;
    const int tokens_per_block = WAVES >> two;
    const int64_t block = logical_block<ORDER>(blockIdx.x, gridDim.x);
    const int64_t t_first = block * tokens_per_block;
    const int64_t t = t_first + (wave >> two);
    const int s = wave & two;
    const bool active = t < p.tokens;

    const int d0 = (lane % L) * kVec;  // this lane's first dimension
    const int hs = lane / L;           // head slot within a wave iteration
    const int H = p.heads;
    uint16_t* const row = p.x[s] + (active ? t : 0) * p.row_stride;

    u32x4 v[U];
    u32x4 tw[TU * 2 * table_vecs<COS_BF16>()];    // per-head cos/sin rows (raw)

    // Head loads first: they depend on nothing, so their latency overlaps
    // the staging of the cos/sin rows and the barrier below.
    float g[8], gp[8];
    if (active) {
        load_chunk<D, PER_HEAD, COS_BF16, U, NT>(p, row, t, 0, hs, d0, v, tw);
        const float* gam = p.gamma[s];
        load_f32x8(gam + d0, g);
        if constexpr (STYLE == kInterleaved) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                gp[i] = g[i ^ 1];
        } else {
            load_f32x8(gam + (d0 + D / 2) % D, gp);
        }
    }

    if constexpr (!PER_HEAD) {
        constexpr int per_chunk = COS_BF16 ? 8 : 4;      // table entries per 16-byte chunk
        constexpr int chunks = D / per_chunk;            // chunks per table row
        const int n_chunks = tokens_per_block * 2 * chunks;
        for (int i = tid; i < n_chunks; i += kThreads) {
            const int r = i / (2 * chunks);
            const int tab = (i / chunks) & 1;
            const int c = i % chunks;
            const int64_t tt = t_first + r;
            if (tt < p.tokens) {
                float* dst = stage + (r * 2 + tab) * D + c * per_chunk;
                const void* src = tab ? p.sin : p.cos;
                if constexpr (COS_BF16) {
                    float f[8];
                    load_table8<true>(src, tt * D + c * per_chunk, f);
                    reinterpret_cast<f32x4*>(dst)[0] = f32x4{f[0], f[1], f[2], f[3]};
                    reinterpret_cast<f32x4*>(dst)[1] = f32x4{f[4], f[5], f[6], f[7]};
                } else {
                    *reinterpret_cast<f32x4*>(dst) =
                        reinterpret_cast<const f32x4*>(static_cast<const float*>(src) + tt * D)[c];
                }
            }
        }
        __syncthreads();
    }
    if (!active)
        return;

    float A[8], B[8];
    if constexpr (!PER_HEAD) {
        const float* row_cs = stage + (wave >> two) * 2 * D;
        float c[8], sn[8];
        load_f32x8(row_cs + d0, c);
        load_f32x8(row_cs + D + d0, sn);
        rotation_coeffs<D, STYLE>(g, gp, c, sn, d0, A, B);
    }

    for (int h0 = 0;;) {
        uint32_t redo = 0;     // bit u: head iteration u is out of range, not stored
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int h = h0 + u * HPI + hs;
            u32x4 out;
            bool in_range;
            if constexpr (PER_HEAD) {
                constexpr int NV = table_vecs<COS_BF16>();
                float c[8], sn[8], Ah[8], Bh[8];
                widen_table<COS_BF16>(&tw[2 * u * NV], c);
                widen_table<COS_BF16>(&tw[(2 * u + 1) * NV], sn);
                rotation_coeffs<D, STYLE>(g, gp, c, sn, d0, Ah, Bh);
                out = head_math<D, STYLE, X_FP16>(v[u], Ah, Bh, p.eps, in_range);
            } else {
                out = head_math<D, STYLE, X_FP16>(v[u], A, B, p.eps, in_range);
            }
            if (h < H) {
                if (__builtin_expect(in_range, 1))
                    store16<(NT & 2) != 0>(row + h * D + d0, out);
                else
                    redo |= 1u << u;
            }
        }
        if (__builtin_expect(redo != 0, 0))
            fix_heads<D, STYLE, PER_HEAD, COS_BF16, X_FP16, U>(p, row, t, h0, hs, d0, redo, g, gp,
                                                             A, B);
        h0 += HPI * U;
        if (h0 >= H)
            break;
        load_chunk<D, PER_HEAD, COS_BF16, U, NT>(p, row, t, h0, hs, d0, v, tw);
    }
}

// Launch configuration of the library's kernels.
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWavesPerBlock * kWave;
constexpr int kNonTemporal = 3;         // Q/K loads and stores are not retained in cache
constexpr int kUnrollPerHeadMax = 10;   // per-head layout also keeps 2 table rows per head
constexpr int kDieRunsFromBlocks = 4096;
// Residency cap: dynamic LDS (never touched by the kernel) that, with the
// kernel's 2-8 KB of staging, takes 58-64 KB per workgroup, so that a
// 160 KB CU holds 2 workgroups (8 waves) of the pass at a time.
constexpr int kCapFromBlocks = 4096;
constexpr int64_t kCapFromFlightBytes = 6144;
constexpr size_t kCapLdsBytes = 56 * 1024;
constexpr int kCapWorkgroupsPerCu = 2;

// ---------------------------------------------------------------- dispatch
//
// Scheduling only (every choice computes bit-identical output):
//   unroll  the smallest of {3, 6, 10, 12} head iterations covering all H
//           heads (capped at 12), so a wave keeps one slice's loads in flight
//           with few padded iterations; the per-head layout, whose table rows
//           take registers too, caps it at 10 (measured on 40 heads: 4 / 8 /
//           10 iterations in flight gave 490 / 479 / 473 us);
//   order   one contiguous run of tokens per die when one buffer is streamed
//           (fused QKV or a single tensor) and the grid has at least
//           kDieRunsFromBlocks workgroups; hardware order otherwise (two
//           separate q/k buffers, or small grids where per-die runs are short);
//   residency  2 workgroups per CU (kCapLdsBytes of dynamic LDS) for the
//           shared layout when the grid has at least kCapFromBlocks
//           workgroups and each wave keeps at least kCapFromFlightBytes of
//           Q/K loads in flight.  More resident waves make the HBM stream
//           slower: on the 32760 x 3*40*128 fused call, 6 / 5 / 4 / 3 / 2 / 1
//           workgroups per CU took 235.9 / 234.1 / 228.9 / 227.9 / 223.4 /
//           313 us; on 75600 tokens 542.8 us uncapped, 502.3 us at 2.  Short
//           grids and small slices need every wave they can get (the 5-head
//           shard: 33.4 us uncapped, 67.7 us at 2), and the per-head layout's
//           registers already hold it to 2-3 waves per SIMD.

using KernelFn = void (*)(Params);

struct Launch {
    int unroll;
    int order;
    int64_t blocks;
    int tokens_per_block;
    size_t dynamic_lds;        // bytes of dynamic LDS per workgroup (the residency cap)
    int workgroups_per_cu;     // the cap it sets, 0 for none
};

Launch plan_launch(int head_dim, int heads, int64_t tokens, int n_tensors, bool separate_pair,
                   bool per_head)
{
    Launch l;
    const int heads_per_iter = kWave / (head_dim / kVec);
    const int iters = (heads + heads_per_iter - 1) / heads_per_iter;
    l.unroll = iters <= 3 ? 3 : iters <= 6 ? 6 : iters <= 10 ? 10 : 12;
    if (per_head && l.unroll > kUnrollPerHeadMax)
        l.unroll = kUnrollPerHeadMax;
    l.tokens_per_block = kWavesPerBlock / n_tensors;
    l.blocks = (tokens + l.tokens_per_block - 1) / l.tokens_per_block;
    l.order = (!separate_pair && l.blocks >= kDieRunsFromBlocks) ? -1 : 0;
    const int heads_in_flight = heads < l.unroll * heads_per_iter ? heads : l.unroll * heads_per_iter;
    const int64_t flight_bytes = (int64_t)heads_in_flight * head_dim * 2;
    const bool cap = !per_head && l.blocks >= kCapFromBlocks && flight_bytes >= kCapFromFlightBytes;
    l.dynamic_lds = cap ? kCapLdsBytes : 0;
    l.workgroups_per_cu = cap ? kCapWorkgroupsPerCu : 0;
    return l;
}

template <int D, int STYLE, bool PH, bool CB, bool XF, int ORDER>
KernelFn kernel_for_unroll(int unroll)
{
    if constexpr (PH) {
        if (unroll == 3)
            return qknorm_rope_kernel<D, STYLE, PH, CB, XF, 3, kWavesPerBlock, kNonTemporal, ORDER>;
        if (unroll == 6)
            return qknorm_rope_kernel<D, STYLE, PH, CB, XF, 6, kWavesPerBlock, kNonTemporal, ORDER>;
        return qknorm_rope_kernel<D, STYLE, PH, CB, XF, kUnrollPerHeadMax, kWavesPerBlock,
                                  kNonTemporal, ORDER>;
    } else {
        if (unroll == 3)
            return qknorm_rope_kernel<D, STYLE, PH, CB, XF, 3, kWavesPerBlock, kNonTemporal, ORDER>;
        if (unroll == 6)
            return qknorm_rope_kernel<D, STYLE, PH, CB, XF, 6, kWavesPerBlock, kNonTemporal, ORDER>;
        if (unroll == 10)
            return qknorm_rope_kernel<D, STYLE, PH, CB, XF, 10, kWavesPerBlock, kNonTemporal, ORDER>;
        return qknorm_rope_kernel<D, STYLE, PH, CB, XF, 12, kWavesPerBlock, kNonTemporal, ORDER>;
    }
}

template <int D, int STYLE, bool PH, bool CB, bool XF>
KernelFn select_order(const Launch& l)
{
    return l.order < 0 ? kernel_for_unroll<D, STYLE, PH, CB, XF, -1>(l.unroll)
                       : kernel_for_unroll<D, STYLE, PH, CB, XF, 0>(l.unroll);
}

template <int D, int STYLE, bool PH, bool CB>
KernelFn select_x(bool xf, const Launch& l)
{
    return xf ? select_order<D, STYLE, PH, CB, true>(l) : select_order<D, STYLE, PH, CB, false>(l);
}

template <int D, int STYLE, bool PH>
KernelFn select_c(bool cb, bool xf, const Launch& l)
{
    return cb ? select_x<D, STYLE, PH, true>(xf, l) : select_x<D, STYLE, PH, false>(xf, l);
}

template <int D, int STYLE>
KernelFn select_l(bool ph, bool cb, bool xf, const Launch& l)
{
    return ph ? select_c<D, STYLE, true>(cb, xf, l) : select_c<D, STYLE, false>(cb, xf, l);
}

template <int D>
KernelFn select_s(int style, bool ph, bool cb, bool xf, const Launch& l)
{
    return style == kRotateHalf ? select_l<D, kRotateHalf>(ph, cb, xf, l)
                                : select_l<D, kInterleaved>(ph, cb, xf, l);
}

KernelFn select_kernel(int head_dim, int style, int cos_layout, int cos_dtype, int dtype,
                       const Launch& l)
{
    const bool ph = cos_layout == QKR_COS_PER_HEAD;
    const bool cb = cos_dtype == QKR_BF16;
    const bool xf = dtype == QKR_FP16;
    if (head_dim == 128)
        return select_s<128>(style, ph, cb, xf, l);
    return head_dim == 64 ? select_s<64>(style, ph, cb, xf, l) : select_s<256>(style, ph, cb, xf, l);
}

int check_config(int32_t head_dim, int32_t cos_layout, int32_t cos_dtype, int32_t style, int32_t dtype)
{
    if (cos_layout != QKR_COS_SHARED && cos_layout != QKR_COS_PER_HEAD)
        return QKR_ERR_ARG;
    if (style != QKR_ROPE_INTERLEAVED && style != QKR_ROPE_ROTATE_HALF)
        return QKR_ERR_ARG;
    if (cos_dtype < QKR_BF16 || cos_dtype > QKR_FP32 || dtype < QKR_BF16 || dtype > QKR_FP32)
        return QKR_ERR_ARG;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256)
        return QKR_ERR_UNSUPPORTED;
    if (cos_dtype == QKR_FP16 || dtype == QKR_FP32)
        return QKR_ERR_UNSUPPORTED;
    return QKR_OK;
}

}  // namespace

extern "C" int qknorm_rope_fused(void* qkv, void* q, void* k, int64_t tokens, int32_t heads,
                                 int32_t head_dim, const float* q_gamma, const float* k_gamma,
                                 float eps, const void* cos, const void* sin, int32_t cos_layout,
                                 int32_t cos_dtype, int32_t style, int32_t dtype, void* stream)
{
    const int cfg = check_config(head_dim, cos_layout, cos_dtype, style, dtype);
    if (cfg != QKR_OK)
        return cfg;
    if (!(eps > 0.0f) || !isfinite(eps))
        return QKR_ERR_ARG;
    if (tokens < 0 || tokens >= QKR_MAX_TOKENS || heads < 1 || heads > QKR_MAX_HEADS)
        return QKR_ERR_SHAPE;
    if (tokens == 0)
        return QKR_OK;

    Params p = {};
    const int64_t hd = (int64_t)heads * head_dim;
    if (qkv) {
        if (q || k)
            return QKR_ERR_MODE;
        if (!q_gamma || !k_gamma)
            return QKR_ERR_NULL;
        uint16_t* base = static_cast<uint16_t*>(qkv);
        p.x[0] = base;
        p.x[1] = base + hd;
        p.gamma[0] = q_gamma;
        p.gamma[1] = k_gamma;
        p.n_tensors = 2;
        p.row_stride = 3 * hd;
        if (!aligned16(qkv))
            return QKR_ERR_ALIGN;
    } else {
        if (!q && !k)
            return QKR_ERR_MODE;
        int n = 0;
        if (q) {
            if (!q_gamma)
                return QKR_ERR_NULL;
            if (!aligned16(q))
                return QKR_ERR_ALIGN;
            p.x[n] = static_cast<uint16_t*>(q);
            p.gamma[n++] = q_gamma;
        }
        if (k) {
            if (!k_gamma)
                return QKR_ERR_NULL;
            if (!aligned16(k))
                return QKR_ERR_ALIGN;
            p.x[n] = static_cast<uint16_t*>(k);
            p.gamma[n++] = k_gamma;
        }
        p.n_tensors = n;
        p.row_stride = hd;
    }
    if (!cos || !sin)
        return QKR_ERR_NULL;
    if (!aligned16(cos) || !aligned16(sin))
        return QKR_ERR_ALIGN;
    for (int s = 0; s < p.n_tensors; ++s)
        if (!aligned16(p.gamma[s]))
            return QKR_ERR_ALIGN;

    // The tensors written must not overlap each other or a read-only input.
    const uint64_t tensor_bytes = (uint64_t)tokens * (uint64_t)hd * 2u;
    const uint64_t table_bytes = (uint64_t)tokens * (uint64_t)head_dim *
                                 (cos_layout == QKR_COS_PER_HEAD ? (uint64_t)heads : 1u) *
                                 (cos_dtype == QKR_FP32 ? 4u : 2u);
    const uint64_t gamma_bytes = (uint64_t)head_dim * 4u;
    const void* written[2] = {qkv ? qkv : p.x[0], qkv ? nullptr : (p.n_tensors == 2 ? p.x[1] : nullptr)};
    const uint64_t written_bytes = qkv ? 3 * tensor_bytes : tensor_bytes;
    if (written[1] && overlaps(written[0], written_bytes, written[1], written_bytes))
        return QKR_ERR_ARG;
    for (const void* w : written) {
        if (!w)
            continue;
        if (overlaps(w, written_bytes, cos, table_bytes) || overlaps(w, written_bytes, sin, table_bytes))
            return QKR_ERR_ARG;
        for (int s = 0; s < p.n_tensors; ++s)
            if (overlaps(w, written_bytes, p.gamma[s], gamma_bytes))
                return QKR_ERR_ARG;
    }

    p.cos = cos;
    p.sin = sin;
    p.tokens = tokens;
    p.heads = heads;
    p.eps = eps;

    const Launch l = plan_launch(head_dim, heads, tokens, p.n_tensors, !qkv && p.n_tensors == 2,
                                 cos_layout == QKR_COS_PER_HEAD);
    KernelFn fn = select_kernel(head_dim, style, cos_layout, cos_dtype, dtype, l);
    void* args[] = {&p};
    hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)l.blocks),
                                     dim3(kBlock), args, l.dynamic_lds,
                                     static_cast<hipStream_t>(stream));
    return err == hipSuccess ? QKR_OK : QKR_ERR_HIP;
}

extern "C" const char* qknorm_rope_strerror(int status)
{
    switch (status) {
    case QKR_OK: return "ok";
    case QKR_ERR_NULL: return "a required pointer is NULL";
    case QKR_ERR_SHAPE: return "a size is out of range or the sizes do not fit together";
    case QKR_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case QKR_ERR_UNSUPPORTED: return "unsupported size or dtype (head_dim 64/128/256; hidden or spatial a multiple of 8)";
    case QKR_ERR_MODE: return "pass either qkv, or q and/or k (not both, not neither)";
    case QKR_ERR_HIP: return "HIP launch or query failed";
    case QKR_ERR_ARG: return "eps not finite and > 0, an enum out of range, or a written buffer overlapping another";
    case QKR_ERR_WORKSPACE: return "workspace missing or smaller than required";
    case QKR_ERR_SCRATCH: return "the call needs more workspace than the library's fixed scratch "
                                 "(QKR_GN_NOALLOC_WORKSPACE_MAX); pass a workspace instead";
    default: return "unknown status";
    }
}

extern "C" int qknorm_rope_version(void) { return QKNORM_ROPE_VERSION; }

extern "C" int qknorm_rope_kernel_info(int32_t head_dim, int32_t heads, int64_t tokens,
                                       int32_t tensors, int32_t cos_layout, int32_t cos_dtype,
                                       int32_t style, int32_t dtype, qkr_kernel_info* out)
{
    if (!out)
        return QKR_ERR_NULL;
    if (tensors != QKR_TENSORS_FUSED && tensors != QKR_TENSORS_PAIR && tensors != QKR_TENSORS_ONE)
        return QKR_ERR_ARG;
    const int cfg = check_config(head_dim, cos_layout, cos_dtype, style, dtype);
    if (cfg != QKR_OK)
        return cfg;
    if (tokens < 0 || tokens >= QKR_MAX_TOKENS || heads < 1 || heads > QKR_MAX_HEADS)
        return QKR_ERR_SHAPE;
    const Launch l = plan_launch(head_dim, heads, tokens, tensors == QKR_TENSORS_ONE ? 1 : 2,
                                 tensors == QKR_TENSORS_PAIR, cos_layout == QKR_COS_PER_HEAD);
    hipFuncAttributes attr;
    KernelFn fn = select_kernel(head_dim, style, cos_layout, cos_dtype, dtype, l);
    if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(fn)) != hipSuccess)
        return QKR_ERR_HIP;
    out->num_vgprs = attr.numRegs;
    out->lds_bytes = (int32_t)attr.sharedSizeBytes;
    out->scratch_bytes = (int32_t)attr.localSizeBytes;
    out->block_threads = kBlock;
    out->tokens_per_block = l.tokens_per_block;
    out->heads_in_flight = l.unroll;
    out->die_runs = l.order < 0 ? 1 : 0;
    out->dynamic_lds_bytes = (int32_t)l.dynamic_lds;
    out->workgroups_per_cu = l.workgroups_per_cu;
    return QKR_OK;
}
