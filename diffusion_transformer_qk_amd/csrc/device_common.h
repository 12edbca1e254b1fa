// device_common.h -- lane-level helpers shared by the gfx950 kernels of this
// library: 16-byte vector access (optionally non-temporal), bf16/fp16 <-> fp32
// packing with round-to-nearest-even, DPP moves, and the die-contiguous block
// order.  Internal header (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace qkr_dev {

constexpr int kWave = 64;
constexpr int kVec = 8;                 // 16-bit elements per 16-byte access
constexpr int kXcds = 8;                // accelerator dies of an MI355X, each with its own L2

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Move of v across lanes with a DPP control (all rows and banks enabled).
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// The same move for a control under which every lane reads a lane of its own
// row (a rotation or permutation within the row): no lane keeps an old value,
// so none is supplied, and the compiler may fold the move into the
// instruction that consumes it.
template <int CTRL>
__device__ __forceinline__ float dpp_in_row(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <bool NT>
__device__ __forceinline__ u32x4 load16(const void* p)
{
    const u32x4* q = static_cast<const u32x4*>(p);
    if constexpr (NT)
        return __builtin_nontemporal_load(q);
    else
        return *q;
}

template <bool NT>
__device__ __forceinline__ void store16(void* p, u32x4 v)
{
    u32x4* q = static_cast<u32x4*>(p);
    if constexpr (NT)
        __builtin_nontemporal_store(v, q);
    else
        *q = v;
}

template <bool FP16>
__device__ __forceinline__ void unpack8(const u32x4 v, float f[8])
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t w = v[k];
        if constexpr (FP16) {
            const f16x2 h = __builtin_bit_cast(f16x2, w);
            f[2 * k] = (float)h.x;
            f[2 * k + 1] = (float)h.y;
        } else {
            f[2 * k] = __uint_as_float(w << 16);
            f[2 * k + 1] = __uint_as_float(w & 0xffff0000u);
        }
    }
}

template <bool FP16>
__device__ __forceinline__ u32x4 pack8(const float o[8])
{
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f32x2 pr = {o[2 * k], o[2 * k + 1]};
        if constexpr (FP16)
            w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, f16x2));
        else
            w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
    }
    return w;
}

__device__ __forceinline__ void load_f32x8(const float* p, float f[8])
{
    const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
    const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = a[i];
        f[4 + i] = b[i];
    }
}

// 1 / sqrt(x) for any positive x, subnormals included: the hardware
// reciprocal square root takes a subnormal input as zero (and returns +inf),
// so a subnormal x is scaled by 2^64 first (exact) and the result by 2^32.
__device__ __forceinline__ float rsqrt_full_range(float x)
{
    return x < 0x1p-126f ? __builtin_amdgcn_rsqf(x * 0x1p64f) * 0x1p32f : __builtin_amdgcn_rsqf(x);
}

// Sum over all 64 lanes of a wave; every lane ends with the same value.
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp<0xB1>(v);      // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);      // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);     // row_half_mirror
    v += dpp<0x140>(v);     // row_mirror: 16-lane row total in every lane
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// Sum over a workgroup of WAVES waves through `slot` (WAVES floats of LDS),
// added in wave order by every thread, so all threads get identical bits.
// Contains one barrier; a slot may be reused once every thread has passed a
// later barrier.
template <int WAVES>
__device__ __forceinline__ float block_sum(float v, float* slot)
{
    v = wave_sum(v);
    if (threadIdx.x % kWave == 0)
        slot[threadIdx.x / kWave] = v;
    __syncthreads();
    float t = slot[0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w)
        t += slot[w];
    return t;
}

// Largest value over all 64 lanes of a wave; every lane ends with it.
__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// Largest value over a workgroup of WAVES waves through `slot` (WAVES floats
// of LDS); the same barrier and slot rules as block_sum.
template <int WAVES>
__device__ __forceinline__ float block_max(float v, float* slot)
{
    v = wave_max(v);
    if (threadIdx.x % kWave == 0)
        slot[threadIdx.x / kWave] = v;
    __syncthreads();
    float t = slot[0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w)
        t = fmaxf(t, slot[w]);
    return t;
}

// Logical block of hardware block `bid`.  The dispatcher deals consecutive
// hardware blocks to consecutive dies; ORDER < 0 remaps that so each die
// walks one contiguous run of blocks (die d gets the d-th eighth of the grid,
// the first blocks % 8 dies one block more); ORDER == 0 keeps hardware order.
template <int ORDER>
__device__ __forceinline__ int64_t logical_block(uint32_t bid, uint32_t blocks)
{
    if constexpr (ORDER == 0) {
        return bid;
    } else {
        const uint32_t die = bid % kXcds, local = bid / kXcds;
        const uint32_t q = blocks / kXcds, r = blocks % kXcds;
        return (int64_t)die * q + (die < r ? die : r) + local;
    }
}

}  // namespace qkr_dev
