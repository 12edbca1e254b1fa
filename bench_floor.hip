// bench_floor.hip -- data-movement floor of the fused QK-norm + RoPE pass's
// access pattern on gfx950.  Measurement only: bench.py (--op floor) times it
// beside the pass; it is built into its own library (bench_floor.so), never
// into libqknorm_rope.so.
//
// The kernel moves exactly the bytes the pass moves, with the pass's work
// mapping and cache policy, and does no arithmetic on them: every 16-byte
// vector of Q and K is loaded non-temporally and stored back unchanged to the
// same address (head_dim 128, one wave per (token, tensor) slice, 16 lanes
// per head, 4 heads per wave iteration, all head iterations' loads in flight
// before the first store, 256-thread workgroups of two tokens, one
// contiguous run of tokens per die from 4096 workgroups on).  With the table,
// each workgroup also stages its tokens' fp32 cos and sin rows in LDS behind
// a barrier, and every lane reads its 8 + 8 entries back, as the pass does.
// The stores depend on the staged entries only through a comparison that is
// never true for a cos/sin table, so the data written equals the data read.
//
// row_stride (elements between tokens) >= 2 * heads * 128: the fused layout's
// 3 * heads * 128 leaves the V gap in every row; 2 * heads * 128 is the same
// bytes with no gaps.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "device_common.h"

namespace {

using namespace qkr_dev;

constexpr int kD = 128;
constexpr int kL = kD / kVec;          // lanes per head
constexpr int kHpi = kWave / kL;       // heads per wave iteration
constexpr int kU = 10;                 // head iterations in flight: up to 40 heads
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kDieRunsFromBlocks = 4096;

struct FloorParams {
    uint16_t* x;
    const float* cos;
    const float* sin;
    int64_t row_stride;
    int64_t tokens;
    int32_t heads;
};

template <bool TABLE, int ORDER>
__global__ __launch_bounds__(kThreads) void floor_kernel(const FloorParams p)
{
    __shared__ float stage[TABLE ? 2 * 2 * kD : 4];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int64_t block = logical_block<ORDER>(blockIdx.x, gridDim.x);
    const int64_t t_first = block * 2;
    const int64_t t = t_first + (wave >> 1);
    const int s = wave & 1;
    const bool active = t < p.tokens;
    const int d0 = (lane % kL) * kVec;
    const int hs = lane / kL;
    const int H = p.heads;
    uint16_t* const row = p.x + (active ? t : 0) * p.row_stride + (int64_t)s * H * kD;

    u32x4 v[kU];
    if (active) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int h = u * kHpi + hs;
            v[u] = h < H ? load16<true>(row + h * kD + d0) : u32x4{0, 0, 0, 0};
        }
    }
    uint32_t flip = 0;
    if constexpr (TABLE) {
        constexpr int chunks = kD / 4;                // 16-byte chunks per fp32 row
        for (int i = tid; i < 2 * 2 * chunks; i += kThreads) {
            const int r = i / (2 * chunks);
            const int tab = (i / chunks) & 1;
            const int c = i % chunks;
            const int64_t tt = t_first + r;
            if (tt < p.tokens)
                reinterpret_cast<f32x4*>(stage + (r * 2 + tab) * kD)[c] =
                    reinterpret_cast<const f32x4*>((tab ? p.sin : p.cos) + tt * kD)[c];
        }
        __syncthreads();
        if (active) {
            float c[8], sn[8];
            load_f32x8(stage + (wave >> 1) * 2 * kD + d0, c);
            load_f32x8(stage + (wave >> 1) * 2 * kD + kD + d0, sn);
            float acc = c[0];
#pragma unroll
            for (int i = 1; i < 8; ++i)
                acc = fmaxf(acc, c[i]);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc = fmaxf(acc, sn[i]);
            flip = acc > 4.0f ? 1u : 0u;              // |cos|, |sin| <= 1: never set
        }
    }
    if (!active)
        return;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int h = u * kHpi + hs;
        if (h < H)
            store16<true>(row + h * kD + d0, v[u] ^ flip);
    }
}

}  // namespace

// Enqueue one floor pass over [tokens] rows of `heads` Q heads and `heads` K
// heads of 128 bf16/fp16 elements (row_stride elements apart) on `stream`.
// cos/sin: fp32 [tokens, 128], read only when with_table != 0.  Returns 0, or
// -1 (NULL pointer), -2 (sizes: tokens < 1 or >= 2^24, heads not in 1..40,
// row_stride < 2 * heads * 128), -3 (pointer not 16-byte aligned), -6 (launch
// failed).
extern "C" int qkr_floor_fused(void* qkv, int64_t tokens, int32_t heads, int64_t row_stride,
                               const float* cos, const float* sin, int32_t with_table,
                               void* stream)
{
    if (!qkv || (with_table && (!cos || !sin)))
        return -1;
    if (tokens < 1 || tokens >= ((int64_t)1 << 24) || heads < 1 || heads > kU * kHpi ||
        row_stride < 2 * (int64_t)heads * kD)
        return -2;
    if ((reinterpret_cast<uintptr_t>(qkv) & 15u) || (row_stride % kVec) ||
        (with_table && ((reinterpret_cast<uintptr_t>(cos) | reinterpret_cast<uintptr_t>(sin)) & 15u)))
        return -3;
    FloorParams p = {static_cast<uint16_t*>(qkv), cos, sin, row_stride, tokens, heads};
    const int64_t blocks = (tokens + 1) / 2;
    const bool runs = blocks >= kDieRunsFromBlocks;
    const void* fn = with_table
        ? (runs ? reinterpret_cast<const void*>(floor_kernel<true, -1>)
                : reinterpret_cast<const void*>(floor_kernel<true, 0>))
        : (runs ? reinterpret_cast<const void*>(floor_kernel<false, -1>)
                : reinterpret_cast<const void*>(floor_kernel<false, 0>));
    void* args[] = {&p};
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), args, 0,
                           static_cast<hipStream_t>(stream)) == hipSuccess ? 0 : -6;
}
