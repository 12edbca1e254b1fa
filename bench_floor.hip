// bench_floor.hip -- data-movement floors of the fused QK-norm + RoPE pass's
// access pattern on gfx950 (and, out of place, of the row-wise AdaLN and
// group-norm steps' bytes).  Measurement only: bench.py (--op floor) times
// these probes beside the pass; they are built into their own library
// (bench_floor.so), never into libqknorm_rope.so.
//
// The probes move the pass's bytes with the pass's work mapping and cache
// policy and do no arithmetic on them: head_dim 128, one wave per (token,
// tensor) slice, 16 lanes per head holding one 16-byte vector each, 4 heads
// per wave iteration, U head iterations' loads in flight before the first
// store (U the smallest of 3, 6, 10, 12 covering the heads, 12 at most per
// chunk of heads, as the pass picks it), 256-thread workgroups of two tokens
// of Q and K (four tokens of a single tensor), and one contiguous run of
// tokens per die from 4096 workgroups on when one buffer is streamed.  Modes:
//   0  Q/K vectors loaded and stored back unchanged, in place;
//   1  mode 0 plus the pass's cos/sin staging: each workgroup stages its
//      tokens' fp32 rows in LDS behind a barrier and every lane reads its
//      8 + 8 entries back (the stores depend on them only through a test
//      that is never true for a cos/sin table, so the data stays unchanged);
//   2  mode 0, but every wave waits for all of its loads and then the
//      workgroup meets at a barrier before the first store (the phase
//      structure of mode 1 without the table bytes);
//   3  loads only: each wave folds its vectors into one word, stored to a
//      sink only if it equals a value the host never passes as `magic`;
//   4  stores only: each vector written with zeros (the data is destroyed);
//   5  mode 0, but every wave waits for all of its loads before its first
//      store (no barrier);
//   6  mode 5 out of place: the vectors read from a single tensor are
//      written to the same positions of another buffer y (the access
//      pattern of a row-wise step that writes a new tensor, such as the
//      AdaLN modulation, when heads * 128 is its row width).
// Modes 2, 5 and 6 make the stores depend on every loaded vector through the
// same fold as mode 3: the data written equals the data read unless the fold
// equals `magic`.
//
// Residency: like the pass, a long grid (at least 4096 workgroups) whose waves
// each keep at least 6 KB in flight reserves 56 KB of dynamic LDS per
// workgroup, which holds a 160 KB CU to 2 workgroups; `cap` 0 launches
// without the reservation, 1 applies the pass's rule.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "device_common.h"

namespace {

using namespace qkr_dev;

constexpr int kD = 128;
constexpr int kL = kD / kVec;          // lanes per head
constexpr int kHpi = kWave / kL;       // heads per wave iteration
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kDieRunsFromBlocks = 4096;
constexpr int kCapFromBlocks = 4096;
constexpr int64_t kCapFromFlightBytes = 6144;
constexpr size_t kCapLdsBytes = 56 * 1024;

struct FloorParams {
    uint16_t* x[2];            // tensor s: head h of token t at x[s] + t * row_stride + h * 128
    const float* cos;
    const float* sin;
    uint32_t* sink;            // mode 3
    uint16_t* y;               // mode 6: the destination, laid out like x[0]
    int64_t row_stride;
    int64_t tokens;
    int32_t heads;
    int32_t n_tensors;
    uint32_t magic;
};

template <int U, int MODE, int ORDER>
__global__ __launch_bounds__(kThreads) void floor_kernel(const FloorParams p)
{
    __shared__ float stage[MODE == 1 ? kWaves * 2 * kD : 4];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // uniform: scalar pointers
    const int lane = tid % kWave;
    const int two = p.n_tensors == 2 ? 1 : 0;
    const int tokens_per_block = kWaves >> two;
    const int64_t block = logical_block<ORDER>(blockIdx.x, gridDim.x);
    const int64_t t_first = block * tokens_per_block;
    const int64_t t = t_first + (wave >> two);
    const int s = wave & two;
    const bool active = t < p.tokens;
    const int d0 = (lane % kL) * kVec;
    const int hs = lane / kL;
    const int H = p.heads;
    uint16_t* const row = p.x[s] + (active ? t : 0) * p.row_stride;

    u32x4 v[U];
    if constexpr (MODE != 4) {
        if (active) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int h = u * kHpi + hs;
                v[u] = h < H ? load16<true>(row + h * kD + d0) : u32x4{0, 0, 0, 0};
            }
        }
    }
    uint32_t flip = 0;
    if constexpr (MODE == 1) {
        constexpr int chunks = kD / 4;                // 16-byte chunks per fp32 row
        for (int i = tid; i < tokens_per_block * 2 * chunks; i += kThreads) {
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
            load_f32x8(stage + (wave >> two) * 2 * kD + d0, c);
            load_f32x8(stage + (wave >> two) * 2 * kD + kD + d0, sn);
            float acc = c[0];
#pragma unroll
            for (int i = 1; i < 8; ++i)
                acc = fmaxf(acc, c[i]);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc = fmaxf(acc, sn[i]);
            flip = acc > 4.0f ? 1u : 0u;              // |cos|, |sin| <= 1: never set
        }
    } else if constexpr (MODE == 2 || MODE == 5 || MODE == 6) {
        if (active) {
            uint32_t acc = 0;
#pragma unroll
            for (int u = 0; u < U; ++u)
                acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
            flip = acc == p.magic ? 1u : 0u;
        }
        if constexpr (MODE == 2)
            __syncthreads();
    }
    if (!active)
        return;
    if constexpr (MODE == 3) {
        uint32_t acc = 0;
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
        if (acc == p.magic)
            p.sink[0] = acc;
        return;
    }
    uint16_t* const dst = MODE == 6 ? p.y + t * p.row_stride : row;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int h = u * kHpi + hs;
        if (h < H) {
            if constexpr (MODE == 4)
                store16<true>(row + h * kD + d0, u32x4{0, 0, 0, 0});
            else
                store16<true>(dst + h * kD + d0, v[u] ^ flip);
        }
    }
}

using FloorFn = void (*)(FloorParams);

template <int U>
FloorFn pick_mode(int mode, bool runs)
{
    switch (mode) {
    case 1: return runs ? floor_kernel<U, 1, -1> : floor_kernel<U, 1, 0>;
    case 2: return runs ? floor_kernel<U, 2, -1> : floor_kernel<U, 2, 0>;
    case 3: return runs ? floor_kernel<U, 3, -1> : floor_kernel<U, 3, 0>;
    case 4: return runs ? floor_kernel<U, 4, -1> : floor_kernel<U, 4, 0>;
    case 5: return runs ? floor_kernel<U, 5, -1> : floor_kernel<U, 5, 0>;
    case 6: return runs ? floor_kernel<U, 6, -1> : floor_kernel<U, 6, 0>;
    default: return runs ? floor_kernel<U, 0, -1> : floor_kernel<U, 0, 0>;
    }
}

}  // namespace

// Enqueue one probe pass over `tokens` rows of `heads` heads of 128 16-bit
// elements in one tensor (x1 == NULL) or two (x0 and x1; for a fused QKV
// buffer x1 = x0 + heads * 128), rows row_stride elements apart, on `stream`.
// cos/sin: fp32 [tokens, 128], read in mode 1 only; sink: one device word,
// written in mode 3 only (and only if a wave's folded data equals magic).
// cap: 1 applies the pass's residency rule, 0 never reserves LDS.  y: mode
// 6's destination, tokens * row_stride elements that do not overlap x0
// (NULL in the other modes); mode 6 takes a single tensor (x1 == NULL).
// Returns 0, or -1 (NULL pointer), -2 (sizes: tokens < 1 or >= 2^24, heads
// not in 1..48, row_stride < heads * 128 for separate tensors or
// < 2 * heads * 128 for a fused buffer, mode not in 0..6, cap not 0 or 1,
// mode 6 with x1), -3 (pointer not 16-byte aligned), -6 (launch failed).
extern "C" int qkr_floor(void* x0, void* x1, int64_t tokens, int32_t heads, int64_t row_stride,
                         const float* cos, const float* sin, uint32_t* sink, uint32_t magic,
                         int32_t mode, int32_t cap, void* y, void* stream)
{
    if (!x0 || (mode == 1 && (!cos || !sin)) || (mode == 3 && !sink) || (mode == 6 && !y))
        return -1;
    const bool fused = x1 && static_cast<uint16_t*>(x1) == static_cast<uint16_t*>(x0) + (int64_t)heads * kD;
    if (tokens < 1 || tokens >= ((int64_t)1 << 24) || heads < 1 || heads > 12 * kHpi ||
        mode < 0 || mode > 6 || (cap != 0 && cap != 1) || (mode == 6 && x1) ||
        row_stride < (fused ? 2 : 1) * (int64_t)heads * kD)
        return -2;
    const uintptr_t bits = reinterpret_cast<uintptr_t>(x0) | reinterpret_cast<uintptr_t>(x1) |
                           (mode == 1 ? reinterpret_cast<uintptr_t>(cos) | reinterpret_cast<uintptr_t>(sin) : 0) |
                           (mode == 6 ? reinterpret_cast<uintptr_t>(y) : 0);
    if ((bits & 15u) || (row_stride % kVec))
        return -3;
    FloorParams p = {{static_cast<uint16_t*>(x0), static_cast<uint16_t*>(x1 ? x1 : x0)},
                     cos, sin, sink, static_cast<uint16_t*>(y), row_stride, tokens, heads, x1 ? 2 : 1,
                     magic};
    const int tokens_per_block = kWaves / p.n_tensors;
    const int64_t blocks = (tokens + tokens_per_block - 1) / tokens_per_block;
    // one run of tokens per die when one buffer is streamed, as the pass does
    const bool runs = (fused || !x1) && blocks >= kDieRunsFromBlocks;
    const int iters = (heads + kHpi - 1) / kHpi;
    FloorFn fn = iters <= 3 ? pick_mode<3>(mode, runs) : iters <= 6 ? pick_mode<6>(mode, runs)
               : iters <= 10 ? pick_mode<10>(mode, runs) : pick_mode<12>(mode, runs);
    const int64_t in_flight = (int64_t)heads * kD * 2;        // heads <= 12 iterations
    const size_t lds = cap && blocks >= kCapFromBlocks && in_flight >= kCapFromFlightBytes
                           ? kCapLdsBytes : 0;
    void* args[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)blocks),
                           dim3(kThreads), args, lds, static_cast<hipStream_t>(stream)) == hipSuccess
               ? 0 : -6;
}
