// The gated MLP activation h = RN_bf16(silu(g) * u) as a pass of its own, for
// the fused int4 calls that run the tiled kernel: there the kernel's loader
// waves would form h again for every 64-row block (and they pace the main
// loop), so h is formed once into the caller's workspace and the tiled kernel
// reads it as plain activations.  The arithmetic is the loaders' own
// (silu_mul_bf16x2), so h -- and every output -- is the same bit for bit.
#include "internal.h"

namespace q4 {

namespace {

struct GatedTable {
    int blk0[kMaxTasks];                 // first workgroup of each segment (unused: INT_MAX)
    const uint16_t* g[kMaxTasks];
    const uint16_t* u[kMaxTasks];
    uint16_t* h[kMaxTasks];
    int pieces[kMaxTasks];               // 16-byte pieces (8 values) of each segment
};

__global__ __launch_bounds__(256) void silu_mul_kernel(GatedTable tt) {
    int t = 0;
#pragma unroll
    for (int i = 1; i < kMaxTasks; ++i) t += ((int)blockIdx.x >= tt.blk0[i]) ? 1 : 0;
    const int p = ((int)blockIdx.x - tt.blk0[t]) * 256 + (int)threadIdx.x;
    if (p >= tt.pieces[t]) return;
    const u32x4 g = reinterpret_cast<const u32x4*>(tt.g[t])[p];
    const u32x4 u = reinterpret_cast<const u32x4*>(tt.u[t])[p];
    reinterpret_cast<u32x4*>(tt.h[t])[p] =
        u32x4{silu_mul_bf16x2(g.x, u.x), silu_mul_bf16x2(g.y, u.y), silu_mul_bf16x2(g.z, u.z), silu_mul_bf16x2(g.w, u.w)};
}

}  // namespace

hipError_t launch_silu_mul(const uint16_t* const* g, const uint16_t* const* u, uint16_t* const* h, const size_t* values, int count,
                           hipStream_t s) {
    GatedTable tt{};
    int grid = 0;
    for (int i = 0; i < kMaxTasks; ++i) tt.blk0[i] = 0x7fffffff;
    for (int i = 0; i < count; ++i) {
        tt.blk0[i] = grid;
        tt.g[i] = g[i];
        tt.u[i] = u[i];
        tt.h[i] = h[i];
        tt.pieces[i] = (int)(values[i] / 8);
        grid += (tt.pieces[i] + 255) / 256;
    }
    return launch_kernel(silu_mul_kernel, dim3(grid), dim3(256), 0, s, tt);
}

}  // namespace q4
