// Diagnostic streaming read: the plain-read reference a GEMV launch of the
// same bytes is measured against.  Each workgroup reads 16 KB of one buffer
// with 16-byte loads, four per lane issued together (the access pattern of
// the streaming GEMV), and XORs them into one word per wave so the loads
// cannot be dropped.
#include "internal.h"

namespace q4 {

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadLoads = 4;
constexpr uint32_t kReadBytesPerWg = kReadThreads * kReadLoads * 16;

struct ReadTable {
    const uint8_t* p[kMaxReadBufs];
    uint32_t bytes[kMaxReadBufs];
    int wg0[kMaxReadBufs + 1];   // first workgroup of each buffer; wg0[count] = grid
    int count;
};

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(ReadTable t, uint32_t* __restrict__ sink) {
    int b = 0;
    for (int i = 1; i < t.count; ++i) b += ((int)blockIdx.x >= t.wg0[i]) ? 1 : 0;
    const uint32_t base = (uint32_t)(blockIdx.x - t.wg0[b]) * kReadBytesPerWg;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(t.p[b], t.bytes[b]);
    u32x4 v[kReadLoads];
#pragma unroll
    for (int k = 0; k < kReadLoads; ++k) v[k] = buf_load16(r, base + (uint32_t)(k * kReadThreads + threadIdx.x) * 16u, 0);
    uint32_t x = 0;
#pragma unroll
    for (int k = 0; k < kReadLoads; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kReadThreads / 64) + (threadIdx.x >> 6)] = x;
}

}  // namespace

size_t stream_read_sink_words(const size_t* bytes, int count) {
    size_t wg = 0;
    for (int i = 0; i < count; ++i) wg += (bytes[i] + kReadBytesPerWg - 1) / kReadBytesPerWg;
    return wg * (kReadThreads / 64);
}

hipError_t launch_stream_read(const void* const* bufs, const size_t* bytes, int count, uint32_t* sink, hipStream_t s) {
    ReadTable t{};
    int grid = 0;
    for (int i = 0; i < count; ++i) {
        t.p[i] = static_cast<const uint8_t*>(bufs[i]);
        t.bytes[i] = (uint32_t)bytes[i];
        t.wg0[i] = grid;
        grid += (int)((bytes[i] + kReadBytesPerWg - 1) / kReadBytesPerWg);
    }
    t.wg0[count] = grid;
    t.count = count;
    return launch_kernel(stream_read_kernel, dim3(grid), dim3(kReadThreads), 0, s, t, sink);
}

}  // namespace q4
