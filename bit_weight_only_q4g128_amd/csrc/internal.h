// Host-side launchers shared between the C ABI (api.cpp) and the kernel
// translation units.  Everything here assumes the arguments were validated.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "formats.h"

namespace q4 {

// Caller-owned events that the next kernel launch of the calling thread
// records at its start and end (set through q4gemv_time_next_launch).
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& pending_launch_events();

template <typename Kernel, typename... Args>
hipError_t launch_kernel(Kernel k, dim3 grid, dim3 block, size_t shmem, hipStream_t st, Args... args) {
    LaunchEvents& ev = pending_launch_events();
    if (ev.start || ev.stop) {
        const LaunchEvents e = ev;
        ev = LaunchEvents{};
        hipExtLaunchKernelGGL(k, grid, block, shmem, st, e.start, e.stop, 0, args...);
    } else {
        hipLaunchKernelGGL(k, grid, block, shmem, st, args...);
    }
    return hipGetLastError();
}

enum Fmt { kFmtQ4 = 0, kFmtNvfp4 = 1, kFmtBf16 = 2 };

// Most GEMVs one launch can carry.
constexpr int kMaxTasks = 8;

// Packed-dot GEMV (wave-per-row-slice, DPP reduction) over `count` <= kMaxTasks
// independent GEMVs of one format and one batch size M (any N, K each).
// Supports any M by looping over batch tiles of at most 8 rows.  Returns
// hipSuccess or the launch error.
hipError_t launch_dot2(Fmt fmt, const GemvArgs* tasks, int count, hipStream_t s);
bool dot2_supported(Fmt fmt, int K);

// Streaming GEMV for M <= kStreamMaxM on rows of 1, 2 or 4 KB; up to
// kMaxTasks GEMVs per launch.  stream_supported() says whether (fmt, M, K)
// qualifies.
constexpr int kStreamMaxM = 4;
constexpr int kStreamMaxShmem = 64 * 1024;
hipError_t launch_stream(Fmt fmt, const GemvArgs* tasks, int count, hipStream_t s);
bool stream_supported(Fmt fmt, int M, int K);
// The streaming kernel over tasks of several formats in one launch (fmts[i]
// per task; every task stream_supported at the one batch size M).
hipError_t launch_stream_mixed(const Fmt* fmts, const GemvArgs* tasks, int count, hipStream_t s);
// The int4 streaming kernel with the fused activation prologue and residual
// epilogue (GemvArgs::up, GemvArgs::resid; either may be null).
hipError_t launch_stream_fused(const GemvArgs* tasks, int count, hipStream_t s);

// Tiled matrix-core GEMV with staged activations (M <= 64, K % 128 == 0) for
// the three weight formats, up to kMaxTasks GEMVs of one format per launch.
// With a workspace of at least mm_workspace_bytes() bytes (zero-filled before
// first use; its counters are left at zero, the rest is scratch), K may be
// split over workgroups; without one every task runs unsplit, which
// mm_supported(fmt, M, K, false) must allow.
bool mm_supported(Fmt fmt, int M, int K, bool split);
// Every workspace starts with this many bytes of arrival counters that each
// call leaves at zero; scratch lies after them.
constexpr size_t kWsCounterBytes = 64 * 1024;
// Bytes between two arrival counters: device-scope atomics on one cache line
// serialize (about 12 ns each), on different lines they proceed in parallel.
constexpr size_t kCtrStride = 128;
constexpr int kCtrWords = (int)(kCtrStride / 4);
// The built-in scratch of the allocation-free entry point (noalloc.hip): its
// size, and its device address on the stream's device (set up on first use:
// address lookup, counters cleared on stream s).
constexpr size_t kNoAllocScratchBytes = 8u << 20;
hipError_t noalloc_scratch(hipStream_t s, void** out);
size_t mm_workspace_bytes(Fmt fmt, const GemvArgs* tasks, int count);
hipError_t launch_mm(Fmt fmt, const GemvArgs* tasks, int count, void* ws, size_t ws_bytes, hipStream_t s);
// Skinny matrix-core GEMV (gemv_skinny.hip): int4, NVFP4 and BF16 tasks
// (fmts[i] per task; the overloads without fmts take int4 tasks), 5 <= M <=
// kSkinnyMaxM, K % 128 == 0, up to kMaxTasks GEMVs of one batch size per
// launch.  A workgroup owns up to 80 rows over a slice of at most 16 groups
// of K (BF16: 8); with a workspace of at least skinny_workspace_bytes() (same
// layout rules as the tiled kernel's: counters first, left at zero) K may be
// split over workgroups; without one every task must fit one slice
// (skinny_supported(fmt, M, K, false)).  GemvArgs::resid is honoured (added
// before the one rounding), GemvArgs::up is not.
constexpr int kSkinnyMaxM = 48;
bool skinny_supported(Fmt fmt, int M, int K, bool split);
size_t skinny_workspace_bytes(const Fmt* fmts, const GemvArgs* tasks, int count);
hipError_t launch_skinny(const Fmt* fmts, const GemvArgs* tasks, int count, void* ws, size_t ws_bytes, hipStream_t s);
bool skinny_supported(int M, int K, bool split);
size_t skinny_workspace_bytes(const GemvArgs* tasks, int count);
hipError_t launch_skinny(const GemvArgs* tasks, int count, void* ws, size_t ws_bytes, hipStream_t s);
// The tiled kernel over NVFP4 and BF16 tasks in one launch (fmts[i] per
// task), with the same workspace rules (sized by mm_workspace_bytes with
// kFmtNvfp4).
hipError_t launch_mm_mixed(const Fmt* fmts, const GemvArgs* tasks, int count, void* ws, size_t ws_bytes, hipStream_t s);
// Prefill GEMM: the int4 tiled kernel over batch chunks of up to 64 rows
// (grid rows), for any M, unsplit; K % 128 == 0 and the K's group
// parameters within the kernel's LDS budget (K <= 16384).
bool mm_chunks_supported(int K);
hipError_t launch_mm_chunks(const GemvArgs& a, hipStream_t s);
// The prefill GEMM kernel (gemm.hip): workgroup tiles of 128 batch rows x
// 64 * nt weight rows (nt = 2 or 4, gemm_tile_nt picks by shape), any M >= 1,
// K % 128 == 0, K < 2^24.
int gemm_tile_nt(int M, int N);
long gemm_tiles(int M, int N, int nt);
hipError_t launch_gemm(const GemvArgs& a, int nt, hipStream_t s);
// The int4 tiled kernel with the fused activation prologue and residual
// epilogue (GemvArgs::up, GemvArgs::resid; either may be null).
hipError_t launch_mm_fused(const GemvArgs* tasks, int count, void* ws, size_t ws_bytes, hipStream_t s);

// h_i = RN_bf16(silu(g_i) * u_i) over values[i] elements (a multiple of 8;
// every array 16-byte aligned) for count <= kMaxTasks segments, one launch.
hipError_t launch_silu_mul(const uint16_t* const* g, const uint16_t* const* u, uint16_t* const* h, const size_t* values, int count,
                           hipStream_t s);

// Top-k sampling from BF16 logits [M, V], one workgroup per row (see
// sample.hip); 1 <= top_k <= min(kMaxTopK, V), V <= kMaxVocab.
constexpr int kMaxTopK = 64;
constexpr int kMaxVocab = 30720;
hipError_t launch_topk_sample(const uint16_t* logits, int M, int V, float temperature, int top_k, const float* u, int32_t* token,
                              int32_t* topk_index, float* topk_prob, hipStream_t s);
// The BF16 head GEMV with top-k sampling in one launch (M = 1,
// streaming row sizes, top_k <= 64): workspace bytes it needs (zero-filled,
// left zero), or 0 if the fused launch does not apply.
size_t head_sample_workspace_bytes(int M, int N, int K, int top_k);
// Top-k sampling split over workgroups of 1024 logits per row, the last
// block of each row merging (a workspace: counters a cache line apart per
// row, then candidates); its workspace bytes (0: not applicable).
constexpr int kSplitBlock = 1024;  // logits per workgroup of the split sampler
size_t topk_sample_split_ws_bytes(int M, int V, int top_k);
hipError_t launch_topk_sample_split(const uint16_t* logits, int M, int V, float temperature, int top_k, const float* u,
                                    int32_t* token, int32_t* topk_index, float* topk_prob, void* ws, hipStream_t s);
hipError_t launch_head_sample(const GemvArgs& a, float temperature, int top_k, const float* u, int32_t* token, int32_t* topk_index,
                              float* topk_prob, void* ws, hipStream_t s);

// 16x16x32 BF16 matrix-core GEMV (any M <= 64), one launch per task.
hipError_t launch_mfma(Fmt fmt, const GemvArgs* tasks, int count, hipStream_t s);

// Diagnostic streaming read of up to kMaxReadBufs device buffers (each under
// 4 GiB) in one launch; sink holds stream_read_sink_words() words.
constexpr int kMaxReadBufs = 32;
size_t stream_read_sink_words(const size_t* bytes, int count);
hipError_t launch_stream_read(const void* const* bufs, const size_t* bytes, int count, uint32_t* sink, hipStream_t s);

// Diagnostic dequantization to fp32 [N, K].
hipError_t launch_q4_dequant(const uint8_t* qw, const uint16_t* sc, const uint16_t* mn, int N, int K, float* w, hipStream_t s);
hipError_t launch_nvfp4_dequant(const uint8_t* qw, const uint8_t* sc, float G, int N, int K, float* w, hipStream_t s);

}  // namespace q4
