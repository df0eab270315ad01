// Streaming GEMV for decode batches M <= 4 (gfx950).
//
// Shaped like a plain streaming read: every lane issues all of its 16-byte
// weight loads (4 per lane, 4 KB per wave) at once, right after two small
// shared loads, and nothing on the weight path waits for anything else.
//
//   * A workgroup (4 waves) owns 16 / CPL consecutive rows, where CPL =
//     chunks per lane = row bytes / 1 KB (1, 2 or 4: K = 2048, 4096, 8192 for
//     the 4-bit formats).  A wave owns 4 / CPL whole rows; load i of a lane is
//     chunk (i % CPL) * 64 + lane of row i / CPL, so every wave-wide load is
//     1 KB of consecutive bytes.
//   * The activations x[0..M) are loaded once per workgroup, turned into the
//     operand layout the packed dot products need (plus per-chunk sums for
//     int4) and kept in LDS; so are the group parameters of the workgroup's
//     rows.  Both loads go out before the weight loads, so waiting for them
//     does not wait for the weights.
//   * Rows past N read zeros through buffer-resource range checks and are
//     not stored.
//
// One launch serves up to kMaxTasks GEMVs of one format and batch size; the
// workgroups of a launch are split between tasks by a prefix table.
//
// Fused int4 instances (kFused) also take, per task, an optional second
// activation array `up` -- the activations become RN_bf16(silu(x) * up),
// formed while x is staged -- and an optional residual added to each output
// before its one rounding (it may be the output array itself: each element
// is read and then written by the same lane).
#include <type_traits>

#include "internal.h"
#include "topk.h"

namespace q4 {

namespace {

constexpr int kLoads = 4;    // 16-byte weight loads per lane
constexpr int kWaves = 4;    // waves per workgroup

struct StreamTable {
    int blk0[kMaxTasks];     // first workgroup of each task (unused: INT_MAX)
    int cpl_log2[kMaxTasks];
    int fmt[kMaxTasks];      // weight format of each task (the mixed-format kernel)
    GemvArgs a[kMaxTasks];
    int count;
};

template <class F> struct Stream;

// int4 g128: LDS holds x as 128+code-matching BF16 pairs [M][K], the chunk
// sums [M][K/32] (fp32) and the rows' (scale | min << 16) words [rows][K/128].
template <> struct Stream<FmtQ4> {
    static constexpr int kAuxPerThread = 1;   // (16 / CPL rows) * (16 * CPL groups) = 256 words
    __host__ __device__ static int x_bytes(int MT, int K) { return MT * K * 2; }
    __host__ __device__ static int sum_bytes(int MT, int K) { return MT * (K / 32) * 4; }
    __host__ __device__ static int aux_bytes() { return 256 * 4; }
};
// NVFP4: x raw [M][K]; the rows' e4m3 scale bytes [rows][K/16].
template <> struct Stream<FmtNvfp4> {
    static constexpr int kAuxPerThread = 4;   // (16 / CPL rows) * (128 * CPL bytes) = 2048 bytes = 1024 halves
    __host__ __device__ static int x_bytes(int MT, int K) { return MT * K * 2; }
    __host__ __device__ static int sum_bytes(int, int) { return 0; }
    __host__ __device__ static int aux_bytes() { return 1024 * 2; }
};
// BF16: x raw [M][K], nothing else.
template <> struct Stream<FmtBf16> {
    static constexpr int kAuxPerThread = 0;
    __host__ __device__ static int x_bytes(int MT, int K) { return MT * K * 2; }
    __host__ __device__ static int sum_bytes(int, int) { return 0; }
    __host__ __device__ static int aux_bytes() { return 0; }
};

template <class F>
__host__ __device__ inline int stream_shmem(int MT, int K) {
    return Stream<F>::x_bytes(MT, K) + Stream<F>::sum_bytes(MT, K) + Stream<F>::aux_bytes();
}

// rows a workgroup owns: 16 / CPL for rows up to 4 KB; one row per 4 / wpr
// waves for the split BF16 rows of 8 and 16 KB
__host__ __device__ inline int rows_per_wg(int cl) { return cl > 2 ? kWaves >> (cl - 2) : kWaves * (kLoads >> cl); }

// 16-byte x pieces per thread (x is MT*K*2 bytes over 256 threads)
template <class F> __host__ __device__ inline int x_pieces(int MT, int K) { return (MT * K / 8 + 255) / 256; }

__device__ __forceinline__ int stream_task(const StreamTable& tt) {
    int t = 0;
#pragma unroll
    for (int i = 1; i < kMaxTasks; ++i) t += ((int)blockIdx.x >= tt.blk0[i]) ? 1 : 0;
    return t;
}

constexpr int kAuxCoherent = 16;   // buffer cache policy sc1: device-coherent, not held in the per-XCD L2

// One output element; kCoh: a device-coherent store (read back by other
// workgroups of the same launch).
template <bool kCoh>
__device__ __forceinline__ void store_y(const GemvArgs& a, size_t off, uint16_t v) {
    if constexpr (kCoh) {
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, (uint32_t)((size_t)a.M * a.N * 2));
        __builtin_amdgcn_raw_buffer_store_b16(v, ry, (int)(off * 2), 0, kAuxCoherent);
    } else {
        a.y[off] = v;
    }
}

// One workgroup block of task `a`: blk is the block's index within the task.
template <class F, int MT, bool kFused, bool kCoh = false>
__device__ __forceinline__ void stream_block(const GemvArgs a, const int cl, const int blk, uint8_t* lds) {
    constexpr int kXP = MT * 4;   // most x pieces a thread stages (K <= 8192 for the 4-bit formats)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int CPL = 1 << cl;
    const int C = 64 << cl;                      // chunks per row
    const uint32_t rowbytes = (uint32_t)C * 16;
    // BF16 rows of 8 or 16 KB (cl = 3, 4) are split over wpr = 2 or 4 waves,
    // each taking the row's part-th quarter/half of its chunks
    const int wpr = cl > 2 ? 1 << (cl - 2) : 1;  // waves per row
    const int rpw = cl > 2 ? 1 : kLoads >> cl;   // rows per wave (a part of one row when wpr > 1)
    const int RW = rows_per_wg(cl);              // rows per workgroup
    const int row0 = blk * RW;
    const int wrow0 = row0 + (cl > 2 ? wave / wpr : wave * rpw);
    const int part = cl > 2 ? wave % wpr : 0;
    const int K = a.K;

    // --- 1. shared inputs: x pieces and group parameters into registers
    const int nxp = x_pieces<F>(MT, K);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)(MT * K * 2));
    u32x4 xr[kXP];
#pragma unroll
    for (int i = 0; i < kXP; ++i)
        xr[i] = i < nxp ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (tid + 256 * i) * 16, 0, 0))
                        : u32x4{0, 0, 0, 0};
    const bool gated = kFused && a.up != nullptr;
    u32x4 xu[kFused ? kXP : 1];
    if constexpr (kFused) {
        if (gated) {
            const __amdgpu_buffer_rsrc_t ru = make_rsrc(a.up, (uint32_t)(MT * K * 2));
#pragma unroll
            for (int i = 0; i < kXP; ++i)
                xu[i] = i < nxp ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ru, (tid + 256 * i) * 16, 0, 0))
                                : u32x4{0, 0, 0, 0};
        }
    }
    int wg_rows = a.N - row0;
    wg_rows = wg_rows < 0 ? 0 : (wg_rows > RW ? RW : wg_rows);
    uint32_t auxr[Stream<F>::kAuxPerThread > 0 ? Stream<F>::kAuxPerThread : 1];
    if constexpr (Stream<F>::kAuxPerThread > 0) {
        if constexpr (std::is_same<F, FmtQ4>::value) {
            const int G = K >> 7;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scale + (size_t)row0 * G, (uint32_t)(wg_rows * G * 2));
            const __amdgpu_buffer_rsrc_t rm = make_rsrc(a.minv + (size_t)row0 * G, (uint32_t)(wg_rows * G * 2));
            auxr[0] = (uint32_t)buf_load2(rs, tid * 2, 0) | ((uint32_t)buf_load2(rm, tid * 2, 0) << 16);
        } else {
            const int SB = K >> 4;   // scale bytes per row
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scale8 + (size_t)row0 * SB, (uint32_t)(wg_rows * SB));
#pragma unroll
            for (int i = 0; i < Stream<F>::kAuxPerThread; ++i) auxr[i] = buf_load2(rs, (tid + 256 * i) * 2, 0);
        }
    }

    // --- 2. the weights: all of this lane's loads at once
    int nrows = a.N - wrow0;
    nrows = nrows < 0 ? 0 : (nrows > rpw ? rpw : nrows);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w + (size_t)wrow0 * rowbytes, (uint32_t)nrows * rowbytes);
    u32x4 q[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const uint32_t r = (uint32_t)(i >> cl), j = (uint32_t)(i & (CPL - 1)) + (uint32_t)(part * kLoads);
        q[i] = buf_load16(rw, r * rowbytes + (j * 64 + lane) * 16, 0);
    }
    // fused: the residuals of the wave's rows (rows past N read as zero)
    float res[kFused ? kLoads : 1][kFused ? MT : 1];
    if constexpr (kFused) {
        const bool has_res = a.resid != nullptr;
        const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.resid, has_res ? (uint32_t)(MT * a.N * 2) : 0u);
#pragma unroll
        for (int r = 0; r < kLoads; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int row = wrow0 + r;
                const bool ok = has_res && r < rpw && row < a.N;
                res[r][m] = ok ? __builtin_bit_cast(float, (uint32_t)buf_load2(rr, (uint32_t)(((size_t)m * a.N + row) * 2), 0) << 16) : 0.f;
            }
    }

    // --- 3. stage x (and int4 chunk sums) and the group parameters in LDS
    uint8_t* xs = lds;
    float* sums = reinterpret_cast<float*>(lds + Stream<F>::x_bytes(MT, K));
    uint8_t* auxs = lds + Stream<F>::x_bytes(MT, K) + Stream<F>::sum_bytes(MT, K);
#pragma unroll
    for (int i = 0; i < kXP; ++i) {
        if (i < nxp) {
            const int p = tid + 256 * i;   // piece index over [MT][K/8]
            const bool in = p < MT * K / 8;
            if constexpr (std::is_same<F, FmtQ4>::value) {
                if (gated)
                    xr[i] = u32x4{silu_mul_bf16x2(xr[i].x, xu[i].x), silu_mul_bf16x2(xr[i].y, xu[i].y),
                                  silu_mul_bf16x2(xr[i].z, xu[i].z), silu_mul_bf16x2(xr[i].w, xu[i].w)};
                uint32_t pr[4];
                xq4_pairs(xr[i].x, xr[i].y, xr[i].z, xr[i].w, pr);
                if (in) *reinterpret_cast<u32x4*>(xs + p * 16) = u32x4{pr[0], pr[1], pr[2], pr[3]};
                // chunk (32 activations) = 4 consecutive pieces = 4 consecutive lanes
                float s = dot2(xr[i].x, 0x3F803F80u, 0.f);
                s = dot2(xr[i].y, 0x3F803F80u, s);
                s = dot2(xr[i].z, 0x3F803F80u, s);
                s = dot2(xr[i].w, 0x3F803F80u, s);
                s += dpp<0xB1>(s);
                s += dpp<0x4E>(s);
                if (in && (lane & 3) == 0) sums[p >> 2] = s;
            } else {
                if (in) *reinterpret_cast<u32x4*>(xs + p * 16) = xr[i];
            }
        }
    }
    if constexpr (std::is_same<F, FmtQ4>::value) {
        reinterpret_cast<uint32_t*>(auxs)[tid] = auxr[0];
    } else if constexpr (std::is_same<F, FmtNvfp4>::value) {
#pragma unroll
        for (int i = 0; i < Stream<F>::kAuxPerThread; ++i) reinterpret_cast<uint16_t*>(auxs)[tid + 256 * i] = (uint16_t)auxr[i];
    }
    __syncthreads();

    // --- 4. rows
    const uint16_t* aux16 = reinterpret_cast<const uint16_t*>(auxs);
    auto read_x = [&](int c, typename F::X (&xc)[MT]) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if constexpr (std::is_same<F, FmtBf16>::value) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(xs + (size_t)m * K * 2 + c * 16);
                xc[m].p[0] = v.x; xc[m].p[1] = v.y; xc[m].p[2] = v.z; xc[m].p[3] = v.w;
            } else {
                const u32x4* src = reinterpret_cast<const u32x4*>(xs + (size_t)m * K * 2 + c * 64);
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const u32x4 v = src[d];
                    xc[m].p[4 * d + 0] = v.x; xc[m].p[4 * d + 1] = v.y; xc[m].p[4 * d + 2] = v.z; xc[m].p[4 * d + 3] = v.w;
                }
                if constexpr (std::is_same<F, FmtQ4>::value) xc[m].sum = sums[m * (K / 32) + c];
            }
        }
    };
    auto read_aux = [&](int rl, int c) {
        typename F::Aux ax{};
        if constexpr (std::is_same<F, FmtQ4>::value) {
            const uint32_t v = reinterpret_cast<const uint32_t*>(auxs)[rl * (K >> 7) + (c >> 2)];
            ax.s = f16_to_f32((uint16_t)(v & 0xFFFFu));
            ax.m = f16_to_f32((uint16_t)(v >> 16));
        } else if constexpr (std::is_same<F, FmtNvfp4>::value) {
            const uint32_t b = aux16[rl * (K >> 5) + c];
            ax.s0 = e4m3_to_f32<0>(b);
            ax.s1 = e4m3_to_f32<1>(b);
        }
        return ax;
    };
    auto finish_row = [&](int r, float (&out)[MT]) {
        const int row = wrow0 + r;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float v = out[m];
            v += dpp<0xB1>(v);
            v += dpp<0x4E>(v);
            v += dpp<0x141>(v);
            v += dpp<0x140>(v);
            v += dpp<0x142, 0xA>(v);
            v += dpp<0x143, 0xC>(v);
            if constexpr (kFused) v += res[r][m];   // (F::finish is the identity for int4)
            if (lane == 63 && row < a.N) store_y<kCoh>(a, (size_t)m * a.N + row, f32_to_bf16(F::finish(a, v)));
            out[m] = 0.f;
        }
    };

    float out[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) out[m] = 0.f;
    if (cl == 0) {
        // one chunk per lane: the lane's activations are the same for every row
        typename F::X xc[MT];
        read_x(lane, xc);
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            F::template accumulate<MT>(q[i], read_aux(wave * rpw + i, lane), xc, out);
            finish_row(i, out);
        }
    } else if (cl <= 2) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int r = i >> cl, c = (i & (CPL - 1)) * 64 + lane;
            typename F::X xc[MT];
            read_x(c, xc);
            F::template accumulate<MT>(q[i], read_aux(wave * rpw + r, c), xc, out);
            if ((i & (CPL - 1)) == CPL - 1) finish_row(r, out);
            if constexpr (kFused) __builtin_amdgcn_sched_barrier(0);
        }
    } else if constexpr (std::is_same<F, FmtBf16>::value) {
        // a part of one row: reduce it in the wave, add the parts of the row in
        // wave order through LDS, and let the row's first wave store it
        __shared__ float parts[kWaves][MT];
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            typename F::X xc[MT];
            read_x((part * kLoads + i) * 64 + lane, xc);
            F::template accumulate<MT>(q[i], read_aux(0, 0), xc, out);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float v = out[m];
            v += dpp<0xB1>(v);
            v += dpp<0x4E>(v);
            v += dpp<0x141>(v);
            v += dpp<0x140>(v);
            v += dpp<0x142, 0xA>(v);
            v += dpp<0x143, 0xC>(v);
            if (lane == 63) parts[wave][m] = v;
        }
        __syncthreads();
        if (part == 0 && lane == 63 && wrow0 < a.N) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float v = parts[wave][m];
                for (int p = 1; p < wpr; ++p) v += parts[wave + p][m];
                store_y<kCoh>(a, (size_t)m * a.N + wrow0, f32_to_bf16(F::finish(a, v)));
            }
        }
    }
}

template <class F, int MT, bool kFused>
__global__ __launch_bounds__(256) void gemv_stream_kernel(StreamTable tt) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int t = stream_task(tt);
    stream_block<F, MT, kFused>(tt.a[t], tt.cpl_log2[t], blockIdx.x - tt.blk0[t], lds);
}

// One launch over tasks of different weight formats (the NVFP4 decode step's
// BF16 projections beside its NVFP4 ones): each workgroup runs its task's
// format; the launch's registers are the widest format's.
template <int MT>
__global__ __launch_bounds__(256) void gemv_stream_mixed_kernel(StreamTable tt) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int t = stream_task(tt);
    const int blk = blockIdx.x - tt.blk0[t];
    switch (tt.fmt[t]) {
        case kFmtQ4: stream_block<FmtQ4, MT, false>(tt.a[t], tt.cpl_log2[t], blk, lds); break;
        case kFmtNvfp4: stream_block<FmtNvfp4, MT, false>(tt.a[t], tt.cpl_log2[t], blk, lds); break;
        default: stream_block<FmtBf16, MT, false>(tt.a[t], tt.cpl_log2[t], blk, lds); break;
    }
}

// rows of 1, 2 or 4 KB (64 << cl chunks); BF16 also 8 and 16 KB rows, split
// over 2 or 4 waves
template <class F> int chunk_log2(int K) {
    const int wpc = F::WPC;
    if (K % wpc) return -1;
    const int C = K / wpc;
    const int max_l = std::is_same<F, FmtBf16>::value ? 4 : 2;
    for (int l = 0; l <= max_l; ++l)
        if (C == (64 << l)) return l;
    return -1;
}

template <class F, int MT, bool kFused>
hipError_t launch_stream_mt(const GemvArgs* tasks, int count, hipStream_t st) {
    StreamTable tt{};
    for (int i = 0; i < kMaxTasks; ++i) tt.blk0[i] = 0x7fffffff;
    int grid = 0, shmem = 0;
    for (int i = 0; i < count; ++i) {
        const int cl = chunk_log2<F>(tasks[i].K);
        const int rw = rows_per_wg(cl);
        tt.blk0[i] = grid;
        tt.cpl_log2[i] = cl;
        tt.a[i] = tasks[i];
        grid += (tasks[i].N + rw - 1) / rw;
        const int sh = stream_shmem<F>(MT, tasks[i].K);
        shmem = sh > shmem ? sh : shmem;
    }
    tt.count = count;
    return launch_kernel(gemv_stream_kernel<F, MT, kFused>, dim3(grid), dim3(256), (size_t)shmem, st, tt);
}

template <class F, bool kFused = false>
hipError_t launch_stream_fmt(const GemvArgs* tasks, int count, hipStream_t st) {
    switch (tasks[0].M) {
        case 1: return launch_stream_mt<F, 1, kFused>(tasks, count, st);
        case 2: return launch_stream_mt<F, 2, kFused>(tasks, count, st);
        case 3: return launch_stream_mt<F, 3, kFused>(tasks, count, st);
        default: return launch_stream_mt<F, 4, kFused>(tasks, count, st);
    }
}

// (256 bytes of margin for the kernel's own LDS: the split rows' partial sums)
template <class F> bool stream_ok(int M, int K) {
    return M >= 1 && M <= kStreamMaxM && chunk_log2<F>(K) >= 0 && stream_shmem<F>(M, K) + 256 <= kStreamMaxShmem;
}

}  // namespace

bool stream_supported(Fmt fmt, int M, int K) {
    switch (fmt) {
        case kFmtQ4: return stream_ok<FmtQ4>(M, K);
        case kFmtNvfp4: return stream_ok<FmtNvfp4>(M, K);
        default: return stream_ok<FmtBf16>(M, K);
    }
}

hipError_t launch_stream(Fmt fmt, const GemvArgs* tasks, int count, hipStream_t s) {
    switch (fmt) {
        case kFmtQ4: return launch_stream_fmt<FmtQ4>(tasks, count, s);
        case kFmtNvfp4: return launch_stream_fmt<FmtNvfp4>(tasks, count, s);
        default: return launch_stream_fmt<FmtBf16>(tasks, count, s);
    }
}

hipError_t launch_stream_fused(const GemvArgs* tasks, int count, hipStream_t s) {
    return launch_stream_fmt<FmtQ4, true>(tasks, count, s);
}

namespace {

template <int MT>
hipError_t launch_stream_mixed_mt(const Fmt* fmts, const GemvArgs* tasks, int count, hipStream_t st) {
    StreamTable tt{};
    for (int i = 0; i < kMaxTasks; ++i) tt.blk0[i] = 0x7fffffff;
    int grid = 0, shmem = 0;
    for (int i = 0; i < count; ++i) {
        const int K = tasks[i].K;
        int cl, sh;
        if (fmts[i] == kFmtQ4) { cl = chunk_log2<FmtQ4>(K); sh = stream_shmem<FmtQ4>(MT, K); }
        else if (fmts[i] == kFmtNvfp4) { cl = chunk_log2<FmtNvfp4>(K); sh = stream_shmem<FmtNvfp4>(MT, K); }
        else { cl = chunk_log2<FmtBf16>(K); sh = stream_shmem<FmtBf16>(MT, K); }
        const int rw = rows_per_wg(cl);
        tt.blk0[i] = grid;
        tt.cpl_log2[i] = cl;
        tt.fmt[i] = fmts[i];
        tt.a[i] = tasks[i];
        grid += (tasks[i].N + rw - 1) / rw;
        shmem = sh > shmem ? sh : shmem;
    }
    tt.count = count;
    return launch_kernel(gemv_stream_mixed_kernel<MT>, dim3(grid), dim3(256), (size_t)shmem, st, tt);
}

}  // namespace

hipError_t launch_stream_mixed(const Fmt* fmts, const GemvArgs* tasks, int count, hipStream_t s) {
    switch (tasks[0].M) {
        case 1: return launch_stream_mixed_mt<1>(fmts, tasks, count, s);
        case 2: return launch_stream_mixed_mt<2>(fmts, tasks, count, s);
        case 3: return launch_stream_mixed_mt<3>(fmts, tasks, count, s);
        default: return launch_stream_mixed_mt<4>(fmts, tasks, count, s);
    }
}


// ---------------------------------------------------------------------------
// The BF16 head GEMV with top-k sampling in the same launch (M = 1).
//
// The workgroups run the streaming BF16 GEMV and store their logits
// device-coherently.  They are grouped into super-blocks of consecutive
// workgroups; the last workgroup to finish in a super-block (an arrival
// counter tree) reads the super-block's logits back and selects, per batch row,
// the top k entries (topk.h).  With one super-block (heads up to 3072 rows)
// that workgroup also sorts and draws; otherwise it publishes the k entries
// as candidates, and the last super-block to finish selects the top k of all
// candidates, sorts and draws.  Nothing waits on another workgroup, and every
// counter is back at zero when the launch ends.  Atomics on one cache line
// serialize (about 12 ns each), so arrivals go through a tree of counters
// on separate lines, with at most 16 arrivals at the first level.  The
// hand-overs are those of
// the split-K completion: device-coherent (sc1) stores, a wait for their
// acknowledgements and a barrier before the counter update, sc1 loads after
// it.
// ---------------------------------------------------------------------------
namespace {

constexpr int kHsE = 12;                       // entries per thread in one selection
constexpr int kHsMaxEntries = 256 * kHsE;      // rows of a super-block, candidates of all
constexpr int kHsFan = 16;                     // workgroups per first-level counter
constexpr int kHsCtrWords = kCtrWords;         // counters a cache line apart

struct HsArgs {
    GemvArgs a;          // the head GEMV; a.y receives the logits
    int cl, nwg;         // row chunking and GEMV workgroups
    int sbw, nsb;        // workgroups per super-block, super-blocks
    int k;
    float temperature;
    const float* u;
    int32_t* token;
    int32_t* topk_index;
    float* topk_prob;
    unsigned* cnt;       // arrival counters, zero, kHsCtrWords apart: [0, nsb) super-blocks,
                         // [nsb] all, [nsb + 1 + g] first-level group g (workgroups 16 g ..)
    uint32_t* cand;      // [M][nsb][k] candidate entries (nsb > 1)
};

template <int MT>
__global__ __launch_bounds__(256) void head_sample_kernel(HsArgs h) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ uint32_t lists[4 * 64];
    __shared__ uint32_t scratch[4 * 64 * kHsE];
    __shared__ unsigned s_prev;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int blk = blockIdx.x;
    stream_block<FmtBf16, MT, false, true>(h.a, h.cl, blk, lds);

    // stage 1: the super-block's rows, once all of its workgroups are done
    // (its first-level groups of 16, then the super-block's count of groups)
    const int g1 = blk / kHsFan;
    const int g1_wgs = (h.nwg - g1 * kHsFan < kHsFan) ? h.nwg - g1 * kHsFan : kHsFan;
    if (!arrive_last(h.cnt + (size_t)(h.nsb + 1 + g1) * kHsCtrWords, g1_wgs, tid, &s_prev)) return;
    const int sb = blk / h.sbw;
    const int sb_wgs = (h.nwg - sb * h.sbw < h.sbw) ? h.nwg - sb * h.sbw : h.sbw;
    if (!arrive_last(h.cnt + (size_t)sb * kHsCtrWords, (sb_wgs + kHsFan - 1) / kHsFan, tid, &s_prev)) return;
    const int N = h.a.N, k = h.k;
    const int rw = rows_per_wg(h.cl);
    const int r0 = sb * h.sbw * rw;
    const int r1 = (N < r0 + sb_wgs * rw) ? N : r0 + sb_wgs * rw;
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(h.a.y, (uint32_t)(MT * N * 2));
#pragma unroll 1
    for (int m = 0; m < MT; ++m) {
        // every load issued before any is used (rows past the block read as
        // zero through the range check and are masked to the empty entry)
        uint32_t v[kHsE];
#pragma unroll
        for (int j = 0; j < kHsE; ++j) {
            const int row = r0 + tid + 256 * j;
            const uint32_t off = row < r1 ? (uint32_t)(m * N + row) * 2u : 0xFFFFFFF0u;
            v[j] = __builtin_amdgcn_raw_buffer_load_b16(ry, (int)off, 0, kAuxCoherent);
        }
#pragma unroll
        for (int j = 0; j < kHsE; ++j) {
            const int row = r0 + tid + 256 * j;
            v[j] = topk_entry(v[j], row) & (row < r1 ? 0xFFFFFFFFu : 0u);
        }
        const uint32_t top = wg_topk<kHsE>(v, k, lists, scratch, wave, lane);
        if (wave == 0) {
            if (h.nsb == 1) {
                draw_sorted(top, k, h.temperature, h.u[m], lane, h.token + m, h.topk_index ? h.topk_index + m * k : nullptr,
                              h.topk_prob ? h.topk_prob + m * k : nullptr);
            } else if (lane < k) {
                const __amdgpu_buffer_rsrc_t rc = make_rsrc(h.cand, (uint32_t)(MT * h.nsb * k * 4));
                __builtin_amdgcn_raw_buffer_store_b32(top, rc, ((m * h.nsb + sb) * k + lane) * 4, 0, kAuxCoherent);
            }
        }
    }
    if (h.nsb == 1) return;

    // stage 2: all super-blocks' candidates
    if (!arrive_last(h.cnt + (size_t)h.nsb * kHsCtrWords, h.nsb, tid, &s_prev)) return;
    const int nc = h.nsb * k;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(h.cand, (uint32_t)(MT * nc * 4));
#pragma unroll 1
    for (int m = 0; m < MT; ++m) {
        uint32_t v[kHsE];
#pragma unroll
        for (int j = 0; j < kHsE; ++j) {
            const int i = tid + 256 * j;
            const uint32_t off = i < nc ? (uint32_t)(m * nc + i) * 4u : 0xFFFFFFF0u;
            v[j] = __builtin_amdgcn_raw_buffer_load_b32(rc, (int)off, 0, kAuxCoherent);
        }
        const uint32_t top = wg_topk<kHsE>(v, k, lists, scratch, wave, lane);
        if (wave == 0)
            draw_sorted(top, k, h.temperature, h.u[m], lane, h.token + m, h.topk_index ? h.topk_index + m * k : nullptr,
                          h.topk_prob ? h.topk_prob + m * k : nullptr);
    }
}

struct HsPlan {
    int cl = -1, rw = 0, nwg = 0, sbw = 0, nsb = 0;
    size_t ws = 0;
};

size_t hs_counter_bytes(const HsPlan& p) {
    return (size_t)(p.nsb + 1 + (p.nwg + kHsFan - 1) / kHsFan) * kHsCtrWords * 4;
}

bool hs_plan(int M, int N, int K, int k, HsPlan& p) {
    // one batch row: the last workgroup selects and draws row after row, so
    // for M > 1 the two launches (one sampling workgroup per row) are faster
    if (M != 1 || k < 1 || k > 64 || N < k || !stream_ok<FmtBf16>(M, K)) return false;
    p.cl = chunk_log2<FmtBf16>(K);
    p.rw = rows_per_wg(p.cl);
    p.nwg = (N + p.rw - 1) / p.rw;
    if (p.nwg * p.rw <= kHsMaxEntries) {
        p.sbw = p.nwg;
        p.nsb = 1;
    } else {
        p.sbw = 128;
        while ((size_t)((p.nwg + p.sbw - 1) / p.sbw) * k > (size_t)kHsMaxEntries) p.sbw *= 2;
        if (p.sbw * p.rw > kHsMaxEntries) return false;
        p.nsb = (p.nwg + p.sbw - 1) / p.sbw;
    }
    p.ws = hs_counter_bytes(p) + (p.nsb > 1 ? (size_t)M * p.nsb * k * 4 : 0);
    return true;
}

template <int MT>
hipError_t launch_hs_mt(const GemvArgs& a, const HsPlan& p, int k, float temperature, const float* u, int32_t* token,
                        int32_t* topk_index, float* topk_prob, void* ws, hipStream_t st) {
    HsArgs h{};
    h.a = a;
    h.cl = p.cl;
    h.nwg = p.nwg;
    h.sbw = p.sbw;
    h.nsb = p.nsb;
    h.k = k;
    h.temperature = temperature;
    h.u = u;
    h.token = token;
    h.topk_index = topk_index;
    h.topk_prob = topk_prob;
    h.cnt = static_cast<unsigned*>(ws);
    h.cand = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + hs_counter_bytes(p));
    return launch_kernel(head_sample_kernel<MT>, dim3(p.nwg), dim3(256), (size_t)stream_shmem<FmtBf16>(MT, a.K), st, h);
}

}  // namespace

size_t head_sample_workspace_bytes(int M, int N, int K, int top_k) {
    HsPlan p;
    return hs_plan(M, N, K, top_k, p) ? p.ws : 0;
}

hipError_t launch_head_sample(const GemvArgs& a, float temperature, int top_k, const float* u, int32_t* token, int32_t* topk_index,
                              float* topk_prob, void* ws, hipStream_t s) {
    HsPlan p;
    if (!hs_plan(a.M, a.N, a.K, top_k, p)) return hipErrorInvalidValue;
    switch (a.M) {
        case 1: return launch_hs_mt<1>(a, p, top_k, temperature, u, token, topk_index, topk_prob, ws, s);
        case 2: return launch_hs_mt<2>(a, p, top_k, temperature, u, token, topk_index, topk_prob, ws, s);
        case 3: return launch_hs_mt<3>(a, p, top_k, temperature, u, token, topk_index, topk_prob, ws, s);
        default: return launch_hs_mt<4>(a, p, top_k, temperature, u, token, topk_index, topk_prob, ws, s);
    }
}

}  // namespace q4
