// Skinny matrix-core GEMV for batched decode with int4 g128 weights
// (5 <= M <= 48, K % 128 == 0; gfx950, v_mfma_f32_16x16x32_bf16).
//
// The decode batch shares one read of the weights: at M = 48 every weight byte
// feeds 48 products ("rumik-oss-1-nvfp4-vllm" card, "Concurrent request
// throughput": one weight read serves many sequences).  The work is cut so
// that a workgroup (eight waves) owns R 16-row tiles over a slice of at most
// 16 groups of K (the whole of K for the hidden-2048 projections), and every
// wave owns distinct groups of that slice: group g0 + 8 r + w for round r of
// wave w.  A wave therefore needs only its own data, and issues all of it at
// once when it starts -- per round the activation fragments of its group (MT
// batch tiles x 4 k-steps, 16 bytes a lane each, from L2) and the group's
// 64 bytes of each of its R x 16 weight rows (one 16-byte load a lane per
// tile, from HBM) -- so a workgroup's whole input is one memory round trip,
// the waves never wait for each other until the end, and each activation byte
// is read once per workgroup.  The group parameters of the workgroup's rows
// are staged in LDS once (one barrier), as fp32 (scale, min - 128 scale).
//
// Per round a wave pairs its activations to match the nibble unpack
// (x0,x4) (x1,x5) (x2,x6) (x3,x7), forms SX (the sum of the group's
// activations per batch row) with an all-ones A operand, and per tile turns
// each lane's 8 codes per k-step into BF16 "128 + code" (v_perm_b32 on the
// 0x43 exponent byte) and accumulates D = sum of (128 + code) * x over the
// group; the group folds as
//     acc += scale * D + (min - 128 scale) * SX,
// exact up to the fp32 roundings (both products and the fold are exact for a
// one-hot x).  The eight waves' partial tiles meet in LDS in a fixed order;
// when K is split over workgroups, each writes its fp32 tile to the caller's
// workspace and the workgroup that arrives last at the row block's counter
// sums the slices in slice order, writes y and resets the counter.
//
// MFMA operand layout (16x16x32): lane l holds A row l % 16 and B column
// l % 16, k-values 8 (l / 16) .. + 8 of the k-step.  For k-step s of a group,
// lane l's k-values are the 8 columns 32 (l / 16) + 8 s .. + 8 of the group
// (in the pairing order): dword s of the lane's 16 weight bytes, and the
// activations at the same columns.  D: lane l holds rows 4 (l / 16) + v
// (v = 0..3) of column l % 16.
#include "internal.h"

namespace q4 {

namespace {

constexpr int kSkWaves = 8;
constexpr int kSkThreads = 64 * kSkWaves;
constexpr int kSkMaxGroups = 16;   // groups per workgroup slice: two rounds of eight waves
constexpr int kSkCoherent = 16;    // buffer cache policy sc1: device-coherent, not held in the per-XCD L2

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8_t as_b8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

struct SkTask {
    GemvArgs a;
    int ks;          // workgroups (K slices) per row block
    int gs;          // groups per slice
    float* part;     // ks > 1: partial tiles [blocks][ks][R * MT][64 lanes] x 4 floats
    unsigned* cnt;   // ks > 1: arrival counters [blocks]
};

struct SkTable {
    int blk0[kMaxTasks];   // first workgroup of each task (unused: INT_MAX)
    SkTask t[kMaxTasks];
};

// LDS: the eight waves' partial tiles [8][R * MT][64 lanes] x 16 bytes
template <int MT, int R>
__host__ __device__ constexpr int sk_lds_bytes() { return kSkWaves * R * MT * 64 * 16; }

// Workgroup barrier that waits only for this wave's LDS traffic, so the
// vector-memory loads in flight stay in flight across it.
__device__ __forceinline__ void lds_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One result tile (16 weight rows x 16 batch rows) to y: lane l holds batch
// rows 16 mt + 4 (l / 16) + v (v = 0..3) of weight row trow + l % 16; the
// task's residual, if any, is added before the one rounding.  (16 lanes
// store 32 contiguous bytes of a batch row.)
__device__ __forceinline__ void sk_write_tile(const SkTask& tk, int trow, int mt, int lane, f32x4 r) {
    const GemvArgs& a = tk.a;
    const int row = trow + (lane & 15);
    if (row >= a.N) return;
    const int m0 = 16 * mt + 4 * (lane >> 4);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = m0 + v;
        if (m >= a.M) break;
        const size_t off = (size_t)m * a.N + row;
        float val = r[v];
        if (a.resid != nullptr) val += __builtin_bit_cast(float, (uint32_t)a.resid[off] << 16);
        a.y[off] = f32_to_bf16(val);
    }
}

template <int MT, int R>
__global__ __launch_bounds__(kSkThreads) void skinny_q4_kernel(SkTable tt) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    int ti = 0;
#pragma unroll
    for (int i = 1; i < kMaxTasks; ++i) ti += ((int)blockIdx.x >= tt.blk0[i]) ? 1 : 0;
    const SkTask& tk = tt.t[ti];
    const GemvArgs& a = tk.a;
    const int KS = tk.ks;
    const int local = (int)blockIdx.x - tt.blk0[ti];
    const int blk = local / KS, ks = local - blk * KS;
    const int G = a.K >> 7;
    const int g0 = ks * tk.gs;
    const int ng = (G - g0 < tk.gs) ? G - g0 : tk.gs;   // groups of this slice, >= 1
    const int nr = (ng + kSkWaves - 1) / kSkWaves;      // rounds per wave: 1 or 2
    const int row0 = blk * 16 * R;
    const int nrows = (a.N - row0 < 16 * R) ? a.N - row0 : 16 * R;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t rowbytes = (uint32_t)a.K >> 1;
    f32x4* red = reinterpret_cast<f32x4*>(lds);   // [8 waves][R * MT][64 lanes]

    // ---- 1. this wave's loads, all at once.  Round r is group g0 + nr w + r
    // (a wave's groups are adjacent, so its weight bytes of a row are whole
    // cache lines).  Per round: the activation fragments (MT x 4 k-steps),
    // then per tile the lane's 16 weight bytes and its row's scale and min
    // (the lane's results share one weight row: row l % 16 of the tile).
    // Loads of a round past the slice fall outside the buffer ranges and
    // read zero, so the wait counts are the same on every path.
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)a.M * (uint32_t)a.K * 2u);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w + (size_t)row0 * rowbytes, (uint32_t)nrows * rowbytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scale + (size_t)row0 * G, (uint32_t)nrows * (uint32_t)G * 2u);
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(a.minv + (size_t)row0 * G, (uint32_t)nrows * (uint32_t)G * 2u);
    const uint32_t xoff0 = ((uint32_t)(lane & 15) * (uint32_t)a.K + 32u * (uint32_t)(lane >> 4)) * 2u;
    const uint32_t woff0 = (uint32_t)(lane & 15) * rowbytes + 16u * (uint32_t)(lane >> 4);
    const uint32_t poff0 = (uint32_t)(lane & 15) * (uint32_t)G * 2u;
    u32x4 X[2][MT][4];
    u32x4 W[2][R];
    uint16_t S16[2][R], M16[2][R];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int gl = nr * wave + r;          // group within the slice
        const bool valid = r < nr && gl < ng;
        const uint32_t g = (uint32_t)(g0 + gl);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint32_t off = valid ? xoff0 + ((uint32_t)(16 * mt) * (uint32_t)a.K + 128u * g + 8u * s) * 2u : 0xFFFFFFF0u;
                X[r][mt][s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
            }
#pragma unroll
        for (int t = 0; t < R; ++t) {
            const uint32_t off = valid ? woff0 + (uint32_t)(16 * t) * rowbytes + 64u * g : 0xFFFFFFF0u;
            W[r][t] = buf_load16(rw, off, 0);
            const uint32_t po = valid ? poff0 + ((uint32_t)(16 * t) * (uint32_t)G + g) * 2u : 0xFFFFFFF0u;
            S16[r][t] = buf_load2(rs, po, 0);
            M16[r][t] = buf_load2(rm, po, 0);
        }
    }

    // ---- 2. the rounds.  D = X . W^T with the activations as the A operand:
    // lane l holds batch rows 4 (l / 16) + v of weight row l % 16.
    const bf16x8_t ones = as_b8(u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    f32x4 acc[R][MT];
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        if (r >= nr || nr * wave + r >= ng) break;   // wave-uniform
        // activations in the pairing of the nibble unpack; SX per batch row
        // (an all-ones B operand: every column of the result is SX)
        u32x4 B[MT][4];
        f32x4 sx[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const u32x4 v = X[r][mt][s];
                uint32_t p[4];
                xq4_pairs(v.x, v.y, v.z, v.w, p);
                B[mt][s] = u32x4{p[0], p[1], p[2], p[3]};
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(B[mt][s]), ones, c, 0, 0, 0);
            }
            sx[mt] = c;
        }
#pragma unroll
        for (int t = 0; t < R; ++t) {
            f32x4 D[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) D[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                uint32_t A[4];
                q4_pairs(W[r][t][s], A);
                const bf16x8_t Wv = as_b8(u32x4{A[0], A[1], A[2], A[3]});
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) D[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(B[mt][s]), Wv, D[mt], 0, 0, 0);
            }
            // acc += scale * D + (min - 128 scale) * SX for the lane's row
            const float sc = f16_to_f32(S16[r][t]);
            const float mq = fmaf(-128.0f, sc, f16_to_f32(M16[r][t]));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[t][mt][v] = fmaf(sc, D[mt][v], fmaf(mq, sx[mt][v], acc[t][mt][v]));
        }
    }

    // ---- 3. the eight waves meet in LDS: each writes its tiles, then each
    // finishes whole tiles, summing the eight in wave order
    constexpr int kTiles = R * MT;
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[(wave * kTiles + t * MT + mt) * 64 + lane] = acc[t][mt];
    lds_sync();
    f32x4 fin[(kTiles + kSkWaves - 1) / kSkWaves];
#pragma unroll
    for (int j = 0; j * kSkWaves < kTiles; ++j) {
        const int p = wave + kSkWaves * j;
        if (p < kTiles) {
            f32x4 v = red[p * 64 + lane];
#pragma unroll
            for (int w = 1; w < kSkWaves; ++w) v += red[(w * kTiles + p) * 64 + lane];
            fin[j] = v;
        }
    }

    // ---- 4. epilogue
    if (KS == 1) {
#pragma unroll
        for (int j = 0; j * kSkWaves < kTiles; ++j) {
            const int p = wave + kSkWaves * j;
            if (p < kTiles) sk_write_tile(tk, row0 + 16 * (p / MT), p % MT, lane, fin[j]);
        }
        return;
    }
    // split K: publish this slice's tiles (device-coherent 16-byte stores, 1 KB
    // contiguous per instruction), then the row block's counter
    const int blocks = (a.N + 16 * R - 1) / (16 * R);
    const __amdgpu_buffer_rsrc_t rpart = make_rsrc(tk.part, (uint32_t)blocks * (uint32_t)KS * (uint32_t)kTiles * 1024u);
#pragma unroll
    for (int j = 0; j * kSkWaves < kTiles; ++j) {
        const int p = wave + kSkWaves * j;
        if (p < kTiles)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, fin[j]), rpart,
                                                   (uint32_t)(((blk * KS + ks) * kTiles + p) * 64 + lane) * 16u, 0, kSkCoherent);
    }
    // The hand-over rests on the device-coherent (sc1) partial accesses, not
    // on agent-scope fences, whose L2 invalidate would evict the activations
    // other workgroups on the XCD are reading: sc1 stores are acknowledged
    // once they reach the device's coherence point, every wave waits for
    // those acknowledgements (vmcnt(0)) before the barrier that precedes the
    // counter update, and the last slice's sc1 loads are issued only after
    // its update returned.  The asm memory clobbers keep the compiler from
    // moving accesses across.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __shared__ unsigned s_prev;
    if (tid == 0) s_prev = __hip_atomic_fetch_add(&tk.cnt[blk], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_prev != (unsigned)(KS - 1)) return;
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j * kSkWaves < kTiles; ++j) {
        const int p = wave + kSkWaves * j;
        if (p >= kTiles) continue;
        // slices in order, four in flight at a time
        f32x4 sum = {0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < KS; s0 += 4) {
            u32x4 pv[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t off = s0 + k < KS ? (uint32_t)(((blk * KS + s0 + k) * kTiles + p) * 64 + lane) * 16u : 0xFFFFFFF0u;
                pv[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rpart, off, 0, kSkCoherent));
            }
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (s0 + k < KS) sum += __builtin_bit_cast(f32x4, pv[k]);
        }
        sk_write_tile(tk, row0 + 16 * (p / MT), p % MT, lane, sum);
    }
    if (tid == 0) __hip_atomic_store(&tk.cnt[blk], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kCUs = 256;

// The launch plan: rows per workgroup (16 R, one R per launch) and per task
// the K slice (the whole of K up to 16 groups, or 16 or 8 groups with a
// workspace).  Cost model per workgroup, in HBM-byte equivalents: its weight
// bytes, its activation bytes (L2, about a fifth of an HBM byte each) and, if
// any slice is split, the partial-tile round trip and counter of the split
// completion; times the number of waves of workgroups over the CUs.
struct SkPlan {
    int R = 0;
    int gs[kMaxTasks];
    int ks[kMaxTasks];
    size_t ws = 0;   // workspace bytes (0: unsplit)
};

constexpr int kSkR[] = {5, 3, 2, 1};

int sk_mt(int M) { return (M + 15) / 16; }

size_t sk_ws_bytes(const GemvArgs* tasks, int count, int R, const int* ks) {
    const int MT = sk_mt(tasks[0].M);
    size_t part = 0, cnt = 0;
    for (int i = 0; i < count; ++i) {
        if (ks[i] <= 1) continue;
        const size_t blocks = (tasks[i].N + 16 * R - 1) / (16 * R);
        part += blocks * ks[i] * R * MT * 1024;
        cnt += blocks * 4;
    }
    if (part == 0) return 0;
    if (cnt > kWsCounterBytes) return (size_t)-1;
    return kWsCounterBytes + part;
}

bool sk_plan(const GemvArgs* tasks, int count, bool can_split, SkPlan& best) {
    const int MT = sk_mt(tasks[0].M);
    double best_cost = 0;
    bool found = false;
    for (int R : kSkR) {
        for (int S : {16, 8}) {
            if (S == 8 && !can_split) continue;
            SkPlan p;
            p.R = R;
            long wgs = 0;
            int smax = 0;
            bool ok = true, split = false;
            for (int i = 0; i < count; ++i) {
                const int G = tasks[i].K >> 7;
                int gs = G <= S ? G : S;
                if (G > kSkMaxGroups && !can_split) { ok = false; break; }
                const int ks = (G + gs - 1) / gs;
                p.gs[i] = gs;
                p.ks[i] = ks;
                split = split || ks > 1;
                smax = gs > smax ? gs : smax;
                wgs += (long)((tasks[i].N + 16 * R - 1) / (16 * R)) * ks;
            }
            if (!ok) continue;
            p.ws = split ? sk_ws_bytes(tasks, count, R, p.ks) : 0;
            if (p.ws == (size_t)-1) continue;
            const double per_wg = 16.0 * R * smax * 64 + 0.19 * smax * MT * 4096 + (split ? 35000.0 : 0.0);
            const double cost = (double)((wgs + kCUs - 1) / kCUs) * per_wg;
            if (!found || cost < best_cost * 0.999) {
                best = p;
                best_cost = cost;
                found = true;
            }
        }
    }
    return found;
}

template <int MT, int R>
hipError_t launch_sk_mt(const GemvArgs* tasks, int count, const SkPlan& p, void* ws, hipStream_t st) {
    SkTable tt{};
    for (int i = 0; i < kMaxTasks; ++i) tt.blk0[i] = 0x7fffffff;
    uint8_t* pc = static_cast<uint8_t*>(ws);
    uint8_t* pp = pc + kWsCounterBytes;
    int grid = 0;
    for (int i = 0; i < count; ++i) {
        const GemvArgs& a = tasks[i];
        const int blocks = (a.N + 16 * R - 1) / (16 * R);
        SkTask& t = tt.t[i];
        tt.blk0[i] = grid;
        t.a = a;
        t.ks = p.ks[i];
        t.gs = p.gs[i];
        if (p.ks[i] > 1) {
            t.cnt = reinterpret_cast<unsigned*>(pc);
            pc += (size_t)blocks * 4;
            t.part = reinterpret_cast<float*>(pp);
            pp += (size_t)blocks * p.ks[i] * R * MT * 1024;
        }
        grid += blocks * p.ks[i];
    }
    constexpr int kShmem = sk_lds_bytes<MT, R>();
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(skinny_q4_kernel<MT, R>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kShmem);
    if (attr != hipSuccess) return attr;
    return launch_kernel(skinny_q4_kernel<MT, R>, dim3(grid), dim3(kSkThreads), (size_t)kShmem, st, tt);
}

template <int MT>
hipError_t launch_sk_r(const GemvArgs* tasks, int count, const SkPlan& p, void* ws, hipStream_t st) {
    switch (p.R) {
        case 5: return launch_sk_mt<MT, 5>(tasks, count, p, ws, st);
        case 3: return launch_sk_mt<MT, 3>(tasks, count, p, ws, st);
        case 2: return launch_sk_mt<MT, 2>(tasks, count, p, ws, st);
        default: return launch_sk_mt<MT, 1>(tasks, count, p, ws, st);
    }
}

}  // namespace

bool skinny_supported(int M, int K, bool split) {
    if (M < 5 || M > kSkinnyMaxM || K % 128 != 0) return false;
    return split || (K >> 7) <= kSkMaxGroups;
}

size_t skinny_workspace_bytes(const GemvArgs* tasks, int count) {
    SkPlan p;
    if (!sk_plan(tasks, count, true, p)) return 0;
    return p.ws;
}

hipError_t launch_skinny(const GemvArgs* tasks, int count, void* ws, size_t ws_bytes, hipStream_t s) {
    SkPlan p;
    const size_t need = skinny_workspace_bytes(tasks, count);
    const bool split = ws != nullptr && need > 0 && ws_bytes >= need;
    if (!sk_plan(tasks, count, split, p)) return hipErrorInvalidValue;
    switch (sk_mt(tasks[0].M)) {
        case 1: return launch_sk_r<1>(tasks, count, p, ws, s);
        case 2: return launch_sk_r<2>(tasks, count, p, ws, s);
        default: return launch_sk_r<3>(tasks, count, p, ws, s);
    }
}

}  // namespace q4
