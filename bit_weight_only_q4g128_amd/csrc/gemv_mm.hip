// Tiled matrix-core GEMV for batched decode (gfx950, v_mfma_f32_16x16x32_bf16):
// int4 g128 weights, and with the same structure NVFP4 and BF16 weights (see
// the end of this comment).
//
// A workgroup owns a block of 64 weight rows and one slice of K (the whole of
// K unless the row blocks alone cannot give every CU the same work; see the
// split plan).  The slice is cut into
// two halves that the workgroup walks side by side, and it runs six waves:
//
//   * four compute waves, one per (32-row pair, K half).  A compute wave
//     issues only weight loads (kPre 128-column groups ahead), so its in-order
//     waits on the vector-memory counter never stall behind anything but its
//     own weights.  Per group it turns its 2 x 16 bytes per lane into BF16
//     "128 + code" operands for its two 16-row tiles and runs 4 k-steps x MT
//     batch tiles x 2 row tiles of MFMA with the activations as the B operand
//     (each activation fragment read from LDS once serves both row tiles),
//     giving D = sum of (128 + code) * x; beside them one chain per batch tile
//     with an all -128 A operand gives C = -128 * SX (SX = sum of x over the
//     group), and the group folds as
//         acc += scale * (D + C) + min * SX   (min staged as -min / 128),
//     exact up to the fp32 rounding of D + C (exact when one product is
//     nonzero);
//   * two loader waves, one per K half, that stream the activations of each
//     128-column group (MT*16 batch rows) from L2 through registers into a
//     double-buffered LDS ring.  Each load reads four whole rows of the group
//     (1 KB contiguous, so every load fills whole cache lines); the writes
//     scatter them into B-fragment order, in the column pairing of the weight
//     operand.

// One barrier per group step keeps the ring in step.  At the end the two K
// halves meet in LDS.  When K is split over several workgroups, each writes
// its fp32 partial tile to a caller-provided workspace; the workgroup that
// arrives last at the block's counter sums the partials in slice order, so the
// result does not depend on timing, writes y and resets the counter to zero.
//
// NVFP4 (VoxCPM2-NVFP4 card, "What was quantized") and BF16 weights run the
// same kernel: the A operand of a k-step is the lane's 8 E2M1 codes times the
// e4m3 scale of their 16-column group, rounded to BF16 (exact: at most 6
// significant bits), or the 16 bytes of BF16 weights themselves (one load per
// k-step, one group in flight); the activations stay in natural column order,
// D accumulates per group without a fold, and NVFP4 outputs are scaled by the
// global scale G.
//
// MFMA operand layout (16x16x32): lane l holds A row l % 16 and B column
// l % 16; for k-step s it holds the 8 columns 32 * (l / 16) + 8 * s .. + 8 of
// the group (any fixed assignment works as long as A and B agree), so one
// 16-byte load per lane fetches all four k-steps of a row's group.  D: lane l
// holds rows 4 * (l / 16) + v (v = 0..3) of column l % 16.
#include <type_traits>

#include "internal.h"

namespace q4 {

namespace {

constexpr int kRows = 64;        // rows per workgroup
constexpr int kCompute = 4;      // compute waves: 2 row pairs x 2 K halves
constexpr int kLoaders = 2;      // activation loader waves, one per K half
constexpr int kThreads = 64 * (kCompute + kLoaders);
constexpr int kLdsBudget = 80 * 1024;   // two workgroups per CU (160 KB of LDS)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Weight formats of the tiled kernel.  kLoads: 16-byte loads per lane for one
// 16-row tile's 128-column group (the group is 64 bytes of a row for the
// 4-bit formats, 256 for BF16); kPre: weight groups a compute lane keeps in
// flight beyond the current one.
template <class F> struct MmFmt;
template <> struct MmFmt<FmtQ4> { static constexpr int kLoads = 1, kPre = 2; };
template <> struct MmFmt<FmtNvfp4> { static constexpr int kLoads = 1, kPre = 2; };
template <> struct MmFmt<FmtBf16> { static constexpr int kLoads = 4, kPre = 1; };
template <class F> __host__ __device__ constexpr bool is_q4() { return std::is_same<F, FmtQ4>::value; }

struct MmTask {
    GemvArgs a;
    int ks;            // workgroups per row block (K slices)
    int gps;           // 128-column groups per slice
    int smw;           // group parameters can be read in pieces of smw (8 or 4) groups, 0: one by one
    int y8;            // y rows can be written 8 bytes at a time (y 8-byte aligned, N % 4 == 0)
    int fmt;           // weight format (the mixed-format kernel)
    float* part;       // partial tiles (ks > 1): [blocks][ks][4 tiles][MT][64 lanes] x 4 floats
    unsigned* cnt;     // arrival counters (ks > 1): [blocks], kCtrStride bytes apart
};

struct MmTable {
    int blk0[kMaxTasks];   // first workgroup of each task (unused: INT_MAX)
    MmTask t[kMaxTasks];
};

// waves per SIMD the register budget is cut for: two 6-wave workgroups per
// CU need four when their waves land unevenly on the SIMDs (up to three batch
// tiles; four tiles fit one workgroup per CU)
template <int MT>
__host__ __device__ constexpr int mm_waves() { return MT <= 3 ? 4 : 2; }
// the fused instances' loaders also hold the up activations: 3 waves per
// SIMD (168 registers) still keep two 6-wave workgroups per CU
template <int MT, bool kFused>
__host__ __device__ constexpr int mm_waves_f() { return kFused && MT <= 3 ? 3 : mm_waves<MT>(); }
// activation groups a loader keeps in flight (registers: 4 * MT pieces each)
template <int MT>
__host__ __device__ constexpr int mm_xp() { return MT <= 1 ? 2 : 1; }
// LDS: ring [2 slots][2 halves][MT][4 k-steps][64 lanes] x 16 bytes, group
// parameters [groups][64 rows] x (scale, min)
template <int MT>
__host__ __device__ constexpr int mm_ring_bytes() { return 2 * 2 * MT * 4 * 64 * 16; }
template <class F, int MT>
__host__ __device__ inline int mm_shmem(int gps) { return mm_ring_bytes<MT>() + (is_q4<F>() ? gps * kRows * 8 : 0); }
// most groups per slice whose parameters fit the LDS budget (int4 only; the
// NVFP4 scales go straight to registers)
template <class F, int MT>
constexpr int mm_max_gps() { return is_q4<F>() ? (kLdsBudget - mm_ring_bytes<MT>()) / (kRows * 8) : (1 << 20); }

// Workgroup barrier for the main loops: waits only for this wave's LDS
// traffic (lgkmcnt) and fences the compiler, so vector-memory loads (the
// weight and activation prefetch) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS slot of fragment lane L in a k-step s fragment (1 KB, 64 slots of 16
// bytes).  The loaders scatter whole activation rows into fragment order, 8
// consecutive lanes of a write landing in four fragments; the XOR puts those 8
// lanes, and any 8 consecutive lanes of a fragment read, on 8 distinct
// 16-byte bank groups (of 128 bytes).
__device__ __forceinline__ int frag_slot(int L, int s) { return L ^ (2 * s + ((L >> 4) & 1)); }

// Workspace layout, the same for every call so that calls with different
// tasks can share one workspace: the arrival counters of all split tasks of a
// call in the first kCntBytes (every call leaves them zero), partial tiles
// after them.
constexpr size_t kCntBytes = kWsCounterBytes;
constexpr int kCoherent = 16;   // buffer cache policy sc1: device-coherent, not held in the per-XCD L2

// slices whose partial tile a reducing wave loads at once (4 * MT registers
// per lane each)
template <int MT>
__host__ __device__ constexpr int mm_reduce_batch() { return 24 / MT; }

// Byte offset of a partial tile: row block blk, K slice ks of KS, row pair
// rp, row tile t, batch tile mt, lane.
template <int MT>
__device__ __forceinline__ uint32_t part_off(int blk, int KS, int ks, int rp, int t, int mt, int lane) {
    return (uint32_t)(((((blk * KS + ks) * 4 + rp * 2 + t) * MT + mt) * 64 + lane) * 16);
}

// y for one 16-row tile: lane l holds rows trow0 + 4 (l / 16) + v (v = 0..3)
// of batch row 16 mt + l % 16; write_y does the two tiles of a row pair.
// (times gs: the NVFP4 global scale, 1 otherwise)
// Fused instances add the residual (read by the lane that then writes the
// same elements, so it may be y itself) before the one rounding; every
// residual read of a call is issued before its first store (with y possibly
// the residual, a read after a store could not be moved ahead of it).
template <int MT>
__device__ __forceinline__ void add_resid_tile(const GemvArgs& a, int trow0, int lane, f32x4 (&rv)[MT]) {
    const int row = trow0 + 4 * (lane >> 4);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + (lane & 15);
        if (m >= a.M || row >= a.N) continue;
        const uint16_t* rs = a.resid + (size_t)m * a.N + row;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (row + q < a.N) rv[mt][q] += __builtin_bit_cast(float, (uint32_t)rs[q] << 16);
    }
}
template <int MT>
__device__ __forceinline__ void store_y_tile(const GemvArgs& a, bool y8, int trow0, int lane, const f32x4 (&rv)[MT]) {
    const int row = trow0 + 4 * (lane >> 4);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + (lane & 15);
        if (m >= a.M || row >= a.N) continue;
        uint16_t* dst = a.y + (size_t)m * a.N + row;
        const f32x4 r = rv[mt];
        if (y8 && row + 3 < a.N) {
            const uint32_t lo = (uint32_t)f32_to_bf16(r.x) | ((uint32_t)f32_to_bf16(r.y) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16(r.z) | ((uint32_t)f32_to_bf16(r.w) << 16);
            *reinterpret_cast<uint2*>(dst) = uint2{lo, hi};
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (row + q < a.N) dst[q] = f32_to_bf16(r[q]);
        }
    }
}
template <int MT, bool kFused = false>
__device__ __forceinline__ void write_y_tile(const GemvArgs& a, bool y8, float gs, int trow0, int lane, const f32x4 (&v)[MT]) {
    f32x4 rv[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) rv[mt] = v[mt] * gs;
    if constexpr (kFused)
        if (a.resid != nullptr) add_resid_tile<MT>(a, trow0, lane, rv);
    store_y_tile<MT>(a, y8, trow0, lane, rv);
}
template <int MT, bool kFused = false>
__device__ __forceinline__ void write_y(const GemvArgs& a, bool y8, float gs, int prow0, int lane, const f32x4 (&v)[2][MT]) {
    f32x4 r0[MT], r1[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        r0[mt] = v[0][mt] * gs;
        r1[mt] = v[1][mt] * gs;
    }
    if constexpr (kFused) {
        if (a.resid != nullptr) {
            add_resid_tile<MT>(a, prow0, lane, r0);
            add_resid_tile<MT>(a, prow0 + 16, lane, r1);
        }
    }
    store_y_tile<MT>(a, y8, prow0, lane, r0);
    store_y_tile<MT>(a, y8, prow0 + 16, lane, r1);
}

// Batch chunking (kChunks, one unsplit task): block row y of the grid takes
// batch rows [16 MT y, 16 MT (y + 1)) -- the prefill GEMM, M in the hundreds or
// thousands, as independent 16 MT-row products over the same weights.
template <bool kChunks, int MT>
__device__ __forceinline__ GemvArgs chunk_args(GemvArgs a) {
    if constexpr (kChunks) {
        const int m0 = (int)blockIdx.y * 16 * MT;
        a.x += (size_t)m0 * a.K;
        a.y += (size_t)m0 * a.N;
        a.M = a.M - m0 < 16 * MT ? a.M - m0 : 16 * MT;
    }
    return a;
}

__device__ __forceinline__ int mm_task(const MmTable& tt) {
    int ti = 0;
#pragma unroll
    for (int i = 1; i < kMaxTasks; ++i) ti += ((int)blockIdx.x >= tt.blk0[i]) ? 1 : 0;
    return ti;
}

// One workgroup of task ti (a row block, or one K slice of it).
template <class F, int MT, bool kFused, bool kChunks>
__device__ __forceinline__ void tiled_body(const MmTable& tt, const int ti, uint8_t* lds) {
    constexpr int kPre = MmFmt<F>::kPre;
    constexpr int kLoads = MmFmt<F>::kLoads;
    constexpr int XP = mm_xp<MT>() < kPre ? mm_xp<MT>() : kPre;
    u32x4* xb = reinterpret_cast<u32x4*>(lds);                                               // [2][2][MT][4][64]
    f32x2* smb = reinterpret_cast<f32x2*>(lds + mm_ring_bytes<MT>());    // [gps][64]

    const GemvArgs a = chunk_args<kChunks, MT>(tt.t[ti].a);
    const int KS = tt.t[ti].ks, gps = tt.t[ti].gps;
    const int local = blockIdx.x - tt.blk0[ti];
    const int blk = local / KS, ks = local - blk * KS;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = a.K >> 7;
    const int g0 = ks * gps;
    int ng = G - g0;
    ng = ng < gps ? ng : gps;                      // groups of this slice (>= 1 by construction)
    const int row0 = blk * kRows;
    const uint32_t rowbytes = std::is_same<F, FmtBf16>::value ? (uint32_t)a.K * 2u : (uint32_t)a.K >> 1;
    const float gs = std::is_same<F, FmtNvfp4>::value ? a.gscale : 1.0f;
    // the two halves of the slice: groups [0, h0) and [h0, ng)
    const int h0 = (ng + 1) >> 1;
    const int h1 = ng - h0;
    // One group step per barrier, in rounds of kPre (h0 rounded up; the split
    // plan's slices make h0 even).  Past a half's last group the loads re-read
    // that group (every load is unconditional, so the wait counts stay exact)
    // and the results are not accumulated.
    const int niter = ((h0 + kPre - 1) / kPre) * kPre;

    if (wave < kCompute) {
        // ------------------------------------------------------------ compute
        const int rp = wave & 1, kh = wave >> 1;
        const int hlen = kh == 0 ? h0 : h1;
        const int hbase = kh == 0 ? 0 : h0;
        const int hlast = hlen > 0 ? hlen - 1 : 0;
        const int hb = hlen > 0 ? hbase : 0;
        const int prow0 = row0 + 32 * rp;
        const bf16x8_t neg128 = as_bf16x8(0xC300C300u, 0xC300C300u, 0xC300C300u, 0xC300C300u);
        int fs[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) fs[s] = frag_slot(lane, s);
        int nr = a.N - prow0;
        nr = __builtin_amdgcn_readfirstlane(nr < 0 ? 0 : (nr > 32 ? 32 : nr));
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w + (size_t)prow0 * rowbytes, (uint32_t)nr * rowbytes);
        // lane l: row l % 16 of the tile, columns 32 (l / 16) .. + 32 of the
        // group (16 * kLoads bytes: one load per k-step for BF16)
        constexpr uint32_t kGroupBytes = 64u * kLoads;
        const uint32_t avoff = (uint32_t)(lane & 15) * rowbytes + (uint32_t)(g0 + hb) * kGroupBytes + (uint32_t)(lane >> 4) * 16u * kLoads;
        auto aload = [&](int i, int t, int j) {
            return buf_load16(rw, avoff + (uint32_t)t * 16u * rowbytes + (uint32_t)(i < hlast ? i : hlast) * kGroupBytes + 16u * j, 0);
        };
        // NVFP4: the lane's two e4m3 scales (its 32 columns are two 16-column groups)
        const uint32_t sbytes = (uint32_t)a.K >> 4;
        const __amdgpu_buffer_rsrc_t rsc = make_rsrc(std::is_same<F, FmtNvfp4>::value ? a.scale8 + (size_t)prow0 * sbytes : nullptr,
                                                     std::is_same<F, FmtNvfp4>::value ? (uint32_t)nr * sbytes : 0u);
        const uint32_t svoff = (uint32_t)(lane & 15) * sbytes + (uint32_t)(g0 + hb) * 8u + (uint32_t)(lane >> 4) * 2u;
        auto sload = [&](int i, int t) -> uint32_t {
            if constexpr (std::is_same<F, FmtNvfp4>::value)
                return buf_load2(rsc, svoff + (uint32_t)t * 16u * sbytes + (uint32_t)(i < hlast ? i : hlast) * 8u, 0);
            else
                return 0u;
        };
        // the loaders' first activation and group-parameter loads go out
        // before this workgroup's weight prefetch, so they do not queue
        // behind it
        lds_barrier();
        u32x4 q[kPre][2][kLoads];
        uint32_t sq[kPre][2];
#pragma unroll
        for (int u = 0; u < kPre; ++u)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int j = 0; j < kLoads; ++j) q[u][t][j] = aload(u, t, j);
                sq[u][t] = sload(u, t);
            }

        f32x4 acc[2][MT];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        lds_barrier();     // parameters and activation step 0 ready

        // one group step; u = i % kPre is the prefetch ring entry
        auto step = [&](const int i, const int u) {
            const int slot = i & 1;
            const u32x4* xs = xb + (size_t)((slot * 2 + kh) * MT) * 4 * 64;
            u32x4 qa[2][kLoads];
            uint32_t sa[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int j = 0; j < kLoads; ++j) {
                    qa[t][j] = q[u][t][j];
                    q[u][t][j] = aload(i + kPre, t, j);
                }
                sa[t] = sq[u][t];
                sq[u][t] = sload(i + kPre, t);
            }
            // the A operand of k-step s for row tile t
            auto a_op = [&](int t, int s) -> bf16x8_t {
                if constexpr (std::is_same<F, FmtBf16>::value) {
                    return as_bf16x8(qa[t][s]);
                } else {
                    const uint32_t w = qa[t][0][s];
                    uint32_t A[4];
                    if constexpr (is_q4<F>()) {
                        q4_pairs(w, A);   // 128 + code, in the (c0,c4) (c1,c5) ... pairing
                    } else {
                        // e2m1 * e4m3, natural column order; k-steps 0-1 and
                        // 2-3 lie in the lane's first and second 16-column group
                        const float sc = s < 2 ? e4m3_to_f32<0>(sa[t]) : e4m3_to_f32<1>(sa[t]);
                        A[0] = nv_pair_scaled<0>(w, sc);
                        A[1] = nv_pair_scaled<1>(w, sc);
                        A[2] = nv_pair_scaled<2>(w, sc);
                        A[3] = nv_pair_scaled<3>(w, sc);
                    }
                    return as_bf16x8(A[0], A[1], A[2], A[3]);
                }
            };
            // int4: D = sum of (128 + code) * x and C = -128 * SX (an all -128
            // A operand against the same fragments leaves -128 * SX of batch
            // row l % 16 in all four results of lane l); otherwise D = sum of
            // w * x over the group
            f32x4 cx[MT], D[2][MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) cx[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) D[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                u32x4 B[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) B[mt] = xs[(mt * 4 + s) * 64 + fs[s]];
                if constexpr (is_q4<F>()) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) cx[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(neg128, as_bf16x8(B[mt]), cx[mt], 0, 0, 0);
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const bf16x8_t Av = a_op(t, s);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        D[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Av, as_bf16x8(B[mt]), D[t][mt], 0, 0, 0);
                }
            }
            if (i < hlen) {
                if constexpr (is_q4<F>()) {
                    // acc += scale * (D + C) + min * SX with min staged as -min / 128;
                    // D + C is the sum of code * x (exact when one product is nonzero)
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const f32x4* sm4 = reinterpret_cast<const f32x4*>(smb + (hbase + i) * kRows + 32 * rp + 16 * t + 4 * (lane >> 4));
                        const f32x4 sm01 = sm4[0], sm23 = sm4[1];
                        const float sc[4] = {sm01.x, sm01.z, sm23.x, sm23.z};
                        const float mq[4] = {sm01.y, sm01.w, sm23.y, sm23.w};
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                acc[t][mt][v] = fmaf(mq[v], cx[mt][v], fmaf(sc[v], D[t][mt][v] + cx[mt][v], acc[t][mt][v]));
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) acc[t][mt] += D[t][mt];
                }
            }
            lds_barrier();
        };
        // whole rounds of kPre steps (a fixed trip structure keeps the
        // compiler's waits on the weight prefetch exact)
        for (int i0 = 0; i0 < niter; i0 += kPre) {
#pragma unroll
            for (int u = 0; u < kPre; ++u) step(i0 + u, u);
        }

        // the two K halves meet: half 1 hands its tiles to half 0 through LDS
        // (the ring is free once every wave has passed the last barrier)
        f32x4* red = reinterpret_cast<f32x4*>(lds);   // [2 row pairs][2 tiles][MT][64]
        if (kh == 1) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) red[((rp * 2 + t) * MT + mt) * 64 + lane] = acc[t][mt];
        }
        __syncthreads();
        if (kh == 0) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[t][mt] += red[((rp * 2 + t) * MT + mt) * 64 + lane];
        }
        // ------------------------------------------------------------ epilogue
        if (KS == 1) {
            __syncthreads();   // every wave meets the same barriers
            if (kh == 0) write_y<MT, kFused>(a, tt.t[ti].y8 != 0, gs, prow0, lane, acc);
            return;
        }
        // split K: publish this slice's partial tile; the last slice to arrive
        // reduces.  Partials are written and read with device-coherent 16-byte
        // accesses (1 KB contiguous per instruction), which do not stop in the
        // per-XCD L2, and every wave waits for its stores to complete before
        // the barrier that precedes the block's counter update, so no
        // cache-wide write-back or invalidate is needed.
        if (kh == 0) {
            const int blocks = (a.N + kRows - 1) / kRows;
            const __amdgpu_buffer_rsrc_t rpart = make_rsrc(tt.t[ti].part, (uint32_t)blocks * KS * 4u * MT * 64u * 16u);
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[t][mt]), rpart,
                                                           part_off<MT>(blk, KS, ks, rp, t, mt, lane), 0, kCoherent);
        }
    } else {
        // ------------------------------------------------------------- loader
        const int L = wave - kCompute;          // the K half this loader feeds
        const int lt = tid - 64 * kCompute;     // 0 .. 64 * kLoaders - 1
        const int hlen = L == 0 ? h0 : h1;
        const int hbase = L == 0 ? 0 : h0;
        const int hlast = hlen > 0 ? hlen - 1 : 0;
        const int hb = hlen > 0 ? hbase : 0;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)(a.M * a.K * 2));
        // piece (mt, s) of step i: four whole batch rows 16 mt + 4 s + l / 16
        // of the group, lane l holding columns 8 (l % 16) .. + 8 (1 KB
        // contiguous per row quartet, so each load fills whole cache lines)
        auto xoff = [&](int i, int p) {
            const int mt = p >> 2, s = p & 3;
            const int m = 16 * mt + 4 * s + (lane >> 4);
            const int g = g0 + hb + (i < hlast ? i : hlast);
            const int k = (g << 7) + 8 * (lane & 15);
            return (uint32_t)((m * a.K + k) * 2);
        };
        auto xload = [&](int i, int p) {
            return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff(i, p), 0, 0));
        };
        // fused: the up activations at the same places (an empty range when
        // the task has none: the loads return zeros and are not used, and
        // every load stays unconditional)
        const bool gated = kFused && a.up != nullptr;
        const __amdgpu_buffer_rsrc_t ru = make_rsrc(a.up, gated ? (uint32_t)(a.M * a.K * 2) : 0u);
        auto uload = [&](int i, int p) {
            return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ru, xoff(i, p), 0, 0));
        };
        // where lane l's piece (mt, s) goes: fragment (mt, k-step l % 4), lane
        // 4 s + l / 16 + 16 ((l / 4) % 4) (its row within the tile plus 16 x
        // its column quarter)
        const int sp = lane & 3;
        const int fl0 = (lane >> 4) + 16 * ((lane >> 2) & 3);
        auto stage = [&](int i, const u32x4 (&xr)[4 * MT], const u32x4 (&ur)[kFused ? 4 * MT : 1]) {
            const int slot = i & 1;
            u32x4* frag = xb + (size_t)((slot * 2 + L) * MT) * 4 * 64;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    u32x4 v = xr[mt * 4 + s];
                    if constexpr (kFused) {
                        if (gated) {
                            const u32x4 u = ur[mt * 4 + s];
                            v = u32x4{silu_mul_bf16x2(v.x, u.x), silu_mul_bf16x2(v.y, u.y), silu_mul_bf16x2(v.z, u.z),
                                      silu_mul_bf16x2(v.w, u.w)};
                        }
                    }
                    u32x4 w = v;
                    if constexpr (is_q4<F>()) {
                        uint32_t pr[4];
                        xq4_pairs(v.x, v.y, v.z, v.w, pr);
                        w = u32x4{pr[0], pr[1], pr[2], pr[3]};
                    }
                    frag[(mt * 4 + sp) * 64 + frag_slot(fl0 + 4 * s, sp)] = w;
                }
        };
        u32x4 xr[XP][4 * MT];
        u32x4 ur[XP][kFused ? 4 * MT : 1];
        auto load_step = [&](int r, int i) {   // step i's x (and up) pieces into ring entry r
#pragma unroll
            for (int p = 0; p < 4 * MT; ++p) xr[r][p] = xload(i, p);
            if constexpr (kFused) {
#pragma unroll
                for (int p = 0; p < 4 * MT; ++p) ur[r][p] = uload(i, p);
            }
        };
#pragma unroll
        for (int u = 0; u < XP; ++u) load_step(u, u);

        // group parameters of the block's rows for the slice, fp32 (scale, min)
        // [group][row], every load of a lane issued before the first is used
        if constexpr (is_q4<F>()) {
            const int smw = tt.t[ti].smw;
            if (smw != 0) {
                // pieces of smw = 8 or 4 groups of one row (16 or 8 bytes): the
                // host sets smw when K/128, the slice start and length are
                // multiples of it and both arrays are aligned to the piece
                int wg_rows = a.N - row0;
                wg_rows = __builtin_amdgcn_readfirstlane(wg_rows > kRows ? kRows : wg_rows);
                const uint32_t rb = (uint32_t)G * 2;
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scale + (size_t)row0 * G, (uint32_t)wg_rows * rb);
                const __amdgpu_buffer_rsrc_t rm = make_rsrc(a.minv + (size_t)row0 * G, (uint32_t)wg_rows * rb);
                const int ppr = ng / smw;                 // pieces per row
                constexpr int kMaxP = 4;                  // 64 rows x (56 groups / 8 or 16 groups / 4) / 128 threads
                u32x4 ps[kMaxP], pm[kMaxP];
    #pragma unroll
                for (int i = 0; i < kMaxP; ++i) {
                    const int c = lt + 64 * kLoaders * i;
                    const int r = c / ppr, pc = c - r * ppr;
                    const uint32_t off = (c < kRows * ppr) ? r * rb + (uint32_t)(g0 + smw * pc) * 2 : 0xFFFFFFF0u;
                    if (smw == 8) {
                        ps[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
                        pm[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rm, off, 0, 0));
                    } else {
                        const u32x2 s2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0));
                        const u32x2 m2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rm, off, 0, 0));
                        ps[i] = u32x4{s2.x, s2.y, 0u, 0u};
                        pm[i] = u32x4{m2.x, m2.y, 0u, 0u};
                    }
                }
                lds_barrier();   // releases the compute waves' weight prefetch
    #pragma unroll
                for (int i = 0; i < kMaxP; ++i) {
                    const int c = lt + 64 * kLoaders * i;
                    if (c < kRows * ppr) {
                        const int r = c / ppr, pc = c - r * ppr;
                        const uint32_t sw[4] = {ps[i].x, ps[i].y, ps[i].z, ps[i].w};
                        const uint32_t mw[4] = {pm[i].x, pm[i].y, pm[i].z, pm[i].w};
    #pragma unroll
                        for (int h = 0; h < 8; ++h) {
                            if (h >= smw) break;
                            const uint16_t sh = (uint16_t)(sw[h >> 1] >> (16 * (h & 1)));
                            const uint16_t mh = (uint16_t)(mw[h >> 1] >> (16 * (h & 1)));
                            smb[(smw * pc + h) * kRows + r] = f32x2{f16_to_f32(sh), -0.0078125f * f16_to_f32(mh)};
                        }
                    }
                }
            } else {
                lds_barrier();   // releases the compute waves' weight prefetch
                // single groups, in batches of 8 per lane
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scale, (uint32_t)a.N * (uint32_t)G * 2u);
                const __amdgpu_buffer_rsrc_t rm = make_rsrc(a.minv, (uint32_t)a.N * (uint32_t)G * 2u);
                for (int e0 = lt; e0 < kRows * ng; e0 += 8 * 64 * kLoaders) {
                    uint16_t sv[8], mv[8];
    #pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int e = e0 + 64 * kLoaders * k;
                        const int r = e / ng, g = e - r * ng;
                        const uint32_t off = e < kRows * ng ? ((uint32_t)(row0 + r) * (uint32_t)G + (uint32_t)(g0 + g)) * 2u : 0xFFFFFFF0u;
                        sv[k] = buf_load2(rs, off, 0);
                        mv[k] = buf_load2(rm, off, 0);
                    }
    #pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int e = e0 + 64 * kLoaders * k;
                        if (e < kRows * ng) {
                            const int r = e / ng, g = e - r * ng;
                            smb[g * kRows + r] = f32x2{f16_to_f32(sv[k]), -0.0078125f * f16_to_f32(mv[k])};
                        }
                    }
                }
            }

        } else {
            lds_barrier();   // releases the compute waves' weight prefetch
        }

        stage(0, xr[0], ur[0]);
        load_step(0, XP);
        lds_barrier();

        // step i stages step i + 1, held in ring entry (i + 1) % XP (i0 is a
        // multiple of kPre, itself a multiple of XP)
        auto lstep = [&](const int i, const int u) {
            const int r = (u + 1) % XP;
            stage(i + 1, xr[r], ur[r]);
            load_step(r, i + 1 + XP);
            lds_barrier();
        };
        for (int i0 = 0; i0 < niter; i0 += kPre) {
#pragma unroll
            for (int u = 0; u < kPre; ++u) lstep(i0 + u, u);
        }
        // the compute waves' two barriers of the half merge and the epilogue
        __syncthreads();
        if (KS == 1) {
            __syncthreads();
            return;
        }
    }

    // --------------------------------------------------- split-K completion
    // The hand-over rests on the device-coherent (sc1) partial accesses, not
    // on agent-scope fences (whose L2 write-back and invalidate cost more
    // than the split saves, and whose invalidate evicts the activations the
    // other workgroups on the XCD are reading): a wave's sc1 stores are
    // acknowledged only once they reach the device's coherence point, the
    // wave waits for those acknowledgements (vmcnt(0)) before the barrier
    // that precedes the counter update, and the last slice's sc1 loads are
    // issued only after its update returned and read at that point.  The
    // asm memory clobbers keep the compiler from moving accesses across.
    unsigned* cnt = tt.t[ti].cnt;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __shared__ unsigned s_prev;
    if (tid == 0) s_prev = __hip_atomic_fetch_add(&cnt[(size_t)blk * kCtrWords], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_prev != (unsigned)(KS - 1)) return;
    asm volatile("" ::: "memory");
    if (wave < kCompute) {
        // each compute wave sums one 16-row tile over the slices, in slice
        // order, with the partial tiles of kRB slices in flight at once
        constexpr int kRB = mm_reduce_batch<MT>();
        const int rp = wave & 1, t = wave >> 1;
        const int blocks = (a.N + kRows - 1) / kRows;
        const __amdgpu_buffer_rsrc_t rpart = make_rsrc(tt.t[ti].part, (uint32_t)blocks * KS * 4u * MT * 64u * 16u);
        f32x4 sum[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) sum[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < KS; s0 += kRB) {
            u32x4 pv[kRB][MT];
#pragma unroll
            for (int k = 0; k < kRB; ++k)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint32_t off = s0 + k < KS ? part_off<MT>(blk, KS, s0 + k, rp, t, mt, lane) : 0xFFFFFFF0u;
                    pv[k][mt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rpart, off, 0, kCoherent));
                }
#pragma unroll
            for (int k = 0; k < kRB; ++k)
                if (s0 + k < KS) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) sum[mt] += __builtin_bit_cast(f32x4, pv[k][mt]);
                }
        }
        write_y_tile<MT, kFused>(a, tt.t[ti].y8 != 0, gs, row0 + 32 * rp + 16 * t, lane, sum);
    }
    if (tid == 0) __hip_atomic_store(&cnt[(size_t)blk * kCtrWords], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class F, int MT, bool kFused = false, bool kChunks = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(mm_waves_f<MT, kFused>()))) void tiled_mm_kernel(MmTable tt) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    tiled_body<F, MT, kFused, kChunks>(tt, mm_task(tt), lds);
}

// One launch over NVFP4 and BF16 tasks (the NVFP4 decode step's BF16 v and down
// beside its NVFP4 projections): each workgroup runs its task's format.  Both
// formats use the same LDS layout (no staged group parameters) and planner.
template <int MT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(mm_waves<MT>()))) void tiled_mm_mixed_kernel(MmTable tt) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int ti = mm_task(tt);
    if (tt.t[ti].fmt == kFmtNvfp4) tiled_body<FmtNvfp4, MT, false, false>(tt, ti, lds);
    else tiled_body<FmtBf16, MT, false, false>(tt, ti, lds);
}

constexpr int kCUs = 256;
constexpr int kMinSlice = 4;     // fewest groups in a K slice (two steps of the two halves)

// groups per slice when G groups are cut into k slices: multiples of 4 where
// K allows (so group parameters load in 8-byte pieces)
inline int slice_groups(int G, int k) {
    int g = (G + k - 1) / k;
    if (G % 4 == 0) g = ((g + 3) / 4) * 4;
    return g;
}

// Split plan.  Each row block of a task is cut into ks[i] K slices of gps[i]
// groups (ks = 1: unsplit).  No split without a workspace, nor when the row
// blocks alone give two workgroups per CU.  Otherwise the tasks with the most
// blocks stay unsplit, one block per CU (at most kCUs blocks), and the other
// tasks are split so that their slices fill the remaining workgroup slots (two
// per CU in all; kCUs when no task stays unsplit), the largest slice as short
// as the slots allow: every CU then streams about the same weight bytes.
// whole[i] says which tasks stayed unsplit by this rule.
template <class F, int MT>
void mm_plan(const GemvArgs* tasks, int count, bool can_split, int* ks, int* gps, bool* whole) {
    int blocks[kMaxTasks], btot = 0;
    for (int i = 0; i < count; ++i) {
        blocks[i] = (tasks[i].N + kRows - 1) / kRows;
        btot += blocks[i];
        ks[i] = 1;
        gps[i] = tasks[i].K >> 7;
        whole[i] = true;
    }
    if (can_split && btot < 2 * kCUs) {
        int cap = kCUs, used = 0;
        for (int i = 0; i < count; ++i) whole[i] = false;
        if (btot >= kCUs) {
            // largest tasks first
            int order[kMaxTasks];
            for (int i = 0; i < count; ++i) order[i] = i;
            for (int a = 0; a < count; ++a)
                for (int b = a + 1; b < count; ++b)
                    if (blocks[order[b]] > blocks[order[a]]) { const int t = order[a]; order[a] = order[b]; order[b] = t; }
            for (int a = 0; a < count; ++a)
                if (used + blocks[order[a]] <= kCUs) {
                    whole[order[a]] = true;
                    used += blocks[order[a]];
                }
            cap = 2 * kCUs - used;
        }
        int tot = 0;
        for (int i = 0; i < count; ++i)
            if (!whole[i]) tot += blocks[i];
        // shorten the longest slice while the slots allow
        while (tot <= cap) {
            int w = -1;
            for (int i = 0; i < count; ++i)
                if (!whole[i] && (w < 0 || gps[i] > gps[w])) w = i;
            if (w < 0) break;
            const int G = tasks[w].K >> 7;
            int k = ks[w] + 1;
            while (k <= G && slice_groups(G, k) >= gps[w]) ++k;
            if (k > G) break;
            const int g = slice_groups(G, k);
            if (g < kMinSlice) break;
            const int kk = (G + g - 1) / g;
            if (tot + blocks[w] * (kk - ks[w]) > cap) break;
            tot += blocks[w] * (kk - ks[w]);
            ks[w] = kk;
            gps[w] = g;
        }
    }
    // every slice's group parameters fit LDS
    const int gmax = (mm_max_gps<F, MT>() / 4) * 4;
    for (int i = 0; i < count; ++i)
        if (gps[i] > gmax) {
            const int G = tasks[i].K >> 7;
            gps[i] = gmax;
            ks[i] = (G + gmax - 1) / gmax;
        }
}

// Workspace a launch needs: 0 when no task is split, or when the counters of
// the split tasks would not fit the counter region (the launch then runs
// unsplit).
template <class F, int MT>
size_t ws_bytes_mt(const GemvArgs* tasks, int count) {
    int ks[kMaxTasks], gps[kMaxTasks];
    bool whole[kMaxTasks];
    mm_plan<F, MT>(tasks, count, true, ks, gps, whole);
    size_t cnt = 0, part = 0;
    for (int i = 0; i < count; ++i) {
        if (ks[i] <= 1) continue;
        const size_t blocks = (tasks[i].N + kRows - 1) / kRows;
        part += blocks * ks[i] * kCompute * MT * 64 * 16;
        cnt += blocks * kCtrStride;
    }
    return (part > 0 && cnt <= kCntBytes) ? kCntBytes + part : 0;
}

// The task's int4 group-parameter load width (smw) and output store width (y8).
template <class F>
void fill_flags(MmTask& tk, const GemvArgs& a, int gps) {
    const int G = a.K >> 7;
    const uintptr_t sa = reinterpret_cast<uintptr_t>(a.scale), ma = reinterpret_cast<uintptr_t>(a.minv);
    if (!is_q4<F>())
        tk.smw = 0;
    else if (G % 8 == 0 && gps % 8 == 0 && gps <= 64 && sa % 16 == 0 && ma % 16 == 0)
        tk.smw = 8;
    else if (G % 4 == 0 && gps % 4 == 0 && gps <= 32 && sa % 8 == 0 && ma % 8 == 0)
        tk.smw = 4;
    else
        tk.smw = 0;
    tk.y8 = (reinterpret_cast<uintptr_t>(a.y) % 8 == 0 && a.N % 4 == 0) ? 1 : 0;
}

// The launch table of a tiled launch: plan the splits, order the tasks
// (unsplit first), lay out the workspace; returns the grid and sets *gmax.
template <class F, int MT>
int build_table(const GemvArgs* tasks, const Fmt* fmts, int count, void* ws, size_t ws_bytes, MmTable& tt, int* gmax_out) {
    int ks[kMaxTasks], gps[kMaxTasks];
    const size_t need = ws_bytes_mt<F, MT>(tasks, count);
    const bool split = ws != nullptr && need > 0 && ws_bytes >= need;
    bool whole[kMaxTasks];
    mm_plan<F, MT>(tasks, count, split, ks, gps, whole);
    // unsplit tasks take the first workgroups, so that the dispatcher spreads
    // their blocks one per CU before the slices fill the second slots
    int order[kMaxTasks], n = 0;
    for (int i = 0; i < count; ++i)
        if (whole[i]) order[n++] = i;
    for (int i = 0; i < count; ++i)
        if (!whole[i]) order[n++] = i;
    for (int i = 0; i < kMaxTasks; ++i) tt.blk0[i] = 0x7fffffff;
    uint8_t* pc = static_cast<uint8_t*>(ws);
    uint8_t* pp = pc + kCntBytes;
    int grid = 0, gmax = 0;
    for (int j = 0; j < count; ++j) {
        const int i = order[j];
        const int blocks = (tasks[i].N + kRows - 1) / kRows;
        tt.blk0[j] = grid;
        tt.t[j].a = tasks[i];
        tt.t[j].ks = ks[i];
        tt.t[j].gps = gps[i];
        fill_flags<F>(tt.t[j], tasks[i], gps[i]);
        tt.t[j].fmt = fmts ? fmts[i] : 0;
        if (ks[i] > 1) {
            tt.t[j].cnt = reinterpret_cast<unsigned*>(pc);
            pc += (size_t)blocks * kCtrStride;
            tt.t[j].part = reinterpret_cast<float*>(pp);
            pp += (size_t)blocks * ks[i] * kCompute * MT * 64 * 16;
        }
        grid += blocks * ks[i];
        gmax = gps[i] > gmax ? gps[i] : gmax;
    }
    *gmax_out = gmax;
    return grid;
}

template <class F, int MT, bool kFused = false>
hipError_t launch_mm_mt(const GemvArgs* tasks, int count, void* ws, size_t ws_bytes, hipStream_t st) {
    MmTable tt{};
    int gmax = 0;
    const int grid = build_table<F, MT>(tasks, nullptr, count, ws, ws_bytes, tt, &gmax);
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(tiled_mm_kernel<F, MT, kFused>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget);
    if (attr != hipSuccess) return attr;
    return launch_kernel(tiled_mm_kernel<F, MT, kFused>, dim3(grid), dim3(kThreads), (size_t)mm_shmem<F, MT>(gmax), st, tt);
}

// NVFP4 and BF16 tasks in one launch (fmts[i] per task), planned as NVFP4:
// the two formats share the planner and the LDS layout.
template <int MT>
hipError_t launch_mm_mixed_mt(const Fmt* fmts, const GemvArgs* tasks, int count, void* ws, size_t ws_bytes, hipStream_t st) {
    MmTable tt{};
    int gmax = 0;
    const int grid = build_table<FmtNvfp4, MT>(tasks, fmts, count, ws, ws_bytes, tt, &gmax);
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(tiled_mm_mixed_kernel<MT>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget);
    if (attr != hipSuccess) return attr;
    return launch_kernel(tiled_mm_mixed_kernel<MT>, dim3(grid), dim3(kThreads), (size_t)mm_shmem<FmtNvfp4, MT>(gmax), st, tt);
}


}  // namespace

template <class F>
bool mm_supported_f(int M, int K, bool split) {
    if (M < 1 || M > 64 || K % 128) return false;
    if (split) return true;
    const int G = K >> 7;
    switch ((M + 15) / 16) {
        case 1: return G <= mm_max_gps<F, 1>();
        case 2: return G <= mm_max_gps<F, 2>();
        case 3: return G <= mm_max_gps<F, 3>();
        default: return G <= mm_max_gps<F, 4>();
    }
}

template <class F>
size_t mm_workspace_bytes_f(const GemvArgs* tasks, int count) {
    switch ((tasks[0].M + 15) / 16) {
        case 1: return ws_bytes_mt<F, 1>(tasks, count);
        case 2: return ws_bytes_mt<F, 2>(tasks, count);
        case 3: return ws_bytes_mt<F, 3>(tasks, count);
        default: return ws_bytes_mt<F, 4>(tasks, count);
    }
}

template <class F, bool kFused = false>
hipError_t launch_mm_f(const GemvArgs* tasks, int count, void* ws, size_t ws_bytes, hipStream_t s) {
    switch ((tasks[0].M + 15) / 16) {
        case 1: return launch_mm_mt<F, 1, kFused>(tasks, count, ws, ws_bytes, s);
        case 2: return launch_mm_mt<F, 2, kFused>(tasks, count, ws, ws_bytes, s);
        case 3: return launch_mm_mt<F, 3, kFused>(tasks, count, ws, ws_bytes, s);
        default: return launch_mm_mt<F, 4, kFused>(tasks, count, ws, ws_bytes, s);
    }
}

bool mm_supported(Fmt fmt, int M, int K, bool split) {
    switch (fmt) {
        case kFmtQ4: return mm_supported_f<FmtQ4>(M, K, split);
        case kFmtNvfp4: return mm_supported_f<FmtNvfp4>(M, K, split);
        default: return mm_supported_f<FmtBf16>(M, K, split);
    }
}

size_t mm_workspace_bytes(Fmt fmt, const GemvArgs* tasks, int count) {
    switch (fmt) {
        case kFmtQ4: return mm_workspace_bytes_f<FmtQ4>(tasks, count);
        case kFmtNvfp4: return mm_workspace_bytes_f<FmtNvfp4>(tasks, count);
        default: return mm_workspace_bytes_f<FmtBf16>(tasks, count);
    }
}

hipError_t launch_mm(Fmt fmt, const GemvArgs* tasks, int count, void* ws, size_t ws_bytes, hipStream_t s) {
    switch (fmt) {
        case kFmtQ4: return launch_mm_f<FmtQ4>(tasks, count, ws, ws_bytes, s);
        case kFmtNvfp4: return launch_mm_f<FmtNvfp4>(tasks, count, ws, ws_bytes, s);
        default: return launch_mm_f<FmtBf16>(tasks, count, ws, ws_bytes, s);
    }
}

hipError_t launch_mm_fused(const GemvArgs* tasks, int count, void* ws, size_t ws_bytes, hipStream_t s) {
    return launch_mm_f<FmtQ4, true>(tasks, count, ws, ws_bytes, s);
}

namespace {

template <int MT>
hipError_t launch_chunks_mt(const GemvArgs& a, hipStream_t st) {
    MmTable tt{};
    for (int i = 0; i < kMaxTasks; ++i) tt.blk0[i] = 0x7fffffff;
    const int G = a.K >> 7;
    tt.blk0[0] = 0;
    tt.t[0].a = a;
    tt.t[0].ks = 1;
    tt.t[0].gps = G;
    fill_flags<FmtQ4>(tt.t[0], a, G);
    const dim3 grid((a.N + kRows - 1) / kRows, (a.M + 16 * MT - 1) / (16 * MT));
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(tiled_mm_kernel<FmtQ4, MT, false, true>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget);
    if (attr != hipSuccess) return attr;
    return launch_kernel(tiled_mm_kernel<FmtQ4, MT, false, true>, grid, dim3(kThreads), (size_t)mm_shmem<FmtQ4, MT>(G), st, tt);
}

// widest batch chunk whose group parameters fit LDS unsplit (0: none)
int chunk_mt(int K) {
    const int G = K >> 7;
    if (K % 128) return 0;
    if (G <= mm_max_gps<FmtQ4, 4>()) return 4;
    if (G <= mm_max_gps<FmtQ4, 2>()) return 2;
    if (G <= mm_max_gps<FmtQ4, 1>()) return 1;
    return 0;
}

}  // namespace

bool mm_chunks_supported(int K) { return chunk_mt(K) > 0; }

hipError_t launch_mm_chunks(const GemvArgs& a, hipStream_t s) {
    switch (chunk_mt(a.K)) {
        case 4: return launch_chunks_mt<4>(a, s);
        case 2: return launch_chunks_mt<2>(a, s);
        default: return launch_chunks_mt<1>(a, s);
    }
}

hipError_t launch_mm_mixed(const Fmt* fmts, const GemvArgs* tasks, int count, void* ws, size_t ws_bytes, hipStream_t s) {
    switch ((tasks[0].M + 15) / 16) {
        case 1: return launch_mm_mixed_mt<1>(fmts, tasks, count, ws, ws_bytes, s);
        case 2: return launch_mm_mixed_mt<2>(fmts, tasks, count, ws, ws_bytes, s);
        case 3: return launch_mm_mixed_mt<3>(fmts, tasks, count, ws, ws_bytes, s);
        default: return launch_mm_mixed_mt<4>(fmts, tasks, count, ws, ws_bytes, s);
    }
}

}  // namespace q4
