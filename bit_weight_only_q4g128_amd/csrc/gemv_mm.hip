// Matrix-core GEMV for batched decode, int4 g128 (gfx950, v_mfma_f32_16x16x32_bf16).
//
// A workgroup owns a block of 64 weight rows and one slice of K (the whole of
// K unless the rows alone cannot fill the chip).  It runs six waves:
//
//   * four compute waves, one 16-row tile each.  A compute wave issues only
//     weight loads (kPre 128-column groups ahead), so its in-order waits on
//     the vector-memory counter never stall behind anything but its own
//     weights.  Per group it turns its 16 bytes per lane into BF16 "128 + code"
//     operands, runs 4 k-steps x MT batch tiles of MFMA with the activations as
//     the B operand, and folds the group as
//         acc += scale * (D - 128 * SX) + min * SX,   SX = sum of x over the group;
//   * two loader waves that stream the activations of each 128-column group
//     (MT*16 batch rows) from L2 into a double-buffered LDS ring, already in
//     B-fragment order and in the column pairing of the weight operand, and
//     compute SX on the way (each loader half of it).
//
// One barrier per group keeps the ring in step.  When K is split over several
// workgroups, each writes its fp32 partial tile to a caller-provided
// workspace; the workgroup that arrives last at the block's counter (release /
// acquire fences around one atomic) sums the partials in slice order, so the
// result does not depend on timing, writes y and resets the counter to zero.
//
// MFMA operand layout (16x16x32): lane l holds A row l % 16 and B column
// l % 16; for k-step s it holds the 8 columns 32 * (l / 16) + 8 * s .. + 8 of
// the group (any fixed assignment works as long as A and B agree), so one
// 16-byte load per lane fetches all four k-steps of a row's group.  D: lane l
// holds rows 4 * (l / 16) + v (v = 0..3) of column l % 16.
#include "internal.h"

namespace q4 {

namespace {

constexpr int kRows = 64;        // rows per workgroup
constexpr int kCompute = 4;      // compute waves (one 16-row tile each)
constexpr int kLoaders = 2;      // activation loader waves
constexpr int kThreads = 64 * (kCompute + kLoaders);
constexpr int kPre = 4;          // weight groups in flight per compute lane
constexpr int kXPre = 2;         // activation groups in flight per loader lane (divides kPre)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

struct MmTask {
    GemvArgs a;
    int ks;            // workgroups per row block (K slices)
    int gps;           // 128-column groups per slice
    int sm16;          // group parameters can be read as 16-byte pieces (see below)
    float* part;       // partial tiles (ks > 1): [blocks][ks][4 waves][MT][64 lanes] x 4 floats
    unsigned* cnt;     // arrival counters (ks > 1): [blocks]
};

struct MmTable {
    int blk0[kMaxTasks];   // first workgroup of each task (unused: INT_MAX)
    MmTask t[kMaxTasks];
};

// Activation ring: NS slots of one 128-column group each, [MT][4 k-steps][64
// lanes] x 16 bytes per slot in B-fragment order.  The loaders keep XD groups
// of direct-to-LDS loads in flight beyond the group they are preparing.
constexpr int kLdsBudget = 80 * 1024;   // two workgroups per CU (160 KB of LDS)
template <int MT>
__host__ __device__ constexpr int mm_ns() { return MT <= 3 ? 5 : 4; }
template <int MT>
__host__ __device__ constexpr int mm_xd() { return mm_ns<MT>() - 2; }
template <int MT>
__host__ __device__ constexpr int mm_slot_bytes() { return MT * 4 * 64 * 16; }
template <int MT>
__host__ __device__ constexpr int mm_sx_bytes() { return mm_ns<MT>() * kLoaders * MT * 16 * 4; }
template <int MT>
__host__ __device__ inline int mm_shmem(int gps) {
    return mm_ns<MT>() * mm_slot_bytes<MT>() + mm_sx_bytes<MT>() + gps * kRows * 8;
}
// most groups per slice whose parameters fit the LDS budget
template <int MT>
constexpr int mm_max_gps() {
    return (kLdsBudget - mm_ns<MT>() * mm_slot_bytes<MT>() - mm_sx_bytes<MT>()) / (kRows * 8);
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most the direct-to-
// LDS loads of XD - 1 groups (2 * MT instructions each) are outstanding.
template <int MT>
constexpr int mm_wait_xd() {
    constexpr int n = (mm_xd<MT>() - 1) * 2 * MT;
    return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}
template <int MT>
constexpr int kWaitXD = mm_wait_xd<MT>();

// Workgroup barrier for the main loops: waits only for this wave's LDS
// traffic (lgkmcnt) and fences the compiler, so vector-memory loads -- the
// weight prefetch and the direct-to-LDS activation loads -- stay in flight
// across it.  (__syncthreads would add a workgroup release fence, which waits
// for every outstanding direct-to-LDS load.)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int MT>
__global__ __launch_bounds__(kThreads) void q4_mm_kernel(MmTable tt) {
    constexpr int NS = mm_ns<MT>();
    constexpr int XD = mm_xd<MT>();
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    u32x4* xb = reinterpret_cast<u32x4*>(lds);                                                  // [NS][MT][4][64]
    float* sxb = reinterpret_cast<float*>(lds + NS * mm_slot_bytes<MT>());                      // [NS][kLoaders][MT*16]
    f32x2* smb = reinterpret_cast<f32x2*>(lds + NS * mm_slot_bytes<MT>() + mm_sx_bytes<MT>());  // [gps][64]

    int ti = 0;
#pragma unroll
    for (int i = 1; i < kMaxTasks; ++i) ti += ((int)blockIdx.x >= tt.blk0[i]) ? 1 : 0;
    const GemvArgs a = tt.t[ti].a;
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
    const uint32_t rowbytes = (uint32_t)a.K >> 1;
    // Groups run in rounds of kPre; past the slice's last group the loads
    // re-read that group (every load is unconditional, so the wait counts
    // stay exact) and the results are not accumulated.
    const int niter = ((ng + kPre - 1) / kPre) * kPre;

    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (wave < kCompute) {
        // ------------------------------------------------------------ compute
        const int trow0 = row0 + 16 * wave;
        int nr = a.N - trow0;
        // uniform; kept in a scalar register so the buffer resource is too
        nr = __builtin_amdgcn_readfirstlane(nr < 0 ? 0 : (nr > 16 ? 16 : nr));
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w + (size_t)trow0 * rowbytes, (uint32_t)nr * rowbytes);
        const uint32_t avoff = (uint32_t)(lane & 15) * rowbytes + ((uint32_t)g0 << 6) + ((uint32_t)(lane >> 4) << 4);
        auto aload = [&](int j) { return buf_load16(rw, avoff + ((uint32_t)(j < ng ? j : ng - 1) << 6), 0); };
        u32x4 q[kPre];
#pragma unroll
        for (int u = 0; u < kPre; ++u) q[u] = aload(u);
        lds_barrier();     // parameters and activation group 0 ready

        // Software pipeline: iteration j issues group j's MFMAs into Dc and
        // folds group j - 1 (Dp, with its SX / scale / min read one iteration
        // earlier) while those run.
        f32x4 Dp[MT];
        float sxp[MT];
        f32x4 smp01 = {0.f, 0.f, 0.f, 0.f}, smp23 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) { Dp[mt] = f32x4{0.f, 0.f, 0.f, 0.f}; sxp[mt] = 0.f; }
        auto fold = [&](const f32x4 (&D)[MT], const float (&sx)[MT], f32x4 sm01, f32x4 sm23) {
            const float sc[4] = {sm01.x, sm01.z, sm23.x, sm23.z};
            const float mn[4] = {sm01.y, sm01.w, sm23.y, sm23.w};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float t = fmaf(-128.f, sx[mt], D[mt][v]);
                    acc[mt][v] = fmaf(mn[v], sx[mt], fmaf(sc[v], t, acc[mt][v]));
                }
        };
        int slot0 = 0;                              // slot of group j0
        for (int j0 = 0; j0 < niter; j0 += kPre) {
#pragma unroll
            for (int u = 0; u < kPre; ++u) {
                const int j = j0 + u;
                int slot = slot0 + u;
                slot = slot >= NS ? slot - NS : slot;
                slot = slot >= NS ? slot - NS : slot;
                slot = slot >= NS ? slot - NS : slot;
                const u32x4* xs = xb + (size_t)slot * MT * 4 * 64 + lane;
                float sxc[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    sxc[mt] = sxb[(slot * kLoaders + 0) * MT * 16 + mt * 16 + (lane & 15)] +
                              sxb[(slot * kLoaders + 1) * MT * 16 + mt * 16 + (lane & 15)];
                const int jc = j < ng ? j : ng - 1;
                const f32x4* sm4 = reinterpret_cast<const f32x4*>(smb + jc * kRows + 16 * wave + 4 * (lane >> 4));
                const f32x4 smc01 = sm4[0], smc23 = sm4[1];
                // fold group j - 1 (its MFMAs ran during the previous iteration)
                if (j >= 1 && j - 1 < ng) fold(Dp, sxp, smp01, smp23);
                // group j: per k-step, three activation fragments and one weight operand
                const u32x4 qa = q[u];
                q[u] = aload(j + kPre);
                const uint32_t qd[4] = {qa.x, qa.y, qa.z, qa.w};
                f32x4 Dc[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) Dc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    u32x4 B[MT];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) B[mt] = xs[(mt * 4 + s) * 64];
                    uint32_t A[4];
                    q4_pairs(qd[s], A);
                    const bf16x8_t Av = as_bf16x8(A[0], A[1], A[2], A[3]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        Dc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Av, as_bf16x8(B[mt]), Dc[mt], 0, 0, 0);
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) { Dp[mt] = Dc[mt]; sxp[mt] = sxc[mt]; }
                smp01 = smc01;
                smp23 = smc23;
                lds_barrier();
            }
            slot0 += kPre % NS;
            slot0 = slot0 >= NS ? slot0 - NS : slot0;
        }
        if (niter - 1 < ng) fold(Dp, sxp, smp01, smp23);
    } else {
        // ------------------------------------------------------------- loader
        // Loader L owns k-steps s = 2L, 2L + 1 of every batch tile.  For group
        // j it issues, per (mt, s), one direct-to-LDS load in which lane l
        // fetches the 8 activations of batch row 16 mt + l % 16 at group
        // columns 32 (l / 16) + 8 s .. + 8, landing exactly where compute lane
        // l reads them; once they have landed it re-pairs them in place to
        // match the weight operand and sums them for SX.
        const int L = wave - kCompute;
        const int lt = tid - 64 * kCompute;   // 0 .. 64 * kLoaders - 1
        const uint16_t* xg = a.x;
        auto issue = [&](int j) {
            const int slot = j % NS;
            const int g = g0 + (j < ng ? j : ng - 1);
#pragma unroll
            for (int i = 0; i < 2 * MT; ++i) {
                const int mt = i >> 1, s = 2 * L + (i & 1);
                int m = 16 * mt + (lane & 15);
                m = m < a.M ? m : a.M - 1;        // padding rows re-read a real row; their columns are dropped
                const uint16_t* src = xg + (size_t)m * a.K + (g << 7) + 32 * (lane >> 4) + 8 * s;
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                                 (__attribute__((address_space(3))) void*)(xb + ((size_t)slot * MT * 4 + mt * 4 + s) * 64),
                                                 16, 0, 0);
            }
        };
        auto prepare = [&](int j) {
            const int slot = j % NS;
            u32x4* base = xb + (size_t)slot * MT * 4 * 64 + lane;
            u32x4 v[MT][2];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int h = 0; h < 2; ++h) v[mt][h] = base[(mt * 4 + 2 * L + h) * 64];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                float sx = 0.f;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t pr[4];
                    xq4_pairs(v[mt][h].x, v[mt][h].y, v[mt][h].z, v[mt][h].w, pr);
                    base[(mt * 4 + 2 * L + h) * 64] = u32x4{pr[0], pr[1], pr[2], pr[3]};
                    sx = dot2(v[mt][h].x, 0x3F803F80u, sx);
                    sx = dot2(v[mt][h].y, 0x3F803F80u, sx);
                    sx = dot2(v[mt][h].z, 0x3F803F80u, sx);
                    sx = dot2(v[mt][h].w, 0x3F803F80u, sx);
                }
                // lanes l, l ^ 16, l ^ 32, l ^ 48 hold the same batch row
                sx += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, sx), 0x401F));
                sx += __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, sx)));
                const int m = 16 * mt + lane;
                if (lane < 16) sxb[(slot * kLoaders + L) * MT * 16 + mt * 16 + lane] = (m < a.M) ? sx : 0.f;
            }
        };
#pragma unroll
        for (int u = 0; u <= XD; ++u) issue(u);

        // group parameters of the block's rows for the slice, fp32 (scale, min) [group][row]
        if (tt.t[ti].sm16) {
            // 16-byte pieces (8 groups of one row), all loads issued at once:
            // the host sets sm16 when K/128, the slice start and length are
            // multiples of 8 and both arrays are 16-byte aligned
            int wg_rows = a.N - row0;
            wg_rows = __builtin_amdgcn_readfirstlane(wg_rows > kRows ? kRows : wg_rows);
            const uint32_t rb = (uint32_t)G * 2;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scale + (size_t)row0 * G, (uint32_t)wg_rows * rb);
            const __amdgpu_buffer_rsrc_t rm = make_rsrc(a.minv + (size_t)row0 * G, (uint32_t)wg_rows * rb);
            const int ppr = ng >> 3;                  // pieces per row
            constexpr int kMaxP = 4;                  // 64 rows * 64 groups / 8 / 128 threads
            u32x4 ps[kMaxP], pm[kMaxP];
#pragma unroll
            for (int i = 0; i < kMaxP; ++i) {
                const int c = lt + 64 * kLoaders * i;
                const int r = c / ppr, pc = c - r * ppr;
                const uint32_t off = (c < kRows * ppr) ? (uint32_t)r * rb + (uint32_t)(g0 + 8 * pc) * 2 : 0xFFFFFFF0u;
                ps[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
                pm[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rm, off, 0, 0));
            }
#pragma unroll
            for (int i = 0; i < kMaxP; ++i) {
                const int c = lt + 64 * kLoaders * i;
                if (c < kRows * ppr) {
                    const int r = c / ppr, pc = c - r * ppr;
                    const uint32_t sw[4] = {ps[i].x, ps[i].y, ps[i].z, ps[i].w};
                    const uint32_t mw[4] = {pm[i].x, pm[i].y, pm[i].z, pm[i].w};
#pragma unroll
                    for (int h = 0; h < 8; ++h) {
                        const uint16_t sh = (uint16_t)(sw[h >> 1] >> (16 * (h & 1)));
                        const uint16_t mh = (uint16_t)(mw[h >> 1] >> (16 * (h & 1)));
                        smb[(8 * pc + h) * kRows + r] = f32x2{f16_to_f32(sh), f16_to_f32(mh)};
                    }
                }
            }
        } else {
            for (int e = lt; e < kRows * ng; e += 64 * kLoaders) {
                const int r = e / ng, g = e - r * ng;
                f32x2 v = {0.f, 0.f};
                if (row0 + r < a.N) {
                    const size_t gi = (size_t)(row0 + r) * G + g0 + g;
                    v = f32x2{f16_to_f32(a.scale[gi]), f16_to_f32(a.minv[gi])};
                }
                smb[g * kRows + r] = v;
            }
        }

        __builtin_amdgcn_s_waitcnt(0);
        prepare(0);
        lds_barrier();

        // iteration j prepares group j + 1 and issues group j + 1 + XD into
        // the slot of group j - 1, which the compute waves finished before
        // the previous barrier
        for (int j0 = 0; j0 < niter; j0 += kPre) {
#pragma unroll
            for (int u = 0; u < kPre; ++u) {
                const int j = j0 + u;
                __builtin_amdgcn_s_waitcnt(kWaitXD<MT>);   // group j + 1 has landed
                prepare(j + 1);
                issue(j + 1 + XD);
                lds_barrier();
            }
        }
        __builtin_amdgcn_s_waitcnt(0);   // no direct-to-LDS load outlives the wave
    }

    // ---------------------------------------------------------------- epilogue
    if (KS == 1) {
        if (wave < kCompute) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = 16 * mt + (lane & 15);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = row0 + 16 * wave + 4 * (lane >> 4) + v;
                    if (m < a.M && row < a.N) a.y[(size_t)m * a.N + row] = f32_to_bf16(acc[mt][v]);
                }
            }
        }
        return;
    }
    // split K: publish this slice's partial tile; the last slice to arrive
    // reduces.  Partials are written and read with device-coherent (agent
    // scope) accesses, which do not stop in the per-XCD L2, and every wave
    // waits for its stores to complete before the barrier that precedes the
    // block's counter update, so no cache-wide write-back or invalidate is
    // needed.
    float* part = tt.t[ti].part;
    unsigned* cnt = tt.t[ti].cnt;
    if (wave < kCompute) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float* dst = part + ((((size_t)blk * KS + ks) * kCompute + wave) * MT * 64 + mt * 64 + lane) * 4;
#pragma unroll
            for (int v = 0; v < 4; ++v) __hip_atomic_store(dst + v, acc[mt][v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's partial stores have completed
    __syncthreads();
    __shared__ unsigned s_prev;
    if (tid == 0) s_prev = __hip_atomic_fetch_add(&cnt[blk], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_prev != (unsigned)(KS - 1)) return;
    if (wave < kCompute) {
        f32x4 sum[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) sum[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float* src = part + ((((size_t)blk * KS + s) * kCompute + wave) * MT * 64 + mt * 64 + lane) * 4;
#pragma unroll
                for (int v = 0; v < 4; ++v) sum[mt][v] += __hip_atomic_load(src + v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = 16 * mt + (lane & 15);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = row0 + 16 * wave + 4 * (lane >> 4) + v;
                if (m < a.M && row < a.N) a.y[(size_t)m * a.N + row] = f32_to_bf16(sum[mt][v]);
            }
        }
    }
    if (tid == 0) __hip_atomic_store(&cnt[blk], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// Split plan: no split while the row blocks alone give >= 256 workgroups;
// otherwise enough slices to reach about 384 workgroups, each slice >= 4
// groups.  Without a workspace every task runs unsplit (the caller has
// checked that its groups fit LDS).
template <int MT>
void mm_plan(const GemvArgs* tasks, int count, bool can_split, int* ks, int* gps) {
    int blocks = 0;
    for (int i = 0; i < count; ++i) blocks += (tasks[i].N + kRows - 1) / kRows;
    int want = 1;
    if (can_split && blocks < 256) want = (384 + blocks - 1) / blocks;
    for (int i = 0; i < count; ++i) {
        const int G = tasks[i].K >> 7;
        if (!can_split) {
            ks[i] = 1;
            gps[i] = G;
            continue;
        }
        // slices of 8 groups (a multiple of the weight prefetch round and of
        // a 16-byte parameter piece) where K allows, at least 4 groups each
        int k = want;
        const int kmax = G >= 8 ? G / 8 : 1;
        if (k > kmax) k = kmax;
        if (k < 1) k = 1;
        int g = (G + k - 1) / k;
        if (G % 8 == 0) g = ((g + 7) / 8) * 8;
        const int gmax = (mm_max_gps<MT>() / 8) * 8;
        if (g > gmax) g = gmax;
        ks[i] = (G + g - 1) / g;
        gps[i] = g;
    }
}

template <int MT>
size_t ws_bytes_mt(const GemvArgs* tasks, int count) {
    int ks[kMaxTasks], gps[kMaxTasks];
    mm_plan<MT>(tasks, count, true, ks, gps);
    size_t bytes = 0;
    for (int i = 0; i < count; ++i) {
        if (ks[i] <= 1) continue;
        const size_t blocks = (tasks[i].N + kRows - 1) / kRows;
        bytes += blocks * ks[i] * kCompute * MT * 64 * 16;
        bytes += ((blocks * 4 + 255) / 256) * 256;
    }
    return bytes;
}

template <int MT>
hipError_t launch_mm_mt(const GemvArgs* tasks, int count, void* ws, size_t ws_bytes, hipStream_t st) {
    int ks[kMaxTasks], gps[kMaxTasks];
    const bool split = ws != nullptr && ws_bytes >= ws_bytes_mt<MT>(tasks, count);
    mm_plan<MT>(tasks, count, split, ks, gps);
    MmTable tt{};
    for (int i = 0; i < kMaxTasks; ++i) tt.blk0[i] = 0x7fffffff;
    uint8_t* p = static_cast<uint8_t*>(ws);
    int grid = 0, gmax = 0;
    for (int i = 0; i < count; ++i) {
        const int blocks = (tasks[i].N + kRows - 1) / kRows;
        tt.blk0[i] = grid;
        tt.t[i].a = tasks[i];
        tt.t[i].ks = ks[i];
        tt.t[i].gps = gps[i];
        const int G = tasks[i].K >> 7;
        tt.t[i].sm16 = (G % 8 == 0 && gps[i] % 8 == 0 && (reinterpret_cast<uintptr_t>(tasks[i].scale) % 16) == 0 &&
                        (reinterpret_cast<uintptr_t>(tasks[i].minv) % 16) == 0) ? 1 : 0;
        if (ks[i] > 1) {
            tt.t[i].part = reinterpret_cast<float*>(p);
            p += (size_t)blocks * ks[i] * kCompute * MT * 64 * 16;
            tt.t[i].cnt = reinterpret_cast<unsigned*>(p);
            p += (((size_t)blocks * 4 + 255) / 256) * 256;
        }
        grid += blocks * ks[i];
        gmax = gps[i] > gmax ? gps[i] : gmax;
    }
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(q4_mm_kernel<MT>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget);
    if (attr != hipSuccess) return attr;
    return launch_kernel(q4_mm_kernel<MT>, dim3(grid), dim3(kThreads), (size_t)mm_shmem<MT>(gmax), st, tt);
}

}  // namespace

bool mm_supported(int M, int K, bool split) {
    if (M < 1 || M > 64 || K % 128) return false;
    if (split) return true;
    const int G = K >> 7;
    switch ((M + 15) / 16) {
        case 1: return G <= mm_max_gps<1>();
        case 2: return G <= mm_max_gps<2>();
        case 3: return G <= mm_max_gps<3>();
        default: return G <= mm_max_gps<4>();
    }
}

size_t mm_workspace_bytes(const GemvArgs* tasks, int count) {
    switch ((tasks[0].M + 15) / 16) {
        case 1: return ws_bytes_mt<1>(tasks, count);
        case 2: return ws_bytes_mt<2>(tasks, count);
        case 3: return ws_bytes_mt<3>(tasks, count);
        default: return ws_bytes_mt<4>(tasks, count);
    }
}

hipError_t launch_mm(const GemvArgs* tasks, int count, void* ws, size_t ws_bytes, hipStream_t s) {
    switch ((tasks[0].M + 15) / 16) {
        case 1: return launch_mm_mt<1>(tasks, count, ws, ws_bytes, s);
        case 2: return launch_mm_mt<2>(tasks, count, ws, ws_bytes, s);
        case 3: return launch_mm_mt<3>(tasks, count, ws, ws_bytes, s);
        default: return launch_mm_mt<4>(tasks, count, ws, ws_bytes, s);
    }
}

}  // namespace q4
