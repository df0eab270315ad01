// Packed-dot GEMV for small decode batches (gfx950).
//
// Each lane owns one or more 16-byte chunks of a weight row and keeps the
// matching activations in registers for the whole kernel, so the activation
// vector is read once per wave while the weights stream past.  A wave-wide
// 128-bit load covers 1 KB of consecutive weight bytes (one int4 row at
// K = 2048, several rows for shorter K, a quarter row at K = 8192).  Nibbles
// become BF16 pairs in registers and meet the activations in
// v_dot2c_f32_bf16; group parameters are applied once per chunk; lanes that
// share a row are summed with DPP.  Long rows are split over the waves of a
// workgroup and their partial sums meet in LDS.
//
// Latency: a wave issues its first weight loads before it touches the
// activations, so both arrive in one memory round trip, and it keeps the next
// batch of weight loads in flight while it computes the current one.
//
// One launch can run several independent GEMVs ("tasks": same format and
// batch size, any N and K); workgroups are assigned to tasks by a prefix table.
#include "internal.h"

namespace q4 {

namespace {

constexpr int kWavesPerWG = 4;
constexpr int kMaxR = 16;
constexpr int kMaxMT = 8;

template <class F> struct FmtTraits;
template <> struct FmtTraits<FmtQ4> { static constexpr int base_cpl = 1; };
template <> struct FmtTraits<FmtNvfp4> { static constexpr int base_cpl = 1; };
template <> struct FmtTraits<FmtBf16> { static constexpr int base_cpl = 4; };

// Per-task launch plan: lanes per row (log2), waves per row (S in 1, 2, 4),
// row-loads per wave (R, a multiple of the in-flight batch U), first block.
struct TaskPlan {
    int lpr_log2, S, R, blk0, staged;
};

struct TaskTable {
    int blk0[kMaxTasks];     // first workgroup of each task (unused slots: INT_MAX)
    GemvArgs a[kMaxTasks];
    TaskPlan p[kMaxTasks];
    int count;
};

template <int CPL> struct Batch { static constexpr int U = (CPL >= 4) ? 1 : 2; };

// Sum over aligned groups of 2^L lanes with L known at compile time.
template <int L>
__device__ __forceinline__ float group_sum_fixed(float v) {
    if (L >= 1) v += dpp<0xB1>(v);
    if (L >= 2) v += dpp<0x4E>(v);
    if (L >= 3) v += dpp<0x141>(v);
    if (L >= 4) v += dpp<0x140>(v);
    if (L >= 5) v += dpp<0x142, 0xA>(v);
    if (L >= 6) v += dpp<0x143, 0xC>(v);
    return v;
}

// LPRT: log2(lanes per row) fixed at compile time, or 0 for "from the plan".
template <class F, int MT, int CPL, int LPRT>
__global__ __launch_bounds__(256) void gemv_dot2_kernel(TaskTable tt) {
    constexpr int U = Batch<CPL>::U;
    __shared__ float red[kWavesPerWG][kMaxR][MT];
    // per wave, two batches of staged group parameters (ping-pong)
    __shared__ __attribute__((aligned(16))) uint8_t stage[F::kStaged ? kWavesPerWG : 1][2][F::kStageBytes > 0 ? F::kStageBytes : 16];

    // which task owns this workgroup
    int t = 0;
#pragma unroll
    for (int i = 1; i < kMaxTasks; ++i) t += ((int)blockIdx.x >= tt.blk0[i]) ? 1 : 0;
    const GemvArgs a = tt.a[t];
    const TaskPlan tp = tt.p[t];
    const int lpr_log2 = LPRT > 0 ? LPRT : tp.lpr_log2;
    const int S = tp.S, R = tp.R;
    const bool staged = F::kStaged && tp.staged;
    const int blk = blockIdx.x - tp.blk0;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int LPR = 1 << lpr_log2;
    const int RPL = 64 >> lpr_log2;
    const int RG = kWavesPerWG / S;
    const int s = wave % S;
    const int rg = wave / S;
    const int sub = lane >> lpr_log2;
    const int li = lane & (LPR - 1);
    const int C = a.K / F::WPC;
    const uint32_t rowbytes = (uint32_t)C * 16;
    const int rowbase = (blk * RG + rg) * R * RPL;
    int nrows = a.N - rowbase;                    // rows of this wave that exist
    nrows = nrows < 0 ? 0 : (nrows > R * RPL ? R * RPL : nrows);

    // Buffer resources start at the wave's first row and end at its last
    // existing row: lanes whose row is past N read zeros.
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w + (size_t)rowbase * rowbytes, (uint32_t)nrows * rowbytes);
    const typename F::AuxRes rx = F::make_aux(a, rowbase, nrows);

    int ch[CPL];
    bool act[CPL];
    uint32_t vw[CPL], vx[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = (j * S + s) * LPR + li;
        act[j] = c < C;
        ch[j] = act[j] ? c : C - 1;
        vw[j] = (uint32_t)sub * rowbytes + (uint32_t)ch[j] * 16;
        vx[j] = F::aux_voff(a, sub, ch[j]);
    }

    // The whole offset goes in the lane offset (which the range check covers);
    // the scalar offset stays 0.
    auto load = [&](int i0, u32x4 (&q)[U][CPL], typename F::Aux (&ax)[U][CPL], u32x4& stg) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = (i0 + u) * RPL;
            const uint32_t sw = (uint32_t)r * rowbytes;
            const uint32_t sx = F::aux_soff(a, r);
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                q[u][j] = buf_load16(rw, vw[j] + sw, 0);
                if (!staged) ax[u][j] = F::load_aux(rx, vx[j] + sx, 0);
            }
        }
        if (staged) stg = F::load_stage(a, rowbase + i0 * RPL, U * RPL, lane);
    };

    typename F::X xc[CPL][MT];
    auto compute = [&](int i0, int buf, const u32x4 (&q)[U][CPL], typename F::Aux (&ax)[U][CPL], const u32x4& stg) {
        if (staged) {
            // one wave writes and reads its own slot: LDS keeps a wave's
            // accesses in order, so no barrier is needed
            uint8_t* slot = stage[F::kStaged ? wave : 0][buf];
            *reinterpret_cast<u32x4*>(slot + lane * 16) = stg;
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < CPL; ++j)
                    ax[u][j] = F::read_stage(reinterpret_cast<const uint16_t*>(slot), a, u * RPL + sub, ch[j]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = rowbase + (i0 + u) * RPL + sub;
            float out[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) out[m] = 0.f;
#pragma unroll
            for (int j = 0; j < CPL; ++j)
                if (act[j]) F::template accumulate<MT>(q[u][j], ax[u][j], xc[j], out);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float v = LPRT > 0 ? group_sum_fixed<LPRT>(out[m]) : group_sum(out[m], LPR);
                if (li == LPR - 1) {
                    if (S == 1) {
                        if (row < a.N && m < a.M) a.y[(size_t)m * a.N + row] = f32_to_bf16(F::finish(a, v));
                    } else {
                        red[wave][i0 + u][m] = v;
                    }
                }
            }
        }
    };

    // weights of the first batch go out before the activations
    u32x4 qa[U][CPL], qb[U][CPL];
    typename F::Aux aa[U][CPL], ab[U][CPL];
    u32x4 sa, sb;
    load(0, qa, aa, sa);
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int m = 0; m < MT; ++m)
            F::load_x(a.x + (size_t)(m < a.M ? m : 0) * a.K, ch[j] * F::WPC, act[j] && m < a.M, xc[j][m]);

    // ping-pong: the next batch is in flight while the current one is used
    for (int i0 = 0;;) {
        const bool nb = i0 + U < R;
        if (nb) load(i0 + U, qb, ab, sb);
        compute(i0, 0, qa, aa, sa);
        if (!nb) break;
        i0 += U;
        const bool na = i0 + U < R;
        if (na) load(i0 + U, qa, aa, sa);
        compute(i0, 1, qb, ab, sb);
        if (!na) break;
        i0 += U;
    }

    if (S > 1) {
        __syncthreads();
        const int total = RG * R * MT;
        for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
            const int m = idx % MT;
            const int i = (idx / MT) % R;
            const int g = idx / (MT * R);
            float v = 0.f;
            for (int w = 0; w < S; ++w) v += red[g * S + w][i][m];
            const int row = (blk * RG + g) * R + i;   // RPL == 1 when S > 1
            if (row < a.N && m < a.M) a.y[(size_t)m * a.N + row] = f32_to_bf16(F::finish(a, v));
        }
    }
}

template <class F>
bool make_plan(int N, int K, TaskPlan& p, int& cpl_out, int& blocks) {
    const int C = K / F::WPC;
    int cpl = FmtTraits<F>::base_cpl;
    const int lanes = (C + cpl - 1) / cpl;
    int S = 1, lpr = 1;
    if (lanes <= 64) {
        while (lpr < lanes) lpr <<= 1;
    } else {
        lpr = 64;
        S = (lanes + 63) / 64;
        if (S > 2) S = 4;
        while (64 * S * cpl < C) cpl *= 2;
        if (cpl > 2 * FmtTraits<F>::base_cpl) return false;
    }
    int lpr_log2 = 0;
    while ((1 << lpr_log2) < lpr) ++lpr_log2;
    const int RPL = 64 / lpr;
    const int loads = (N + RPL - 1) / RPL;
    const int U = (cpl >= 4) ? 1 : 2;
    // Aim for ~8 waves per CU; small matrices get one batch per wave.
    const int target_waves = 2048;
    int R = (int)(((long)loads * S + target_waves - 1) / target_waves);
    if (R < 1) R = 1;
    if (R > kMaxR) R = kMaxR;
    R = ((R + U - 1) / U) * U;
    const int RG = kWavesPerWG / S;
    p.lpr_log2 = lpr_log2;
    p.S = S;
    p.R = R;
    p.staged = 0;
    cpl_out = cpl;
    blocks = (loads + R * RG - 1) / (R * RG);
    return true;
}

template <class F, int MT, int CPL>
hipError_t launch_mt(const TaskTable& tt, int grid, bool lpr64, hipStream_t st) {
    // rows of 64 lanes (K = 2048 / 8192 for the 4-bit formats) get the
    // straight-line reduction; batch tiles above 4 rows share the generic one
    if (lpr64 && MT <= 4) return launch_kernel(gemv_dot2_kernel<F, MT, CPL, 6>, dim3(grid), dim3(256), 0, st, tt);
    return launch_kernel(gemv_dot2_kernel<F, MT, CPL, 0>, dim3(grid), dim3(256), 0, st, tt);
}

template <class F, int CPL>
hipError_t launch_cpl(const TaskTable& tt, int M, int grid, bool lpr64, hipStream_t st) {
    switch (M) {
        case 1: return launch_mt<F, 1, CPL>(tt, grid, lpr64, st);
        case 2: return launch_mt<F, 2, CPL>(tt, grid, lpr64, st);
        case 3: return launch_mt<F, 3, CPL>(tt, grid, lpr64, st);
        case 4: return launch_mt<F, 4, CPL>(tt, grid, lpr64, st);
        case 5: return launch_mt<F, 5, CPL>(tt, grid, lpr64, st);
        case 6: return launch_mt<F, 6, CPL>(tt, grid, lpr64, st);
        case 7: return launch_mt<F, 7, CPL>(tt, grid, lpr64, st);
        default: return launch_mt<F, 8, CPL>(tt, grid, lpr64, st);
    }
}

// Tasks are grouped by chunks-per-lane (a template parameter); each group is
// one launch per batch tile of at most 8 rows.
template <class F>
hipError_t launch_fmt(const GemvArgs* tasks, int count, hipStream_t st) {
    const int base = FmtTraits<F>::base_cpl;
    for (int pass = 0; pass < 2; ++pass) {
        const int want_cpl = pass == 0 ? base : 2 * base;
        const int M = tasks[0].M;
        for (int m0 = 0; m0 < M; m0 += kMaxMT) {
            TaskTable tt{};
            for (int i = 0; i < kMaxTasks; ++i) tt.blk0[i] = 0x7fffffff;
            tt.blk0[0] = 0;
            int grid = 0;
            for (int i = 0; i < count; ++i) {
                TaskPlan p;
                int cpl, blocks;
                if (!make_plan<F>(tasks[i].N, tasks[i].K, p, cpl, blocks)) return hipErrorInvalidValue;
                if (cpl != want_cpl) continue;
                GemvArgs a = tasks[i];
                a.M = (M - m0) < kMaxMT ? (M - m0) : kMaxMT;
                a.x = tasks[i].x + (size_t)m0 * tasks[i].K;
                a.y = tasks[i].y + (size_t)m0 * tasks[i].N;
                p.blk0 = grid;
                // int4 group parameters go through LDS when their 16-byte
                // loads are aligned (see FmtQ4)
                p.staged = (F::kStaged && (tasks[i].K % 1024) == 0 && (reinterpret_cast<uintptr_t>(tasks[i].scale) % 16) == 0 &&
                            (reinterpret_cast<uintptr_t>(tasks[i].minv) % 16) == 0) ? 1 : 0;
                tt.blk0[tt.count] = grid;
                tt.a[tt.count] = a;
                tt.p[tt.count] = p;
                ++tt.count;
                grid += blocks;
            }
            if (tt.count == 0) break;
            bool lpr64 = true;
            for (int i = 0; i < tt.count; ++i) lpr64 = lpr64 && tt.p[i].lpr_log2 == 6;
            const int mt = (M - m0) < kMaxMT ? (M - m0) : kMaxMT;
            hipError_t e = (pass == 0) ? launch_cpl<F, FmtTraits<F>::base_cpl>(tt, mt, grid, lpr64, st)
                                       : launch_cpl<F, 2 * FmtTraits<F>::base_cpl>(tt, mt, grid, lpr64, st);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace

bool dot2_supported(Fmt fmt, int K) {
    TaskPlan p;
    int cpl, blocks;
    switch (fmt) {
        case kFmtQ4: return make_plan<FmtQ4>(1, K, p, cpl, blocks);
        case kFmtNvfp4: return make_plan<FmtNvfp4>(1, K, p, cpl, blocks);
        default: return make_plan<FmtBf16>(1, K, p, cpl, blocks);
    }
}

hipError_t launch_dot2(Fmt fmt, const GemvArgs* tasks, int count, hipStream_t s) {
    switch (fmt) {
        case kFmtQ4: return launch_fmt<FmtQ4>(tasks, count, s);
        case kFmtNvfp4: return launch_fmt<FmtNvfp4>(tasks, count, s);
        default: return launch_fmt<FmtBf16>(tasks, count, s);
    }
}

}  // namespace q4
