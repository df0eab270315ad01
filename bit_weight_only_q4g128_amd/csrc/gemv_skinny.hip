// Skinny matrix-core GEMV for batched decode (5 <= M <= 48, K % 128 == 0;
// gfx950, v_mfma_f32_16x16x32_bf16): int4 g128 weights, and in the same
// launch NVFP4 and BF16 ones (the NVFP4 decode step keeps v and down in BF16).
//
// The decode batch shares one read of the weights: at M = 48 every weight byte
// feeds 48 products ("rumik-oss-1-nvfp4-vllm" card, "Concurrent request
// throughput": one weight read serves many sequences).  A workgroup (eight
// waves) owns R 16-row tiles over a slice of at most 16 groups of K (the whole
// of K for the hidden-2048 projections); each wave owns one or two adjacent
// groups of the slice (its rounds) for all R tiles, so a wave needs only its
// own data and the waves meet only once, at the end.
//
// Memory.  A wave issues everything it will need as soon as it starts: its
// rows' scales for its groups and a share of the workgroup's mins, the first
// round's activations (MT x 16 batch rows x 256 bytes) -- these straight into
// LDS with buffer_load ... lds, into regions of their own, so no barrier is
// involved -- and the weights of both its rounds, straight into registers
// (from MT = 2 on, the weights once the first part has landed: see there).
// The workgroup's vector-memory path delivers cache lines at a bounded rate,
// so every load reads whole 128-byte lines: four activation rows per
// instruction, and for the weights eight rows x the wave's two adjacent
// groups (128 bytes), the lanes then exchanging chunks with DPP row shifts to
// reach the matrix-core operand layout.  The second round's activations
// follow once the first round has computed (the region it read out at its
// start is then free, and the loads ahead of them have drained).  Every
// buffer offset is scalar
// plus one per-lane base, so the address arithmetic costs no vector
// instructions.
//
// Arithmetic per round: the activation fragments are read from LDS (an XOR
// swizzle of the 16-byte chunks by row makes every read conflict-free) and
// paired as (x0,x4) (x1,x5) (x2,x6) (x3,x7) to match the nibble unpack; an
// all-ones B operand gives SX (the group's activation sum per batch row); per
// tile each lane's 8 codes per k-step become BF16 "128 + code" (v_perm_b32 on
// the 0x43 exponent byte) and the MFMAs accumulate D = sum of (128 + code) * x
// with the activations as the A operand, so a lane's four results share one
// weight row; the round folds as acc += scale * D (one FMA per result).  The
// remaining term, sum over groups of (min - 128 scale) * SX, is a product of
// a [batch x groups] and a [groups x rows] matrix: it is formed once per
// workgroup, after the waves meet, with fp32 MFMAs (v_mfma_f32_16x16x4f32)
// from the SX and group parameters left in LDS.  Every product is exact, and
// for a one-hot x so is every sum.
//
// The eight waves' tiles meet in LDS and are summed in wave order; when K is
// split over workgroups, each adds its min term and writes its fp32 tiles to
// the caller's workspace, and the workgroup that arrives last at the row
// block's counter sums the slices in slice order, writes y and resets the
// counter.
//
// NVFP4 rounds read their codes exactly as int4 rounds do (64 bytes of a row
// per group, two groups per cache line).  Each 8-code dword becomes BF16
// pairs e2m1 * e4m3 -- exact: at most 6 significant bits -- with the lane's
// 16-column block scale staged in LDS, in natural column order (the
// activations are not paired); the MFMAs accumulate across groups directly
// and the global scale multiplies each finished output once.  BF16 rounds
// take one group of 128 columns per wave (256 bytes of a row, two cache
// lines; slices of 8 groups): the same row-shift exchange turns eight-row
// whole-line loads into the operand layout, k-step s taking 16-byte chunk
// 8 (s / 2) + 2 (l / 16) + s % 2 of the group.  Neither has a min term.
//
// MFMA operand layout (16x16x32): lane l holds A row l % 16 and B column
// l % 16, k-values 8 (l / 16) .. + 8 of the k-step.  For k-step s of a group,
// lane l's k-values are the 8 columns 32 (l / 16) + 8 s .. + 8 of the group
// (in the pairing order): dword s of the lane's 16 weight bytes, and the
// activations at the same columns.  D: lane l holds rows 4 (l / 16) + v
// (v = 0..3; here batch rows) of column l % 16 (here a weight row).
#include "internal.h"

namespace q4 {

namespace {

constexpr int kSkWaves = 8;
constexpr int kSkThreads = 64 * kSkWaves;
constexpr int kSkMaxGroups = 16;   // groups per workgroup slice: two rounds of eight waves
constexpr int kSkCoherent = 16;    // buffer cache policy sc1: device-coherent, not held in the per-XCD L2

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ bf16x8_t as_b8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

struct SkTask {
    GemvArgs a;
    int fmt;         // Fmt of the task's weights
    int ks;          // workgroups (K slices) per row block
    int gs;          // groups per slice
    float* part;     // ks > 1: partial tiles [blocks][ks][R * MT][64 lanes] x 4 floats
    unsigned* cnt;   // ks > 1: arrival counters [blocks], kCtrStride bytes apart
};

struct SkTable {
    int blk0[kMaxTasks];   // first workgroup of each task (unused: INT_MAX)
    SkTask t[kMaxTasks];
};

// LDS layout (bytes):
//   [0, kArea)           per wave, kWave bytes: one round of activations,
//                        MT * 16 rows x 256 bytes; after its rounds, the
//                        wave's result tiles [R * MT][64 lanes] x 16 bytes
//   [kArea, + kPar)      per wave: the scales of its 16 R rows for its two
//                        group slots -- int4: [16 R][2] dwords holding the
//                        fp16 value in the low half (a 2-byte load to LDS
//                        writes one zero-extended dword per lane); NVFP4:
//                        [16 R][2][2] dwords, the group's eight e4m3 bytes --
//                        padded to whole 64-lane loads
//   [.., + kMin)         the mins of the workgroup's 16 R rows for the slice's
//                        groups, [16 R][17] dwords (fp16 in the low half; the
//                        17th word of a row is padding, so that one group's
//                        mins of 16 consecutive rows sit in 16 distinct
//                        banks), padded to whole 64-lane loads of all eight
//                        waves
//   [.., + kSx)          SX per group of the slice and batch row, fp32 [16][16 MT]
// FM: the formats a launch carries (bit 0 int4, bit 1 NVFP4, bit 2 BF16);
// only their code is compiled into an instance
template <int MT, int R, int FM>
struct SkLds {
    static constexpr int kX = MT * 16 * 256;
    static constexpr int kWave = (kX > R * MT * 1024) ? kX : R * MT * 1024;
    static constexpr int kArea = kSkWaves * kWave;
    static constexpr int kParArr = (((FM & 2) ? 64 : 32) * R + 63) / 64 * 64;   // dwords per wave, whole 64-lane loads
    static constexpr int kPar = kSkWaves * kParArr * 4;
    static constexpr int kMinPitch = kSkMaxGroups + 1;                                         // dwords per row
    static constexpr int kMinLoads = ((16 * R * kMinPitch + 63) / 64 + kSkWaves - 1) / kSkWaves;   // per wave
    static constexpr int kMin = kSkWaves * kMinLoads * 64 * 4;
    static constexpr int kSx = kSkMaxGroups * 16 * MT * 4;
    static constexpr int kBytes = kArea + kPar + kMin + kSx;
};

// Workgroup barrier that waits only for this wave's LDS traffic, so the
// vector-memory loads in flight stay in flight across it.
__device__ __forceinline__ void lds_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt immediates (gfx9 encoding): vmcnt(n) only, lgkmcnt(0) only
__host__ __device__ constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kLgkm0 = 0xC07F;

// One result tile (16 weight rows x 16 batch rows) to y: lane l holds batch
// rows 16 mt + 4 (l / 16) + v (v = 0..3) of weight row trow + l % 16; res
// holds the task's residual at the same elements (BF16 bits, zero without a
// residual), added before the one rounding.  (16 lanes store 32 contiguous
// bytes of a batch row.)
__device__ __forceinline__ void sk_write_tile(const SkTask& tk, int trow, int mt, int lane, f32x4 r, const uint32_t (&res)[4]) {
    const GemvArgs& a = tk.a;
    const int row = trow + (lane & 15);
    if (row >= a.N) return;
    const int m0 = 16 * mt + 4 * (lane >> 4);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = m0 + v;
        if (m >= a.M) break;
        a.y[(size_t)m * a.N + row] = f32_to_bf16(r[v] + __builtin_bit_cast(float, res[v] << 16));
    }
}

template <int MT, int R, int FM>
__global__ __launch_bounds__(kSkThreads) void skinny_q4_kernel(SkTable tt) {
    using L = SkLds<MT, R, FM>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    int ti = 0;
#pragma unroll
    for (int i = 1; i < kMaxTasks; ++i) ti += ((int)blockIdx.x >= tt.blk0[i]) ? 1 : 0;
    const SkTask& tk = tt.t[ti];
    const GemvArgs& a = tk.a;
    const bool q4f = (FM & 1) && (FM == 1 || tk.fmt == kFmtQ4);
    const bool nvf = (FM & 2) && (FM == 2 || tk.fmt == kFmtNvfp4);
    const bool bff = (FM & 4) && (FM == 4 || tk.fmt == kFmtBf16);
    const int KS = tk.ks;
    const int local = (int)blockIdx.x - tt.blk0[ti];
    const int blk = local / KS, ks = local - blk * KS;
    const int G = a.K >> 7;
    const int g0 = ks * tk.gs;
    const int ng = (G - g0 < tk.gs) ? G - g0 : tk.gs;   // groups of this slice, >= 1
    const int nr = (ng + kSkWaves - 1) / kSkWaves;      // rounds per wave: 1 or 2 (BF16: 1)
    const int row0 = blk * 16 * R;
    const int nrows = (a.N - row0 < 16 * R) ? a.N - row0 : 16 * R;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t rowbytes = bff ? (uint32_t)a.K * 2u : (uint32_t)a.K >> 1;
    const int nv = ng - nr * wave;                       // this wave's valid rounds (may be <= 0)

    uint8_t* xbuf = lds + wave * L::kWave;
    uint32_t* par = reinterpret_cast<uint32_t*>(lds + L::kArea);               // scales [8][kParArr]
    uint32_t* mtab = reinterpret_cast<uint32_t*>(lds + L::kArea + L::kPar);    // mins [16 R][16]
    float* sxt = reinterpret_cast<float*>(lds + L::kArea + L::kPar + L::kMin);  // [16][16 MT]

    // ---- 1. issue: group parameters (to LDS), round-0 activations (to LDS),
    // all weights (to registers).  Out-of-range offsets read zero.
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scale + (size_t)row0 * G, (uint32_t)nrows * (uint32_t)G * 2u);
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(a.minv + (size_t)row0 * G, (uint32_t)nrows * (uint32_t)G * 2u);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)a.M * (uint32_t)a.K * 2u);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w + (size_t)row0 * rowbytes, (uint32_t)nrows * rowbytes);
    // scales, per wave.  int4: element e = 64 i + lane is (row e / 2, slot
    // e % 2) -> group g0 + nr w + slot.  NVFP4: dword e = 64 i + lane is (row
    // e / 4, slot (e / 2) % 2, half e % 2) -> bytes 4 half .. 4 half + 3 of the
    // eight e4m3 scales of group g0 + nr w + slot.
    if (q4f) {
        constexpr int kPI = (16 * R * 2 + 63) / 64;
#pragma unroll
        for (int i = 0; i < kPI; ++i) {
            const int e = 64 * i + lane;
            const int row = e >> 1, slot = e & 1;
            const bool ok = row < 16 * R && slot < nv;
            const uint32_t off = ok ? ((uint32_t)row * (uint32_t)G + (uint32_t)(g0 + nr * wave + slot)) * 2u : 0xFFFFFFF0u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(par + wave * L::kParArr + 64 * i), 2, off, 0, 0, 0);
        }
    } else if (nvf) {
        const uint32_t sb = (uint32_t)a.K >> 4;   // scale bytes per row
        const __amdgpu_buffer_rsrc_t r8 = make_rsrc(a.scale8 + (size_t)row0 * sb, (uint32_t)nrows * sb);
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int e = 64 * i + lane;
            const int row = e >> 2, slot = (e >> 1) & 1, hf = e & 1;
            const bool ok = row < 16 * R && slot < nv;
            const uint32_t off = ok ? (uint32_t)row * sb + (uint32_t)(g0 + nr * wave + slot) * 8u + 4u * (uint32_t)hf : 0xFFFFFFF0u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r8, (lds_void*)(par + wave * L::kParArr + 64 * i), 4, off, 0, 0, 0);
        }
    }
    // int4 mins, once per workgroup (they are read only after the waves
    // meet): element e = 64 (wave + 8 j) + lane is (row e / 17, group e % 17
    // of the slice; group 16 is the padding word, never loaded); four rows'
    // slices of a whole-K task share one cache line
#pragma unroll
    for (int j = 0; j < L::kMinLoads; ++j) {
        if (!q4f) break;
        const int e = 64 * (wave + kSkWaves * j) + lane;
        const int row = e / L::kMinPitch, gi = e - L::kMinPitch * row;
        const bool ok = row < 16 * R && gi < ng;
        const uint32_t off = ok ? ((uint32_t)row * (uint32_t)G + (uint32_t)(g0 + gi)) * 2u : 0xFFFFFFF0u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rm, (lds_void*)(mtab + 64 * (wave + kSkWaves * j)), 2, off, 0, 0, 0);
    }
    // activations of round r: instruction i covers batch rows 4 i .. 4 i + 3;
    // lane l writes position p = l % 16 of row m = 4 i + l / 16 and fetches
    // the row's 16-byte chunk p ^ (m % 16) of the group
    const int xm_l = lane >> 4, xp = lane & 15;
    auto issue_x = [&](int r) {
        const bool ok = r < nv;
        const uint32_t gcol = (uint32_t)(g0 + nr * wave + r) * 128u;
#pragma unroll
        for (int i = 0; i < 4 * MT; ++i) {
            const int m = 4 * i + xm_l;
            const uint32_t off = ok ? ((uint32_t)m * (uint32_t)a.K + gcol + 8u * (uint32_t)(xp ^ (m & 15))) * 2u : 0xFFFFFFF0u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(xbuf + 1024 * i), 16, off, 0, 0, 0);
        }
    };
    if (nv > 0) issue_x(0);   // (a wave without a group of the slice fills nothing)
    // weights.  A wave's two groups are adjacent, 128 bytes of each row (one
    // cache line), so a load instruction reads eight rows in whole lines:
    // lane l reads row l % 8 of the tile's lower (L0) or upper (L1) eight
    // rows, 16-byte chunk l / 16 of the first group (l % 16 < 8) or of the
    // second (l % 16 >= 8).  (A wave with one group reads that group's chunk
    // l / 16 in both halves of the lane range.)  The row and group parts of
    // the offset are scalar.
    // BF16: the wave's one group is 256 bytes of each row, two cache lines;
    // a load reads eight rows of one line, lane l row l % 8, 16-byte chunk
    // l / 8 (L0/L1: the first line, L2/L3: the second).
    const bool pair = nr == 2;
    const uint32_t woff = bff ? (uint32_t)(lane & 7) * rowbytes + 16u * (uint32_t)(lane >> 3)
                              : (uint32_t)(lane & 7) * rowbytes + 16u * (uint32_t)(lane >> 4) + (pair ? 64u * (uint32_t)((lane >> 3) & 1) : 0u);
    const __amdgpu_buffer_rsrc_t rw0 = nv > 0 ? rw : make_rsrc(a.w, 0u);
    const uint32_t gb = (uint32_t)(g0 + nr * wave) * (bff ? 256u : 64u);
    // The two waves that share a SIMD issue vector-memory instructions oldest
    // first, so a wave that issued all its loads at once would queue the other
    // wave's activations behind its own weights; from two batch tiles on a
    // wave first waits for its parameters and activations, and the SIMD's
    // other wave issues its own meanwhile (at one batch tile the wait costs
    // more than it saves).
    if constexpr (MT >= 2) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
    }
    u32x4 L0[R], L1[R], L2[R], L3[R];
#pragma unroll
    for (int t = 0; t < R; ++t) {
        L0[t] = buf_load16(rw0, woff, (uint32_t)(16 * t) * rowbytes + gb);
        L1[t] = buf_load16(rw0, woff, (uint32_t)(16 * t + 8) * rowbytes + gb);
        if (bff) {
            L2[t] = buf_load16(rw0, woff, (uint32_t)(16 * t) * rowbytes + gb + 128u);
            L3[t] = buf_load16(rw0, woff, (uint32_t)(16 * t + 8) * rowbytes + gb + 128u);
        }
    }

    // ---- 2. the rounds
    const bf16x8_t ones = as_b8(u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    f32x4 acc[R][MT];
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int kWLoads = 2 * R;   // weight loads issued after the round-0 activations (BF16: twice as many)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int gl = nr * wave + r;   // group within the slice
        if (r >= nr) break;             // wave-uniform
        if (r >= nv) {
            // a slot past the slice: no SX for it
            if (lane < 16 * MT && (lane & 3) == 0)
                *reinterpret_cast<f32x4*>(sxt + gl * 16 * MT + lane) = f32x4{0.f, 0.f, 0.f, 0.f};
            continue;
        }
        // this round's activations (and, in round 0, the parameters) are in LDS
        if (r == 0) {
            if (bff) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kWLoads));
            else __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWLoads));
        } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        // k-step s: lane l takes 8 columns of the group -- 4-bit formats:
        // 32 (l / 16) + 8 s .. (dword s of the lane's weight chunk); BF16:
        // chunk 8 (s / 2) + 2 (l / 16) + s % 2 (line s / 2 after the exchange)
        u32x4 X[MT][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int m = 16 * mt + (lane & 15);
                const int chunk = bff ? 8 * (s >> 1) + 2 * (lane >> 4) + (s & 1) : 4 * (lane >> 4) + s;
                X[mt][s] = *reinterpret_cast<const u32x4*>(xbuf + m * 256 + 16 * (chunk ^ (m & 15)));
            }
        if (!q4f) {
            // NVFP4 and BF16: weights in natural column order, no group fold
#pragma unroll
            for (int t = 0; t < R; ++t) {
                if (nvf) {
                    // the lane's scales for k-steps 0-1 and 2-3: 16-column
                    // blocks 2 (l / 16) and 2 (l / 16) + 1 of the group
                    const uint32_t sw = par[wave * L::kParArr + 4 * (16 * t + (lane & 15)) + 2 * r + (lane >> 5)] >> (16 * ((lane >> 4) & 1));
                    const float sc0 = e4m3_to_f32<0>(sw), sc1 = e4m3_to_f32<1>(sw);
                    u32x4 Wt;
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        Wt[d] = r == 0 ? (uint32_t)__builtin_amdgcn_update_dpp((int)L0[t][d], (int)L1[t][d], 0x118, 0xF, 0xC, false)
                                       : (uint32_t)__builtin_amdgcn_update_dpp((int)L1[t][d], (int)L0[t][d], 0x108, 0xF, 0x3, false);
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const float sc = s < 2 ? sc0 : sc1;
                        const bf16x8_t Wv = as_b8(u32x4{nv_pair_scaled<0>(Wt[s], sc), nv_pair_scaled<1>(Wt[s], sc),
                                                        nv_pair_scaled<2>(Wt[s], sc), nv_pair_scaled<3>(Wt[s], sc)});
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(X[mt][s]), Wv, acc[t][mt], 0, 0, 0);
                    }
                } else {
                    // BF16: rows 0-7 of the tile in L0 / L2, rows 8-15 in L1 / L3;
                    // chunk 2 (l / 16) + s % 2 of row l % 16 comes from this lane or
                    // eight lanes away (the same exchange as the 4-bit rounds)
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const u32x4 La = s < 2 ? L0[t] : L2[t], Lb = s < 2 ? L1[t] : L3[t];
                        u32x4 Wv;
#pragma unroll
                        for (int d = 0; d < 4; ++d)
                            Wv[d] = (s & 1) == 0 ? (uint32_t)__builtin_amdgcn_update_dpp((int)La[d], (int)Lb[d], 0x118, 0xF, 0xC, false)
                                                 : (uint32_t)__builtin_amdgcn_update_dpp((int)Lb[d], (int)La[d], 0x108, 0xF, 0x3, false);
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(X[mt][s]), as_b8(Wv), acc[t][mt], 0, 0, 0);
                    }
                }
            }
            if (r == 0 && nr > 1 && nv > 1) {
                __builtin_amdgcn_s_waitcnt(kLgkm0);
                issue_x(1);
            }
            continue;
        }
        uint32_t sc16[R];   // this lane's row: the scale of this round's group (fp16 in the low half)
#pragma unroll
        for (int t = 0; t < R; ++t) sc16[t] = par[wave * L::kParArr + 2 * (16 * t + (lane & 15)) + r];
        // pairing; SX (all-ones B operand: every column of the result is SX)
        u32x4 B[MT][4];
        f32x4 sx[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const u32x4 v = X[mt][s];
                uint32_t p[4];
                xq4_pairs(v.x, v.y, v.z, v.w, p);
                B[mt][s] = u32x4{p[0], p[1], p[2], p[3]};
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(B[mt][s]), ones, c, 0, 0, 0);
            }
            sx[mt] = c;
        }
        // lanes 0, 16, 32, 48 hold SX of batch rows 16 mt + 4 (l / 16) + v
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            if ((lane & 15) == 0) *reinterpret_cast<f32x4*>(sxt + gl * 16 * MT + 16 * mt + 4 * (lane >> 4)) = sx[mt];
#pragma unroll
        for (int t = 0; t < R; ++t) {
            f32x4 D[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) D[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            // the operand (lane l: row l % 16, chunk l / 16 of the round's
            // group): lanes l % 16 >= 8 take their chunk from eight lanes
            // down in L1 (round 0), lanes l % 16 < 8 from eight lanes up in
            // L0 (round 1) -- DPP row shifts, within rows of 16 lanes
            u32x4 Wt;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                Wt[d] = r == 0 ? (uint32_t)__builtin_amdgcn_update_dpp((int)L0[t][d], (int)L1[t][d], 0x118, 0xF, 0xC, false)
                               : (uint32_t)__builtin_amdgcn_update_dpp((int)L1[t][d], (int)L0[t][d], 0x108, 0xF, 0x3, false);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                uint32_t A[4];
                q4_pairs(Wt[s], A);
                const bf16x8_t Wv = as_b8(u32x4{A[0], A[1], A[2], A[3]});
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) D[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(B[mt][s]), Wv, D[mt], 0, 0, 0);
            }
            const float sc = f16_to_f32((uint16_t)sc16[t]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[t][mt][v] = fmaf(sc, D[mt][v], acc[t][mt][v]);
        }
        // the second round's activations, into the region this round read
        // out at its start: issued only now, since an issue waits for room in
        // the workgroup's queue of loads, which the weights still fill while
        // the first round computes
        if (r == 0 && nr > 1 && nv > 1) {
            __builtin_amdgcn_s_waitcnt(kLgkm0);   // (the fragment reads of the region are long complete)
            issue_x(1);
        }
    }

    // ---- 3. the waves meet: each wave's tiles to its own LDS region as soon
    // as it is done (it has read its last round out of the region), then each
    // wave finishes whole tiles: the eight waves' tiles summed in wave order,
    // plus the min term
    //   sum over the slice's groups of SX[batch][g] * (min - 128 scale)[g][row]
    // as fp32 MFMAs over chunks of four groups.  Every wave's loads into LDS
    // (its share of the group parameters, its activations) are complete
    // before the barrier.
    constexpr int kTiles = R * MT;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    // the residual of the wave's output tiles (p = wave + 8 j, as in the
    // epilogue), fetched now so that its latency hides behind the meeting of
    // the waves: one element per lane and batch row (zero without a residual,
    // or past M or N).  Each element is read only by the lane that then
    // writes it, so the residual may be y itself.
    constexpr int kJ = (kTiles + kSkWaves - 1) / kSkWaves;
    uint32_t res[kJ][4];
    if (a.resid == nullptr) {
#pragma unroll
        for (int j = 0; j < kJ; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) res[j][v] = 0u;
    } else {
        const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.resid, (uint32_t)a.M * (uint32_t)a.N * 2u);
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            const int p = wave + kSkWaves * j;
            const int row = row0 + 16 * (p / MT) + (lane & 15);
            const int m0 = 16 * (p % MT) + 4 * (lane >> 4);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const bool ok = p < kTiles && row < a.N && m0 + v < a.M;
                const uint32_t off = ok ? ((uint32_t)(m0 + v) * (uint32_t)a.N + (uint32_t)row) * 2u : 0xFFFFFFF0u;
                res[j][v] = __builtin_amdgcn_raw_buffer_load_b16(rr, off, 0, 0);
            }
        }
    }
    f32x4* myred = reinterpret_cast<f32x4*>(xbuf);
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) myred[(t * MT + mt) * 64 + lane] = acc[t][mt];
    lds_sync();
    f32x4 fin[(kTiles + kSkWaves - 1) / kSkWaves];
    const int nsh = nr - 1;   // group g of the slice belongs to wave g >> nsh, slot g & nsh
#pragma unroll
    for (int j = 0; j * kSkWaves < kTiles; ++j) {
        const int p = wave + kSkWaves * j;
        if (p < kTiles) {
            const int t = p / MT, mt = p - t * MT;
            const int row = 16 * t + (lane & 15);
            // operands of the min term for all four chunks first (LDS reads in flight together)
            float av[kSkMaxGroups / 4], sv[kSkMaxGroups / 4], mv[kSkMaxGroups / 4];
#pragma unroll
            for (int c = 0; c < kSkMaxGroups / 4; ++c) {
                if (!q4f) break;
                const int g = 4 * c + (lane >> 4);
                const int gi = g < ng ? g : 0;
                const int w2 = gi >> nsh, slot = gi & nsh;
                av[c] = sxt[gi * 16 * MT + 16 * mt + (lane & 15)];
                sv[c] = f16_to_f32((uint16_t)par[w2 * L::kParArr + 2 * row + slot]);
                mv[c] = f16_to_f32((uint16_t)mtab[L::kMinPitch * row + gi]);
            }
            f32x4 v = reinterpret_cast<const f32x4*>(lds)[p * 64 + lane];
#pragma unroll
            for (int w = 1; w < kSkWaves; ++w) v += reinterpret_cast<const f32x4*>(lds + w * L::kWave)[p * 64 + lane];
            if (q4f) {
                f32x4 dm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < kSkMaxGroups / 4; ++c) {
                    const bool ok = 4 * c + (lane >> 4) < ng;
                    dm = __builtin_amdgcn_mfma_f32_16x16x4f32(ok ? av[c] : 0.0f, ok ? fmaf(-128.0f, sv[c], mv[c]) : 0.0f, dm, 0, 0, 0);
                }
                fin[j] = v + dm;
            } else {
                fin[j] = nvf ? v * a.gscale : v;   // NVFP4: the global scale, once per output
            }
        }
    }

    // ---- 4. epilogue
    if (KS == 1) {
#pragma unroll
        for (int j = 0; j * kSkWaves < kTiles; ++j) {
            const int p = wave + kSkWaves * j;
            if (p < kTiles) sk_write_tile(tk, row0 + 16 * (p / MT), p % MT, lane, fin[j], res[j]);
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
    if (tid == 0) s_prev = __hip_atomic_fetch_add(&tk.cnt[(size_t)blk * kCtrWords], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
        sk_write_tile(tk, row0 + 16 * (p / MT), p % MT, lane, sum, res[j]);
    }
    if (tid == 0) __hip_atomic_store(&tk.cnt[(size_t)blk * kCtrWords], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
        cnt += blocks * kCtrStride;
    }
    if (part == 0) return 0;
    if (cnt > kWsCounterBytes) return (size_t)-1;
    return kWsCounterBytes + part;
}

// weight bytes per row and group of 128 columns (int4 counts its codes only)
int sk_group_bytes(int fmt) { return fmt == kFmtBf16 ? 256 : fmt == kFmtNvfp4 ? 72 : 64; }
// most groups per slice: BF16 rounds are one group per wave
int sk_max_groups(int fmt) { return fmt == kFmtBf16 ? kSkMaxGroups / 2 : kSkMaxGroups; }

bool sk_plan(const Fmt* fmts, const GemvArgs* tasks, int count, bool can_split, SkPlan& best) {
    const int MT = sk_mt(tasks[0].M);
    double best_cost = 0;
    bool found = false;
    for (int R : kSkR) {
        for (int S : {16, 8}) {
            if (S == 8 && !can_split) continue;
            SkPlan p;
            p.R = R;
            long wgs = 0;
            double per_wg = 0;
            bool ok = true, split = false;
            for (int i = 0; i < count; ++i) {
                const int G = tasks[i].K >> 7, cap = sk_max_groups(fmts[i]);
                const int S1 = S < cap ? S : cap;
                int gs = G <= S1 ? G : S1;
                if (G > cap && !can_split) { ok = false; break; }
                const int ks = (G + gs - 1) / gs;
                p.gs[i] = gs;
                p.ks[i] = ks;
                split = split || ks > 1;
                const double c = 16.0 * R * gs * sk_group_bytes(fmts[i]) + 0.19 * gs * MT * 4096;
                per_wg = c > per_wg ? c : per_wg;
                wgs += (long)((tasks[i].N + 16 * R - 1) / (16 * R)) * ks;
            }
            if (!ok) continue;
            p.ws = split ? sk_ws_bytes(tasks, count, R, p.ks) : 0;
            if (p.ws == (size_t)-1) continue;
            per_wg += split ? 35000.0 : 0.0;
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

template <int MT, int R, int FM>
hipError_t launch_sk_fm(const SkTable& tt, int grid, hipStream_t st) {
    constexpr int kShmem = SkLds<MT, R, FM>::kBytes;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(skinny_q4_kernel<MT, R, FM>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kShmem);
    if (attr != hipSuccess) return attr;
    return launch_kernel(skinny_q4_kernel<MT, R, FM>, dim3(grid), dim3(kSkThreads), (size_t)kShmem, st, tt);
}

template <int MT, int R>
hipError_t launch_sk_mt(const Fmt* fmts, const GemvArgs* tasks, int count, const SkPlan& p, void* ws, hipStream_t st) {
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
        t.fmt = fmts[i];
        t.ks = p.ks[i];
        t.gs = p.gs[i];
        if (p.ks[i] > 1) {
            t.cnt = reinterpret_cast<unsigned*>(pc);
            pc += (size_t)blocks * kCtrStride;
            t.part = reinterpret_cast<float*>(pp);
            pp += (size_t)blocks * p.ks[i] * R * MT * 1024;
        }
        grid += blocks * p.ks[i];
    }
    int fm = 0;
    for (int i = 0; i < count; ++i) fm |= 1 << fmts[i];
    if (fm == 1) return launch_sk_fm<MT, R, 1>(tt, grid, st);
    if (!(fm & 1)) return launch_sk_fm<MT, R, 6>(tt, grid, st);
    return launch_sk_fm<MT, R, 7>(tt, grid, st);
}

template <int MT>
hipError_t launch_sk_r(const Fmt* fmts, const GemvArgs* tasks, int count, const SkPlan& p, void* ws, hipStream_t st) {
    switch (p.R) {
        case 5: return launch_sk_mt<MT, 5>(fmts, tasks, count, p, ws, st);
        case 3: return launch_sk_mt<MT, 3>(fmts, tasks, count, p, ws, st);
        case 2: return launch_sk_mt<MT, 2>(fmts, tasks, count, p, ws, st);
        default: return launch_sk_mt<MT, 1>(fmts, tasks, count, p, ws, st);
    }
}

}  // namespace

bool skinny_supported(Fmt fmt, int M, int K, bool split) {
    if (M < 5 || M > kSkinnyMaxM || K % 128 != 0) return false;
    return split || (K >> 7) <= sk_max_groups(fmt);
}

size_t skinny_workspace_bytes(const Fmt* fmts, const GemvArgs* tasks, int count) {
    SkPlan p;
    if (!sk_plan(fmts, tasks, count, true, p)) return 0;
    return p.ws;
}

hipError_t launch_skinny(const Fmt* fmts, const GemvArgs* tasks, int count, void* ws, size_t ws_bytes, hipStream_t s) {
    SkPlan p;
    const size_t need = skinny_workspace_bytes(fmts, tasks, count);
    const bool split = ws != nullptr && need > 0 && ws_bytes >= need;
    if (!sk_plan(fmts, tasks, count, split, p)) return hipErrorInvalidValue;
    switch (sk_mt(tasks[0].M)) {
        case 1: return launch_sk_r<1>(fmts, tasks, count, p, ws, s);
        case 2: return launch_sk_r<2>(fmts, tasks, count, p, ws, s);
        default: return launch_sk_r<3>(fmts, tasks, count, p, ws, s);
    }
}

// int4 tasks only
namespace {
struct AllQ4 {
    Fmt f[kMaxTasks];
    AllQ4() {
        for (Fmt& x : f) x = kFmtQ4;
    }
};
}  // namespace

bool skinny_supported(int M, int K, bool split) { return skinny_supported(kFmtQ4, M, K, split); }
size_t skinny_workspace_bytes(const GemvArgs* tasks, int count) { return skinny_workspace_bytes(AllQ4().f, tasks, count); }
hipError_t launch_skinny(const GemvArgs* tasks, int count, void* ws, size_t ws_bytes, hipStream_t s) {
    return launch_skinny(AllQ4().f, tasks, count, ws, ws_bytes, s);
}

}  // namespace q4
