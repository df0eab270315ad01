// Matrix-core GEMV for batched decode (gfx950, v_mfma_f32_16x16x32_bf16).
//
// Weights are the A operand (16 rows x 32 columns per instruction), the batch
// is the B operand (32 columns x 16 batch rows), so one instruction covers 16
// output features for 16 sequences.  Each lane dequantizes its own 8 columns of
// A in registers; only group scales go through LDS.  Lane l holds A row
// (l % 16) and column block (l / 16); B uses the same column blocks, so any
// fixed order of the 8 columns inside a block is valid as long as A and B
// agree.
//
// A workgroup (4 waves) owns RT row tiles of 16 rows.  The K dimension is cut
// into 128-column steps and each wave walks a contiguous quarter of them,
// keeping the weights and activations of the next step in flight while it
// computes the current one.  The four partial tiles meet in LDS and are summed
// in a fixed order, so results do not depend on timing.
#include "internal.h"

namespace q4 {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4 mfma(bf16x8_t a, bf16x8_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

constexpr f32x4 kZero4 = {0.f, 0.f, 0.f, 0.f};
constexpr u32x4 kZeroU4 = {0u, 0u, 0u, 0u};

// Raw activations of one 128-column step: x[m][k0 + 32*kb + 8*d .. +8] for
// the lane's batch row m = 16*mt + (lane % 16); zero for padding rows and
// columns past K.
template <int MTILES>
__device__ __forceinline__ void load_xraw(const GemvArgs& a, int col, int kb, int k0, u32x4 (&xr)[MTILES][4]) {
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt) {
        const int m = 16 * mt + col;
        const bool ok = m < a.M;
        const u32x4* src = reinterpret_cast<const u32x4*>(a.x + (size_t)(ok ? m : 0) * a.K + k0 + 32 * kb);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const bool okd = ok && (k0 + 32 * kb + 8 * d) < a.K;
            xr[mt][d] = okd ? src[d] : kZeroU4;
        }
    }
}

// Sum the four waves' partial tiles (fixed order) and store bf16 y = acc*mul.
// `red` must hold 3 * RT * MTILES * 256 floats.
template <int MTILES, int RT>
__device__ __forceinline__ void reduce_store(const GemvArgs& a, float* red, int row0, int lane, int wave, f32x4 (&acc)[RT][MTILES],
                                             float mul) {
    const int col = lane & 15, kb = lane >> 4;
    if (wave > 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    red[(((wave - 1) * RT + rt) * MTILES + mt) * 256 + v * 64 + lane] = acc[rt][mt][v];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt) {
            const int m = 16 * mt + col;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float s = acc[rt][mt][v];
#pragma unroll
                for (int w = 0; w < 3; ++w) s += red[((w * RT + rt) * MTILES + mt) * 256 + v * 64 + lane];
                const int row = row0 + 16 * rt + 4 * kb + v;
                if (m < a.M && row < a.N) a.y[(size_t)m * a.N + row] = f32_to_bf16(s * mul);
            }
        }
}

__device__ __forceinline__ void step_range(int steps, int wave, int& s0, int& s1) {
    const int per = (steps + 3) >> 2;
    s0 = wave * per;
    if (s0 > steps) s0 = steps;
    s1 = s0 + per < steps ? s0 + per : steps;
}

// ---------------------------------------------------------------------------
// int4 g128 min/max.  A holds 128 + code (exact in BF16); per 128-column group
//   D = sum (128 + c) x,  SX = sum x   (SX from an all-ones A operand)
//   y += s * (D - 128 SX) + min * SX
// Scale and min of the workgroup's rows are staged once into LDS as
// [group][row] dwords (scale | min << 16).
// ---------------------------------------------------------------------------
template <int MTILES, int RT>
__global__ __launch_bounds__(256) void q4_mfma_kernel(GemvArgs a) {
    extern __shared__ uint32_t lds_u32[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, kb = lane >> 4;
    const int G = a.K >> 7;
    const int row0 = blockIdx.x * RT * 16;
    uint32_t* sm = lds_u32;                                         // [G][16*RT]
    float* red = reinterpret_cast<float*>(lds_u32 + (size_t)G * 16 * RT);

    int g0, g1;
    step_range(G, wave, g0, g1);
    const size_t rowbytes = (size_t)a.K >> 1;
    const uint8_t* wrow[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        int r = row0 + 16 * rt + col;
        r = r < a.N ? r : a.N - 1;
        wrow[rt] = a.w + (size_t)r * rowbytes + 16 * kb;
    }

    // first step's operands go out before the scale staging
    u32x4 qn[RT];
    u32x4 xn[MTILES][4];
    if (g0 < g1) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) qn[rt] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[rt] + 64 * g0));
        load_xraw<MTILES>(a, col, kb, 128 * g0, xn);
    }

    const int nrows = a.N - row0;
    for (int i = threadIdx.x; i < 16 * RT * G; i += 256) {
        const int r = i / G, g = i - r * G;
        uint32_t v = 0;
        if (r < nrows) {
            const size_t gi = (size_t)(row0 + r) * G + g;
            v = (uint32_t)a.scale[gi] | ((uint32_t)a.minv[gi] << 16);
        }
        sm[g * 16 * RT + r] = v;
    }
    __syncthreads();

    const bf16x8_t ones = as_bf16x8(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
    f32x4 acc[RT][MTILES];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt) acc[rt][mt] = kZero4;

    for (int g = g0; g < g1; ++g) {
        u32x4 q[RT];
        bf16x8_t B[MTILES][4];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) q[rt] = qn[rt];
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t p[4];
                xq4_pairs(xn[mt][d].x, xn[mt][d].y, xn[mt][d].z, xn[mt][d].w, p);
                B[mt][d] = as_bf16x8(p[0], p[1], p[2], p[3]);
            }
        if (g + 1 < g1) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) qn[rt] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[rt] + 64 * (g + 1)));
            load_xraw<MTILES>(a, col, kb, 128 * (g + 1), xn);
        }
        f32x4 SX[MTILES];
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt) {
            SX[mt] = kZero4;
#pragma unroll
            for (int d = 0; d < 4; ++d) SX[mt] = mfma(ones, B[mt][d], SX[mt]);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            f32x4 D[MTILES];
#pragma unroll
            for (int mt = 0; mt < MTILES; ++mt) D[mt] = kZero4;
            const uint32_t qd[4] = {q[rt].x, q[rt].y, q[rt].z, q[rt].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t p[4];
                q4_pairs(qd[d], p);
                const bf16x8_t A = as_bf16x8(p[0], p[1], p[2], p[3]);
#pragma unroll
                for (int mt = 0; mt < MTILES; ++mt) D[mt] = mfma(A, B[mt][d], D[mt]);
            }
            const u32x4 smv = *reinterpret_cast<const u32x4*>(sm + g * 16 * RT + 16 * rt + 4 * kb);
            const uint32_t smw[4] = {smv.x, smv.y, smv.z, smv.w};
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float s = f16_to_f32((uint16_t)(smw[v] & 0xFFFFu));
                const float mn = f16_to_f32((uint16_t)(smw[v] >> 16));
#pragma unroll
                for (int mt = 0; mt < MTILES; ++mt) {
                    const float sx = SX[mt][v];
                    const float t = fmaf(-128.f, sx, D[mt][v]);
                    const float r = fmaf(s, t, acc[rt][mt][v]);
                    acc[rt][mt][v] = fmaf(mn, sx, r);
                }
            }
        }
    }
    reduce_store<MTILES, RT>(a, red, row0, lane, wave, acc, 1.0f);
}

// ---------------------------------------------------------------------------
// NVFP4.  A holds e2m1(code) * e4m3(scale) rounded to BF16 -- exact, since the
// product has at most 6 significant bits and lies in [2^-10, 2688] -- so the
// group scale is inside the operand; G multiplies the finished sum.  (The
// hardware's scaled FP4 conversions apply only the exponent of their scale
// operand, so the e4m3 factor is a separate fp32 multiply.)
// ---------------------------------------------------------------------------

template <int MTILES, int RT>
__global__ __launch_bounds__(256) void nvfp4_mfma_kernel(GemvArgs a) {
    extern __shared__ uint32_t lds_u32[];
    float* red = reinterpret_cast<float*>(lds_u32);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, kb = lane >> 4;
    const int row0 = blockIdx.x * RT * 16;
    const size_t rowbytes = (size_t)a.K >> 1;
    const size_t srow = (size_t)a.K >> 4;
    const int steps = (a.K + 127) >> 7;
    int g0, g1;
    step_range(steps, wave, g0, g1);

    const uint8_t* wrow[RT];
    const uint8_t* srowp[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        int r = row0 + 16 * rt + col;
        r = r < a.N ? r : a.N - 1;
        wrow[rt] = a.w + (size_t)r * rowbytes + 16 * kb;
        srowp[rt] = a.scale8 + (size_t)r * srow + 2 * kb;
    }
    auto load_step = [&](int g, u32x4 (&q)[RT], uint32_t (&sb)[RT], u32x4 (&xr)[MTILES][4]) {
        const bool kin = (128 * g + 32 * kb) < a.K;   // the lane's 32 columns
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            q[rt] = kin ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[rt] + 64 * g)) : kZeroU4;
            sb[rt] = kin ? ((uint32_t)srowp[rt][8 * g] | ((uint32_t)srowp[rt][8 * g + 1] << 8)) : 0u;
        }
        load_xraw<MTILES>(a, col, kb, 128 * g, xr);
    };

    f32x4 acc[RT][MTILES];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt) acc[rt][mt] = kZero4;

    u32x4 qn[RT];
    uint32_t sbn[RT];
    u32x4 xn[MTILES][4];
    if (g0 < g1) load_step(g0, qn, sbn, xn);
    for (int g = g0; g < g1; ++g) {
        u32x4 q[RT];
        uint32_t sb[RT];
        bf16x8_t B[MTILES][4];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) { q[rt] = qn[rt]; sb[rt] = sbn[rt]; }
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
            for (int d = 0; d < 4; ++d) B[mt][d] = as_bf16x8(xn[mt][d]);
        if (g + 1 < g1) load_step(g + 1, qn, sbn, xn);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const float s0 = e4m3_to_f32<0>(sb[rt]), s1 = e4m3_to_f32<1>(sb[rt]);
            const uint32_t qd[4] = {q[rt].x, q[rt].y, q[rt].z, q[rt].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const float s = d < 2 ? s0 : s1;
                const bf16x8_t A = as_bf16x8(nv_pair_scaled<0>(qd[d], s), nv_pair_scaled<1>(qd[d], s),
                                             nv_pair_scaled<2>(qd[d], s), nv_pair_scaled<3>(qd[d], s));
#pragma unroll
                for (int mt = 0; mt < MTILES; ++mt) acc[rt][mt] = mfma(A, B[mt][d], acc[rt][mt]);
            }
        }
    }
    reduce_store<MTILES, RT>(a, red, row0, lane, wave, acc, a.gscale);
}

// ---------------------------------------------------------------------------
// BF16 weights: A is read straight from memory.
// ---------------------------------------------------------------------------
template <int MTILES, int RT>
__global__ __launch_bounds__(256) void bf16_mfma_kernel(GemvArgs a) {
    extern __shared__ uint32_t lds_u32[];
    float* red = reinterpret_cast<float*>(lds_u32);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, kb = lane >> 4;
    const int row0 = blockIdx.x * RT * 16;
    const int steps = (a.K + 127) >> 7;
    int g0, g1;
    step_range(steps, wave, g0, g1);
    const uint16_t* wrow[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        int r = row0 + 16 * rt + col;
        r = r < a.N ? r : a.N - 1;
        wrow[rt] = reinterpret_cast<const uint16_t*>(a.w) + (size_t)r * a.K + 32 * kb;
    }
    auto load_step = [&](int g, u32x4 (&w)[RT][4], u32x4 (&xr)[MTILES][4]) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const bool okd = (128 * g + 32 * kb + 8 * d) < a.K;
                w[rt][d] = okd ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[rt] + 128 * g + 8 * d)) : kZeroU4;
            }
        load_xraw<MTILES>(a, col, kb, 128 * g, xr);
    };
    f32x4 acc[RT][MTILES];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt) acc[rt][mt] = kZero4;

    u32x4 wn[RT][4];
    u32x4 xn[MTILES][4];
    if (g0 < g1) load_step(g0, wn, xn);
    for (int g = g0; g < g1; ++g) {
        u32x4 w[RT][4];
        bf16x8_t B[MTILES][4];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int d = 0; d < 4; ++d) w[rt][d] = wn[rt][d];
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
            for (int d = 0; d < 4; ++d) B[mt][d] = as_bf16x8(xn[mt][d]);
        if (g + 1 < g1) load_step(g + 1, wn, xn);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const bf16x8_t A = as_bf16x8(w[rt][d]);
#pragma unroll
                for (int mt = 0; mt < MTILES; ++mt) acc[rt][mt] = mfma(A, B[mt][d], acc[rt][mt]);
            }
    }
    reduce_store<MTILES, RT>(a, red, row0, lane, wave, acc, 1.0f);
}

template <int MTILES, int RT>
hipError_t launch_one(Fmt fmt, const GemvArgs& a, hipStream_t st) {
    const int grid = (a.N + 16 * RT - 1) / (16 * RT);
    const size_t red_bytes = (size_t)3 * RT * MTILES * 256 * sizeof(float);
    switch (fmt) {
        case kFmtQ4: {
            const size_t shmem = (size_t)(a.K >> 7) * 16 * RT * sizeof(uint32_t) + red_bytes;
            return launch_kernel(q4_mfma_kernel<MTILES, RT>, dim3(grid), dim3(256), shmem, st, a);
        }
        case kFmtNvfp4:
            return launch_kernel(nvfp4_mfma_kernel<MTILES, RT>, dim3(grid), dim3(256), red_bytes, st, a);
        default:
            return launch_kernel(bf16_mfma_kernel<MTILES, RT>, dim3(grid), dim3(256), red_bytes, st, a);
    }
}

// Two row tiles per workgroup once that still leaves >= 256 workgroups (and
// the int4 scale staging fits the 64 KB LDS budget).
template <int MTILES>
hipError_t launch_rt(Fmt fmt, const GemvArgs& a, hipStream_t st) {
    const int tiles = (a.N + 15) / 16;
    const size_t lds_rt2 = (size_t)(a.K >> 7) * 16 * 2 * sizeof(uint32_t) + (size_t)3 * 2 * MTILES * 256 * sizeof(float);
    if (tiles >= 512 && (fmt != kFmtQ4 || lds_rt2 <= 65536)) return launch_one<MTILES, 2>(fmt, a, st);
    return launch_one<MTILES, 1>(fmt, a, st);
}

}  // namespace

hipError_t launch_mfma(Fmt fmt, const GemvArgs* tasks, int count, hipStream_t st) {
    for (int i = 0; i < count; ++i) {
        const GemvArgs& a = tasks[i];
        const int mtiles = (a.M + 15) / 16;
        hipError_t e;
        switch (mtiles) {
            case 1: e = launch_rt<1>(fmt, a, st); break;
            case 2: e = launch_rt<2>(fmt, a, st); break;
            case 3: e = launch_rt<3>(fmt, a, st); break;
            default: e = launch_rt<4>(fmt, a, st); break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q4
