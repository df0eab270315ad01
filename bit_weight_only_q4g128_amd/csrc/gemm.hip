// Prefill GEMM for int4 g128 weights (gfx950, v_mfma_f32_16x16x32_bf16):
// y[m, n] = RN_bf16(sum_k x[m, k] * w[n, k]) for many batch rows m, with
// w[n, k] = code[n, k] * scale[n, k / 128] + min[n, k / 128] (rumik-oss-1-int4
// card, "Format"; the int4 prefill matmul of its "Running it" section and of
// the Rumik TTS Fast Inference post, "What Made It Faster").
//
// A workgroup (eight waves) owns a tile of 128 batch rows x BN = 64 * NT
// weight rows and walks all of K one 128-column group at a time.  Each wave
// computes 64 batch rows x 16 * NT weight rows.  Per group every thread loads
// its share of the next group into registers while the waves compute the
// current one from LDS, then writes it to the other LDS buffer; one barrier
// per group.
//
//   * activations: 128 rows x 128 columns of BF16, each 8-column chunk stored
//     in the pair order (x0,x4)(x1,x5)(x2,x6)(x3,x7) that matches the nibble
//     unpacking of the weights; 16-byte chunk c of row r sits at chunk
//     c ^ (r % 16) of its 256-byte row, so the 16 rows of one fragment read,
//     and the 16 chunks of one row that 16 consecutive lanes stage, fall in
//     16 distinct 16-byte bank slots;
//   * weight codes stay packed in LDS (BN rows x 64 bytes, as four planes of
//     16 bytes per row, one per 32-column k-step): each wave turns its lane's
//     dword of 8 codes into the BF16 values 128 + code (exact) right before
//     its MFMAs, so LDS holds and serves a quarter of the bytes of a
//     dequantized tile;
//   * the fp32 scale s and m' = min - 128 * s of every weight row, and
//     SX = sum of the group's activations of every batch row (fp32, summed by
//     the threads that stage them).
//
// The MFMAs give D = sum over the group of (128 + code) * x per output (the
// group's first k-step starts from zero), and the wave folds y += s * D; every
// fourth group (and after the last) one fp32 MFMA per tile adds the term
// sum over those groups of m' * SX (a 16 x 4 by 4 x 16 product: m' and SX
// of the last groups stay in an eight-slot LDS ring).  The result is
// sum (code * s + min) * x up to fp32 rounding (every product in D is exact).
//
// MFMA operand layout (16x16x32): lane l holds A row l % 16 (a weight row) and
// B column l % 16 (a batch row), for k-step h the 8 columns 32 h + 8 (l / 16)
// .. + 8 of the group; D: lane l holds weight rows 4 (l / 16) + v, v = 0..3,
// of batch row l % 16.
//
// Workgroups are dealt to the eight XCDs in turn; the tile order gives each
// XCD a contiguous range of tiles, walked in super-rows of 8 batch blocks so
// the workgroups resident together share weight and activation blocks in
// their L2.
#include "internal.h"

namespace q4 {

namespace {

constexpr int kThreads = 512;
constexpr int kBM = 128;                 // batch rows per workgroup
constexpr int kXPitch = 256;             // LDS bytes per activation row (128 BF16, chunks swizzled)
constexpr int kSuper = 8;                // batch blocks per super-row of the tile order
constexpr uint32_t kOnes = 0x3F803F80u;  // BF16 pair (1, 1)

typedef __bf16 bf16x8_g __attribute__((ext_vector_type(8)));

__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

// sum of the 8 BF16 values of a chunk, added to acc (fp32)
__device__ __forceinline__ float sum8(const u32x4& v, float acc) {
    return dot2(v.w, kOnes, dot2(v.z, kOnes, dot2(v.y, kOnes, dot2(v.x, kOnes, acc))));
}

// LDS layout: two group buffers, then the rings of m' and SX
constexpr int kRing = 8;
template <int NT>
struct GemmLayout {
    static constexpr int kBN = 64 * NT;
    static constexpr int kX = 0;                                // [kBM][kXPitch]
    static constexpr int kCodes = kX + kBM * kXPitch;            // [4 planes][kBN][16]
    static constexpr int kS = kCodes + kBN * 64;                // float [kBN]
    static constexpr int kBuf = kS + kBN * 4;
    static constexpr int kRingM = 2 * kBuf;                     // float [kRing][kBN]
    static constexpr int kRingSX = kRingM + kRing * kBN * 4;    // float [kRing][kBM]
    static constexpr int kBytes = kRingSX + kRing * kBM * 4;
};

template <int NT>
__global__ __launch_bounds__(kThreads) void gemm_q4_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ qw,
                                                            const uint16_t* __restrict__ scale, const uint16_t* __restrict__ minv,
                                                            uint16_t* __restrict__ y, int M, int N, int K, int nM, int nN) {
    constexpr int BN = 64 * NT;
    using Lay = GemmLayout<NT>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    // tile order: XCD-contiguous ranges, super-rows of kSuper batch blocks
    const int T = nM * nN;
    const int b = blockIdx.x, xcd = b & 7, q8 = T >> 3, r8 = T & 7;
    const int tile = xcd * q8 + (xcd < r8 ? xcd : r8) + (b >> 3);
    const int per_super = kSuper * nN;
    const int sup = tile / per_super, within = tile - sup * per_super;
    const int rows_here = (nM - sup * kSuper) < kSuper ? (nM - sup * kSuper) : kSuper;
    const int mb = sup * kSuper + within % rows_here, nb = within / rows_here;
    const int m0 = mb * kBM, n0 = nb * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1, lq = lane >> 4, lr = lane & 15;
    const int G = K >> 7;
    const int rows_m = (M - m0) < kBM ? (M - m0) : kBM;
    const int rows_n = (N - n0) < BN ? (N - n0) : BN;

    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (size_t)m0 * K, (uint32_t)rows_m * (uint32_t)K * 2u);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(qw + (size_t)n0 * (K >> 1), (uint32_t)rows_n * (uint32_t)(K >> 1));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(scale + (size_t)n0 * G, (uint32_t)rows_n * (uint32_t)G * 2u);
    const __amdgpu_buffer_rsrc_t rn = make_rsrc(minv + (size_t)n0 * G, (uint32_t)rows_n * (uint32_t)G * 2u);

    // loader roles per group: activation chunk xc of rows xr + 32 i (i < 4);
    // code chunks (planes) cp and cp + 2 of row cr for tid < 2 BN; the
    // scale/min pair of row tid for tid < BN
    const int xr = tid >> 4, xc = tid & 15;
    const uint32_t vx = (uint32_t)xr * (uint32_t)K * 2u + (uint32_t)xc * 16u;
    const uint32_t vx32 = 32u * (uint32_t)K * 2u;
    const int cr = tid >> 1, cp = tid & 1;
    const bool has_code = tid < 2 * BN, has_scale = tid < BN;
    const uint32_t vc = (uint32_t)cr * (uint32_t)(K >> 1) + (uint32_t)cp * 16u;
    const uint32_t vs = (uint32_t)tid * (uint32_t)G * 2u;

    u32x4 px[4], pc[2];
    pc[0] = pc[1] = u32x4{0, 0, 0, 0};
    uint16_t ps = 0, pm = 0;

    auto load = [&](int g) {
        const uint32_t sx0 = (uint32_t)g * 256u;
#pragma unroll
        for (int i = 0; i < 4; ++i) px[i] = ld16(rx, vx + (uint32_t)i * vx32, sx0);
        if (has_code) {
            pc[0] = ld16(rc, vc, (uint32_t)g * 64u);
            pc[1] = ld16(rc, vc, (uint32_t)g * 64u + 32u);
        }
        if (has_scale) {
            ps = buf_load2(rs, vs, (uint32_t)g * 2u);
            pm = buf_load2(rn, vs, (uint32_t)g * 2u);
        }
    };
    auto store = [&](int g) {
        uint8_t* B = lds + (g & 1) * Lay::kBuf;
        float* ringM = reinterpret_cast<float*>(lds + Lay::kRingM) + (g & (kRing - 1)) * BN;
        float* ringSX = reinterpret_cast<float*>(lds + Lay::kRingSX) + (g & (kRing - 1)) * kBM;
        uint32_t p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xq4_pairs(px[i].x, px[i].y, px[i].z, px[i].w, p);
            const int row = xr + 32 * i;
            *reinterpret_cast<u32x4*>(B + Lay::kX + row * kXPitch + ((xc ^ (row & 15)) << 4)) = u32x4{p[0], p[1], p[2], p[3]};
        }
        if (has_code) {
            *reinterpret_cast<u32x4*>(B + Lay::kCodes + cp * BN * 16 + cr * 16) = pc[0];
            *reinterpret_cast<u32x4*>(B + Lay::kCodes + (cp + 2) * BN * 16 + cr * 16) = pc[1];
        }
        if (has_scale) {
            const float s = f16_to_f32(ps);
            reinterpret_cast<float*>(B + Lay::kS)[tid] = s;
            ringM[tid] = __builtin_fmaf(-128.0f, s, f16_to_f32(pm));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float gs = group_sum(sum8(px[i], 0.f), 16);
            if (xc == 15) ringSX[xr + 32 * i] = gs;
        }
    };

    f32x4 D[NT][4], Y[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u) Y[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};

    load(0);
    store(0);
    __syncthreads();

    // row 64 wm + 16 u + lr (row % 16 == lr), chunk 4 h + lq, swizzled
    const int xrow = (64 * wm + lr) * kXPitch;
    int xoff[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) xoff[h] = xrow + (((4 * h + lq) ^ lr) << 4);
    const int crow = (16 * NT * wn + lr) * 16 + 4 * lq;
    for (int g = 0; g < G; ++g) {
        const bool more = g + 1 < G;
        if (more) load(g + 1);
        const uint8_t* B = lds + (g & 1) * Lay::kBuf;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            bf16x8_g a[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint32_t cw = *reinterpret_cast<const uint32_t*>(B + Lay::kCodes + h * BN * 16 + crow + 256 * t);
                uint32_t p[4];
                q4_pairs(cw, p);
                a[t] = __builtin_bit_cast(bf16x8_g, u32x4{p[0], p[1], p[2], p[3]});
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bf16x8_g xf = *reinterpret_cast<const bf16x8_g*>(B + Lay::kX + xoff[h] + 16 * u * kXPitch);
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    D[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t], xf, h == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : D[t][u], 0, 0, 0);
            }
        }
        {
            const float* S = reinterpret_cast<const float*>(B + Lay::kS);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const f32x4 s4 = *reinterpret_cast<const f32x4*>(S + 16 * NT * wn + 16 * t + 4 * lq);
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int v = 0; v < 4; ++v) Y[t][u][v] = __builtin_fmaf(s4[v], D[t][u][v], Y[t][u][v]);
            }
        }
        if ((g & 3) == 3 || !more) {
            // y += m' . SX over groups g0 .. g: lane l holds m' of weight row
            // l % 16 and SX of batch row l % 16 for group g0 + l / 16
            const int g0 = g & ~3, gl = g0 + lq;
            const bool live = gl <= g;
            const float* ringM = reinterpret_cast<const float*>(lds + Lay::kRingM) + (gl & (kRing - 1)) * BN;
            const float* ringSX = reinterpret_cast<const float*>(lds + Lay::kRingSX) + (gl & (kRing - 1)) * kBM;
            float am[NT], bs[4];
#pragma unroll
            for (int t = 0; t < NT; ++t) am[t] = live ? ringM[16 * NT * wn + 16 * t + lr] : 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u) bs[u] = live ? ringSX[64 * wm + 16 * u + lr] : 0.f;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int u = 0; u < 4; ++u) Y[t][u] = __builtin_amdgcn_mfma_f32_16x16x4f32(am[t], bs[u], Y[t][u], 0, 0, 0);
        }
        if (more) store(g + 1);
        __syncthreads();
    }

    // y: lane holds weight rows n .. n + 3 of batch row m for each (t, u)
    // 8-byte stores only where every row start is 8-byte aligned (y itself
    // need only be 2-byte aligned)
    const bool vec = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int m = m0 + 64 * wm + 16 * u + lr;
        if (m >= M) continue;
        uint16_t* yrow = y + (size_t)m * N;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int n = n0 + 16 * NT * wn + 16 * t + 4 * lq;
            const uint32_t lo = (uint32_t)f32_to_bf16(Y[t][u][0]) | ((uint32_t)f32_to_bf16(Y[t][u][1]) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16(Y[t][u][2]) | ((uint32_t)f32_to_bf16(Y[t][u][3]) << 16);
            if (vec && n + 3 < N) {
                *reinterpret_cast<uint2*>(yrow + n) = make_uint2(lo, hi);
            } else {
                if (n < N) yrow[n] = (uint16_t)lo;
                if (n + 1 < N) yrow[n + 1] = (uint16_t)(lo >> 16);
                if (n + 2 < N) yrow[n + 2] = (uint16_t)hi;
                if (n + 3 < N) yrow[n + 3] = (uint16_t)(hi >> 16);
            }
        }
    }
}

template <int NT>
hipError_t launch_gemm_nt(const GemvArgs& a, hipStream_t s) {
    const int nM = (a.M + kBM - 1) / kBM, nN = (a.N + 64 * NT - 1) / (64 * NT);
    constexpr int kShmem = GemmLayout<NT>::kBytes;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_q4_kernel<NT>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kShmem);
    if (attr != hipSuccess) return attr;
    return launch_kernel(gemm_q4_kernel<NT>, dim3(nM * nN), dim3(kThreads), (size_t)kShmem, s, a.x, a.w, a.scale, a.minv, a.y,
                         a.M, a.N, a.K, nM, nN);
}

}  // namespace

long gemm_tiles(int M, int N, int nt) { return (long)((M + kBM - 1) / kBM) * ((N + 64 * nt - 1) / (64 * nt)); }

int gemm_tile_nt(int M, int N) { return gemm_tiles(M, N, 4) >= 256 ? 4 : 2; }

hipError_t launch_gemm(const GemvArgs& a, int nt, hipStream_t s) {
    return nt == 4 ? launch_gemm_nt<4>(a, s) : launch_gemm_nt<2>(a, s);
}

}  // namespace q4
