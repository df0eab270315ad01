// Weight-format policies for the packed-dot GEMV kernel.
//
// A "chunk" is the 16 bytes of weight data one lane loads with one 128-bit
// load.  For the 4-bit formats that is 32 consecutive weights of one row; for
// BF16 it is 8.  Each policy says how to hold the matching activations in
// registers, how to fetch the per-chunk group parameters, and how to turn a
// chunk into a partial dot product for every batch row.
#pragma once

#include "common.h"

namespace q4 {

struct GemvArgs {
    const uint16_t* x;       // [M, K] bf16
    const uint8_t* w;        // packed weights, row-major
    const uint16_t* scale;   // int4: fp16 [N, K/128]
    const uint16_t* minv;    // int4: fp16 [N, K/128]
    const uint8_t* scale8;   // nvfp4: e4m3 [N, K/16]
    float gscale;            // nvfp4: per-matrix global scale (multiplier)
    uint16_t* y;             // [M, N] bf16
    int M, N, K;
};

// ---------------------------------------------------------------------------
// int4 g128 min/max (rumik-oss-1-int4 card, "Format")
//
//   w[n,k] = code * scale[n, k/128] + min[n, k/128]
//
// A chunk (32 weights) lies inside one 128-column group, so per chunk
//   sum_k w*x = scale * sum_k code*x + min * sum_k x.
// The packed dot products produce sum (128+code)*x; subtracting 128*sum x
// recovers sum code*x.
// ---------------------------------------------------------------------------
struct FmtQ4 {
    static constexpr int WPC = 32;       // weights per chunk
    static constexpr int XW = 16;        // activation dwords per chunk
    struct X { uint32_t p[16]; float sum; };
    struct Aux { float s, m; };

    __device__ static void load_x(const uint16_t* xrow, int k0, bool active, X& xc) {
        if (!active) {
#pragma unroll
            for (int i = 0; i < 16; ++i) xc.p[i] = 0;
            xc.sum = 0.f;
            return;
        }
        const u32x4* src = reinterpret_cast<const u32x4*>(xrow + k0);
        float s = 0.f;
        // 32 activations = 16 dwords; block d (8 activations) = dwords 4d..4d+3.
        uint32_t w[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4 v = src[i];
            w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            xq4_pairs(w[4 * d], w[4 * d + 1], w[4 * d + 2], w[4 * d + 3], &xc.p[4 * d]);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) s += bf16lo(w[i]) + bf16hi(w[i]);
        xc.sum = s;
    }

    __device__ static Aux load_aux(const GemvArgs& a, int row, int chunk) {
        const size_t gi = (size_t)row * (a.K >> 7) + (chunk >> 2);
        Aux r;
        r.s = f16_to_f32(a.scale[gi]);
        r.m = f16_to_f32(a.minv[gi]);
        return r;
    }

    template <int MT>
    __device__ static void accumulate(u32x4 q, const Aux& ax, const X (&xc)[MT], float (&out)[MT]) {
        float acc[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = 0.f;
        const uint32_t qd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t p[4];
            q4_pairs(qd[d], p);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[m] = dot2(p[j], xc[m].p[4 * d + j], acc[m]);
            }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float t = fmaf(-128.f, xc[m].sum, acc[m]);   // sum code*x
            out[m] += fmaf(ax.s, t, ax.m * xc[m].sum);
        }
    }
    __device__ static float finish(const GemvArgs&, float v) { return v; }
};

// ---------------------------------------------------------------------------
// NVFP4 weight-only (VoxCPM2-NVFP4 card, "What was quantized")
//
//   w[n,k] = e2m1(code) * e4m3(scale[n, k/16]) * G
//
// A chunk (32 weights) covers two 16-groups.  Per group the E2M1 values are
// exact in BF16, so sum e2m1*x comes from packed dot products; the e4m3 group
// scale multiplies that sum and G multiplies the finished row sum.
// ---------------------------------------------------------------------------
struct FmtNvfp4 {
    static constexpr int WPC = 32;
    static constexpr int XW = 16;
    struct X { uint32_t p[16]; };
    struct Aux { float s0, s1; };

    __device__ static void load_x(const uint16_t* xrow, int k0, bool active, X& xc) {
        const u32x4* src = reinterpret_cast<const u32x4*>(xrow + k0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4 v = active ? src[i] : u32x4{0, 0, 0, 0};
            xc.p[4 * i + 0] = v.x; xc.p[4 * i + 1] = v.y; xc.p[4 * i + 2] = v.z; xc.p[4 * i + 3] = v.w;
        }
    }

    __device__ static Aux load_aux(const GemvArgs& a, int row, int chunk) {
        const uint8_t* p = a.scale8 + (size_t)row * (a.K >> 4) + 2 * chunk;
        const uint32_t b = (uint32_t)p[0] | ((uint32_t)p[1] << 8);
        Aux r;
        r.s0 = e4m3_to_f32<0>(b);
        r.s1 = e4m3_to_f32<1>(b);
        return r;
    }

    template <int MT>
    __device__ static void accumulate(u32x4 q, const Aux& ax, const X (&xc)[MT], float (&out)[MT]) {
        const uint32_t qd[4] = {q.x, q.y, q.z, q.w};
        float a0[MT], a1[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) { a0[m] = 0.f; a1[m] = 0.f; }
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t p[4];
            p[0] = e2m1x2_to_bf16x2<0>(qd[d]);
            p[1] = e2m1x2_to_bf16x2<1>(qd[d]);
            p[2] = e2m1x2_to_bf16x2<2>(qd[d]);
            p[3] = e2m1x2_to_bf16x2<3>(qd[d]);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float t = (d < 2) ? a0[m] : a1[m];
#pragma unroll
                for (int j = 0; j < 4; ++j) t = dot2(p[j], xc[m].p[4 * d + j], t);
                if (d < 2) a0[m] = t; else a1[m] = t;
            }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) out[m] += fmaf(ax.s0, a0[m], ax.s1 * a1[m]);
    }
    __device__ static float finish(const GemvArgs& a, float v) { return v * a.gscale; }
};

// ---------------------------------------------------------------------------
// BF16 weights (the audio head, and v/down when they stay dense)
// ---------------------------------------------------------------------------
struct FmtBf16 {
    static constexpr int WPC = 8;
    static constexpr int XW = 4;
    struct X { uint32_t p[4]; };
    struct Aux {};

    __device__ static void load_x(const uint16_t* xrow, int k0, bool active, X& xc) {
        u32x4 v = active ? *reinterpret_cast<const u32x4*>(xrow + k0) : u32x4{0, 0, 0, 0};
        xc.p[0] = v.x; xc.p[1] = v.y; xc.p[2] = v.z; xc.p[3] = v.w;
    }
    __device__ static Aux load_aux(const GemvArgs&, int, int) { return Aux{}; }

    template <int MT>
    __device__ static void accumulate(u32x4 q, const Aux&, const X (&xc)[MT], float (&out)[MT]) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float t = out[m];
            t = dot2(q.x, xc[m].p[0], t);
            t = dot2(q.y, xc[m].p[1], t);
            t = dot2(q.z, xc[m].p[2], t);
            t = dot2(q.w, xc[m].p[3], t);
            out[m] = t;
        }
    }
    __device__ static float finish(const GemvArgs&, float v) { return v; }
};

}  // namespace q4
