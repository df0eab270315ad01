// Weight-format policies for the packed-dot GEMV kernel.
//
// A "chunk" is the 16 bytes of weight data one lane loads with one 128-bit
// load.  For the 4-bit formats that is 32 consecutive weights of one row; for
// BF16 it is 8.  Each policy says how to hold the matching activations in
// registers, how to fetch the per-chunk group parameters (through buffer
// resources based at the wave's first row, so rows past N read as zero), and
// how to turn a chunk into a partial dot product for every batch row.
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
    // fused int4 calls only (kernels instantiated with kFused), else null:
    const uint16_t* up;      // [M, K] bf16: the activations are RN_bf16(silu(x) * up)
    const uint16_t* resid;   // [M, N] bf16: y = RN_bf16(x W^T + resid); may equal y
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
    struct X { uint32_t p[16]; float sum; };
    struct Aux { float s, m; };
    struct AuxRes { __amdgpu_buffer_rsrc_t s, m; };

    __device__ static void load_x(const uint16_t* xrow, int k0, bool active, X& xc) {
        if (!active) {
#pragma unroll
            for (int i = 0; i < 16; ++i) xc.p[i] = 0;
            xc.sum = 0.f;
            return;
        }
        const u32x4* src = reinterpret_cast<const u32x4*>(xrow + k0);
        // 32 activations = 16 dwords; block d (8 activations) = dwords 4d..4d+3.
        uint32_t w[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4 v = src[i];
            w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) xq4_pairs(w[4 * d], w[4 * d + 1], w[4 * d + 2], w[4 * d + 3], &xc.p[4 * d]);
        // sum of the 32 activations: packed dot products against (1.0, 1.0)
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            s0 = dot2(w[i], 0x3F803F80u, s0);
            s1 = dot2(w[i + 1], 0x3F803F80u, s1);
        }
        xc.sum = s0 + s1;
    }

    // Batch staging: the scale and min blocks of one batch of rows are
    // contiguous ([rows][K/128] fp16 each, at most 512 bytes for the batch
    // shapes the GEMV plans use), so lanes 0-31 fetch the scales and lanes
    // 32-63 the mins with one 16-byte load each; the block then goes through
    // LDS to the lanes that need it.  Used when every such load is 16-byte
    // aligned: K % 1024 == 0 and both arrays 16-byte aligned (the host
    // decides, per task).
    static constexpr bool kStaged = true;
    static constexpr int kStageBytes = 1024;
    // row0: first row of the batch.  Plain global loads: the two halves of
    // the wave read different arrays, which a buffer resource (uniform per
    // wave) cannot express without a readfirstlane loop.  With K % 1024 == 0
    // every array is a whole number of 16-byte pieces, so the bound check
    // per piece is exact.
    // rows: rows in the batch (the block is rows * K/128 fp16 per array).
    __device__ static u32x4 load_stage(const GemvArgs& a, int row0, int rows, int lane) {
        const size_t G = (size_t)(a.K >> 7);
        const uint32_t piece = (uint32_t)(lane & 31) * 16;
        const size_t off = (size_t)row0 * G * 2 + piece;
        const uint8_t* base = reinterpret_cast<const uint8_t*>(lane < 32 ? a.scale : a.minv);
        const bool ok = piece < (uint32_t)rows * G * 2 && off < (size_t)a.N * G * 2;
        return ok ? *reinterpret_cast<const u32x4*>(base + off) : u32x4{0, 0, 0, 0};
    }
    // row_in_batch: row offset inside the staged batch
    __device__ static Aux read_stage(const uint16_t* st, const GemvArgs& a, int row_in_batch, int chunk) {
        const int i = row_in_batch * (a.K >> 7) + (chunk >> 2);
        Aux x;
        x.s = f16_to_f32(st[i]);
        x.m = f16_to_f32(st[256 + i]);
        return x;
    }

    // group parameters of rows [row0, row0 + rows)
    __device__ static AuxRes make_aux(const GemvArgs& a, int row0, int rows) {
        const size_t G = (size_t)(a.K >> 7);
        AuxRes r;
        r.s = make_rsrc(a.scale + (size_t)row0 * G, (uint32_t)(rows * G * 2));
        r.m = make_rsrc(a.minv + (size_t)row0 * G, (uint32_t)(rows * G * 2));
        return r;
    }
    __device__ static uint32_t aux_voff(const GemvArgs& a, int sub_row, int chunk) {
        return (uint32_t)(sub_row * (a.K >> 7) + (chunk >> 2)) * 2;
    }
    __device__ static uint32_t aux_soff(const GemvArgs& a, int rows) { return (uint32_t)(rows * (a.K >> 7)) * 2; }
    __device__ static Aux load_aux(const AuxRes& r, uint32_t voff, uint32_t soff) {
        Aux x;
        x.s = f16_to_f32(buf_load2(r.s, voff, soff));
        x.m = f16_to_f32(buf_load2(r.m, voff, soff));
        return x;
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
    struct X { uint32_t p[16]; };
    struct Aux { float s0, s1; };
    struct AuxRes { __amdgpu_buffer_rsrc_t s; };

    __device__ static void load_x(const uint16_t* xrow, int k0, bool active, X& xc) {
        const u32x4* src = reinterpret_cast<const u32x4*>(xrow + k0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4 v = active ? src[i] : u32x4{0, 0, 0, 0};
            xc.p[4 * i + 0] = v.x; xc.p[4 * i + 1] = v.y; xc.p[4 * i + 2] = v.z; xc.p[4 * i + 3] = v.w;
        }
    }

    static constexpr bool kStaged = false;
    static constexpr int kStageBytes = 0;
    __device__ static u32x4 load_stage(const GemvArgs&, int, int, int) { return u32x4{0, 0, 0, 0}; }
    __device__ static Aux read_stage(const uint16_t*, const GemvArgs&, int, int) { return Aux{}; }

    __device__ static AuxRes make_aux(const GemvArgs& a, int row0, int rows) {
        const size_t rb = (size_t)(a.K >> 4);
        AuxRes r;
        r.s = make_rsrc(a.scale8 + (size_t)row0 * rb, (uint32_t)(rows * rb));
        return r;
    }
    __device__ static uint32_t aux_voff(const GemvArgs& a, int sub_row, int chunk) {
        return (uint32_t)(sub_row * (a.K >> 4) + 2 * chunk);
    }
    __device__ static uint32_t aux_soff(const GemvArgs& a, int rows) { return (uint32_t)(rows * (a.K >> 4)); }
    __device__ static Aux load_aux(const AuxRes& r, uint32_t voff, uint32_t soff) {
        const uint32_t b = buf_load2(r.s, voff, soff);
        Aux x;
        x.s0 = e4m3_to_f32<0>(b);
        x.s1 = e4m3_to_f32<1>(b);
        return x;
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
    struct X { uint32_t p[4]; };
    struct Aux {};
    struct AuxRes {};

    __device__ static void load_x(const uint16_t* xrow, int k0, bool active, X& xc) {
        u32x4 v = active ? *reinterpret_cast<const u32x4*>(xrow + k0) : u32x4{0, 0, 0, 0};
        xc.p[0] = v.x; xc.p[1] = v.y; xc.p[2] = v.z; xc.p[3] = v.w;
    }
    static constexpr bool kStaged = false;
    static constexpr int kStageBytes = 0;
    __device__ static u32x4 load_stage(const GemvArgs&, int, int, int) { return u32x4{0, 0, 0, 0}; }
    __device__ static Aux read_stage(const uint16_t*, const GemvArgs&, int, int) { return Aux{}; }
    __device__ static AuxRes make_aux(const GemvArgs&, int, int) { return AuxRes{}; }
    __device__ static uint32_t aux_voff(const GemvArgs&, int, int) { return 0; }
    __device__ static uint32_t aux_soff(const GemvArgs&, int) { return 0; }
    __device__ static Aux load_aux(const AuxRes&, uint32_t, uint32_t) { return Aux{}; }

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
