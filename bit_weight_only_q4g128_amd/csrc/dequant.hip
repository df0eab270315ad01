// Diagnostic dequantization to fp32, one thread per 8 weights.  These use the
// same conversion helpers as the GEMV kernels, so a bitwise comparison of their
// output checks the device-side format decoding.
#include "internal.h"

namespace q4 {

namespace {

// rumik-oss-1-int4 card, "Format": w = code * scale[n, k/128] + min[n, k/128];
// code*scale is exact in fp32, so one fma rounds exactly once.
__global__ __launch_bounds__(256) void q4_dequant_kernel(const uint8_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                                                         const uint16_t* __restrict__ mn, int N, int K, float* __restrict__ w) {
    const size_t total = (size_t)N * (K >> 3);
    const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const size_t row = t / (K >> 3);
    const int k0 = (int)(t - row * (K >> 3)) * 8;
    const uint32_t d = *reinterpret_cast<const uint32_t*>(qw + row * (K >> 1) + (k0 >> 1));
    const size_t gi = row * (K >> 7) + (k0 >> 7);
    const float s = f16_to_f32(sc[gi]);
    const float m = f16_to_f32(mn[gi]);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = fmaf((float)((d >> (4 * i)) & 0xFu), s, m);
    f32x4* out = reinterpret_cast<f32x4*>(w + row * K + k0);
    out[0] = f32x4{v[0], v[1], v[2], v[3]};
    out[1] = f32x4{v[4], v[5], v[6], v[7]};
}

// VoxCPM2-NVFP4 card, "What was quantized": w = e2m1(code) * e4m3(scale) * G;
// the first product is exact, the multiply by G rounds once.
__global__ __launch_bounds__(256) void nvfp4_dequant_kernel(const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sc, float G,
                                                            int N, int K, float* __restrict__ w) {
    const size_t total = (size_t)N * (K >> 3);
    const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const size_t row = t / (K >> 3);
    const int k0 = (int)(t - row * (K >> 3)) * 8;
    const uint32_t d = *reinterpret_cast<const uint32_t*>(qw + row * (K >> 1) + (k0 >> 1));
    const float s = e4m3_to_f32<0>((uint32_t)sc[row * (K >> 4) + (k0 >> 4)]);
    const f32x2 p0 = e2m1x2_to_f32x2<0>(d), p1 = e2m1x2_to_f32x2<1>(d);
    const f32x2 p2 = e2m1x2_to_f32x2<2>(d), p3 = e2m1x2_to_f32x2<3>(d);
    const float e[8] = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float es = e[i] * s;   // exact
        v[i] = es * G;               // the single rounding
    }
    f32x4* out = reinterpret_cast<f32x4*>(w + row * K + k0);
    out[0] = f32x4{v[0], v[1], v[2], v[3]};
    out[1] = f32x4{v[4], v[5], v[6], v[7]};
}

}  // namespace

hipError_t launch_q4_dequant(const uint8_t* qw, const uint16_t* sc, const uint16_t* mn, int N, int K, float* w, hipStream_t s) {
    const size_t total = (size_t)N * (K >> 3);
    const unsigned grid = (unsigned)((total + 255) / 256);
    return launch_kernel(q4_dequant_kernel, dim3(grid), dim3(256), 0, s, qw, sc, mn, N, K, w);
}

hipError_t launch_nvfp4_dequant(const uint8_t* qw, const uint8_t* sc, float G, int N, int K, float* w, hipStream_t s) {
    const size_t total = (size_t)N * (K >> 3);
    const unsigned grid = (unsigned)((total + 255) / 256);
    return launch_kernel(nvfp4_dequant_kernel, dim3(grid), dim3(256), 0, s, qw, sc, G, N, K, w);
}

}  // namespace q4
