// Device helpers shared by the gfx950 kernels: bit-level BF16/FP16/FP8/FP4
// conversions, nibble-to-BF16 unpacking, packed-BF16 dot products and
// wavefront reductions built on DPP.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// fp16 bits -> fp32 (exact, subnormals kept).
// RN_bf16(silu(g) * u) for the two BF16 values of each of g and u packed in
// a dword (low half = first element); silu(g) = g / (1 + e^-g) evaluated in
// fp32 with the hardware exp2 and reciprocal (a few fp32 ulps, far below one
// BF16 step), then rounded to BF16 once.
__device__ __forceinline__ float silu_mul(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(-1.44269504088896341f * g);   // e^-g
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}
__device__ __forceinline__ uint32_t silu_mul_bf16x2(uint32_t g, uint32_t u) {
    const uint32_t lo = f32_to_bf16(silu_mul(bf16lo(g), bf16lo(u)));
    const uint32_t hi = f32_to_bf16(silu_mul(bf16hi(g), bf16hi(u)));
    return lo | (hi << 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// OCP float8_e4m3fn byte (selected by SEL from a dword) -> fp32, exact.
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_f32_fp8(w, SEL);
}

// Two E2M1 codes (byte SEL of a dword: low nibble first) -> BF16 pair, exact.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
}

// Two E2M1 codes -> two fp32 values, exact.
template <int SEL>
__device__ __forceinline__ f32x2 e2m1x2_to_f32x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Two E2M1 codes (byte SEL of dw) times an e4m3 group scale s -> a BF16 pair,
// exact: the product has at most 6 significant bits and lies in [2^-10, 2688].
// (The hardware's scaled FP4 conversions apply only the exponent of their scale
// operand, so the e4m3 factor is a separate fp32 multiply.)
template <int SEL>
__device__ __forceinline__ uint32_t nv_pair_scaled(uint32_t dw, float s) {
    f32x2 v = e2m1x2_to_f32x2<SEL>(dw);
    const float lo = v.x * s, hi = v.y * s;
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ---------------------------------------------------------------------------
// int4 nibbles -> BF16 pairs holding 128 + code (exact)
//
// A dword holds 8 codes c0..c7 (c_i in bits 4i..4i+3; the even column sits in
// the low nibble of each byte).  A code in the low mantissa bits of the BF16
// pattern 0x4300 (= 128.0) reads as exactly 128 + c.  The even nibbles
// (c0 c2 c4 c6) and odd nibbles (c1 c3 c5 c7) are first isolated one per byte;
// v_perm_b32 then interleaves them with the 0x43 high byte, 3 + 4 instructions
// per 8 codes.  The pairs come out as (c0,c4) (c1,c5) (c2,c6) (c3,c7);
// activations are paired the same way by xq4_pairs() so the dot products see
// matching columns.
// ---------------------------------------------------------------------------
constexpr uint32_t kMagicBytes = 0x43434343u;

__device__ __forceinline__ void q4_pairs(uint32_t d, uint32_t p[4]) {
    const uint32_t lo = d & 0x0F0F0F0Fu;          // bytes c0 c2 c4 c6
    const uint32_t hi = (d >> 4) & 0x0F0F0F0Fu;   // bytes c1 c3 c5 c7
    p[0] = __builtin_amdgcn_perm(kMagicBytes, lo, 0x04020400u);   // (c0, c4)
    p[1] = __builtin_amdgcn_perm(kMagicBytes, hi, 0x04020400u);   // (c1, c5)
    p[2] = __builtin_amdgcn_perm(kMagicBytes, lo, 0x04030401u);   // (c2, c6)
    p[3] = __builtin_amdgcn_perm(kMagicBytes, hi, 0x04030401u);   // (c3, c7)
}

// ---------------------------------------------------------------------------
// buffer resources: 128-bit loads with an SGPR base and a 32-bit lane offset;
// offsets at or past num_records read as zero.
// ---------------------------------------------------------------------------
constexpr int kBufferFlags = 0x00020000;   // raw buffer, 32-bit data format (gfx9)
constexpr int kAuxStream = 2;              // nt: read-once streaming data

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kAuxStream));
}
__device__ __forceinline__ uint16_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}

// 8 consecutive BF16 activations (4 dwords, natural order) -> the pairing
// (x0,x4) (x1,x5) (x2,x6) (x3,x7) that matches q4_pairs().
__device__ __forceinline__ void xq4_pairs(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, uint32_t p[4]) {
    p[0] = __builtin_amdgcn_perm(w2, w0, 0x05040100u);
    p[1] = __builtin_amdgcn_perm(w2, w0, 0x07060302u);
    p[2] = __builtin_amdgcn_perm(w3, w1, 0x05040100u);
    p[3] = __builtin_amdgcn_perm(w3, w1, 0x07060302u);
}

// acc + a.lo*b.lo + a.hi*b.hi with BF16 pairs a, b and fp32 acc.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}

// ---------------------------------------------------------------------------
// wavefront reductions (DPP; gfx9 row = 16 lanes)
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over aligned groups of `lanes` lanes (lanes in {1,2,4,...,64}).  After
// the call the lane with (lane % lanes) == lanes-1 holds its group's sum (for
// lanes <= 16 every lane of the group does).
__device__ __forceinline__ float group_sum(float v, int lanes) {
    if (lanes >= 2) v += dpp<0xB1>(v);          // quad_perm [1,0,3,2]
    if (lanes >= 4) v += dpp<0x4E>(v);          // quad_perm [2,3,0,1]
    if (lanes >= 8) v += dpp<0x141>(v);         // row_half_mirror
    if (lanes >= 16) v += dpp<0x140>(v);        // row_mirror
    if (lanes >= 32) v += dpp<0x142, 0xA>(v);   // row_bcast:15 into rows 1, 3
    if (lanes >= 64) v += dpp<0x143, 0xC>(v);   // row_bcast:31 into rows 2, 3
    return v;
}

}  // namespace q4
