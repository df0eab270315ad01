"""Plain, slow, obviously-correct CPU reference (test infrastructure only).

Conventions: every input arrives as raw bits (uint8 / uint16 NumPy arrays) in
the layouts the pages give; decoding happens here from the bit fields, so no
conversion routine of the code under test is reused.

Readings of points the pages leave open:
  * NVFP4 nibble order is taken to be the int4 card's (low nibble = even
    column); the VoxCPM2 card only says "4-bit float".
  * E2M1 is the OCP microscaling FP4: bit 3 sign, bits 2..1 exponent with
    bias 1, bit 0 mantissa.
  * float8_e4m3fn is the OCP FP8 E4M3 "fn" variant: bias 7, no infinities,
    S.1111.111 is NaN, largest finite 448.
  * The per-matrix global scale G multiplies: w = e2m1 * e4m3 * G, rounded to
    fp32 once.
  * y = x . W^T with W stored [N, K] (the nn.Linear convention the per-module
    names imply); no bias.
  * Sampling from the head (temperature 0.8, top-k 30 in the fast-inference
    post): the k largest BF16 logits, ties to the lower index, in order of
    (logit descending, index ascending); softmax of logit / T over those k;
    the token is the first in that order whose cumulative probability
    exceeds the caller's uniform u in [0, 1) (inverse CDF).
  * The MLP activation between the gate/up and down projections is SiLU
    gating, h = silu(gate) * up (the pages name gate, up and down projections
    but not the activation; SiLU gating is the one those three names go with),
    rounded to BF16 once; residual adds round once with the product.
"""
from __future__ import annotations

import numpy as np

GROUP_Q4 = 128      # rumik-oss-1-int4 card, "Format": scale/min are [N, K/128]
GROUP_NVFP4 = 16    # VoxCPM2-NVFP4 card, "What was quantized": group size 16


def _u(a, dtype):
    return np.ascontiguousarray(np.asarray(a)).astype(dtype, copy=False)


# ----------------------------------------------------------------------------
# nibble unpacking  (rumik-oss-1-int4, "Format": two 4-bit codes per byte,
# low nibble = even column)
# ----------------------------------------------------------------------------
def unpack_nibbles(qweight) -> np.ndarray:
    """uint8 [N, K/2] -> codes uint8 [N, K]: code[n, 2j] = low nibble of
    byte [n, j], code[n, 2j+1] = high nibble."""
    b = _u(qweight, np.uint8)
    assert b.ndim == 2
    n, half = b.shape
    codes = np.empty((n, 2 * half), dtype=np.uint8)
    codes[:, 0::2] = b & 0x0F
    codes[:, 1::2] = b >> 4
    return codes


# ----------------------------------------------------------------------------
# scalar formats, decoded from their bit fields into exact float64 values
# ----------------------------------------------------------------------------
def fp16_value(bits) -> np.ndarray:
    """IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
    Subnormals decode exactly (no flush to zero)."""
    b = _u(bits, np.uint16).astype(np.int64)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = b & 0x3FF
    normal = np.ldexp((f + 1024).astype(np.float64), (e - 25).astype(np.int64))
    sub = np.ldexp(f.astype(np.float64), -24)
    mag = np.where(e == 0, sub, normal)
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return sign * mag


def bf16_value(bits) -> np.ndarray:
    """bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits (the upper
    half of an IEEE binary32)."""
    b = _u(bits, np.uint16).astype(np.int64)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    normal = np.ldexp((f + 128).astype(np.float64), (e - 134).astype(np.int64))
    sub = np.ldexp(f.astype(np.float64), -133)
    mag = np.where(e == 0, sub, normal)
    mag = np.where(e == 255, np.where(f == 0, np.inf, np.nan), mag)
    return sign * mag


def e4m3fn_value(bits) -> np.ndarray:
    """float8_e4m3fn: 1 sign, 4 exponent (bias 7), 3 fraction bits; exponent 0
    is subnormal (f * 2^-9); S.1111.111 is NaN; there is no infinity."""
    b = _u(bits, np.uint8).astype(np.int64)
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 3) & 0xF
    f = b & 0x7
    normal = np.ldexp((f + 8).astype(np.float64), (e - 10).astype(np.int64))
    sub = np.ldexp(f.astype(np.float64), -9)
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 15) & (f == 7), np.nan, mag)
    return sign * mag


def e2m1_value(codes) -> np.ndarray:
    """E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa;
    exponent 0 is subnormal (m * 0.5).  Code 8 is -0."""
    c = _u(codes, np.uint8).astype(np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    normal = np.ldexp((m + 2).astype(np.float64), (e - 2).astype(np.int64))
    sub = 0.5 * m.astype(np.float64)
    return sign * np.where(e == 0, sub, normal)


# ----------------------------------------------------------------------------
# dequantization to fp32
# ----------------------------------------------------------------------------
def q4g128_dequant_f32(qweight, scale_bits, min_bits) -> np.ndarray:
    """rumik-oss-1-int4, "Format": w[n,k] = code[n,k]*scale[n,k//128] +
    min[n,k//128], with scale and min fp16 [N, K/128].

    The fp64 evaluation is exact for finite inputs (code*scale has at most
    4+11 significant bits and the sum spans at most 44 bits, all multiples of
    2^-24 below 2^20), so casting to fp32 rounds exactly once."""
    codes = unpack_nibbles(qweight).astype(np.float64)
    n, k = codes.shape
    assert k % GROUP_Q4 == 0
    s = fp16_value(scale_bits).reshape(n, k // GROUP_Q4)
    m = fp16_value(min_bits).reshape(n, k // GROUP_Q4)
    w = codes * np.repeat(s, GROUP_Q4, axis=1) + np.repeat(m, GROUP_Q4, axis=1)
    return w.astype(np.float32)


def nvfp4g16_dequant_f32(qweight, scale_bits, global_scale) -> np.ndarray:
    """VoxCPM2-NVFP4, "What was quantized": w[n,k] = e2m1(code[n,k]) *
    e4m3(scale[n,k//16]) * G with G the per-matrix fp32 global scale.

    e2m1*e4m3 is exact (<= 2+4 significant bits); times G (24 bits) is still
    exact in fp64, so the cast to fp32 is the single rounding."""
    codes = unpack_nibbles(qweight)
    n, k = codes.shape
    assert k % GROUP_NVFP4 == 0
    v = e2m1_value(codes)
    s = e4m3fn_value(scale_bits).reshape(n, k // GROUP_NVFP4)
    g = np.float64(np.float32(global_scale))
    w = (v * np.repeat(s, GROUP_NVFP4, axis=1)) * g
    return w.astype(np.float32)


def bf16_dequant_f32(w_bits) -> np.ndarray:
    """BF16 weights widened to fp32 (exact)."""
    return bf16_value(w_bits).astype(np.float32)


# ----------------------------------------------------------------------------
# the product
# ----------------------------------------------------------------------------
def gemv_f64(x_bits, w32) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * w[n, k] in fp64 (x BF16 bits [M, K], w fp32
    [N, K]).  Returns fp64 [M, N]."""
    x = bf16_value(x_bits)
    x = x.reshape(-1, x.shape[-1])
    w = np.asarray(w32, dtype=np.float32).astype(np.float64)
    assert x.shape[1] == w.shape[1]
    return x @ w.T


def q4g128_gemv(x_bits, qweight, scale_bits, min_bits) -> np.ndarray:
    return gemv_f64(x_bits, q4g128_dequant_f32(qweight, scale_bits, min_bits))


def nvfp4g16_gemv(x_bits, qweight, scale_bits, global_scale) -> np.ndarray:
    return gemv_f64(x_bits, nvfp4g16_dequant_f32(qweight, scale_bits, global_scale))


def bf16_gemv(x_bits, w_bits) -> np.ndarray:
    return gemv_f64(x_bits, bf16_dequant_f32(w_bits))


# ----------------------------------------------------------------------------
# the decode step's elementwise neighbours (Rumik TTS Fast Inference post,
# "What Made It Faster": residual and normalization work fused around the
# weight-only projections; the gated MLP activation between gate/up and down)
# ----------------------------------------------------------------------------
def bf16_round_bits(v) -> np.ndarray:
    """fp64 values -> BF16 bit patterns, round to nearest with ties to even,
    from the format's definition: 8 significant bits, fp32's exponent range,
    subnormal step 2^-133, magnitudes that round past the largest finite
    value -> infinity; NaN -> 0x7FC0."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))        # a = m 2^ex, m in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, -126)     # floor(log2 a), clamped to the normal range
    step = np.ldexp(1.0, e - 7)
    r = np.rint(a / step) * step                      # a / step is exact; rint ties to even
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    with np.errstate(over="ignore"):
        f = np.where(np.signbit(v), -r, r).astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(v), np.uint16(0x7FC0), bits)


def _bf16_tie(a) -> np.ndarray:
    """|a| lies exactly halfway between two neighbouring BF16 values."""
    a = np.abs(np.asarray(a, dtype=np.float64))
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    step = np.ldexp(1.0, np.maximum(ex.astype(np.int64) - 1, -126) - 7)
    n = a / step
    return (a > 0) & np.isfinite(a) & (n - np.floor(n) == 0.5)


def silu_mul_bf16(g_bits, u_bits) -> np.ndarray:
    """h = RN_bf16(silu(g) * u) with silu(g) = g / (1 + e^-g), for BF16 g and
    u (bit patterns), rounded to BF16 once.

    Written as P * sigma(g) with P = g * u, which is exact in fp64 (two 8-bit
    significands), and sigma(g) = 1 / (1 + e^-g) in fp64.  For large g the
    fp64 product equals P although the exact value is P (1 - sigma(-g)),
    slightly smaller in magnitude; that only changes the rounding when P lies
    exactly halfway between two BF16 values, and then the exact value rounds
    to the neighbour nearer zero."""
    g = bf16_value(g_bits)
    u = bf16_value(u_bits)
    P = g * u
    with np.errstate(over="ignore"):
        v = P / (1.0 + np.exp(-g))
    lost = (g > 0) & (v == P) & _bf16_tie(P)
    toward_zero = bf16_round_bits(P * (1.0 - 2.0 ** -40))
    return np.where(lost, toward_zero, bf16_round_bits(v))


def gemv_residual_f64(x_bits, w32, r_bits) -> np.ndarray:
    """y = x . W^T + r in fp64, before its one rounding to BF16 (r BF16 bits
    [M, N])."""
    y = gemv_f64(x_bits, w32)
    return y + bf16_value(r_bits).reshape(y.shape)


# ----------------------------------------------------------------------------
# sampling from the head (Rumik TTS Fast Inference post, "The Result":
# temperature 0.8, top-k 30 over the audio-token head)
# ----------------------------------------------------------------------------
def sample_topk(logit_bits, temperature, top_k, u):
    """Per batch row m of BF16 logits [M, V]: the top_k largest logits (ties
    to the lower index), ordered by (logit descending, index ascending); their
    probabilities softmax(logit / T) over those k, in fp64; the sampled token,
    the first of that order whose cumulative probability exceeds u[m].
    Returns (token [M] int64, index [M, k] int64, prob [M, k] fp64)."""
    lg = bf16_value(logit_bits)
    lg = lg.reshape(-1, lg.shape[-1])
    M, V = lg.shape
    assert 1 <= top_k <= V
    u = np.asarray(u, dtype=np.float64).reshape(M)
    index = np.empty((M, top_k), np.int64)
    prob = np.empty((M, top_k), np.float64)
    token = np.empty(M, np.int64)
    for m in range(M):
        order = np.lexsort((np.arange(V), -lg[m]))[:top_k]   # primary: logit descending; then index
        z = lg[m, order] / temperature
        e = np.exp(z - z[0])
        p = e / e.sum()
        c = np.cumsum(p)
        pick = int(np.searchsorted(c, u[m], side="right"))
        index[m], prob[m], token[m] = order, p, order[min(pick, top_k - 1)]
    return token, index, prob
