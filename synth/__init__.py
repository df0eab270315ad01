"""Seeded synthetic inputs for the 4-bit weight-only dequant-GEMV workloads.

This module produces *bytes*: BF16 activations, packed 4-bit codes with their
group scales, and BF16 weights.  It holds none of the arithmetic of the method
under test (no decoding, no dequantization, no matrix product).  It is the one
piece of code shared by the CPU oracle's tests and the GPU path's tests and
benchmark; both sides receive the same tensors from here.

The formats follow the pages:
  * rumik-oss-1-int4 model card, section "Format": qweight uint8 [N, K/2] with
    two 4-bit codes per byte (low nibble = even column), fp16 scale and min of
    shape [N, K/128].
  * VoxCPM2-NVFP4 model card, section "What was quantized": E2M1 4-bit float
    codes, symmetric, group size 16, float8_e4m3fn group scales and one fp32
    global scale per matrix.

Quantizers here only exist to turn Gaussian BF16 matrices into realistic
format bytes (the pages name "min/max" rounding and plain RTN); they are not
timed and nothing downstream depends on their tie-breaking.

Everything is torch so that the same generator runs on the CPU (tests, small
shapes) and on the GPU (benchmark, ~1.2 GB of weights).  CPU generation is
deterministic across machines; GPU generation is deterministic per device
type.  Seeds are tuples hashed to a 63-bit integer.
"""
from __future__ import annotations

import hashlib
from typing import Dict, Tuple

import torch

# Projection shapes (N rows = output features, K = input features) of one
# decoder layer at hidden size 2048 with FFN width 8192.  The rumik-oss-1-int4
# card ("Format") lists the seven per-layer projections; hidden 2048 comes from
# the embedding shape on the same card.
LAYER_SHAPES: Dict[str, Tuple[int, int]] = {
    "q": (2048, 2048),
    "k": (512, 2048),
    "v": (512, 2048),
    "o": (2048, 2048),
    "gate": (8192, 2048),
    "up": (8192, 2048),
    "down": (2048, 8192),
}
LAYER_ORDER = ("q", "k", "v", "o", "gate", "up", "down")
# BF16 audio head (rumik-oss-1-int4 card, "Format": head.audio_weight
# [16385, 2048]) and the current-codebook slice of 2049 rows (Rumik TTS Fast
# Inference, "What Made It Faster", Figure 3).
HEAD_FULL = (16385, 2048)
HEAD_SLICE = (2049, 2048)
# VoxCPM2-NVFP4 card, "What was quantized": v_proj and down_proj stay BF16.
NVFP4_BF16_PROJ = ("v", "down")
N_LAYERS = 36
GROUP_Q4 = 128
GROUP_NVFP4 = 16


def seed_int(*parts) -> int:
    """Stable 63-bit integer from any tuple of str/int parts."""
    h = hashlib.sha256(repr(tuple(parts)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def make_gen(seed, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed if isinstance(seed, int) else seed_int(*seed))
    return g


# ----------------------------------------------------------------------------
# activations and BF16 weights
# ----------------------------------------------------------------------------
def randn_bf16(shape, std: float, seed, device="cpu") -> torch.Tensor:
    g = make_gen(seed, device)
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def x_bf16(M: int, K: int, seed, device="cpu") -> torch.Tensor:
    """Activations: BF16 N(0, 1), shape [M, K]."""
    return randn_bf16((M, K), 1.0, ("x", seed, M, K), device)


def bf16_matrix(N: int, K: int, seed, device="cpu", std: float = 0.02) -> torch.Tensor:
    """Dense BF16 weight [N, K] drawn from N(0, std^2)."""
    return randn_bf16((N, K), std, ("w", seed, N, K), device)


# ----------------------------------------------------------------------------
# int4 g128 min/max
# ----------------------------------------------------------------------------
def pack_nibbles(codes: torch.Tensor) -> torch.Tensor:
    """[N, K] codes in 0..15 -> uint8 [N, K/2]; even column in the low nibble."""
    c = codes.to(torch.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).contiguous()


def quantize_g128_minmax(w: torch.Tensor):
    """Min/max (asymmetric RTN) quantization per 128-column group.

    scale = fp16((max - min) / 15), min = fp16(group min),
    code = clip(round_half_even((w - min) / scale), 0, 15), code = 0 where
    scale == 0.  Returns (qweight uint8 [N, K/2], scale fp16 [N, K/128],
    min fp16 [N, K/128]).
    """
    N, K = w.shape
    assert K % GROUP_Q4 == 0
    wf = w.to(torch.float32).reshape(N, K // GROUP_Q4, GROUP_Q4)
    lo = wf.amin(dim=2)
    hi = wf.amax(dim=2)
    scale16 = ((hi - lo) / 15.0).to(torch.float16)
    min16 = lo.to(torch.float16)
    s = scale16.to(torch.float32).unsqueeze(2)
    m = min16.to(torch.float32).unsqueeze(2)
    safe = torch.where(s == 0, torch.ones_like(s), s)
    q = torch.round((wf - m) / safe)
    q = torch.where(s == 0, torch.zeros_like(q), q).clamp_(0, 15)
    codes = q.to(torch.uint8).reshape(N, K)
    return pack_nibbles(codes), scale16.contiguous(), min16.contiguous()


def q4_matrix(N: int, K: int, seed, device="cpu", std: float = 0.02):
    """min/max-quantized N(0, std^2) BF16 matrix -> (qweight, scale, min)."""
    return quantize_g128_minmax(bf16_matrix(N, K, seed, device, std))


def q4_layer(seed, device="cpu") -> Dict[str, tuple]:
    """All seven projections of one hidden-2048 decoder layer, int4 g128."""
    return {name: q4_matrix(*LAYER_SHAPES[name], (seed, name), device) for name in LAYER_ORDER}


def config0(seed: int = 0, device="cpu"):
    """Single 256x512 int4 g128 matrix with uniform codes, M = 1.

    codes uniform in 0..15; scale fp16 ~ U[1e-3, 2e-2]; min = fp16(-7.5*scale
    + N(0, 1e-3)) evaluated in fp64 and rounded once; x BF16 N(0, 1).
    """
    N, K = 256, 512
    g = make_gen(("config0", seed), "cpu")
    codes = torch.randint(0, 16, (N, K), generator=g, dtype=torch.int64)
    scale16 = (torch.rand((N, K // GROUP_Q4), generator=g, dtype=torch.float64) * (2e-2 - 1e-3) + 1e-3).to(torch.float16)
    noise = torch.randn((N, K // GROUP_Q4), generator=g, dtype=torch.float64) * 1e-3
    min16 = (-7.5 * scale16.to(torch.float64) + noise).to(torch.float16)
    x = (torch.randn((1, K), generator=g, dtype=torch.float32)).to(torch.bfloat16)
    out = dict(x=x, qweight=pack_nibbles(codes), scale=scale16.contiguous(), min=min16.contiguous())
    return {k: v.to(device) for k, v in out.items()}


# ----------------------------------------------------------------------------
# NVFP4 (E2M1 codes, group 16, e4m3 group scales, fp32 global scale)
# ----------------------------------------------------------------------------
# Magnitude thresholds between neighbouring E2M1 values {0,.5,1,1.5,2,3,4,6}
# and whether a value exactly on the threshold rounds up (ties to the value
# whose mantissa bit is 0).
_E2M1_THRESH = ((0.25, False), (0.75, True), (1.25, False), (1.75, True), (2.5, False), (3.5, True), (5.0, False))


def _e2m1_encode(r: torch.Tensor) -> torch.Tensor:
    a = r.abs()
    mag = torch.zeros_like(a, dtype=torch.int32)
    for t, up in _E2M1_THRESH:
        mag += (a >= t if up else a > t).to(torch.int32)
    sign = (r < 0).to(torch.int32) << 3
    return (mag | sign).to(torch.uint8)


def quantize_nvfp4(w: torch.Tensor):
    """Plain RTN NVFP4: G = amax/(6*448); s_g = e4m3(absmax_g/6/G) saturated at
    448; code = e2m1(w/(s_g*G)) with ties to even and |.| clamped at 6;
    codes 0 where s_g == 0.  Returns (qweight uint8 [N,K/2], scale_e4m3 bits
    uint8 [N,K/16], G python float (exactly an fp32 value))."""
    N, K = w.shape
    assert K % GROUP_NVFP4 == 0
    wf = w.to(torch.float32)
    amax = wf.abs().amax()
    G = (amax / (6.0 * 448.0)).to(torch.float32)
    if float(G) == 0.0:
        G = torch.tensor(1.0, dtype=torch.float32, device=w.device)
    wg = wf.reshape(N, K // GROUP_NVFP4, GROUP_NVFP4)
    sg = (wg.abs().amax(dim=2) / 6.0 / G).clamp(max=448.0)
    s8 = sg.to(torch.float8_e4m3fn)
    sdec = s8.to(torch.float32).unsqueeze(2) * G
    safe = torch.where(sdec == 0, torch.ones_like(sdec), sdec)
    r = (wg / safe).clamp(-6.0, 6.0)
    r = torch.where(sdec == 0, torch.zeros_like(r), r)
    codes = _e2m1_encode(r).reshape(N, K)
    return pack_nibbles(codes), s8.view(torch.uint8).contiguous(), float(G)


def nvfp4_matrix(N: int, K: int, seed, device="cpu", std: float = 0.02):
    return quantize_nvfp4(bf16_matrix(N, K, seed, device, std))


# ----------------------------------------------------------------------------
# bit-pattern views for the numpy oracle
# ----------------------------------------------------------------------------
def bits16(t: torch.Tensor):
    """bf16/fp16 tensor -> numpy uint16 bit patterns (on CPU)."""
    import numpy as np
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bits8(t: torch.Tensor):
    import numpy as np
    return t.detach().cpu().contiguous().view(torch.uint8).numpy().view(np.uint8)
