"""Helpers for the GPU parity tests: moving generator output to the device
and the acceptance rule.

Acceptance for a GEMV output element (m, n), with y the BF16 result widened
exactly and y_ref the oracle's fp64 value:

    |y - y_ref| <= 1e-3 * ||w32[n, :]||_2 * ||x[m, :]||_2 + ulp_bf16(|y_ref|)

ulp_bf16(v) = 2^(max(floor(log2 v), -126) - 7), ulp_bf16(0) = 2^-133.  The
first term covers fp32 accumulation in any order (and, for the matrix-core
paths, nothing more: every product there is exact); the second covers the
final round-to-nearest to BF16.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

REL_TOL = 1e-3


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    v = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.maximum(e, -126)
    return np.where(v > 0, np.ldexp(1.0, (e - 7).astype(np.int64)), 2.0 ** -133)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def check_gemv(y_gpu: torch.Tensor, y_ref: np.ndarray, w32: np.ndarray, x_bits: np.ndarray, what: str = ""):
    y = bf16_to_f64(y_gpu)
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    x64 = oracle.bf16_value(x_bits).reshape(y.shape[0], -1)
    wn = np.linalg.norm(np.asarray(w32, dtype=np.float64), axis=1)
    xn = np.linalg.norm(x64, axis=1)
    bound = REL_TOL * xn[:, None] * wn[None, :] + ulp_bf16(y_ref)
    err = np.abs(y - y_ref)
    bad = ~(err <= bound)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first at {tuple(i)}: "
                             f"y={y[tuple(i)]!r} ref={y_ref[tuple(i)]!r} bound={bound[tuple(i)]!r}")
    return float((err / bound).max())


def same_bits_f32(a: np.ndarray, b: np.ndarray) -> bool:
    """fp32 arrays equal element by element; +0 == -0 and NaN == NaN."""
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(nan | (a == b)))


def rn_bf16_bits(w32: np.ndarray) -> np.ndarray:
    """Reference rounding of fp32 values to BF16 bits (round to nearest even),
    via torch's conversion, for the one-hot checks."""
    return torch.from_numpy(np.ascontiguousarray(w32, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def gpu(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda").contiguous()


def onehot_x(K: int, ks) -> torch.Tensor:
    x = torch.zeros(len(ks), K, dtype=torch.bfloat16)
    for m, k in enumerate(ks):
        x[m, k] = 1.0
    return x


def x_bits(x: torch.Tensor) -> np.ndarray:
    return synth.bits16(x)
