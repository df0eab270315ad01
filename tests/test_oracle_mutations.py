"""Planted mistakes in a private copy of the oracle must each fail some pin.

The copy is a fresh module object built from oracle/reference.py, so internal
calls (e.g. q4g128_gemv -> gemv_f64) pick up the planted mistake.  Nothing
here touches the real oracle module or the GPU.
"""
import importlib.util
import os
import types

import numpy as np
import pytest

from oracle_pins import ALL_PINS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REF_PATH = os.path.join(ROOT, "oracle", "reference.py")


def fresh_oracle() -> types.ModuleType:
    spec = importlib.util.spec_from_file_location("oracle_mutant", REF_PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _m_swap_nibbles(O):
    def unpack_nibbles(qweight):
        b = np.ascontiguousarray(qweight).astype(np.uint8)
        c = np.empty((b.shape[0], 2 * b.shape[1]), np.uint8)
        c[:, 0::2] = b >> 4
        c[:, 1::2] = b & 0x0F
        return c
    O.unpack_nibbles = unpack_nibbles


def _m_drop_min(O):
    orig = O.q4g128_dequant_f32

    def q4g128_dequant_f32(qw, sc, mn):
        return orig(qw, sc, np.zeros_like(np.asarray(mn)))
    O.q4g128_dequant_f32 = q4g128_dequant_f32


def _m_negate_min(O):
    orig = O.q4g128_dequant_f32

    def q4g128_dequant_f32(qw, sc, mn):
        return orig(qw, sc, np.asarray(mn, np.uint16) ^ np.uint16(0x8000))
    O.q4g128_dequant_f32 = q4g128_dequant_f32


def _m_group64(O):
    O.GROUP_Q4 = 64


def _m_group_index_mod(O):
    def q4g128_dequant_f32(qw, sc, mn):
        codes = O.unpack_nibbles(qw).astype(np.float64)
        n, k = codes.shape
        s = O.fp16_value(sc).reshape(n, k // 128)
        m = O.fp16_value(mn).reshape(n, k // 128)
        return (codes * np.tile(s, (1, 128)) + np.tile(m, (1, 128))).astype(np.float32)
    O.q4g128_dequant_f32 = q4g128_dequant_f32


def _m_fp16_bias(O):
    orig = O.fp16_value
    O.fp16_value = lambda bits: orig(bits) * 2.0


def _m_fp16_ftz(O):
    orig = O.fp16_value

    def fp16_value(bits):
        b = np.asarray(bits, np.uint16)
        v = orig(b)
        return np.where((b & 0x7C00) == 0, 0.0 * v, v)
    O.fp16_value = fp16_value


def _m_e4m3_bias8(O):
    orig = O.e4m3fn_value
    O.e4m3fn_value = lambda bits: orig(bits) * 0.5


def _m_e4m3_no_nan(O):
    def e4m3fn_value(bits):
        b = np.asarray(bits, np.uint8).astype(np.int64)
        sign = np.where((b >> 7) & 1, -1.0, 1.0)
        e = (b >> 3) & 0xF
        f = b & 0x7
        return sign * np.where(e == 0, np.ldexp(f.astype(float), -9), np.ldexp((f + 8).astype(float), (e - 10)))
    O.e4m3fn_value = e4m3fn_value


def _m_e2m1_sub(O):
    orig = O.e2m1_value

    def e2m1_value(codes):
        c = np.asarray(codes, np.uint8)
        v = orig(c)
        return np.where((c & 7) == 1, v * 0.5, v)
    O.e2m1_value = e2m1_value


def _m_e2m1_nosign(O):
    orig = O.e2m1_value
    O.e2m1_value = lambda codes: np.abs(orig(codes))


def _m_nvfp4_double_round(O):
    def nvfp4g16_dequant_f32(qw, sc, G):
        codes = O.unpack_nibbles(qw)
        n, k = codes.shape
        v = O.e2m1_value(codes)
        s = (O.e4m3fn_value(sc).reshape(n, k // 16) * np.float64(np.float32(G))).astype(np.float32).astype(np.float64)
        return (v * np.repeat(s, 16, axis=1)).astype(np.float32)
    O.nvfp4g16_dequant_f32 = nvfp4g16_dequant_f32


def _m_gemv_drop_last_k(O):
    def gemv_f64(x_bits, w32):
        x = O.bf16_value(x_bits).reshape(-1, np.asarray(w32).shape[1])
        w = np.asarray(w32, np.float32).astype(np.float64)
        return x[:, :-1] @ w[:, :-1].T
    O.gemv_f64 = gemv_f64


def _m_gemv_transposed(O):
    def gemv_f64(x_bits, w32):
        x = O.bf16_value(x_bits).reshape(-1, np.asarray(w32).shape[1])
        w = np.asarray(w32, np.float32).astype(np.float64)
        return w @ x.T
    O.gemv_f64 = gemv_f64


def _m_gemv_fp32(O):
    def gemv_f64(x_bits, w32):
        x = O.bf16_value(x_bits).reshape(-1, np.asarray(w32).shape[1]).astype(np.float32)
        w = np.asarray(w32, np.float32)
        return (x @ w.T).astype(np.float64)
    O.gemv_f64 = gemv_f64


def _m_bf16_bias(O):
    orig = O.bf16_value
    O.bf16_value = lambda bits: orig(bits) * 2.0


def _m_round_truncate(O):
    # keep the upper half of the fp32 bits: rounds toward zero
    O.bf16_round_bits = lambda v: (np.asarray(v, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _m_round_via_fp32(O):
    orig = O.bf16_round_bits
    O.bf16_round_bits = lambda v: orig(np.asarray(v, np.float64).astype(np.float32).astype(np.float64))


def _m_round_ties_away(O):
    orig = O.bf16_round_bits

    def bf16_round_bits(v):
        v = np.asarray(v, np.float64)
        return orig(v + np.sign(v) * np.abs(v) * 2.0 ** -30)
    O.bf16_round_bits = bf16_round_bits


def _m_silu_no_gate(O):
    def silu_mul_bf16(g_bits, u_bits):
        g, u = O.bf16_value(g_bits), O.bf16_value(u_bits)
        return O.bf16_round_bits(u / (1.0 + np.exp(-g)))
    O.silu_mul_bf16 = silu_mul_bf16


def _m_silu_sign(O):
    def silu_mul_bf16(g_bits, u_bits):
        g, u = O.bf16_value(g_bits), O.bf16_value(u_bits)
        return O.bf16_round_bits(g / (1.0 + np.exp(g)) * u)
    O.silu_mul_bf16 = silu_mul_bf16


def _m_residual_transposed(O):
    def gemv_residual_f64(x_bits, w32, r_bits):
        y = O.gemv_f64(x_bits, w32)
        return y + O.bf16_value(r_bits).reshape(y.shape[::-1]).T
    O.gemv_residual_f64 = gemv_residual_f64


def _sample_mutant(O, order_fn=None, temp=None, side="right", over_all=False):
    def sample_topk(logit_bits, temperature, top_k, u):
        lg = O.bf16_value(logit_bits)
        lg = lg.reshape(-1, lg.shape[-1])
        M, V = lg.shape
        u = np.asarray(u, dtype=np.float64).reshape(M)
        index = np.empty((M, top_k), np.int64)
        prob = np.empty((M, top_k), np.float64)
        token = np.empty(M, np.int64)
        T = temperature if temp is None else temp
        for m in range(M):
            order = (order_fn or (lambda v: np.lexsort((np.arange(V), -v))))(lg[m])[:top_k]
            z = lg[m, order] / T
            e = np.exp(z - z[0])
            tot = np.exp(lg[m] / T - z[0]).sum() if over_all else e.sum()
            p = e / tot
            pick = int(np.searchsorted(np.cumsum(p), u[m], side=side))
            index[m], prob[m], token[m] = order, p, order[min(pick, top_k - 1)]
        return token, index, prob
    O.sample_topk = sample_topk


def _m_sample_ties_high(O):
    _sample_mutant(O, order_fn=lambda v: np.lexsort((-np.arange(v.size), -v)))


def _m_sample_smallest(O):
    _sample_mutant(O, order_fn=lambda v: np.lexsort((np.arange(v.size), v)))


def _m_sample_no_temperature(O):
    _sample_mutant(O, temp=1.0)


def _m_sample_cdf_at_least(O):
    _sample_mutant(O, side="left")


def _m_sample_softmax_over_all(O):
    _sample_mutant(O, over_all=True)


MUTANTS = [
    _m_swap_nibbles, _m_drop_min, _m_negate_min, _m_group64, _m_group_index_mod,
    _m_fp16_bias, _m_fp16_ftz, _m_e4m3_bias8, _m_e4m3_no_nan, _m_e2m1_sub,
    _m_e2m1_nosign, _m_nvfp4_double_round, _m_gemv_drop_last_k, _m_gemv_transposed,
    _m_gemv_fp32, _m_bf16_bias, _m_round_truncate, _m_round_via_fp32, _m_round_ties_away, _m_silu_no_gate,
    _m_silu_sign, _m_residual_transposed, _m_sample_ties_high, _m_sample_smallest, _m_sample_no_temperature,
    _m_sample_cdf_at_least, _m_sample_softmax_over_all,
]


@pytest.mark.parametrize("mutate", MUTANTS, ids=lambda f: f.__name__[3:])
def test_planted_mistake_is_caught(mutate):
    O = fresh_oracle()
    mutate(O)
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(O)
        except Exception as e:  # AssertionError or a shape error both count
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"no pin caught mutant {mutate.__name__}"


def test_unmutated_copy_passes_all_pins():
    O = fresh_oracle()
    for pin in ALL_PINS:
        with np.errstate(all="ignore"):
            pin(O)
