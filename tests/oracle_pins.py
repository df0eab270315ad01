"""Pins for the CPU oracle: checks against facts fixed outside the oracle.

Each ``pin_*`` takes an oracle namespace ``O`` (the real ``oracle`` package, or
a copy with one planted mistake) and raises AssertionError on disagreement.
``test_oracle_pins.py`` runs them on the real oracle; ``test_oracle_mutations.py``
plants plausible mistakes into a copy and checks that some pin fails.

Sources of truth used here (never the oracle's own formulas):
  * hand-worked golden fixtures under tests/golden/ (each cites its page or
    standard);
  * exhaustive comparison with numpy's float16 and torch's bfloat16 /
    float8_e4m3fn conversions (library routines);
  * exact rational arithmetic (fractions.Fraction) on tiny inputs;
  * integer-weight special cases where the product is exact in Python ints;
  * the nibble packer of the input generator (an independent implementation
    of the inverse map);
  * for the fused neighbours: torch's fp32 -> bf16 rounding, integer rounding
    of exact rationals, and e^x from the decimal module at 60 digits.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln.split()


def _same(a, b):
    """bitwise-equal float arrays, NaN == NaN, +0 == -0 not allowed unless both 0 with same sign."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return bool(np.all(both_nan | eq))


def _f32_of_fraction(fr: Fraction) -> np.float32:
    """Round an exact rational to fp32 (correct when fr is exactly an fp64
    value, which holds for every product checked here)."""
    d = float(fr)
    assert Fraction(d) == fr, "value not exact in fp64"
    return np.float32(d)


# ----------------------------------------------------------------------------
# nibble order
# ----------------------------------------------------------------------------
def pin_nibble_hand(O):
    for tag, *rest in _lines("q4g128_hand.txt"):
        if tag != "nibble":
            continue
        byte, lo, hi = int(rest[0], 16), int(rest[1]), int(rest[2])
        c = O.unpack_nibbles(np.array([[byte]], dtype=np.uint8))
        assert c.shape == (1, 2), c.shape
        assert int(c[0, 0]) == lo and int(c[0, 1]) == hi, (hex(byte), c)


def pin_nibble_roundtrip(O):
    g = torch.Generator().manual_seed(11)
    codes = torch.randint(0, 16, (7, 96), generator=g)
    packed = synth.pack_nibbles(codes).numpy()
    back = O.unpack_nibbles(packed)
    assert np.array_equal(back, codes.numpy().astype(np.uint8))
    # every byte value: unpack then repack with the generator's packer
    allb = np.arange(256, dtype=np.uint8).reshape(1, 256)
    c = O.unpack_nibbles(allb)
    rep = synth.pack_nibbles(torch.from_numpy(c.astype(np.int64))).numpy()
    assert np.array_equal(rep, allb)


# ----------------------------------------------------------------------------
# scalar decoders
# ----------------------------------------------------------------------------
def pin_fp16(O):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    assert _same(O.fp16_value(bits), ref)
    for hx, val in _lines("fp16_points.txt"):
        assert _same(O.fp16_value(np.array([int(hx, 16)], dtype=np.uint16)), [float(val)]), hx


def pin_bf16(O):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(O.bf16_value(bits), ref)


def pin_e4m3(O):
    bits = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(bits.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(O.e4m3fn_value(bits), ref)
    for hx, val in _lines("e4m3fn_points.txt"):
        assert _same(O.e4m3fn_value(np.array([int(hx, 16)], dtype=np.uint8)), [float(val)]), hx


def pin_e2m1(O):
    for code, val in _lines("e2m1_table.txt"):
        assert _same(O.e2m1_value(np.array([int(code)], dtype=np.uint8)), [float(val)]), code


# ----------------------------------------------------------------------------
# dequantization
# ----------------------------------------------------------------------------
def pin_q4_dequant_hand(O):
    for tag, *rest in _lines("q4g128_hand.txt"):
        if tag != "dequant":
            continue
        code, sb, mb, exp = int(rest[0]), int(rest[1], 16), int(rest[2], 16), float(rest[3])
        # one row, K = 128, the code at every column
        qw = np.full((1, 64), code | (code << 4), dtype=np.uint8)
        w = O.q4g128_dequant_f32(qw, np.array([[sb]], np.uint16), np.array([[mb]], np.uint16))
        assert w.dtype == np.float32 and w.shape == (1, 128)
        assert _same(w, np.full((1, 128), exp)), (code, hex(sb), hex(mb), w[0, 0], exp)


def pin_q4_group_boundary(O):
    qw = np.full((1, 128), 0x11, dtype=np.uint8)  # K = 256, all codes 1
    sc = np.array([[0x3C00, 0x4000]], dtype=np.uint16)
    mn = np.array([[0x0000, 0x3800]], dtype=np.uint16)
    w = O.q4g128_dequant_f32(qw, sc, mn)
    for k0, k1, val in _lines("q4g128_group_boundary.txt"):
        assert np.all(w[0, int(k0): int(k1) + 1] == float(val)), (k0, k1, val)


def _rand_fp16_bits(rng, shape, subnormal_frac=0.2):
    """finite fp16 bit patterns: mostly normal in a realistic range, some subnormal."""
    vals = rng.uniform(-4, 4, size=shape).astype(np.float16).view(np.uint16)
    sub = rng.integers(1, 1024, size=shape, dtype=np.uint16) | (rng.integers(0, 2, size=shape, dtype=np.uint16) << 15)
    pick = rng.random(shape) < subnormal_frac
    return np.where(pick, sub, vals).astype(np.uint16)


def pin_q4_dequant_exact(O):
    """Exact rational dequant on random tiny matrices, every element bitwise."""
    rng = np.random.default_rng(5)
    for (n, k) in ((3, 128), (2, 384)):
        qw = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        sc = _rand_fp16_bits(rng, (n, k // 128))
        mn = _rand_fp16_bits(rng, (n, k // 128))
        w = O.q4g128_dequant_f32(qw, sc, mn)
        sv = sc.view(np.float16).astype(np.float64)
        mv = mn.view(np.float16).astype(np.float64)
        for r in range(n):
            for j in range(k // 2):
                b = int(qw[r, j])
                for kk, code in ((2 * j, b % 16), (2 * j + 1, b // 16)):
                    g = kk // 128
                    exact = Fraction(code) * Fraction(sv[r, g]) + Fraction(mv[r, g])
                    assert _same([w[r, kk]], [_f32_of_fraction(exact)]), (r, kk)


def pin_nvfp4_dequant_exact(O):
    """All 16 codes x all 256 scale bytes x several global scales, exact
    rational product rounded once to fp32, bitwise."""
    codes = np.arange(16, dtype=np.uint8)
    scales = np.arange(256, dtype=np.uint8)
    # one row per scale byte; each row holds the 16 codes (one group)
    qw = np.tile(synth.pack_nibbles(torch.from_numpy(codes.astype(np.int64)).view(1, 16)).numpy(), (256, 1))
    sc = scales.reshape(256, 1)
    e2 = [float(v) for _, v in _lines("e2m1_table.txt")]
    sref = torch.from_numpy(scales.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for G in (1.0, float(np.float32(1.0 / 3.0)), float(np.float32(0.02 / 2688.0)), float(np.float32(1.0 + 2 ** -23)), 2.0 ** -20):
        w = O.nvfp4g16_dequant_f32(qw, sc, G)
        assert w.dtype == np.float32 and w.shape == (256, 16)
        for si in range(256):
            for c in range(16):
                if math.isnan(sref[si]):
                    assert np.isnan(w[si, c]), (si, c)
                    continue
                exact = Fraction(e2[c]) * Fraction(sref[si]) * Fraction(G)
                if exact == 0:  # +0 and -0 are both accepted for a zero weight
                    assert w[si, c] == 0, (si, c)
                else:
                    ref = _f32_of_fraction(exact)
                    assert _same([w[si, c]], [ref]), (G, hex(si), c, w[si, c], ref)


def pin_bf16_dequant(O):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    assert _same(O.bf16_dequant_f32(bits), ref)


# ----------------------------------------------------------------------------
# the product
# ----------------------------------------------------------------------------
def _bf16_bits_from_float(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _exact_gemv(xv, wv):
    """sum over k of Fraction products; xv [M][K], wv [N][K] of python floats."""
    M, N = len(xv), len(wv)
    return [[sum((Fraction(xv[m][k]) * Fraction(wv[n][k]) for k in range(len(xv[m]))), Fraction(0)) for n in range(N)] for m in range(M)]


def _check_vs_exact(y, xv, wv):
    ex = _exact_gemv(xv, wv)
    for m in range(len(xv)):
        for n in range(len(wv)):
            mag = sum(abs(Fraction(xv[m][k]) * Fraction(wv[n][k])) for k in range(len(xv[m])))
            err = abs(Fraction(float(y[m, n])) - ex[m][n])
            assert err <= Fraction(1, 10 ** 12) * mag + Fraction(1, 10 ** 300), (m, n, float(err), float(mag))


def pin_q4_gemv_exact(O):
    rng = np.random.default_rng(7)
    for (M, N, K) in ((1, 5, 128), (3, 8, 256), (2, 3, 128)):
        qw = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        sc = rng.uniform(1e-3, 2e-2, size=(N, K // 128)).astype(np.float16).view(np.uint16)
        mn = (-7.5 * sc.view(np.float16).astype(np.float64)).astype(np.float16).view(np.uint16)
        x = _bf16_bits_from_float(rng.standard_normal((M, K)))
        y = O.q4g128_gemv(x, qw, sc, mn)
        assert y.shape == (M, N) and y.dtype == np.float64
        # independent dequant: numpy float16 decode + Fraction arithmetic
        sv = sc.view(np.float16).astype(np.float64)
        mv = mn.view(np.float16).astype(np.float64)
        wv = []
        for n in range(N):
            row = []
            for kk in range(K):
                b = int(qw[n, kk // 2])
                code = b % 16 if kk % 2 == 0 else b // 16
                row.append(float(_f32_of_fraction(Fraction(code) * Fraction(sv[n, kk // 128]) + Fraction(mv[n, kk // 128]))))
            wv.append(row)
        xv = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy().tolist()
        _check_vs_exact(y, xv, wv)


def pin_nvfp4_gemv_exact(O):
    rng = np.random.default_rng(8)
    e2 = [float(v) for _, v in _lines("e2m1_table.txt")]
    for (M, N, K) in ((1, 4, 32), (3, 6, 64)):
        qw = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        sc = rng.integers(0x08, 0x7E, size=(N, K // 16), dtype=np.uint8)
        G = float(np.float32(rng.uniform(1e-6, 1e-3)))
        x = _bf16_bits_from_float(rng.standard_normal((M, K)))
        y = O.nvfp4g16_gemv(x, qw, sc, G)
        sv = torch.from_numpy(sc.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        wv = []
        for n in range(N):
            row = []
            for kk in range(K):
                b = int(qw[n, kk // 2])
                code = b % 16 if kk % 2 == 0 else b // 16
                row.append(float(_f32_of_fraction(Fraction(e2[code]) * Fraction(sv[n, kk // 16]) * Fraction(G))))
            wv.append(row)
        xv = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy().tolist()
        _check_vs_exact(y, xv, wv)


def pin_bf16_gemv_library(O):
    """bf16 weights: the oracle must equal torch's float64 matmul of the
    converted tensors (a library routine), up to fp64 summation order."""
    g = torch.Generator().manual_seed(3)
    for (M, N, K) in ((1, 7, 64), (4, 33, 256)):
        x = torch.randn(M, K, generator=g).to(torch.bfloat16)
        w = (torch.randn(N, K, generator=g) * 0.02).to(torch.bfloat16)
        y = O.bf16_gemv(synth.bits16(x), synth.bits16(w))
        ref = (x.double() @ w.double().T).numpy()
        mag = (x.double().abs() @ w.double().abs().T).numpy()
        assert y.shape == (M, N)
        assert np.all(np.abs(y - ref) <= 1e-13 * mag + 1e-300)


def pin_integer_weights(O):
    """scale = 1, min = 0: w is the code itself; with small-integer x the
    product is an integer computed exactly with Python ints."""
    rng = np.random.default_rng(9)
    M, N, K = 2, 6, 256
    qw = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    sc = np.full((N, K // 128), 0x3C00, np.uint16)
    mn = np.zeros((N, K // 128), np.uint16)
    xi = rng.integers(-8, 9, size=(M, K))
    x = _bf16_bits_from_float(xi.astype(np.float32))
    y = O.q4g128_gemv(x, qw, sc, mn)
    for m in range(M):
        for n in range(N):
            acc = 0
            for j in range(K // 2):
                b = int(qw[n, j])
                acc += (b & 15) * int(xi[m, 2 * j]) + (b >> 4) * int(xi[m, 2 * j + 1])
            assert y[m, n] == acc, (m, n, y[m, n], acc)


# ----------------------------------------------------------------------------
# fused neighbours: BF16 rounding from fp64, the SiLU-gated activation, the
# product plus a residual
# ----------------------------------------------------------------------------
def _rn_bf16_exact(fr: Fraction) -> int:
    """Exact rational -> BF16 bits by integer arithmetic, ties to even."""
    sign = 0x8000 if fr < 0 else 0
    a = abs(fr)
    if a == 0:
        return sign
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    n = a / Fraction(2) ** (e - 7)
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    if fl == 256:
        fl, e = 128, e + 1
    if e > 127:
        return sign | 0x7F80
    if fl >= 128:
        return sign | ((e + 127) << 7) | (fl - 128)
    return sign | fl                       # subnormal (e == -126)


def pin_bf16_round_library(O):
    """fp32-representable inputs: RN_bf16 from fp64 must equal torch's fp32 ->
    bf16 conversion (round to nearest even), ties and subnormals included."""
    rng = np.random.default_rng(11)
    v = (rng.standard_normal(60000) * np.exp2(rng.integers(-140, 120, 60000))).astype(np.float32)
    b = rng.integers(0, 0x7F7F, 20000).astype(np.uint32) << 16          # BF16 values ...
    ties = (b | 0x8000).view(np.float32)                                 # ... plus half a step: exact ties
    near = (b | 0x7FFF).view(np.float32)                                 # just below the next tie
    v = np.concatenate([v, ties, -ties, near, np.float32([0.0, -0.0, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134])])
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.bf16_round_bits(v.astype(np.float64))
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} mismatches, first {v[bad[0]]!r}: {got[bad[0]]:#06x} vs {want[bad[0]]:#06x}"


def pin_bf16_round_exact(O):
    """fp64 inputs between fp32 values: one rounding of the exact value (no
    detour through fp32), checked by integer arithmetic."""
    vals = []
    for base in (1.0, 1.5, -3.25, 2.0 ** -120, 2.0 ** -130, 6.0e37):
        step = 2.0 ** (math.floor(math.log2(abs(base))) - 7) if abs(base) >= 2.0 ** -126 else 2.0 ** -133
        for frac in (0.5, 1.5):
            for eps in (2.0 ** -30, -2.0 ** -30, 2.0 ** -45):
                vals.append(base + (frac + eps) * step * (1 if base > 0 else -1))
    got = O.bf16_round_bits(np.array(vals))
    want = [_rn_bf16_exact(Fraction(v)) for v in vals]
    assert [int(g) for g in got] == want, [(v, int(g), w) for v, g, w in zip(vals, got, want) if int(g) != w]


def pin_silu_mul_decimal(O):
    """h = RN_bf16(silu(g) * u) against an independent evaluation: e^-g by the
    decimal module at 60 digits, exact rational product, integer rounding."""
    import decimal
    ctx = decimal.Context(prec=60)
    rng = np.random.default_rng(12)
    mags = np.exp2(rng.uniform(-12, 5.5, 1500))
    g = np.concatenate([mags, -mags, [0.0, 1.0, -1.0, 20.0, -20.0, 88.0, -88.0]])
    g_bits = torch.from_numpy(g.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for u in (1.0, -0.75, 3.5, 2.0 ** -20, 1000.0):
        u_bits = np.full(g_bits.shape, torch.tensor(u, dtype=torch.bfloat16).view(torch.int16).item() & 0xFFFF, np.uint16)
        got = O.silu_mul_bf16(g_bits, u_bits)
        for gb, hb in zip(g_bits, got):
            gv = Fraction(float(torch.tensor(int(gb), dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()))
            e = ctx.exp(ctx.minus(decimal.Decimal(gv.numerator) / decimal.Decimal(gv.denominator)))
            s = gv / (1 + Fraction(e))
            want = _rn_bf16_exact(s * Fraction(u))
            if s == 0:   # an exact zero carries the IEEE sign of the product g * u
                want = 0x8000 if (gb >> 15) ^ (u < 0) else 0
            assert int(hb) == want, (float(gv), u, hex(int(hb)), hex(want))


def pin_residual_exact(O):
    """Integer weights, activations and residual: x . W^T + r is an exact
    integer, which the oracle must return exactly, per element."""
    rng = np.random.default_rng(13)
    M, N, K = 3, 5, 256
    codes = rng.integers(0, 16, size=(N, K))
    x = rng.integers(-8, 9, size=(M, K))
    r = rng.integers(-64, 65, size=(M, N))
    w32 = codes.astype(np.float32)
    xb = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    rb = torch.from_numpy(r.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.gemv_residual_f64(xb, w32, rb)
    want = [[sum(int(x[m, k]) * int(codes[n, k]) for k in range(K)) + int(r[m, n]) for n in range(N)] for m in range(M)]
    assert got.shape == (M, N) and np.array_equal(got, np.array(want, dtype=np.float64))


# ----------------------------------------------------------------------------
# sampling from the head
# ----------------------------------------------------------------------------
def _bf16_bits_of(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def pin_sample_decimal(O):
    """Top-k, softmax and the inverse-CDF draw against an independent
    evaluation: Python's sorted() for the order, e^x from the decimal module
    at 50 digits for the probabilities, an explicit walk for the draw."""
    import decimal
    ctx = decimal.Context(prec=50)
    rng = np.random.default_rng(21)
    V, k, T = 97, 30, 0.8
    for trial in range(12):
        vals = np.round(rng.standard_normal(V) * 3, 1)
        vals[rng.integers(0, V, 6)] = vals[0]                  # ties
        bits = _bf16_bits_of(vals.tolist())
        lv = [float(torch.tensor(int(b), dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()) for b in bits]
        order = sorted(range(V), key=lambda i: (-lv[i], i))[:k]
        dT = decimal.Decimal(repr(T))
        z = [ctx.divide(decimal.Decimal(repr(lv[i])), dT) for i in order]
        e = [ctx.exp(ctx.subtract(zi, z[0])) for zi in z]
        s = sum(e, decimal.Decimal(0))
        p = [float(ctx.divide(ei, s)) for ei in e]
        us = rng.uniform(0, 1, 5)
        tok, idx, prob = O.sample_topk(np.stack([bits] * 5), T, k, us)
        for r in range(5):
            assert list(idx[r]) == order, (trial, r)
            assert np.allclose(prob[r], p, rtol=1e-12, atol=0)
            acc, want = decimal.Decimal(0), order[-1]
            for i, ei in zip(order, e):
                acc += ctx.divide(ei, s)
                if acc > decimal.Decimal(repr(float(us[r]))):
                    want = i
                    break
            assert tok[r] == want, (trial, r)


def pin_sample_invariants(O):
    """k = 1 is the argmax (lowest index among equals) with probability 1;
    adding a constant to every logit (exactly) changes nothing; the draw is
    monotone in u; u on an exact CDF boundary is not exceeded by it."""
    rng = np.random.default_rng(22)
    vals = rng.integers(-40, 40, size=(3, 200)).astype(np.float64)
    vals[1, 17] = vals[1, 150] = vals[1].max() + 3                # a tie at the top
    bits = _bf16_bits_of(vals.tolist())
    tok, idx, prob = O.sample_topk(bits, 0.8, 1, [0.3, 0.9, 0.999])
    assert list(tok) == [int(np.argmax(vals[m])) for m in range(3)] and tok[1] == 17
    assert np.all(prob == 1.0)
    shifted = _bf16_bits_of((vals + 64).tolist())
    for u in ([0.1, 0.5, 0.9], [0.0, 0.7, 0.99]):
        a = O.sample_topk(bits, 0.8, 30, u)
        b = O.sample_topk(shifted, 0.8, 30, u)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and np.allclose(a[2], b[2], rtol=1e-12)
    us = np.linspace(0, 0.999, 40)
    toks, idxs, _ = O.sample_topk(np.stack([bits[0]] * 40), 0.8, 30, us)
    pos = [list(idxs[i]).index(toks[i]) for i in range(40)]
    assert pos == sorted(pos) and pos[0] == 0
    # two equal logits well above the rest: p = 1/2 each (to 1e-30); u = 1/2 is not exceeded by
    # the first cumulative probability, so the second is drawn
    two = _bf16_bits_of([[0.0] * 10 + [100.0, 100.0]])
    assert O.sample_topk(two, 1.0, 2, [0.5])[0][0] == 11
    assert O.sample_topk(two, 1.0, 2, [0.49])[0][0] == 10


ALL_PINS = [
    pin_nibble_hand,
    pin_nibble_roundtrip,
    pin_fp16,
    pin_bf16,
    pin_e4m3,
    pin_e2m1,
    pin_q4_dequant_hand,
    pin_q4_group_boundary,
    pin_q4_dequant_exact,
    pin_nvfp4_dequant_exact,
    pin_bf16_dequant,
    pin_q4_gemv_exact,
    pin_nvfp4_gemv_exact,
    pin_bf16_gemv_library,
    pin_integer_weights,
    pin_bf16_round_library,
    pin_bf16_round_exact,
    pin_silu_mul_decimal,
    pin_residual_exact,
    pin_sample_decimal,
    pin_sample_invariants,
]
