"""GPU parity of the fused int4 calls (q4g128_gemv_fused through the C ABI).

  * With neither `up` nor `residual` a fused call must equal the plain kernel
    it runs on (streaming for M <= 4, tiled otherwise) bit for bit.
  * The activation prologue h = RN_bf16(silu(g) * u) is read out exactly:
    rows whose g and u are nonzero in one column j only, and weight row j
    one-hot at column j (code 1, scale 1, min 0), give y[m, j] = h[m, j] with
    every sum in the kernel exact.  h may differ from the oracle by one BF16
    step only where the exact value lies within the fp32 evaluation error of a
    rounding boundary.
  * Otherwise against the oracle within gpu_util.check_gemv's tolerance:
    y = RN_bf16(h . W^T) and y = RN_bf16(x . W^T + r); an in-place residual
    (residual is y) equals the out-of-place result bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_gemv, gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_weight_only_q4g128_amd as m
    return m


def mat(N, K, seed):
    qw, sc, mn = synth.q4_matrix(N, K, seed)
    w32 = oracle.q4g128_dequant_f32(qw.numpy(), synth.bits16(sc), synth.bits16(mn))
    return (gpu(qw), gpu(sc), gpu(mn)), w32


def bits(t):
    return synth.bits16(t)


def workspace(q4, items):
    n = q4.q4g128_fused_workspace_bytes(items)
    return torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda") if n else None


def task(dev, x, **kw):
    d = dict(x=x, qweight=dev[0], scale=dev[1], min=dev[2])
    d.update(kw)
    return d


@pytest.mark.parametrize("M,N,K", [(1, 2048, 2048), (3, 300, 8192), (4, 1000, 4096), (5, 2048, 2048), (48, 2048, 8192),
                                   (64, 130, 2048)])
def test_fused_without_extras_equals_plain_kernel(q4, M, N, K):
    dev, _ = mat(N, K, ("fz-plain", M, N, K))
    x = gpu(synth.x_bf16(M, K, ("fz-plain-x", M)))
    v = q4.VARIANT_STREAM if M <= 4 else q4.VARIANT_TILED
    ref = q4.q4g128_gemv(x, *dev, variant=v)
    (y,) = q4.q4g128_gemv_fused([task(dev, x)])
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


def _tie_distance(v):
    """relative distance of |v| to the nearest BF16 rounding boundary"""
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    step = np.ldexp(1.0, np.maximum(ex.astype(np.int64) - 1, -126) - 7)
    n = a / step
    return np.abs(n - np.floor(n) - 0.5) * step / np.where(a > 0, a, 1.0)


@pytest.mark.parametrize("M,split", [(4, False), (48, False), (48, True), (64, False)])
def test_fused_silu_readout_bitwise(q4, M, split):
    K = N = 2048
    # weight row j one-hot at column j: codes 1 on the diagonal, scale 1, min 0
    codes = torch.zeros(N, K, dtype=torch.int64)
    codes[torch.arange(N), torch.arange(N)] = 1
    qw = gpu(synth.pack_nibbles(codes))
    sc = gpu(torch.ones(N, K // 128, dtype=torch.float16))
    mn = gpu(torch.zeros(N, K // 128, dtype=torch.float16))
    g_all, u_all, h_all = [], [], []
    rng = np.random.default_rng(M + 100 * split)
    for rep in range(24):
        cols = rng.choice(K, size=M, replace=False)
        gv = (rng.standard_normal(M) * np.exp2(rng.integers(-3, 5, M))).astype(np.float32)
        uv = (rng.standard_normal(M) * np.exp2(rng.integers(-3, 4, M))).astype(np.float32)
        if rep == 0:
            gv[:4] = [0.0, -0.0, 30.0, -30.0]
        g = torch.zeros(M, K, dtype=torch.bfloat16)
        u = torch.zeros(M, K, dtype=torch.bfloat16)
        g[torch.arange(M), torch.from_numpy(cols)] = torch.from_numpy(gv).to(torch.bfloat16)
        u[torch.arange(M), torch.from_numpy(cols)] = torch.from_numpy(uv).to(torch.bfloat16)
        items = [dict(x=gpu(g), up=gpu(u), qweight=qw, scale=sc, min=mn)]
        (y,) = q4.q4g128_gemv_fused(items, workspace=workspace(q4, items) if split else None)
        yb = bits(y)
        gb, ub = bits(g), bits(u)
        for m in range(M):
            j = cols[m]
            g_all.append(gb[m, j]); u_all.append(ub[m, j]); h_all.append(yb[m, j])
    g_all, u_all, h_all = np.array(g_all, np.uint16), np.array(u_all, np.uint16), np.array(h_all, np.uint16)
    want = oracle.silu_mul_bf16(g_all, u_all)
    # the read-out is a sum, which turns a -0 term into +0: compare zeros unsigned
    h_all = np.where(h_all == 0x8000, np.uint16(0), h_all)
    want = np.where(want == 0x8000, np.uint16(0), want)
    bad = np.flatnonzero(h_all != want)
    gv64, uv64 = oracle.bf16_value(g_all), oracle.bf16_value(u_all)
    exact = gv64 / (1.0 + np.exp(-gv64)) * uv64
    for i in bad:
        # only a value within the fp32 evaluation error of a rounding boundary
        # may round the other way, and then by one step
        assert _tie_distance(exact[i]) < 2.0 ** -20, (float(gv64[i]), float(uv64[i]), hex(h_all[i]), hex(want[i]))
        assert abs(int(h_all[i]) - int(want[i])) == 1
    assert bad.size <= 2, bad.size


@pytest.mark.parametrize("M,N,K,split", [(1, 2048, 8192, False), (3, 1000, 8192, False), (4, 2048, 2048, False),
                                         (5, 2048, 8192, False), (16, 2048, 8192, True), (48, 2048, 8192, True),
                                         (48, 37, 2048, False), (64, 2048, 4096, True)])
def test_fused_silu_against_oracle(q4, M, N, K, split):
    dev, w32 = mat(N, K, ("fz-silu", N, K))
    g = synth.x_bf16(M, K, ("fz-g", M, K))
    u = synth.x_bf16(M, K, ("fz-u", M, K))
    items = [task(dev, gpu(g), up=gpu(u))]
    (y,) = q4.q4g128_gemv_fused(items, workspace=workspace(q4, items) if split else None)
    hb = oracle.silu_mul_bf16(bits(g), bits(u))
    check_gemv(y, oracle.gemv_f64(hb, w32), w32, hb, f"fused silu M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K,split", [(1, 2048, 2048, False), (2, 2048, 8192, False), (4, 777, 2048, False),
                                         (5, 2048, 2048, False), (48, 2048, 2048, True), (48, 2048, 8192, True),
                                         (64, 300, 2048, False)])
def test_fused_residual_against_oracle_and_in_place(q4, M, N, K, split):
    dev, w32 = mat(N, K, ("fz-res", N, K))
    x = synth.x_bf16(M, K, ("fz-res-x", M, K))
    r = synth.x_bf16(M, N, ("fz-res-r", M, N))
    items = [task(dev, gpu(x), residual=gpu(r))]
    ws = workspace(q4, items) if split else None
    (y,) = q4.q4g128_gemv_fused(items, workspace=ws)
    xb = bits(x)
    check_gemv(y, oracle.gemv_residual_f64(xb, w32, bits(r)), w32, xb, f"fused residual M={M} N={N} K={K}")
    # in place: the residual buffer is the output
    yr = gpu(r)
    (y2,) = q4.q4g128_gemv_fused([task(dev, gpu(x), residual=yr, out=yr)], workspace=ws)
    assert y2.data_ptr() == yr.data_ptr()
    assert torch.equal(yr.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("M", [5, 48, 64])
def test_fused_tiled_prologue_pass_equals_loader_path(q4, M):
    """A full workspace forms h in a separate pass; one sized for the split-K
    part only keeps the loader-side activation (tiled kernel).  At M = 64 both
    run the tiled kernel with the same plan and h: bit for bit equal.  For
    5 <= M <= 48 the pass feeds the skinny kernel instead: both against the
    oracle."""
    dev, _ = mat(2048, 8192, ("fz-pass",))
    g, u = gpu(synth.x_bf16(M, 8192, ("fz-pass-g", M))), gpu(synth.x_bf16(M, 8192, ("fz-pass-u", M)))
    r = gpu(synth.x_bf16(M, 2048, ("fz-pass-r", M)))
    items = [task(dev, g, up=u, residual=r)]
    full = q4.q4g128_fused_workspace_bytes(items)
    # the same call without up: just the split-K part of the same plan
    split_only = q4.q4g128_fused_workspace_bytes([task(dev, g, residual=r)])
    assert full > split_only
    (y_pass,) = q4.q4g128_gemv_fused(items, workspace=torch.zeros(full, dtype=torch.uint8, device="cuda"))
    ws2 = torch.zeros(max(split_only, 256), dtype=torch.uint8, device="cuda")
    (y_load,) = q4.q4g128_gemv_fused(items, workspace=ws2)
    if M > 48:
        assert torch.equal(y_pass.view(torch.int16), y_load.view(torch.int16))
    else:
        w32 = oracle.q4g128_dequant_f32(dev[0].cpu().numpy(), bits(dev[1]), bits(dev[2]))
        hb = oracle.silu_mul_bf16(bits(g), bits(u))
        want = oracle.gemv_residual_f64(hb, w32, bits(r))
        check_gemv(y_pass, want, w32, hb, f"fused pass (skinny) M={M}")
        check_gemv(y_load, want, w32, hb, f"fused loader (tiled) M={M}")


@pytest.mark.parametrize("M,split", [(1, False), (48, True)])
def test_fused_layer_mlp_tail(q4, M, split):
    """down(silu(gate) * up) + residual, and o(attn) + residual, in ONE call
    (two tasks with different extras)."""
    dd, wd = mat(2048, 8192, ("fz-down",))
    do, wo = mat(2048, 2048, ("fz-o",))
    g, u = synth.x_bf16(M, 8192, ("fz-tail-g", M)), synth.x_bf16(M, 8192, ("fz-tail-u", M))
    a = synth.x_bf16(M, 2048, ("fz-tail-a", M))
    r1, r2 = synth.x_bf16(M, 2048, ("fz-tail-r1", M)), synth.x_bf16(M, 2048, ("fz-tail-r2", M))
    items = [task(dd, gpu(g), up=gpu(u), residual=gpu(r1)), task(do, gpu(a), residual=gpu(r2))]
    y_down, y_o = q4.q4g128_gemv_fused(items, workspace=workspace(q4, items) if split else None)
    hb = oracle.silu_mul_bf16(bits(g), bits(u))
    check_gemv(y_down, oracle.gemv_residual_f64(hb, wd, bits(r1)), wd, hb, f"fused down M={M}")
    ab = bits(a)
    check_gemv(y_o, oracle.gemv_residual_f64(ab, wo, bits(r2)), wo, ab, f"fused o M={M}")


def test_fused_rejects_and_odd_shapes(q4):
    dev, _ = mat(64, 2048, ("fz-bad",))
    x = gpu(synth.x_bf16(1, 2048, "fz-bad-x"))
    U = gpu(synth.x_bf16(1, 2048, "fz-bad-u"))
    with pytest.raises(q4.Q4GemvError):      # task 1 writes over task 0's up activations
        q4.q4g128_gemv_fused([task(dev, x, up=U), task(dev, x, out=U[:, :64])])
    big = torch.zeros(1, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(q4.Q4GemvError):      # a residual partly overlapping its output
        q4.q4g128_gemv_fused([task(dev, x, residual=big[:, 1:65], out=big[:, :64])])
    # K = 1152 at M = 1 is not a streaming shape: the tiled kernel runs it
    d2, _ = mat(64, 1152, ("fz-odd",))
    x2 = gpu(synth.x_bf16(1, 1152, "fz-odd-x"))
    (y,) = q4.q4g128_gemv_fused([task(d2, x2)])
    assert torch.equal(y.view(torch.int16), q4.q4g128_gemv(x2, *d2, variant=q4.VARIANT_TILED).view(torch.int16))


@pytest.mark.parametrize("M", [16, 48])
def test_fused_unsplit_then_split_call_share_workspace(q4, M):
    """A gated call whose tiled plan needs no K split (K = 512) keeps its h
    past the arrival counters; a split call on the same workspace afterwards
    must then find the counters at zero and produce the oracle's result."""
    d1, w1 = mat(256, 512, ("fz-ws-a", M))
    g, u = synth.x_bf16(M, 512, ("fz-ws-g", M)), synth.x_bf16(M, 512, ("fz-ws-u", M))
    items = [task(d1, gpu(g), up=gpu(u))]
    d2, w2 = mat(2048, 8192, ("fz-ws-b",))
    x2 = synth.x_bf16(M, 8192, ("fz-ws-x2", M))
    grouped = [(gpu(x2), *d2, None)]
    n = max(q4.q4g128_fused_workspace_bytes(items), q4.q4g128_workspace_bytes(grouped))
    assert q4.q4g128_workspace_bytes(grouped) > 0, "the second call must plan a K split"
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    (y1,) = q4.q4g128_gemv_fused(items, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[:64 * 1024].count_nonzero()) == 0, "counter region written by the fused call"
    (y2,) = q4.q4g128_gemv_grouped(grouped, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[:64 * 1024].count_nonzero()) == 0
    hb = oracle.silu_mul_bf16(bits(g), bits(u))
    check_gemv(y1, oracle.gemv_f64(hb, w1), w1, hb, f"fused K=512 M={M}")
    xb = bits(x2)
    check_gemv(y2, oracle.gemv_f64(xb, w2), w2, xb, f"split after fused M={M}")
