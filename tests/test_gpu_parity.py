"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bitwise: device dequantization, and one-hot activations (a single nonzero
term makes every variant's sum exact, so y must equal RN_bf16(w32)).
Within tolerance (gpu_util.check_gemv): every workload of the pages' shapes
and the edge shapes.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_gemv, gpu, onehot_x, rn_bf16_bits, same_bits_f32, x_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_weight_only_q4g128_amd as m
    return m


VARIANTS = [1, 2]  # dot2, mfma
VNAME = {0: "auto", 1: "dot2", 2: "mfma", 3: "stream", 4: "tiled", 6: "skinny"}
FMT = {"q4": 0, "nv": 1, "bf": 2}


def vlist(q4, fmt, M, K):
    """auto, dot2 and mfma, plus the streaming, tiled and skinny kernels where they accept (M, K)."""
    return ([0, 1, 2] + ([3] if q4.variant_name(FMT[fmt], 3, M, 1, K) == "stream" else [])
            + ([4] if q4.variant_name(FMT[fmt], 4, M, 1, K) == "tiled" else [])
            + ([6] if q4.variant_name(FMT[fmt], 6, M, 1, K) == "skinny" else []))


# ----------------------------------------------------------------------------
# dequantization, bitwise
# ----------------------------------------------------------------------------
def test_q4_dequant_bitwise(q4):
    rng = np.random.default_rng(1)
    for (N, K) in ((256, 512), (33, 1536), (4, 128)):
        qw = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        sc = rng.uniform(-3, 3, size=(N, K // 128)).astype(np.float16).view(np.uint16)
        mn = rng.uniform(-3, 3, size=(N, K // 128)).astype(np.float16).view(np.uint16)
        # sprinkle subnormal scales/mins and the fp16 extremes
        sc.flat[::7] = rng.integers(1, 1024, size=sc.flat[::7].shape)
        mn.flat[::5] = 0x8001
        sc.flat[1] = 0x7BFF
        ref = oracle.q4g128_dequant_f32(qw, sc, mn)
        w = q4.q4g128_dequant_f32(gpu(torch.from_numpy(qw)), gpu(torch.from_numpy(sc.view(np.int16))).view(torch.float16),
                                  gpu(torch.from_numpy(mn.view(np.int16))).view(torch.float16))
        assert same_bits_f32(w.cpu().numpy(), ref), (N, K)


def test_nvfp4_dequant_bitwise_exhaustive(q4):
    # 256 rows = every e4m3 scale byte; each row holds all 16 codes twice
    codes = torch.arange(16).repeat(2).view(1, 32)
    qw = synth.pack_nibbles(codes).repeat(256, 1)
    sc = torch.stack([torch.arange(256, dtype=torch.int64), torch.arange(256, dtype=torch.int64)], 1).to(torch.uint8)
    for G in (1.0, float(np.float32(1 / 3)), float(np.float32(0.02 / 2688)), 2.0 ** -20, float(np.float32(1 + 2 ** -23))):
        ref = oracle.nvfp4g16_dequant_f32(qw.numpy(), sc.numpy(), G)
        w = q4.nvfp4g16_dequant_f32(gpu(qw), gpu(sc), G)
        assert same_bits_f32(w.cpu().numpy(), ref), G


# ----------------------------------------------------------------------------
# one-hot activations: bitwise for every variant
# ----------------------------------------------------------------------------
def _onehot_ks(K, M, seed):
    rng = np.random.default_rng(seed)
    ks = list(rng.choice(K, size=M, replace=False)) if M <= K else list(rng.integers(0, K, size=M))
    ks[0] = 0
    if M > 1:
        ks[-1] = K - 1
    return [int(k) for k in ks]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("M", [1, 3, 8, 16, 48])
def test_q4_onehot_bitwise(q4, variant, M):
    N, K = 200, 1024
    qw, sc, mn = synth.q4_matrix(N, K, ("onehot", M))
    w32 = oracle.q4g128_dequant_f32(qw.numpy(), synth.bits16(sc), synth.bits16(mn))
    ks = _onehot_ks(K, M, M)
    x = onehot_x(K, ks)
    y = q4.q4g128_gemv(gpu(x), gpu(qw), gpu(sc), gpu(mn), variant=variant)
    got = y.cpu().float().numpy()
    exp = torch.from_numpy(rn_bf16_bits(w32[:, ks].T).view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(got, exp), (VNAME[variant], M, np.argwhere(got != exp)[:4])


@pytest.mark.parametrize("variant", VARIANTS + [4])
@pytest.mark.parametrize("M", [1, 4, 17, 48])
def test_nvfp4_onehot_bitwise(q4, variant, M):
    N, K = 150, 512
    qw, s8, G = synth.nvfp4_matrix(N, K, ("onehot-nv", M))
    w32 = oracle.nvfp4g16_dequant_f32(qw.numpy(), s8.numpy(), G)
    ks = _onehot_ks(K, M, 100 + M)
    x = onehot_x(K, ks)
    y = q4.nvfp4g16_gemv(gpu(x), gpu(qw), gpu(s8), G, variant=variant)
    got = synth.bits16(y.cpu())
    exp = rn_bf16_bits(w32[:, ks].T)
    # +0 / -0 are equal values
    gotv = torch.from_numpy(got.view(np.int16)).view(torch.bfloat16).float().numpy()
    expv = torch.from_numpy(exp.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(gotv, expv), (VNAME[variant], M)


@pytest.mark.parametrize("variant", VARIANTS + [4])
@pytest.mark.parametrize("M", [1, 5, 32, 64])
def test_bf16_onehot_bitwise(q4, variant, M):
    N, K = 77, 256
    w = synth.bf16_matrix(N, K, ("onehot-bf", M))
    ks = _onehot_ks(K, M, 200 + M)
    y = q4.bf16_gemv(gpu(onehot_x(K, ks)), gpu(w), variant=variant)
    assert np.array_equal(y.cpu().float().numpy(), w[:, ks].T.float().numpy()), (VNAME[variant], M)


def _runs_on(fmt, variant, name, cases):
    """The (K, M) cases a forced variant accepts (the host-side choice, no GPU
    needed); the others are shapes that variant does not take -- the automatic
    choice runs them on another kernel, tested elsewhere (e.g. M = 4, K = 8192
    in test_q4_down_shape_M4_auto)."""
    try:
        import bit_weight_only_q4g128_amd as m
    except ImportError:
        return cases
    return [(K, M) for K, M in cases if m.variant_name(fmt, variant, M, 1, K) == name]


# the streaming kernel takes rows of 1, 2 or 4 KB only, and activations within its LDS budget
@pytest.mark.parametrize("K,M", _runs_on(0, 3, "stream", [(K, M) for K in (2048, 4096, 8192) for M in (1, 2, 3, 4)]))
def test_q4_onehot_bitwise_stream(q4, K, M):
    N = 37   # rows past N in the last workgroup
    qw, sc, mn = synth.q4_matrix(N, K, ("onehot-st", K, M))
    w32 = oracle.q4g128_dequant_f32(qw.numpy(), synth.bits16(sc), synth.bits16(mn))
    ks = _onehot_ks(K, M, 300 + M)
    y = q4.q4g128_gemv(gpu(onehot_x(K, ks)), gpu(qw), gpu(sc), gpu(mn), variant=3)
    got = y.cpu().float().numpy()
    exp = torch.from_numpy(rn_bf16_bits(w32[:, ks].T).view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(got, exp), (K, M, np.argwhere(got != exp)[:4])


@pytest.mark.parametrize("K,M", _runs_on(1, 3, "stream", [(K, M) for K in (2048, 8192) for M in (1, 3, 4)]))
def test_nvfp4_onehot_bitwise_stream(q4, K, M):
    N = 21
    qw, s8, G = synth.nvfp4_matrix(N, K, ("onehot-nv-st", K, M))
    w32 = oracle.nvfp4g16_dequant_f32(qw.numpy(), s8.numpy(), G)
    ks = _onehot_ks(K, M, 400 + M)
    y = q4.nvfp4g16_gemv(gpu(onehot_x(K, ks)), gpu(qw), gpu(s8), G, variant=3)
    gotv = torch.from_numpy(synth.bits16(y.cpu()).view(np.int16)).view(torch.bfloat16).float().numpy()
    expv = torch.from_numpy(rn_bf16_bits(w32[:, ks].T).view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(gotv, expv), (K, M)


@pytest.mark.parametrize("K", [512, 2048, 4096, 8192])
@pytest.mark.parametrize("M", [1, 3])
def test_bf16_onehot_bitwise_stream(q4, K, M):
    N = 70
    w = synth.bf16_matrix(N, K, ("onehot-bf-st", K, M))
    ks = _onehot_ks(K, M, 500 + M)
    y = q4.bf16_gemv(gpu(onehot_x(K, ks)), gpu(w), variant=3)
    assert np.array_equal(y.cpu().float().numpy(), w[:, ks].T.float().numpy()), (K, M)


# the tiled matrix-core kernel (int4): ragged row blocks, groups past a round
# of eight, every batch-tile count
@pytest.mark.parametrize("K,M", _runs_on(0, 4, "tiled", [(K, M) for K in (128, 1152, 2048, 8192) for M in (5, 16, 17, 33, 48, 64)]))
def test_q4_onehot_bitwise_tiled(q4, K, M):
    N = 70
    qw, sc, mn = synth.q4_matrix(N, K, ("onehot-tl", K, M))
    w32 = oracle.q4g128_dequant_f32(qw.numpy(), synth.bits16(sc), synth.bits16(mn))
    ks = _onehot_ks(K, M, 600 + M)
    y = q4.q4g128_gemv(gpu(onehot_x(K, ks)), gpu(qw), gpu(sc), gpu(mn), variant=4)
    got = y.cpu().float().numpy()
    exp = torch.from_numpy(rn_bf16_bits(w32[:, ks].T).view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(got, exp), (K, M, np.argwhere(got != exp)[:4])


# ----------------------------------------------------------------------------
# the pages' shapes, within tolerance
# ----------------------------------------------------------------------------
def test_config0_single_matrix(q4):
    d = synth.config0(0)
    w32 = oracle.q4g128_dequant_f32(d["qweight"].numpy(), synth.bits16(d["scale"]), synth.bits16(d["min"]))
    ref = oracle.gemv_f64(synth.bits16(d["x"]), w32)
    for v in (0, 1, 2):
        y = q4.q4g128_gemv(gpu(d["x"]), gpu(d["qweight"]), gpu(d["scale"]), gpu(d["min"]), variant=v)
        check_gemv(y, ref, w32, synth.bits16(d["x"]), f"config0 {VNAME[v]}")


_LAYER_CACHE = {}


def _layer_q4():
    if "q4" not in _LAYER_CACHE:
        lay = synth.q4_layer(("layer", 0))
        w32 = {n: oracle.q4g128_dequant_f32(t[0].numpy(), synth.bits16(t[1]), synth.bits16(t[2])) for n, t in lay.items()}
        _LAYER_CACHE["q4"] = (lay, w32)
    return _LAYER_CACHE["q4"]


@pytest.mark.parametrize("M", [1, 3, 16, 48])
@pytest.mark.parametrize("proj", synth.LAYER_ORDER)
def test_q4_layer(q4, proj, M):
    lay, w32 = _layer_q4()
    qw, sc, mn = lay[proj]
    N, K = synth.LAYER_SHAPES[proj]
    x = synth.x_bf16(M, K, ("layer-x", proj))
    ref = oracle.gemv_f64(x_bits(x), w32[proj])
    for v in vlist(q4, "q4", M, K):
        y = q4.q4g128_gemv(gpu(x), gpu(qw), gpu(sc), gpu(mn), variant=v)
        check_gemv(y, ref, w32[proj], x_bits(x), f"{proj} M={M} {VNAME[v]}")


@pytest.mark.parametrize("M", [1, 48])
@pytest.mark.parametrize("proj", synth.LAYER_ORDER)
def test_nvfp4_layer(q4, proj, M):
    N, K = synth.LAYER_SHAPES[proj]
    x = synth.x_bf16(M, K, ("nv-x", proj))
    if proj in synth.NVFP4_BF16_PROJ:
        w = synth.bf16_matrix(N, K, ("nv-layer", proj))
        w32 = oracle.bf16_dequant_f32(synth.bits16(w))
        ref = oracle.gemv_f64(x_bits(x), w32)
        for v in vlist(q4, "bf", M, K):
            check_gemv(q4.bf16_gemv(gpu(x), gpu(w), variant=v), ref, w32, x_bits(x), f"bf16 {proj} M={M} {VNAME[v]}")
        return
    qw, s8, G = synth.nvfp4_matrix(N, K, ("nv-layer", proj))
    w32 = oracle.nvfp4g16_dequant_f32(qw.numpy(), s8.numpy(), G)
    ref = oracle.gemv_f64(x_bits(x), w32)
    for v in vlist(q4, "nv", M, K):
        y = q4.nvfp4g16_gemv(gpu(x), gpu(qw), gpu(s8), G, variant=v)
        check_gemv(y, ref, w32, x_bits(x), f"nvfp4 {proj} M={M} {VNAME[v]}")


@pytest.mark.parametrize("M", [1, 48])
@pytest.mark.parametrize("shape", [synth.HEAD_FULL, synth.HEAD_SLICE])
def test_bf16_head(q4, shape, M):
    N, K = shape
    w = synth.bf16_matrix(N, K, ("head", N))
    x = synth.x_bf16(M, K, ("head-x", N))
    w32 = oracle.bf16_dequant_f32(synth.bits16(w))
    ref = oracle.gemv_f64(x_bits(x), w32)
    for v in vlist(q4, "bf", M, K):
        check_gemv(q4.bf16_gemv(gpu(x), gpu(w), variant=v), ref, w32, x_bits(x), f"head {N} M={M} {VNAME[v]}")


# ----------------------------------------------------------------------------
# edge shapes: ragged N, short/odd K, every batch size
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("N,K", [(1, 128), (7, 256), (17, 384), (65, 1536), (130, 4096), (33, 11008), (5, 16384),
                                 (1, 2048), (23, 8192), (4097, 2048)])
def test_q4_edge_shapes(q4, N, K):
    qw, sc, mn = synth.q4_matrix(N, K, ("edge", N, K))
    w32 = oracle.q4g128_dequant_f32(qw.numpy(), synth.bits16(sc), synth.bits16(mn))
    for M in (1, 2, 5, 8, 9, 16, 33, 64):
        x = synth.x_bf16(M, K, ("edge-x", N, K, M))
        ref = oracle.gemv_f64(x_bits(x), w32)
        for v in vlist(q4, "q4", M, K):
            y = q4.q4g128_gemv(gpu(x), gpu(qw), gpu(sc), gpu(mn), variant=v)
            check_gemv(y, ref, w32, x_bits(x), f"edge N={N} K={K} M={M} {VNAME[v]}")


@pytest.mark.parametrize("N,K", [(1, 32), (9, 96), (31, 160), (66, 2080), (3, 2048), (45, 4096), (18, 8192)])
def test_nvfp4_edge_shapes(q4, N, K):
    qw, s8, G = synth.nvfp4_matrix(N, K, ("edge-nv", N, K))
    w32 = oracle.nvfp4g16_dequant_f32(qw.numpy(), s8.numpy(), G)
    for M in (1, 3, 8, 12, 40):
        x = synth.x_bf16(M, K, ("edge-nv-x", N, K, M))
        ref = oracle.gemv_f64(x_bits(x), w32)
        for v in vlist(q4, "nv", M, K):
            check_gemv(q4.nvfp4g16_gemv(gpu(x), gpu(qw), gpu(s8), G, variant=v), ref, w32, x_bits(x),
                       f"nv edge N={N} K={K} M={M} {VNAME[v]}")


@pytest.mark.parametrize("N,K", [(1, 8), (3, 24), (19, 136), (40, 1000), (129, 2056), (1, 512), (21, 1024), (257, 2048),
                                 (37, 4096), (65, 8192), (2, 8192)])
def test_bf16_edge_shapes(q4, N, K):
    w = synth.bf16_matrix(N, K, ("edge-bf", N, K))
    w32 = oracle.bf16_dequant_f32(synth.bits16(w))
    for M in (1, 2, 7, 16, 20):
        x = synth.x_bf16(M, K, ("edge-bf-x", N, K, M))
        ref = oracle.gemv_f64(x_bits(x), w32)
        for v in vlist(q4, "bf", M, K):
            check_gemv(q4.bf16_gemv(gpu(x), gpu(w), variant=v), ref, w32, x_bits(x), f"bf edge N={N} K={K} M={M} {VNAME[v]}")


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("variant", VARIANTS + [3])
def test_q4_power_of_two_scaling_is_bitwise(q4, variant):
    N, K, M = 300, 2048, 4
    qw, sc, mn = (gpu(t) for t in synth.q4_matrix(N, K, ("pow2",)))
    x = synth.x_bf16(M, K, ("pow2-x",))
    y1 = q4.q4g128_gemv(gpu(x), qw, sc, mn, variant=variant)
    y2 = q4.q4g128_gemv(gpu((x.float() * 8).to(torch.bfloat16)), qw, sc, mn, variant=variant)
    assert torch.equal((y1.float() * 8).to(torch.bfloat16), y2)


@pytest.mark.parametrize("variant", VARIANTS + [6])
def test_q4_row_permutation_is_bitwise(q4, variant):
    N, K, M = 256, 2048, 16
    qw, sc, mn = synth.q4_matrix(N, K, ("perm",))
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(0))
    x = gpu(synth.x_bf16(M, K, ("perm-x",)))
    y1 = q4.q4g128_gemv(x, gpu(qw), gpu(sc), gpu(mn), variant=variant)
    y2 = q4.q4g128_gemv(x, gpu(qw[perm]), gpu(sc[perm]), gpu(mn[perm]), variant=variant)
    assert torch.equal(y1[:, perm.cuda()], y2)


@pytest.mark.parametrize("variant", VARIANTS + [3])
def test_q4_repeat_runs_are_bitwise_identical(q4, variant):
    N, K, M = 2048, 8192, 3
    qw, sc, mn = (gpu(t) for t in synth.q4_matrix(N, K, ("det",)))
    x = gpu(synth.x_bf16(M, K, ("det-x",)))
    y0 = q4.q4g128_gemv(x, qw, sc, mn, variant=variant)
    for _ in range(20):
        assert torch.equal(q4.q4g128_gemv(x, qw, sc, mn, variant=variant), y0)


def test_q4_batched_equals_stacked_singles(q4):
    N, K, M = 512, 2048, 6
    qw, sc, mn = synth.q4_matrix(N, K, ("stack",))
    w32 = oracle.q4g128_dequant_f32(qw.numpy(), synth.bits16(sc), synth.bits16(mn))
    x = synth.x_bf16(M, K, ("stack-x",))
    yb = q4.q4g128_gemv(gpu(x), gpu(qw), gpu(sc), gpu(mn))
    ys = torch.cat([q4.q4g128_gemv(gpu(x[m:m + 1]), gpu(qw), gpu(sc), gpu(mn)) for m in range(M)], 0)
    ref = oracle.gemv_f64(x_bits(x), w32)
    check_gemv(yb, ref, w32, x_bits(x), "batched")
    check_gemv(ys, ref, w32, x_bits(x), "singles")


@pytest.mark.parametrize("variant", [0, 1, 2])
def test_output_fully_overwritten(q4, variant):
    N, K, M = 100, 512, 20
    qw, sc, mn = (gpu(t) for t in synth.q4_matrix(N, K, ("poison",)))
    x = gpu(synth.x_bf16(M, K, ("poison-x",)))
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    q4.q4g128_gemv(x, qw, sc, mn, out=out, variant=variant)
    assert not torch.isnan(out).any()


def test_stream_ordering_on_side_stream(q4):
    N, K, M = 1024, 2048, 2
    qw, sc, mn = (gpu(t) for t in synth.q4_matrix(N, K, ("stream",)))
    x = gpu(synth.x_bf16(M, K, ("stream-x",)))
    ref = q4.q4g128_gemv(x, qw, sc, mn)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = q4.q4g128_gemv(x, qw, sc, mn)
    s.synchronize()
    assert torch.equal(y, ref)


# ----------------------------------------------------------------------------
# grouped launches: same kernels, several GEMVs per launch
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M", [1, 3, 8, 48])
def test_q4_grouped_equals_single_calls(q4, M):
    lay, w32 = _layer_q4()
    xin = gpu(synth.x_bf16(M, 2048, ("grp-xin", M)))
    xat = gpu(synth.x_bf16(M, 2048, ("grp-xat", M)))
    xff = gpu(synth.x_bf16(M, 8192, ("grp-xff", M)))
    xs = {"q": xin, "k": xin, "v": xin, "gate": xin, "up": xin, "o": xat, "down": xff}
    dev = {p: tuple(gpu(t) for t in lay[p]) for p in synth.LAYER_ORDER}
    for stage in (("q", "k", "v", "gate", "up"), ("o", "down")):
        for v in [0, 1, 2] + ([3] if M <= 4 else [4, 6]):
            try:
                outs = q4.q4g128_gemv_grouped([(xs[p], *dev[p], None) for p in stage], variant=v)
            except q4.Q4GemvError:
                # a forced variant that some task of the stage cannot run
                assert v != 0
                continue
            for p, y in zip(stage, outs):
                xb = x_bits(xs[p].cpu())
                check_gemv(y, oracle.gemv_f64(xb, w32[p]), w32[p], xb, f"grouped {p} M={M} {VNAME[v]}")
                if v != 0:
                    # the same kernel: grouping must not change a single bit
                    ys = q4.q4g128_gemv(xs[p], *dev[p], variant=v)
                    assert torch.equal(y, ys), (p, M, VNAME[v])


@pytest.mark.parametrize("M", [16, 48])
def test_q4_grouped_split_k_workspace(q4, M):
    # o and down alone are 64 row blocks, so with a workspace K is split over
    # workgroups; the result must match the oracle and the unsplit call within
    # tolerance and repeat bitwise on the same workspace without re-zeroing it
    lay, w32 = _layer_q4()
    xat = gpu(synth.x_bf16(M, 2048, ("split-xat", M)))
    xff = gpu(synth.x_bf16(M, 8192, ("split-xff", M)))
    items = [(xat, *(gpu(t) for t in lay["o"]), None), (xff, *(gpu(t) for t in lay["down"]), None)]
    nbytes = q4.q4g128_workspace_bytes(items)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    outs = q4.q4g128_gemv_grouped(items, workspace=ws)
    plain = q4.q4g128_gemv_grouped(items)
    for p, x, y, yp in zip(("o", "down"), (xat, xff), outs, plain):
        xb = x_bits(x.cpu())
        ref = oracle.gemv_f64(xb, w32[p])
        check_gemv(y, ref, w32[p], xb, f"split {p} M={M}")
        check_gemv(yp, ref, w32[p], xb, f"unsplit {p} M={M}")
    for _ in range(5):
        again = q4.q4g128_gemv_grouped(items, workspace=ws)
        assert all(torch.equal(a, b) for a, b in zip(again, outs))


def test_q4_workspace_shared_by_different_calls(q4):
    # the two grouped calls of a decode layer (q/k/v/gate/up, then o/down) at
    # M = 48 take turns on one workspace sized for the larger; every call must
    # find its counters at zero, so each round matches the oracle and the
    # first round bitwise
    M = 48
    lay, w32 = _layer_q4()
    xin = gpu(synth.x_bf16(M, 2048, ("wsh-xin",)))
    xat = gpu(synth.x_bf16(M, 2048, ("wsh-xat",)))
    xff = gpu(synth.x_bf16(M, 8192, ("wsh-xff",)))
    xs = {"q": xin, "k": xin, "v": xin, "gate": xin, "up": xin, "o": xat, "down": xff}
    dev = {p: tuple(gpu(t) for t in lay[p]) for p in synth.LAYER_ORDER}
    stages = [("q", "k", "v", "gate", "up"), ("o", "down")]
    items = [[(xs[p], *dev[p], None) for p in st] for st in stages]
    need = max(q4.q4g128_workspace_bytes(it) for it in items)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    first = None
    for rnd in range(3):
        outs = [q4.q4g128_gemv_grouped(it, workspace=ws) for it in items]
        if first is None:
            first = outs
            for st, ys in zip(stages, outs):
                for p, y in zip(st, ys):
                    xb = x_bits(xs[p].cpu())
                    check_gemv(y, oracle.gemv_f64(xb, w32[p]), w32[p], xb, f"shared ws {p}")
        else:
            for ys, y0 in zip(outs, first):
                assert all(torch.equal(a, b) for a, b in zip(ys, y0)), rnd


def test_q4_split_k_small_tasks(q4):
    # a few short matrices: split into as many slices as K allows, one-hot exact
    N, K, M = 100, 2048, 20
    qw, sc, mn = synth.q4_matrix(N, K, ("split-small",))
    w32 = oracle.q4g128_dequant_f32(qw.numpy(), synth.bits16(sc), synth.bits16(mn))
    ks = _onehot_ks(K, M, 77)
    items = [(gpu(onehot_x(K, ks)), gpu(qw), gpu(sc), gpu(mn), None)]
    # a workspace larger than any plan needs: the tiled kernel splits K, the
    # skinny kernel's plan for this shape stays unsplit
    ws = torch.zeros(8 << 20, dtype=torch.uint8, device="cuda")
    exp = torch.from_numpy(rn_bf16_bits(w32[:, ks].T).view(np.int16)).view(torch.bfloat16).float().numpy()
    for v in (4, 6, 0):
        y = q4.q4g128_gemv_grouped(items, variant=v, workspace=ws)[0]
        assert np.array_equal(y.cpu().float().numpy(), exp), VNAME[v]


@pytest.mark.parametrize("M", [5, 20, 48, 64])
def test_q4_split_k_mixed_tasks_onehot_and_random(q4, M):
    # with a workspace, a launch whose row blocks cannot fill the GPU splits
    # the tasks whose K allows it over several workgroups and runs the others
    # (K = 128, 384, 1152) whole; one-hot activations must come out exact and
    # random ones within tolerance, and repeat bitwise on the reused workspace
    shapes = [(70, 128), (200, 1152), (130, 2048), (64, 4096), (1000, 384)]
    mats = [synth.q4_matrix(N, K, ("sk", N, K)) for N, K in shapes]
    w32s = [oracle.q4g128_dequant_f32(m[0].numpy(), synth.bits16(m[1]), synth.bits16(m[2])) for m in mats]
    for kind in ("onehot", "random"):
        xs, kss = [], []
        for i, (N, K) in enumerate(shapes):
            if kind == "onehot":
                ks = _onehot_ks(K, M, 900 + 7 * i + M)
                kss.append(ks)
                xs.append(gpu(onehot_x(K, ks)))
            else:
                xs.append(gpu(synth.x_bf16(M, K, ("sk-x", K, M))))
        items = [(x, *(gpu(t) for t in m), None) for x, m in zip(xs, mats)]
        nbytes = q4.q4g128_workspace_bytes(items)
        assert nbytes > 0
        ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        outs = q4.q4g128_gemv_grouped(items, variant=4, workspace=ws)
        for i, ((N, K), w32, x, y) in enumerate(zip(shapes, w32s, xs, outs)):
            if kind == "onehot":
                exp = torch.from_numpy(rn_bf16_bits(w32[:, kss[i]].T).view(np.int16)).view(torch.bfloat16).float().numpy()
                got = y.cpu().float().numpy()
                assert np.array_equal(got, exp), (N, K, M, np.argwhere(got != exp)[:4])
            else:
                xb = x_bits(x.cpu())
                check_gemv(y, oracle.gemv_f64(xb, w32), w32, xb, f"stream-k N={N} K={K} M={M}")
        for _ in range(3):
            again = q4.q4g128_gemv_grouped(items, variant=4, workspace=ws)
            assert all(torch.equal(a, b) for a, b in zip(again, outs))


def _nv_mats(shapes, tag):
    mats = [synth.nvfp4_matrix(N, K, (tag, N, K)) for N, K in shapes]
    return mats, [oracle.nvfp4g16_dequant_f32(m[0].numpy(), m[1].numpy(), m[2]) for m in mats]


def _bf_mats(shapes, tag):
    mats = [synth.bf16_matrix(N, K, (tag, N, K)) for N, K in shapes]
    return mats, [oracle.bf16_dequant_f32(synth.bits16(w)) for w in mats]


@pytest.mark.parametrize("fmt", ["nv", "bf"])
@pytest.mark.parametrize("M", [5, 20, 48, 64])
def test_nvfp4_bf16_grouped_split_k_onehot_and_random(q4, fmt, M):
    # the tiled kernel for NVFP4 and BF16 weights through the grouped calls:
    # with a workspace the launch splits K; ragged N (rows past N in the last
    # block), one-hot activations exact, random ones within tolerance, and
    # repeats bitwise on the reused workspace
    shapes = [(70, 512), (200, 1152), (130, 2048), (64, 4096), (33, 8192)]
    mats, w32s = (_nv_mats if fmt == "nv" else _bf_mats)(shapes, "g" + fmt)
    grouped = q4.nvfp4g16_gemv_grouped if fmt == "nv" else q4.bf16_gemv_grouped
    wsbytes = q4.nvfp4g16_workspace_bytes if fmt == "nv" else q4.bf16_workspace_bytes
    for kind in ("onehot", "random"):
        xs, kss = [], []
        for i, (N, K) in enumerate(shapes):
            if kind == "onehot":
                ks = _onehot_ks(K, M, 1300 + 7 * i + M)
                kss.append(ks)
                xs.append(gpu(onehot_x(K, ks)))
            else:
                xs.append(gpu(synth.x_bf16(M, K, ("g-x", fmt, K, M))))
        if fmt == "nv":
            items = [(x, gpu(m[0]), gpu(m[1]), m[2], None) for x, m in zip(xs, mats)]
        else:
            items = [(x, gpu(m), None) for x, m in zip(xs, mats)]
        nbytes = wsbytes(items)
        assert nbytes > 0
        ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        outs = grouped(items, variant=4, workspace=ws)
        unsplit = grouped(items, variant=4)
        for i, ((N, K), w32, x, y, y1) in enumerate(zip(shapes, w32s, xs, outs, unsplit)):
            if kind == "onehot":
                exp = torch.from_numpy(rn_bf16_bits(w32[:, kss[i]].T).view(np.int16)).view(torch.bfloat16).float().numpy()
                for got in (y.cpu().float().numpy(), y1.cpu().float().numpy()):
                    assert np.array_equal(got, exp), (fmt, N, K, M, np.argwhere(got != exp)[:4])
            else:
                xb = x_bits(x.cpu())
                ref = oracle.gemv_f64(xb, w32)
                check_gemv(y, ref, w32, xb, f"{fmt} grouped split N={N} K={K} M={M}")
                check_gemv(y1, ref, w32, xb, f"{fmt} grouped unsplit N={N} K={K} M={M}")
        for _ in range(3):
            again = grouped(items, variant=4, workspace=ws)
            assert all(torch.equal(a, b) for a, b in zip(again, outs))


@pytest.mark.parametrize("fmt", ["nv", "bf"])
@pytest.mark.parametrize("M", [1, 3, 48])
def test_nvfp4_bf16_grouped_equals_single_calls(q4, fmt, M):
    # the automatic choice for a group (streaming kernel at M <= 4, tiled
    # kernel above) against one call per task with the same kernel
    shapes = [(512, 2048), (2048, 2048), (2049, 2048)]
    mats, _ = (_nv_mats if fmt == "nv" else _bf_mats)(shapes, "ge" + fmt)
    x = gpu(synth.x_bf16(M, 2048, ("ge-x", fmt, M)))
    if fmt == "nv":
        outs = q4.nvfp4g16_gemv_grouped([(x, gpu(m[0]), gpu(m[1]), m[2], None) for m in mats])
        singles = [q4.nvfp4g16_gemv(x, gpu(m[0]), gpu(m[1]), m[2]) for m in mats]
    else:
        outs = q4.bf16_gemv_grouped([(x, gpu(m), None) for m in mats])
        singles = [q4.bf16_gemv(x, gpu(m)) for m in mats]
    for a, b in zip(outs, singles):
        assert torch.equal(a, b)


def test_q4_grouped_mixed_k(q4):
    # K = 16384 needs two chunks per lane, K = 384 one: the call splits into two launches
    shapes = [(64, 16384), (100, 384), (7, 2048)]
    mats = [synth.q4_matrix(N, K, ("mix", N, K)) for N, K in shapes]
    xs = [gpu(synth.x_bf16(2, K, ("mix-x", K))) for _, K in shapes]
    outs = q4.q4g128_gemv_grouped([(x, *(gpu(t) for t in m), None) for x, m in zip(xs, mats)])
    for (N, K), m, x, y in zip(shapes, mats, xs, outs):
        w32 = oracle.q4g128_dequant_f32(m[0].numpy(), synth.bits16(m[1]), synth.bits16(m[2]))
        xb = x_bits(x.cpu())
        check_gemv(y, oracle.gemv_f64(xb, w32), w32, xb, f"mixed N={N} K={K}")


@pytest.mark.parametrize("variant", [1, 2, 3])
def test_q4_scale_arrays_only_2byte_aligned(q4, variant):
    # scale/min as views one element into larger buffers: 2-byte but not
    # 16-byte aligned, so the kernels must not assume wider alignment
    N, K, M = 300, 2048, 2
    qw, sc, mn = synth.q4_matrix(N, K, ("misaligned",))
    big_s = torch.zeros(sc.numel() + 8, dtype=torch.float16, device="cuda")
    big_m = torch.zeros(mn.numel() + 8, dtype=torch.float16, device="cuda")
    big_s[1:1 + sc.numel()] = sc.flatten().cuda()
    big_m[1:1 + mn.numel()] = mn.flatten().cuda()
    s_view = big_s[1:1 + sc.numel()].view(N, K // 128)
    m_view = big_m[1:1 + mn.numel()].view(N, K // 128)
    assert s_view.data_ptr() % 16 != 0
    x = gpu(synth.x_bf16(M, K, ("misaligned-x",)))
    y = q4.q4g128_gemv(x, gpu(qw), s_view, m_view, variant=variant)
    y_ref = q4.q4g128_gemv(x, gpu(qw), gpu(sc), gpu(mn), variant=variant)
    assert torch.equal(y, y_ref)
    w32 = oracle.q4g128_dequant_f32(qw.numpy(), synth.bits16(sc), synth.bits16(mn))
    xb = x_bits(x.cpu())
    check_gemv(y, oracle.gemv_f64(xb, w32), w32, xb, "misaligned scales")


def test_launch_timing_hook(q4):
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    a, z = ctypes.c_void_p(), ctypes.c_void_p()
    assert hip.hipEventCreate(ctypes.byref(a)) == 0 and hip.hipEventCreate(ctypes.byref(z)) == 0
    qw, sc, mn = (gpu(t) for t in synth.q4_matrix(8192, 2048, ("timing",)))
    x = gpu(synth.x_bf16(1, 2048, ("timing-x",)))
    q4.q4g128_gemv(x, qw, sc, mn)
    torch.cuda.synchronize()
    assert q4.lib.q4gemv_time_next_launch(a, z) == 0
    y = q4.q4g128_gemv(x, qw, sc, mn)
    y2 = q4.q4g128_gemv(x, qw, sc, mn)     # not timed: the events are used once
    torch.cuda.synchronize()
    assert hip.hipEventSynchronize(z) == 0
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), a, z) == 0
    assert 0.0 < ms.value < 5.0, ms.value
    assert torch.equal(y, y2)
    hip.hipEventDestroy(a)
    hip.hipEventDestroy(z)


def test_stream_read_touches_every_byte(q4):
    # the diagnostic read XORs every 32-bit word of its buffers into the sink
    g = torch.Generator().manual_seed(5)
    bufs = [torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, generator=g) for n in (4096 * 7 + 12, 4, 100000)]
    dev = [b.cuda() for b in bufs]
    words = q4.stream_read_sink_words(dev)
    assert words > 0
    sink = torch.full((words,), -1, dtype=torch.int32, device="cuda")
    q4.stream_read(dev, sink)
    expect = 0
    for b in bufs:
        expect ^= int(np.bitwise_xor.reduce(b.numpy().view(np.uint32)))
    got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
    assert got == expect


# the down projection's shape at M = 4, where the automatic choice is the
# packed-dot kernel (the streaming kernel's LDS budget excludes K = 8192 at
# this M): one-hot bitwise and the synthetic layer weights within tolerance
def test_q4_down_shape_M4_auto(q4):
    N, K, M = 2048, 8192, 4
    name = q4.variant_name(0, 0, M, N, K)
    lay, w32 = _layer_q4()
    qw, sc, mn = lay["down"]
    ks = _onehot_ks(K, M, 700)
    y = q4.q4g128_gemv(gpu(onehot_x(K, ks)), gpu(qw), gpu(sc), gpu(mn))
    got = y.cpu().float().numpy()
    exp = torch.from_numpy(rn_bf16_bits(w32["down"][:, ks].T).view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(got, exp), (name, np.argwhere(got != exp)[:4])
    x = synth.x_bf16(M, K, ("down-M4-x",))
    ref = oracle.gemv_f64(x_bits(x), w32["down"])
    check_gemv(q4.q4g128_gemv(gpu(x), gpu(qw), gpu(sc), gpu(mn)), ref, w32["down"], x_bits(x), f"down M=4 {name}")


# the skinny matrix-core kernel (int4, 5 <= M <= 48): the planner's row-block
# height follows the row count (N about 4000, 8000, 12000, 20000 at K = 2048
# give 16, 32, 48 and 80 rows per workgroup), N ragged against every block and
# not a multiple of 4 (element stores); one-hot bitwise, random activations
# within tolerance
@pytest.mark.parametrize("N", [4001, 8003, 12005, 20007])
@pytest.mark.parametrize("M", [5, 16, 33, 48])
def test_q4_skinny_row_blocks(q4, N, M):
    K = 2048
    assert q4.variant_name(0, 0, M, N, K) == "skinny"
    qw, sc, mn = synth.q4_matrix(N, K, ("skinny-rb", N))
    w32 = _w32_cached(("skinny-rb", N), qw, sc, mn)
    dev = (gpu(qw), gpu(sc), gpu(mn))
    ks = _onehot_ks(K, M, 800 + M)
    y = q4.q4g128_gemv(gpu(onehot_x(K, ks)), *dev, variant=6)
    got = y.cpu().float().numpy()
    exp = torch.from_numpy(rn_bf16_bits(w32[:, ks].T).view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(got, exp), (N, M, np.argwhere(got != exp)[:4])
    x = synth.x_bf16(M, K, ("skinny-rb-x", N, M))
    check_gemv(q4.q4g128_gemv(gpu(x), *dev, variant=6), oracle.gemv_f64(x_bits(x), w32), w32, x_bits(x), f"skinny N={N} M={M}")


_W32 = {}


def _w32_cached(key, qw, sc, mn):
    if key not in _W32:
        _W32[key] = oracle.q4g128_dequant_f32(qw.numpy(), synth.bits16(sc), synth.bits16(mn))
    return _W32[key]


# K beyond one workgroup slice (16 groups) needs a workspace: slices of 8 or
# 16 groups, a ragged last slice (K = 11008: 86 groups), and K below a slice
@pytest.mark.parametrize("K", [128, 1152, 4096, 8192, 11008, 16384])
@pytest.mark.parametrize("M", [5, 17, 48])
def test_q4_skinny_split_k_onehot_and_random(q4, K, M):
    N = 300
    qw, sc, mn = synth.q4_matrix(N, K, ("skinny-sk", K))
    w32 = _w32_cached(("skinny-sk", K), qw, sc, mn)
    dev = (gpu(qw), gpu(sc), gpu(mn))
    ks = _onehot_ks(K, M, 850 + M)
    for kind in ("onehot", "random"):
        x = gpu(onehot_x(K, ks)) if kind == "onehot" else gpu(synth.x_bf16(M, K, ("skinny-sk-x", K, M)))
        items = [(x, *dev, None)]
        need = q4.q4g128_workspace_bytes(items)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
        (y,) = q4.q4g128_gemv_grouped(items, variant=6, workspace=ws)
        (y2,) = q4.q4g128_gemv_grouped(items, variant=6, workspace=ws)
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "repeat on the reused workspace"
        assert int(ws[:64 * 1024].count_nonzero()) == 0
        if kind == "onehot":
            exp = torch.from_numpy(rn_bf16_bits(w32[:, ks].T).view(np.int16)).view(torch.bfloat16).float().numpy()
            got = y.cpu().float().numpy()
            assert np.array_equal(got, exp), (K, M, np.argwhere(got != exp)[:4])
        else:
            xb = x_bits(x.cpu())
            check_gemv(y, oracle.gemv_f64(xb, w32), w32, xb, f"skinny split K={K} M={M}")


# the skinny kernel on NVFP4 and BF16 weights (forced, and through the
# grouped calls with a workspace): slices of 16 NVFP4 groups or 8 BF16 groups
# of 128 columns, a ragged last slice (K = 1152: 9 groups), a slice of fewer
# groups than waves (K = 640) and below one group's worth of waves (K = 128),
# N ragged against every row block; one-hot bitwise (the e2m1 x e4m3 weights
# are exact in BF16 and G is applied once), random within tolerance, repeats
# bitwise on the reused workspace, which is left with its counters at zero
@pytest.mark.parametrize("fmt", ["nv", "bf"])
@pytest.mark.parametrize("K", [128, 640, 1152, 2048, 8192])
@pytest.mark.parametrize("M", [5, 17, 48])
def test_nvfp4_bf16_skinny_onehot_and_random(q4, fmt, K, M):
    N = 300
    mats, w32s = (_nv_mats if fmt == "nv" else _bf_mats)([(N, K)], "sk" + fmt)
    m, w32 = mats[0], w32s[0]
    grouped = q4.nvfp4g16_gemv_grouped if fmt == "nv" else q4.bf16_gemv_grouped
    wsbytes = q4.nvfp4g16_workspace_bytes if fmt == "nv" else q4.bf16_workspace_bytes
    ks = _onehot_ks(K, M, 870 + M)
    for kind in ("onehot", "random"):
        x = gpu(onehot_x(K, ks)) if kind == "onehot" else gpu(synth.x_bf16(M, K, ("sk-x", fmt, K, M)))
        items = [(x, gpu(m[0]), gpu(m[1]), m[2], None)] if fmt == "nv" else [(x, gpu(m), None)]
        ws = torch.zeros(max(wsbytes(items), 256), dtype=torch.uint8, device="cuda")
        (y,) = grouped(items, variant=6, workspace=ws)
        (y2,) = grouped(items, variant=6, workspace=ws)
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "repeat on the reused workspace"
        assert int(ws[:64 * 1024].count_nonzero()) == 0
        if kind == "onehot":
            exp = torch.from_numpy(rn_bf16_bits(w32[:, ks].T).view(np.int16)).view(torch.bfloat16).float().numpy()
            got = y.cpu().float().numpy()
            assert np.array_equal(got, exp), (fmt, K, M, np.argwhere(got != exp)[:4])
        else:
            xb = x_bits(x.cpu())
            check_gemv(y, oracle.gemv_f64(xb, w32), w32, xb, f"{fmt} skinny K={K} M={M}")


@pytest.mark.parametrize("fmt", ["nv", "bf"])
@pytest.mark.parametrize("N", [16385, 4001])
def test_nvfp4_bf16_skinny_row_blocks_unsplit(q4, fmt, N):
    # one slice per row block (no workspace): tall matrices whose row count is
    # ragged against the planner's blocks
    K, M = 1024, 48
    mats, w32s = (_nv_mats if fmt == "nv" else _bf_mats)([(N, K)], "skr" + fmt)
    m, w32 = mats[0], w32s[0]
    x = synth.x_bf16(M, K, ("skr-x", fmt, N))
    if fmt == "nv":
        y = q4.nvfp4g16_gemv(gpu(x), gpu(m[0]), gpu(m[1]), m[2], variant=6)
    else:
        y = q4.bf16_gemv(gpu(x), gpu(m), variant=6)
    check_gemv(y, oracle.gemv_f64(x_bits(x), w32), w32, x_bits(x), f"{fmt} skinny unsplit N={N}")


@pytest.mark.parametrize("shift", [1, 2, 3])
def test_nvfp4_skinny_scales_any_alignment(q4, shift):
    """The e4m3 scale array has no alignment rule: the skinny kernel reads a
    row's group scales as 4-byte pieces, which must come out right from any
    byte address (the array placed 1, 2, 3 bytes into a larger buffer)."""
    N, K, M = 300, 2048, 48
    qw, s8, G = synth.nvfp4_matrix(N, K, ("nv-mis",))
    w32 = oracle.nvfp4g16_dequant_f32(qw.numpy(), s8.numpy(), G)
    buf = torch.zeros(N * (K // 16) + 8, dtype=torch.uint8, device="cuda")
    s8v = buf[shift:shift + N * (K // 16)].view(N, K // 16)
    s8v.copy_(gpu(s8))
    x = synth.x_bf16(M, K, ("nv-mis-x", shift))
    y = q4.nvfp4g16_gemv(gpu(x), gpu(qw), s8v, G, variant=6)
    check_gemv(y, oracle.gemv_f64(x_bits(x), w32), w32, x_bits(x), f"nvfp4 skinny scales +{shift}")


def test_q4_skinny_misaligned_params_and_output(q4):
    """Group parameters only 2-byte aligned (element loads instead of 16-byte
    pieces) and an output that is only 2-byte aligned (element stores)."""
    N, K, M = 260, 2048, 48
    qw, sc, mn = synth.q4_matrix(N, K, ("skinny-mis",))
    w32 = oracle.q4g128_dequant_f32(qw.numpy(), synth.bits16(sc), synth.bits16(mn))
    scb = torch.zeros(N * (K // 128) + 1, dtype=torch.float16, device="cuda")
    mnb = torch.zeros_like(scb)
    scv, mnv = scb[1:].view(N, K // 128), mnb[1:].view(N, K // 128)
    scv.copy_(gpu(sc)); mnv.copy_(gpu(mn))
    yb = torch.full((M * N + 1,), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = yb[1:].view(M, N)
    x = synth.x_bf16(M, K, ("skinny-mis-x",))
    q4.q4g128_gemv(gpu(x), gpu(qw), scv, mnv, out=y, variant=6)
    check_gemv(y, oracle.gemv_f64(x_bits(x), w32), w32, x_bits(x), "skinny misaligned")
    assert bool(torch.isnan(yb[0].float()))
