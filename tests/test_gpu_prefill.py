"""GPU parity of the int4 prefill GEMM (q4g128_gemm through the C ABI).

Both kernels (VARIANT_GEMM: 128-row batch tiles over all of K; VARIANT_TILED:
the tiled decode kernel over batch chunks) against the oracle within
gpu_util.check_gemv's tolerance for M from 65 to 517 (ragged last tiles and
chunks), ragged N and the layer's K values; at the largest prefill shape the
benchmark times (M = 4096, N = 8192, K = 2048) on sampled batch rows.  The
chunked kernel bitwise against the tiled decode kernel run on each batch chunk
alone (the same arithmetic per chunk); M <= 64 under the automatic choice
equals the GEMV's.
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


@pytest.mark.parametrize("variant", ["GEMM", "TILED", "AUTO"])
@pytest.mark.parametrize("M,N,K", [(65, 2048, 2048), (128, 300, 2048), (200, 2048, 8192), (517, 1000, 4096), (257, 130, 8192),
                                   (300, 515, 2048)])
def test_gemm_against_oracle(q4, M, N, K, variant):
    dev, w32 = mat(N, K, ("gemm", N, K))
    x = synth.x_bf16(M, K, ("gemm-x", M, K))
    y = q4.q4g128_gemm(gpu(x), *dev, variant=getattr(q4, "VARIANT_" + variant))
    xb = synth.bits16(x)
    check_gemv(y, oracle.gemv_f64(xb, w32), w32, xb, f"gemm {variant} M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N", [(1, 2048), (17, 64), (64, 2048)])
def test_gemm_kernel_small_batches(q4, M, N):
    """The large-tile kernel at batch sizes the automatic choice gives to the GEMV."""
    dev, w32 = mat(N, 2048, ("gemm-smallb", N))
    x = synth.x_bf16(M, 2048, ("gemm-smallb-x", M))
    y = q4.q4g128_gemm(gpu(x), *dev, variant=q4.VARIANT_GEMM)
    xb = synth.bits16(x)
    check_gemv(y, oracle.gemv_f64(xb, w32), w32, xb, f"gemm kernel M={M} N={N}")


@pytest.mark.parametrize("M,N,K", [(130, 37, 128), (129, 6, 640), (1, 1, 128), (77, 260, 384), (300, 515, 1152)])
def test_gemm_kernel_odd_shapes(q4, M, N, K):
    """The large-tile kernel where the min term's four-group sets end early
    (K / 128 = 1, 3, 5, 9 groups), N is not a multiple of 4 or below one
    16-row tile, and M ends inside a 16-row batch tile."""
    dev, w32 = mat(N, K, ("gemm-odd", N, K))
    x = synth.x_bf16(M, K, ("gemm-odd-x", M, K))
    y = q4.q4g128_gemm(gpu(x), *dev, variant=q4.VARIANT_GEMM)
    xb = synth.bits16(x)
    check_gemv(y, oracle.gemv_f64(xb, w32), w32, xb, f"gemm kernel M={M} N={N} K={K}")


def test_gemm_full_size_sampled_rows(q4):
    """M = 4096, N = 8192, K = 2048 (256-row weight tiles, 1024 workgroups):
    every output of 24 sampled batch rows (first, last, tile edges, random)
    against the oracle; the whole output finite."""
    M, N, K = 4096, 8192, 2048
    dev, w32 = mat(N, K, ("gemm-full",))
    x = synth.x_bf16(M, K, ("gemm-full-x",))
    y = q4.q4g128_gemm(gpu(x), *dev)
    assert torch.isfinite(y.float()).all()
    rows = sorted({0, 1, 127, 128, 129, 2047, 2048, 4094, 4095} | set(int(r) for r in np.random.default_rng(7).choice(M, 15, replace=False)))
    xb = synth.bits16(x)[rows]
    check_gemv(y[rows], oracle.gemv_f64(xb, w32), w32, xb, "gemm M=4096 N=8192 K=2048 sampled rows")


@pytest.mark.parametrize("M,K,chunk", [(192, 2048, 64), (200, 2048, 64), (100, 8192, 32), (70, 4096, 64)])
def test_gemm_chunks_equal_tiled_decode_calls(q4, M, K, chunk):
    dev, _ = mat(2048, K, ("gemm-chunks", K))
    x = gpu(synth.x_bf16(M, K, ("gemm-chunks-x", M, K)))
    y = q4.q4g128_gemm(x, *dev, variant=q4.VARIANT_TILED)
    for m0 in range(0, M, chunk):
        part = x[m0:m0 + chunk].contiguous()
        ref = q4.q4g128_gemv(part, *dev, variant=q4.VARIANT_TILED)
        assert torch.equal(y[m0:m0 + chunk].view(torch.int16), ref.view(torch.int16)), (M, K, m0)


@pytest.mark.parametrize("M", [1, 4, 48, 64])
def test_gemm_small_m_is_the_gemv(q4, M):
    dev, _ = mat(2048, 2048, ("gemm-small",))
    x = gpu(synth.x_bf16(M, 2048, ("gemm-small-x", M)))
    assert torch.equal(q4.q4g128_gemm(x, *dev).view(torch.int16), q4.q4g128_gemv(x, *dev).view(torch.int16))


def test_gemm_rejects(q4):
    dev, w32 = mat(64, 32768, ("gemm-bad",))
    x = synth.x_bf16(100, 32768, "gemm-bad-x")
    with pytest.raises(q4.Q4GemvError):          # K beyond the chunked kernel's unsplit LDS budget
        q4.q4g128_gemm(gpu(x), *dev, variant=q4.VARIANT_TILED)
    with pytest.raises(q4.Q4GemvError):          # not a prefill variant
        q4.q4g128_gemm(gpu(x), *dev, variant=q4.VARIANT_STREAM)
    xb = synth.bits16(x)                         # the automatic choice takes the large-tile kernel there
    check_gemv(q4.q4g128_gemm(gpu(x), *dev), oracle.gemv_f64(xb, w32), w32, xb, "gemm K=32768")
    d2, w2 = mat(64, 16384, ("gemm-16k",))       # the widest K: 16-row chunks
    x2 = synth.x_bf16(70, 16384, "gemm-16k-x")
    xb = synth.bits16(x2)
    check_gemv(q4.q4g128_gemm(gpu(x2), *d2), oracle.gemv_f64(xb, w2), w2, xb, "gemm K=16384")


def test_gemm_kernel_output_only_2_byte_aligned(q4):
    """y need only be 2-byte aligned: an output view 2 bytes into a buffer
    (N % 4 == 0, where aligned rows take 8-byte stores) must get the same
    values as an aligned output."""
    M, N, K = 130, 256, 2048
    dev, w32 = mat(N, K, ("gemm-misal", N, K))
    x = gpu(synth.x_bf16(M, K, ("gemm-misal-x",)))
    y_al = q4.q4g128_gemm(x, *dev, variant=q4.VARIANT_GEMM)
    buf = torch.full((M * N + 8,), float("nan"), dtype=torch.bfloat16, device="cuda")
    y_mis = buf[1:1 + M * N].view(M, N)
    q4.q4g128_gemm(x, *dev, out=y_mis, variant=q4.VARIANT_GEMM)
    assert torch.equal(y_mis.view(torch.int16), y_al.view(torch.int16))
    assert bool(torch.isnan(buf[0].float())) and bool(torch.isnan(buf[1 + M * N:].float()).all())
