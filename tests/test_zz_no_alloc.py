"""The allocation-free grouped int4 call (q4g128_gemv_grouped_noalloc, built-in
split-K scratch) against the same call with a caller workspace
(q4g128_gemv_grouped_ws): same plan and kernels, so bit-identical outputs,
and both within the oracle's acceptance bound.  Two calls in a row, the
second with a smaller input, so the second finds the first one's leftovers
in the shared array; an oversized plan is rejected before anything runs."""
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


def _items(M, shapes, tag):
    devs, w32s, xs = [], [], []
    for i, (N, K) in enumerate(shapes):
        qw, sc, mn = synth.q4_matrix(N, K, ("noalloc", tag, i))
        w32s.append(oracle.q4g128_dequant_f32(qw.numpy(), synth.bits16(sc), synth.bits16(mn)))
        devs.append((gpu(qw), gpu(sc), gpu(mn)))
        xs.append(synth.x_bf16(M, K, ("noalloc-x", tag, i)))
    return devs, w32s, xs


def test_noalloc_equals_workspace_call_twice(q4):
    # o and down at M = 48, then down alone at M = 16 (K = 8192 is split over
    # workgroups in both)
    for M, shapes, tag in ((48, [(2048, 2048), (2048, 8192)], "a"), (16, [(2048, 8192)], "b")):
        print(f"noalloc: M={M} shapes={shapes}", flush=True)
        devs, w32s, xs = _items(M, shapes, tag)
        items = [(gpu(x), *d, None) for x, d in zip(xs, devs)]
        need = q4.q4g128_workspace_bytes(items)
        assert 0 < need <= q4.NOALLOC_SCRATCH_BYTES
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        ref = q4.q4g128_gemv_grouped(items, workspace=ws)
        got = q4.q4g128_gemv_grouped_noalloc(items)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"M={M} task {i}"
            xb = synth.bits16(xs[i])
            check_gemv(a, oracle.gemv_f64(xb, w32s[i]), w32s[i], xb, f"noalloc M={M} task {i}")


def test_noalloc_rejects_oversized_plan(q4):
    # a 32768 x 8192 matrix at M = 64 plans about 17 MB of partial tiles
    x = torch.zeros(64, 8192, dtype=torch.bfloat16, device="cuda")
    qw = torch.zeros(32768, 4096, dtype=torch.uint8, device="cuda")
    sc = torch.zeros(32768, 64, dtype=torch.float16, device="cuda")
    items = [(x, qw, sc, sc.clone(), None)]
    assert q4.q4g128_workspace_bytes(items) > q4.NOALLOC_SCRATCH_BYTES
    y = torch.full((64, 32768), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(q4.Q4GemvError) as e:
        q4.q4g128_gemv_grouped_noalloc([(x, qw, sc, sc.clone(), y)])
    assert e.value.status == -7
    torch.cuda.synchronize()
    assert bool(torch.isnan(y.float()).all()), "a rejected call wrote its output"
