"""GPU parity of mixed-format grouped GEMVs (q4gemv_grouped_mixed).

At M <= 4 one streaming launch carries int4, NVFP4 and BF16 tasks: each
output must equal the single-format streaming call bit for bit.  At 5 <= M <=
48 one skinny launch carries them, and NVFP4 with BF16 above that one tiled
launch: checked against the oracle.
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


def tasks_for(M):
    q = synth.q4_matrix(300, 4096, ("mx-q4",))
    n1 = synth.nvfp4_matrix(2048, 2048, ("mx-nv1",))
    n2 = synth.nvfp4_matrix(777, 8192 if M < 4 else 4096, ("mx-nv2", M))
    b = synth.bf16_matrix(512, 2048, ("mx-bf",))
    xq = synth.x_bf16(M, 4096, ("mx-xq", M))
    x1 = synth.x_bf16(M, 2048, ("mx-x1", M))
    x2 = synth.x_bf16(M, n2[0].shape[1] * 2, ("mx-x2", M))
    return [("nvfp4g16", gpu(x1), gpu(n1[0]), gpu(n1[1]), n1[2], None),
            ("bf16", gpu(x1), gpu(b), None),
            ("q4g128", gpu(xq), *(gpu(t) for t in q), None),
            ("nvfp4g16", gpu(x2), gpu(n2[0]), gpu(n2[1]), n2[2], None)], dict(q=q, n1=n1, n2=n2, b=b, xq=xq, x1=x1, x2=x2)


def single(q4, t, variant, ws=None):
    kind = t[0]
    if kind == "q4g128":
        return q4.q4g128_gemv_grouped([(t[1], t[2], t[3], t[4], None)], variant=variant, workspace=ws)[0]
    if kind == "nvfp4g16":
        return q4.nvfp4g16_gemv_grouped([(t[1], t[2], t[3], t[4], None)], variant=variant, workspace=ws)[0]
    return q4.bf16_gemv_grouped([(t[1], t[2], None)], variant=variant, workspace=ws)[0]


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_mixed_one_launch_equals_single_format_calls(q4, M):
    items, _ = tasks_for(M)
    outs = q4.gemv_grouped_mixed(items)
    for t, y in zip(items, outs):
        ref = single(q4, t, q4.VARIANT_STREAM)
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), (M, t[0])


def _check_tasks(outs, src, tag):
    xb1, xbq, xb2 = synth.bits16(src["x1"]), synth.bits16(src["xq"]), synth.bits16(src["x2"])
    n1, n2, q, b = src["n1"], src["n2"], src["q"], src["b"]
    w_n1 = oracle.nvfp4g16_dequant_f32(n1[0].numpy(), n1[1].numpy(), n1[2])
    w_b = oracle.bf16_dequant_f32(synth.bits16(b))
    w_q = oracle.q4g128_dequant_f32(q[0].numpy(), synth.bits16(q[1]), synth.bits16(q[2]))
    w_n2 = oracle.nvfp4g16_dequant_f32(n2[0].numpy(), n2[1].numpy(), n2[2])
    for y, w, xb, name in ((outs[0], w_n1, xb1, "nvfp4"), (outs[1], w_b, xb1, "bf16"), (outs[2], w_q, xbq, "int4"),
                           (outs[3], w_n2, xb2, "nvfp4 second")):
        check_gemv(y, oracle.gemv_f64(xb, w), w, xb, f"{tag} {name}")


@pytest.mark.parametrize("M", [5, 16, 48])
def test_mixed_one_skinny_launch(q4, M):
    """At 5 <= M <= 48 int4, NVFP4 and BF16 tasks run as one skinny launch:
    every output against the oracle, equal to itself on a second run on the
    same workspace (whose counters are left at zero)."""
    items, src = tasks_for(M)
    n = q4.mixed_workspace_bytes(items)
    ws = torch.zeros(max(n, 256), dtype=torch.uint8, device="cuda")
    outs = q4.gemv_grouped_mixed(items, workspace=ws)
    again = q4.gemv_grouped_mixed(items, workspace=ws)
    for y, z in zip(outs, again):
        assert torch.equal(y.view(torch.int16), z.view(torch.int16)), M
    assert int(ws[:64 * 1024].count_nonzero()) == 0
    _check_tasks(outs, src, f"mixed skinny M={M}")


@pytest.mark.parametrize("M", [5, 48, 64])
def test_mixed_one_launch_nvfp4_bf16(q4, M):
    """NVFP4 and BF16 tasks run as one launch (the skinny kernel at M <= 48,
    the tiled kernel above): each output checked against the oracle, and
    equal to itself on a second run (the workspace counters are left at
    zero)."""
    n1 = synth.nvfp4_matrix(2048, 2048, ("mxt-nv",))
    b = synth.bf16_matrix(512, 2048, ("mxt-bf",))
    bd = synth.bf16_matrix(2048, 8192, ("mxt-bfd",))
    x = synth.x_bf16(M, 2048, ("mxt-x", M))
    xd = synth.x_bf16(M, 8192, ("mxt-xd", M))
    items = [("nvfp4g16", gpu(x), gpu(n1[0]), gpu(n1[1]), n1[2], None), ("bf16", gpu(x), gpu(b), None),
             ("bf16", gpu(xd), gpu(bd), None)]
    ws = torch.zeros(q4.mixed_workspace_bytes(items), dtype=torch.uint8, device="cuda")
    outs = q4.gemv_grouped_mixed(items, workspace=ws)
    again = q4.gemv_grouped_mixed(items, workspace=ws)
    for y, z in zip(outs, again):
        assert torch.equal(y.view(torch.int16), z.view(torch.int16))
    xb, xdb = synth.bits16(x), synth.bits16(xd)
    w_n = oracle.nvfp4g16_dequant_f32(n1[0].numpy(), n1[1].numpy(), n1[2])
    w_b = oracle.bf16_dequant_f32(synth.bits16(b))
    w_d = oracle.bf16_dequant_f32(synth.bits16(bd))
    for y, w, xx, name in ((outs[0], w_n, xb, "nvfp4"), (outs[1], w_b, xb, "bf16"), (outs[2], w_d, xdb, "bf16 K=8192")):
        check_gemv(y, oracle.gemv_f64(xx, w), w, xx, f"mixed tiled {name} M={M}")


def test_mixed_against_oracle(q4):
    items, src = tasks_for(1)
    _check_tasks(q4.gemv_grouped_mixed(items), src, "mixed stream")
