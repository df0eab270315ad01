"""The decode step composed of library calls, captured in one HIP graph and
replayed, against the CPU oracle.

The pages' engines replay the whole decode step as a graph (Rumik TTS Fast
Inference post, "What Made It Faster"; rumik-oss-1-int4 card, "Running it").
Here a reduced step -- three hidden-2048 layers and the 2049-row head -- is
built from the same calls the benchmark times: per layer one grouped launch
for the projections that read the layer input (q, k, v, gate, up) and one for
o and down, either plain grouped calls or the fused call (o adds the layer
input as its residual, down reads silu(gate) * up), and the NVFP4 step's
mixed-format launches (NVFP4 q, k, o, gate, up; BF16 v, down).  Unlike the
benchmark the layers are chained: the next layer's input is this layer's o
output, and down reads the up (or gate and up) outputs, so a stale or
misordered buffer anywhere shows in the result.  Every call of a step shares
one split-K workspace.

Checked after each of three replays (outputs poisoned with NaN before each):
every output bitwise equal to the eager run of the same calls, the
workspace's arrival counters back at zero, and -- once -- every output of the
eager run against the oracle, computed from that stage's actual inputs, at
the acceptance bound.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_gemv, x_bits

pytestmark = pytest.mark.gpu

N_LAYERS = 3
STAGE1 = ("q", "k", "v", "gate", "up")
COUNTER_BYTES = 64 * 1024


@pytest.fixture(scope="module")
def q4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_weight_only_q4g128_amd as m
    return m


_W = {}


def _weights(fmt):
    """Host weights and their oracle fp32 dequantization, per layer."""
    if fmt not in _W:
        layers = []
        for i in range(N_LAYERS):
            lay, w32 = {}, {}
            for p in synth.LAYER_ORDER:
                N, K = synth.LAYER_SHAPES[p]
                if fmt == "q4":
                    t = synth.q4_matrix(N, K, ("step-graph", i, p))
                    w32[p] = oracle.q4g128_dequant_f32(t[0].numpy(), synth.bits16(t[1]), synth.bits16(t[2]))
                elif p in synth.NVFP4_BF16_PROJ:
                    t = synth.bf16_matrix(N, K, ("step-graph-nvbf", i, p))
                    w32[p] = oracle.bf16_dequant_f32(synth.bits16(t))
                else:
                    t = synth.nvfp4_matrix(N, K, ("step-graph-nv", i, p))
                    w32[p] = oracle.nvfp4g16_dequant_f32(t[0].numpy(), t[1].numpy(), t[2])
                lay[p] = t
            layers.append((lay, w32))
        head = synth.bf16_matrix(*synth.HEAD_SLICE, ("step-graph-head",))
        _W[fmt] = (layers, head, oracle.bf16_dequant_f32(synth.bits16(head)))
    return _W[fmt]


def _dev(t):
    if isinstance(t, tuple):
        return tuple(_dev(a) for a in t)
    return t.cuda() if isinstance(t, torch.Tensor) else t


class Step:
    """The reduced step's calls, buffers and oracle checks."""

    def __init__(self, q4, fmt, M, mode):
        self.q4, self.fmt, self.M, self.mode = q4, fmt, M, mode
        layers, head, self.head_w32 = _weights(fmt)
        self.w32 = [w for _, w in layers]
        self.lay = [{p: _dev(t) for p, t in lay.items()} for lay, _ in layers]
        self.head = head.cuda()
        self.h0 = synth.x_bf16(M, 2048, ("step-graph-x", M)).cuda()
        bf = dict(dtype=torch.bfloat16, device="cuda")
        self.ys = [{p: torch.empty(M, synth.LAYER_SHAPES[p][0], **bf) for p in synth.LAYER_ORDER} for _ in range(N_LAYERS)]
        self.yh = torch.empty(M, synth.HEAD_SLICE[0], **bf)
        self.ws = None
        self.calls = self._plan()

    def layer_input(self, i):
        return self.h0 if i == 0 else self.ys[i - 1]["o"]

    def _stage_items(self, i):
        """(stage-1 items, stage-2 items) of layer i in the call's item format."""
        lay, ys, h = self.lay[i], self.ys[i], self.layer_input(i)
        if self.fmt == "q4":
            s1 = [(h, *lay[p], ys[p]) for p in STAGE1]
            if self.mode == "fused":
                s2 = [dict(x=ys["q"], qweight=lay["o"][0], scale=lay["o"][1], min=lay["o"][2], residual=h, out=ys["o"]),
                      dict(x=ys["gate"], up=ys["up"], qweight=lay["down"][0], scale=lay["down"][1], min=lay["down"][2],
                           out=ys["down"])]
            else:
                s2 = [(ys["q"], *lay["o"], ys["o"]), (ys["up"], *lay["down"], ys["down"])]
            return s1, s2

        def tag(p, x):
            if p in synth.NVFP4_BF16_PROJ:
                return ("bf16", x, lay[p], ys[p])
            return ("nvfp4g16", x, *lay[p], ys[p])
        return [tag(p, h) for p in STAGE1], [tag("o", ys["q"]), tag("down", ys["up"])]

    def _plan(self):
        q4 = self.q4
        stages = [self._stage_items(i) for i in range(N_LAYERS)]
        hitems = [(self.layer_input(N_LAYERS), self.head, self.yh)]
        need = [q4.bf16_workspace_bytes(hitems)]
        for s1, s2 in stages:
            if self.fmt == "q4":
                need.append(q4.q4g128_workspace_bytes(s1))
                need.append(q4.q4g128_fused_workspace_bytes(s2) if self.mode == "fused" else q4.q4g128_workspace_bytes(s2))
            else:
                need += [q4.mixed_workspace_bytes(s1), q4.mixed_workspace_bytes(s2)]
        n = max(need)
        if n:
            # one shared workspace, at least the counter region, zero-filled once
            self.ws = torch.zeros(max(n, COUNTER_BYTES), dtype=torch.uint8, device="cuda")
        ws = self.ws
        calls = []
        for s1, s2 in stages:
            if self.fmt == "q4":
                calls.append(lambda s1=s1: q4.q4g128_gemv_grouped(s1, workspace=ws))
                if self.mode == "fused":
                    calls.append(lambda s2=s2: q4.q4g128_gemv_fused(s2, workspace=ws))
                else:
                    calls.append(lambda s2=s2: q4.q4g128_gemv_grouped(s2, workspace=ws))
            else:
                calls.append(lambda s1=s1: q4.gemv_grouped_mixed(s1, workspace=ws))
                calls.append(lambda s2=s2: q4.gemv_grouped_mixed(s2, workspace=ws))
        calls.append(lambda: q4.bf16_gemv_grouped(hitems, workspace=ws))
        return calls

    def outputs(self):
        return [y for ys in self.ys for y in ys.values()] + [self.yh]

    def run(self):
        for c in self.calls:
            c()

    def check_oracle(self):
        """Each stage against the oracle from its own (eager) inputs."""
        worst = 0.0
        for i in range(N_LAYERS):
            ys, w32, h = self.ys[i], self.w32[i], self.layer_input(i)
            hb = x_bits(h.cpu())
            for p in STAGE1:
                worst = max(worst, check_gemv(ys[p], oracle.gemv_f64(hb, w32[p]), w32[p], hb, f"layer {i} {p}"))
            qb = x_bits(ys["q"].cpu())
            ub = x_bits(ys["up"].cpu())
            if self.fmt == "q4" and self.mode == "fused":
                ref_o = oracle.gemv_residual_f64(qb, w32["o"], hb)
                act = oracle.silu_mul_bf16(x_bits(ys["gate"].cpu()), ub)
            else:
                ref_o = oracle.gemv_f64(qb, w32["o"])
                act = ub
            worst = max(worst, check_gemv(ys["o"], ref_o, w32["o"], qb, f"layer {i} o"))
            worst = max(worst, check_gemv(ys["down"], oracle.gemv_f64(act, w32["down"]), w32["down"], act, f"layer {i} down"))
        hb = x_bits(self.layer_input(N_LAYERS).cpu())
        worst = max(worst, check_gemv(self.yh, oracle.gemv_f64(hb, self.head_w32), self.head_w32, hb, "head"))
        return worst


CASES = [("q4", 1, "grouped"), ("q4", 48, "grouped"), ("q4", 1, "fused"), ("q4", 48, "fused"), ("q4", 16, "grouped"),
         ("nv", 1, "mixed"), ("nv", 48, "mixed")]


@pytest.mark.parametrize("fmt,M,mode", CASES)
def test_step_graph_replay(q4, fmt, M, mode):
    print(f"step graph: {fmt} M={M} {mode}", flush=True)
    st = Step(q4, fmt, M, mode)
    # eager run (outside capture), then the oracle on its results
    st.run()
    torch.cuda.synchronize()
    eager = [y.clone() for y in st.outputs()]
    assert all(bool(torch.isfinite(y.float()).all()) for y in eager)
    st.check_oracle()
    if st.ws is not None:
        assert int(st.ws[:COUNTER_BYTES].count_nonzero()) == 0, "arrival counters not left at zero (eager)"
    # capture the same calls once, replay three times
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    for r in range(3):
        for y in st.outputs():
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(st.outputs(), eager)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {r}: output {k} differs from the eager run"
        if st.ws is not None:
            assert int(st.ws[:COUNTER_BYTES].count_nonzero()) == 0, f"replay {r}: arrival counters not left at zero"
    del g
