"""Decode-step weight-stream benchmark for the 4-bit dequant-GEMV library.

One step = one pass of the whole hot path over one batch: 36 int4 g128 layers
of the hidden-2048 shapes (q, k, v, o, gate, up, down; FFN width 8192), then
the BF16 audio-head GEMV (16385 x 2048).  Weights are seeded synthetic
(min/max-quantized N(0, 0.02) BF16 matrices), about 1.24 GB, generated on the
GPU and resident in HBM before timing.  The step is captured once into a HIP
graph and replayed; `value` is total algorithmic bytes (packed weights + group
scales + activations read + outputs written) per second at batch M = 1.  The
same step at M = 48 is reported alongside, and the step with the layer's
second launch as one fused int4 call (o + residual; down of silu(gate) * up +
residual), with per-call times of those fused calls against the same work
unfused.

Also reported on the same JSON line:
  * roofline: the int4 GEMV kernel used at M = 1 (the streaming kernel), its
    algorithmic bytes per launch over its average launch duration (HIP events
    around each launch on the launch stream), against the 8 TB/s HBM peak,
    with the HBM bytes per launch measured by rocprofv3 counters; the same for
    the matrix-core kernel at M = 48 under roofline_M48;
  * cpu_baseline: the CPU oracle (NumPy, fp64) timed on a bounded sample of
    the same workload on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) + decode steps/s, 4-bit GEMV at M=1 and M=48"
PEAK_GBS = 8000.0
N_LAYERS = 36


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def q4_wbytes(N, K):
    """weight bytes of one int4 g128 matrix: codes + fp16 scale + fp16 min."""
    return N * K // 2 + N * (K // 128) * 4


def q4_bytes(N, K, M):
    """algorithmic bytes of one int4 g128 GEMV: weights + x + y."""
    return q4_wbytes(N, K) + M * K * 2 + M * N * 2


class Workload:
    def __init__(self, q4, synth, torch, head_rows: int):
        self.q4, self.torch = q4, torch
        dev = "cuda"
        t0 = time.time()
        self.layers = []
        for i in range(N_LAYERS):
            self.layers.append({p: synth.q4_matrix(*synth.LAYER_SHAPES[p], ("step", i, p), device=dev) for p in synth.LAYER_ORDER})
        # the full audio head and the current-codebook slice (a step uses one or the other)
        self.heads = {rows: synth.bf16_matrix(rows, 2048, ("step-head", rows), device=dev)
                      for rows in (synth.HEAD_FULL[0], synth.HEAD_SLICE[0])}
        self.head = self.heads[head_rows]
        torch.cuda.synchronize()
        log(f"bench: generated {N_LAYERS} int4 layers + bf16 heads {sorted(self.heads)}x2048 in {time.time() - t0:.1f}s")
        self.shapes = synth.LAYER_SHAPES
        self.order = synth.LAYER_ORDER
        self.head_rows = head_rows
        self.io = {}
        self.res = {}
        self.ws = {}
        self.yh = {}

    def head_out(self, M, rows):
        if (M, rows) not in self.yh:
            self.yh[(M, rows)] = self.torch.empty((M, rows), dtype=self.torch.bfloat16, device="cuda")
        return self.yh[(M, rows)]

    def buffers(self, M):
        if M not in self.io:
            t = self.torch
            import synth
            # input of q/k/v/gate/up, stand-in attention output for o, stand-in FFN activation for down
            xin = synth.x_bf16(M, 2048, ("bench-xin", M), device="cuda")
            xattn = synth.x_bf16(M, 2048, ("bench-xattn", M), device="cuda")
            xffn = synth.x_bf16(M, 8192, ("bench-xffn", M), device="cuda")
            xs = {"q": xin, "k": xin, "v": xin, "gate": xin, "up": xin, "o": xattn, "down": xffn}
            ys = {p: t.empty((M, self.shapes[p][0]), dtype=t.bfloat16, device="cuda") for p in self.order}
            yh = self.head_out(M, self.head_rows)
            self.io[M] = (xs, ys, xin, yh)
            # stand-in residual-stream inputs of the fused o and down calls
            self.res[M] = (synth.x_bf16(M, 2048, ("bench-res-o", M), device="cuda"),
                           synth.x_bf16(M, 2048, ("bench-res-down", M), device="cuda"))
        return self.io[M]

    def launches(self, M, mode="grouped", head_rows=None):
        """[(callable, weight_bytes, is_q4)] for one step, in stream order.

        plain:   one launch per projection (7 per layer) and one for the head.
        grouped: per layer, q, k, v, gate, up (they read the same activations)
                 in one launch and o, down (independent of each other in a
                 parallel block) in another; then the head.
        fused:   as grouped, but the o, down launch is one fused int4 call: o
                 adds a residual, down reads silu(gate) * up -- the outputs of
                 the layer's first launch -- and adds a residual.
        """
        xs, ys, xin, _ = self.buffers(M)
        head_rows = head_rows or self.head_rows
        head, yh = self.heads[head_rows], self.head_out(M, head_rows)
        out = []
        q4 = self.q4
        for lay in self.layers:
            if mode == "plain":
                for p in self.order:
                    qw, sc, mn = lay[p]
                    N, K = self.shapes[p]
                    out.append((lambda x=xs[p], qw=qw, sc=sc, mn=mn, y=ys[p]: q4.q4g128_gemv(x, qw, sc, mn, out=y),
                                q4_wbytes(N, K), True))
            else:
                for stage in (("q", "k", "v", "gate", "up"), ("o", "down")):
                    wb = sum(q4_wbytes(*self.shapes[p]) for p in stage)
                    if mode == "fused" and stage[0] == "o":
                        ro, rd = self.res[M]
                        fitems = [dict(x=xs["o"], qweight=lay["o"][0], scale=lay["o"][1], min=lay["o"][2], residual=ro, out=ys["o"]),
                                  dict(x=ys["gate"], up=ys["up"], qweight=lay["down"][0], scale=lay["down"][1], min=lay["down"][2],
                                       residual=rd, out=ys["down"])]
                        ws = self.workspace(M, None, q4.q4g128_fused_workspace_bytes(fitems))
                        out.append((lambda fitems=fitems, ws=ws: q4.q4g128_gemv_fused(fitems, workspace=ws), wb, True))
                        continue
                    items = [(xs[p], *lay[p], ys[p]) for p in stage]
                    ws = self.workspace(M, items)
                    out.append((lambda items=items, ws=ws: q4.q4g128_gemv_grouped(items, workspace=ws), wb, True))
        if mode in ("grouped", "fused") and M > 4:
            # the head as a one-task grouped call, so that it may split K
            hitems = [(xin, head, yh)]
            hws = self.workspace(M, hitems, self.q4.bf16_workspace_bytes(hitems))
            out.append((lambda: q4.bf16_gemv_grouped(hitems, workspace=hws), head_rows * 2048 * 2, False))
        else:
            out.append((lambda: q4.bf16_gemv(xin, head, out=yh), head_rows * 2048 * 2, False))
        return out

    def outputs(self, M, head_rows=None):
        """The step's output buffers (per projection the last layer's, and the head's)."""
        xs, ys, _, _ = self.buffers(M)
        return [ys[p] for p in self.order] + [self.head_out(M, head_rows or self.head_rows)]

    def workspace(self, M, items, need=None):
        """One split-K workspace per batch size (zero-filled once), shared by
        every grouped and fused call of the step (the calls run in stream
        order; a fused call's activation pass uses the space after its split-K
        part)."""
        if need is None:
            need = self.q4.q4g128_workspace_bytes(items)
        if need == 0:
            return None
        ws = self.ws.get(M)
        if ws is None or ws.numel() < need:
            ws = self.torch.zeros(need, dtype=self.torch.uint8, device="cuda")
            self.ws[M] = ws
        return ws

    def step_bytes(self, M, mode="grouped", head_rows=None):
        """Algorithmic bytes of one step: packed weights + group scales, each
        distinct activation vector read once (layer input, attention output,
        FFN activation, head input), every output written once; the fused
        step reads the gate and up outputs instead of the FFN activation,
        plus two residuals per layer."""
        head_rows = head_rows or self.head_rows
        w = sum(b for _, b, _ in self.launches(M, "plain", head_rows))
        per_layer_x = (2048 + 2048 + (2 * 8192 + 2 * 2048 if mode == "fused" else 8192)) * M * 2
        per_layer_y = sum(self.shapes[p][0] for p in self.order) * M * 2
        head_io = 2048 * M * 2 + head_rows * M * 2
        return w + N_LAYERS * (per_layer_x + per_layer_y) + head_io


def nvfp4_wbytes(N, K):
    """weight bytes of one NVFP4 matrix: E2M1 codes + e4m3 group-16 scales + the fp32 global scale."""
    return N * K // 2 + N * (K // 16) + 4


class Nvfp4Workload:
    """The same decode step with NVFP4 weights: q, k, o, gate, up NVFP4 (E2M1
    codes, e4m3 scales per 16 columns, one fp32 global scale) and v, down BF16,
    as the VoxCPM2-NVFP4 card quantizes them; then the same BF16 head.  plain:
    one launch per projection; grouped: per layer the NVFP4 q, k, gate, up with
    the BF16 v in one mixed-format call and the NVFP4 o with the BF16 down in
    another (one launch each: the streaming kernel at M <= 4, the skinny
    matrix-core kernel at 5 <= M <= 48), then the head."""

    def __init__(self, q4, synth, torch, int4_wl):
        self.q4, self.torch = q4, torch
        t0 = time.time()
        self.layers = []
        for i in range(N_LAYERS):
            lay = {}
            for p in synth.LAYER_ORDER:
                N, K = synth.LAYER_SHAPES[p]
                if p in synth.NVFP4_BF16_PROJ:
                    lay[p] = synth.bf16_matrix(N, K, ("nvfp4-step-bf16", i, p), device="cuda")
                else:
                    lay[p] = synth.nvfp4_matrix(N, K, ("nvfp4-step", i, p), device="cuda")
            self.layers.append(lay)
        torch.cuda.synchronize()
        log(f"bench: generated {N_LAYERS} NVFP4 layers (v, down BF16) in {time.time() - t0:.1f}s")
        self.bf16_proj = synth.NVFP4_BF16_PROJ
        self.int4 = int4_wl
        self.shapes, self.order = synth.LAYER_SHAPES, synth.LAYER_ORDER
        self.ws = {}

    def weight_bytes_of(self, p):
        N, K = self.shapes[p]
        return N * K * 2 if p in self.bf16_proj else nvfp4_wbytes(N, K)

    def workspace(self, M, need):
        """One split-K workspace per batch size, shared by the step's grouped
        calls of both formats (they run in stream order)."""
        if need == 0:
            return None
        ws = self.ws.get(M)
        if ws is None or ws.numel() < need:
            ws = self.torch.zeros(need, dtype=self.torch.uint8, device="cuda")
            self.ws[M] = ws
        return ws

    def launches(self, M, mode="plain"):
        xs, ys, xin, yh = self.int4.buffers(M)
        q4, out = self.q4, []
        if mode == "grouped":
            # size the shared workspace for the largest call first
            plan = []
            for lay in self.layers:
                for stage in (("q", "k", "gate", "up", "v"), ("o", "down")):
                    if len(stage) > 1:
                        # NVFP4 q, k, gate, up with the BF16 v, and the NVFP4 o with the
                        # BF16 down: one launch each
                        items = [("bf16", xs[p], lay[p], ys[p]) if p in self.bf16_proj else ("nvfp4g16", xs[p], *lay[p], ys[p])
                                 for p in stage]
                        plan.append((q4.gemv_grouped_mixed, items, q4.mixed_workspace_bytes(items), stage))
                    elif stage[0] in self.bf16_proj:
                        items = [(xs[p], lay[p], ys[p]) for p in stage]
                        plan.append((q4.bf16_gemv_grouped, items, q4.bf16_workspace_bytes(items), stage))
                    else:
                        items = [(xs[p], *lay[p], ys[p]) for p in stage]
                        plan.append((q4.nvfp4g16_gemv_grouped, items, q4.nvfp4g16_workspace_bytes(items), stage))
            hitems = [(xin, self.int4.head, yh)]
            hneed = q4.bf16_workspace_bytes(hitems) if M > 4 else 0
            ws = self.workspace(M, max([n for _, _, n, _ in plan] + [hneed]))
            for fn, items, n, stage in plan:
                wb = sum(self.weight_bytes_of(p) for p in stage)
                out.append((lambda fn=fn, items=items, w=(ws if n else None): fn(items, workspace=w), wb,
                            stage[0] not in self.bf16_proj))
            # the head as a one-task grouped call, so that it may split K
            out.append((lambda: q4.bf16_gemv_grouped(hitems, workspace=(ws if hneed else None)), self.int4.head_rows * 2048 * 2,
                        False))
            return out
        for lay in self.layers:
            for p in self.order:
                if p in self.bf16_proj:
                    out.append((lambda x=xs[p], w=lay[p], y=ys[p]: q4.bf16_gemv(x, w, out=y), self.weight_bytes_of(p), False))
                else:
                    qw, s8, G = lay[p]
                    out.append((lambda x=xs[p], qw=qw, s8=s8, G=G, y=ys[p]: q4.nvfp4g16_gemv(x, qw, s8, G, out=y),
                                self.weight_bytes_of(p), True))
        head = self.int4.head
        out.append((lambda: q4.bf16_gemv(xin, head, out=yh), self.int4.head_rows * 2048 * 2, False))
        return out

    def step_bytes(self, M):
        w = sum(b for _, b, _ in self.launches(M))
        per_layer_x = (2048 + 2048 + 8192) * M * 2
        per_layer_y = sum(self.shapes[p][0] for p in self.order) * M * 2
        head_io = 2048 * M * 2 + self.int4.head_rows * M * 2
        return w + N_LAYERS * (per_layer_x + per_layer_y) + head_io


def weight_bytes(wl):
    """Packed weights + group parameters of one step (the head's BF16 rows
    included): the bytes the weight stream must read."""
    return sum(b for _, b, _ in wl.launches(1, "plain"))


def graph_us(torch, fn, reps=20, iters=20):
    """Microseconds per call of fn, captured `reps` times in one graph."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        g.replay()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / (iters * reps) * 1e3


def fused_calls(torch, q4, synth, wl, M):
    """The fused int4 calls of one layer against the same work unfused
    (torch's silu, multiply and add around the plain grouped GEMV) and the
    plain GEMV alone, microseconds per call in graphs; plus the fused down
    call's algorithmic bytes per second (weights, gate and up, residual, y)."""
    import torch.nn.functional as Fn
    lay = wl.layers[0]
    g = synth.x_bf16(M, 8192, ("bench-fz-g", M), device="cuda")
    u = synth.x_bf16(M, 8192, ("bench-fz-u", M), device="cuda")
    a = synth.x_bf16(M, 2048, ("bench-fz-a", M), device="cuda")
    wl.buffers(M)
    ro, rd = wl.res[M]
    h = torch.empty_like(g)
    yd = torch.empty((M, 2048), dtype=torch.bfloat16, device="cuda")
    yo = torch.empty_like(yd)
    d, o = lay["down"], lay["o"]
    fd = [dict(x=g, up=u, qweight=d[0], scale=d[1], min=d[2], residual=rd, out=yd)]
    fo = [dict(x=a, qweight=o[0], scale=o[1], min=o[2], residual=ro, out=yo)]
    need = max(q4.q4g128_fused_workspace_bytes(fd), q4.q4g128_fused_workspace_bytes(fo),
               q4.q4g128_workspace_bytes([(h, *d, yd)]), q4.q4g128_workspace_bytes([(a, *o, yo)]))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda") if need else None

    def unfused_down():
        h.copy_((Fn.silu(g.float()) * u.float()).to(torch.bfloat16))
        q4.q4g128_gemv_grouped([(h, *d, yd)], workspace=ws)
        yd.add_(rd)

    def unfused_o():
        q4.q4g128_gemv_grouped([(a, *o, yo)], workspace=ws)
        yo.add_(ro)

    rec = {}
    for name, fused, unfused, plain in (
            ("down_silu_up_residual", lambda: q4.q4g128_gemv_fused(fd, workspace=ws), unfused_down,
             lambda: q4.q4g128_gemv_grouped([(h, *d, yd)], workspace=ws)),
            ("o_residual", lambda: q4.q4g128_gemv_fused(fo, workspace=ws), unfused_o,
             lambda: q4.q4g128_gemv_grouped([(a, *o, yo)], workspace=ws))):
        rec[name] = {"fused_us": round(graph_us(torch, fused), 2), "unfused_us": round(graph_us(torch, unfused), 2),
                     "plain_gemv_us": round(graph_us(torch, plain), 2)}
    down_bytes = q4_wbytes(2048, 8192) + 2 * M * 8192 * 2 + 2 * M * 2048 * 2
    rec["down_silu_up_residual"]["fused_GB_s"] = round(down_bytes / (rec["down_silu_up_residual"]["fused_us"] * 1e-6) / 1e9, 1)
    return rec


def head_sample_calls(torch, q4, synth, M):
    """Sampling from the head at temperature 0.8, top-k 30 (caller-supplied
    uniforms), 2049- and 16385-row heads: the head GEMV alone, GEMV +
    sampling as two launches, the workspace form (one launch at M = 1, the
    GEMV and the split sampler for a batch), and the sampler alone;
    microseconds per call."""
    rec = {}
    x = synth.x_bf16(M, 2048, ("bench-hs-x", M), device="cuda")
    u = torch.rand(M, generator=torch.Generator(device="cuda").manual_seed(M), device="cuda")
    for N in (2049, 16385):
        w = synth.bf16_matrix(N, 2048, ("bench-hs-w", N), device="cuda")
        lg = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        r = {"gemv_us": round(graph_us(torch, lambda: q4.bf16_gemv(x, w, out=lg)), 2),
             "gemv_and_sample_us": round(graph_us(torch, lambda: q4.bf16_head_sample(x, w, u, logits=lg)), 2),
             "sample_only_us": round(graph_us(torch, lambda: q4.sample_topk(lg, u)), 2)}
        need = q4.bf16_head_sample_workspace_bytes(M, N, 2048, 30)
        if need:
            ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
            key = "gemv_and_sample_one_launch_us" if M == 1 else "gemv_and_split_sample_us"
            r[key] = round(graph_us(torch, lambda: q4.bf16_head_sample(x, w, u, logits=lg, workspace=ws)), 2)
            r["workspace_form_over_gemv"] = round(r[key] / r["gemv_us"], 2)
        rec[f"head{N}"] = r
    return rec


def prefill_calls(torch, q4, synth):
    """The int4 prefill GEMM (q4g128_gemm, the automatic kernel choice) on the
    layer's projection shapes at M = 1024 and 4096 tokens: microseconds and
    TFLOP/s against the 2.5 PFLOP/s dense BF16 matrix-core peak, beside the
    tiled decode kernel over batch chunks (VARIANT_TILED) and torch's BF16 GEMM
    (the vendor library) on weights dequantized to BF16 beforehand."""
    rec = {}
    for (N, K) in ((2048, 2048), (8192, 2048), (2048, 8192)):
        qd = tuple(t.cuda() for t in synth.q4_matrix(N, K, ("bench-prefill", N, K)))
        wd = q4.q4g128_dequant_f32(*qd).to(torch.bfloat16)
        for M in (1024, 4096):
            x = synth.x_bf16(M, K, ("bench-prefill-x", M, K), device="cuda")
            y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            us = graph_us(torch, lambda: q4.q4g128_gemm(x, *qd, out=y), reps=5, iters=10)
            uc = graph_us(torch, lambda: q4.q4g128_gemm(x, *qd, out=y, variant=q4.VARIANT_TILED), reps=5, iters=10)
            ub = graph_us(torch, lambda: torch.matmul(x, wd.t(), out=y), reps=5, iters=10)
            fl = 2.0 * M * N * K
            rec[f"N{N}_K{K}_M{M}"] = {"int4_us": round(us, 1), "int4_TFLOP_s": round(fl / us / 1e6, 1),
                                      "frac_of_bf16_mfma_peak": round(fl / us / 1e6 / 2500.0, 3),
                                      "int4_batch_chunks_kernel_us": round(uc, 1),
                                      "bf16_library_on_dequantized_us": round(ub, 1)}
    return rec


def projection_calls(torch, q4, wl):
    """Each projection alone (the automatic kernel choice) at M = 1, 3, 16, 48:
    one launch per layer over the 36 layers' distinct copies, captured in one
    graph and replayed, so gate, up and down (36 x 8.9 MB) overflow the
    256 MB memory-side cache while q, o (80 MB) and k, v (20 MB) stay in it.
    Microseconds and algorithmic GB/s per launch."""
    rec = {}
    for M in (1, 3, 16, 48):
        x = {K: wl.torch.zeros((M, K), dtype=wl.torch.bfloat16, device="cuda").normal_() for K in (2048, 8192)}
        for p in wl.order:
            N, K = wl.shapes[p]
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            items = [[(x[K], *lay[p], y)] for lay in wl.layers]
            ws = wl.workspace(M, items[0])
            calls = [lambda it=it: q4.q4g128_gemv_grouped(it, workspace=ws) for it in items]
            us = graph_us(torch, lambda: [c() for c in calls], reps=1, iters=20) / len(calls)
            rec[f"{p}_M{M}"] = {"us": round(us, 2), "GB_s": round(q4_bytes(N, K, M) / (us * 1e-6) / 1e9, 1),
                                "cached": q4_wbytes(N, K) * N_LAYERS < 256e6}
    return rec


def read_ceiling(torch, q4, wl, steps, warmup, head=True):
    """Plain-read reference for the M=1 grouped step: the same 73 launches,
    each replaced by the library's diagnostic stream_read over exactly the
    weight buffers (codes, scales, mins; the head's BF16 rows) that GEMV launch
    streams, captured and replayed like the step (head=False: the 72 layer
    launches only).  Returns (ms per step, weight bytes read)."""
    groups = []
    for lay in wl.layers:
        for stage in (("q", "k", "v", "gate", "up"), ("o", "down")):
            groups.append([t for p in stage for t in lay[p]])
    if head:
        groups.append([wl.head])
    sinks = [torch.empty(q4.stream_read_sink_words(g), dtype=torch.int32, device="cuda") for g in groups]
    nbytes = sum(t.numel() * t.element_size() for g in groups for t in g)
    return graph_ms(torch, lambda: [q4.stream_read(g, k) for g, k in zip(groups, sinks)], steps, warmup), nbytes


def launch_floor(torch, q4, steps, n=72):
    """The cost of a launch that moves almost nothing: n diagnostic reads of
    4 KB each (distinct buffers) back to back in one graph; ms per launch."""
    bufs = [torch.ones(4096, dtype=torch.uint8, device="cuda") for _ in range(n)]
    sinks = [torch.empty(q4.stream_read_sink_words([b]), dtype=torch.int32, device="cuda") for b in bufs]
    return graph_ms(torch, lambda: [q4.stream_read([b], k) for b, k in zip(bufs, sinks)], steps, 3) / n


def single_launch_read(torch, q4, steps, nbytes=1 << 30):
    """The achievable streaming-read rate of one launch: the diagnostic
    stream_read over one contiguous 1 GiB device buffer, replayed in a graph.
    Returns (ms per launch, GB/s)."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.empty(q4.stream_read_sink_words([buf]), dtype=torch.int32, device="cuda")
    ms = graph_ms(torch, lambda: q4.stream_read([buf], sink), steps, 3)
    del buf
    return ms, nbytes / (ms * 1e-3) / 1e9


def graph_ms(torch, fn, steps, warmup):
    """Milliseconds per replay of fn captured once into a graph (events on
    the stream the graph is replayed on)."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        g.replay()
    e.record()
    e.synchronize()
    del g
    return s.elapsed_time(e) / steps


def time_graph(torch, wl, M, steps, warmup, mode, head_rows=None):
    """The step at batch M captured once into a hipGraph and replayed.  Before
    timing, one replay is checked bit for bit against the same calls run
    eagerly (outputs poisoned in between).  Returns ms per step."""
    return replay_checked(torch, wl.launches(M, mode, head_rows), wl.outputs(M, head_rows), steps, warmup, f"M={M} {mode}")


def replay_checked(torch, calls, outs, steps, warmup, what):
    for f, _, _ in calls:  # eager run outside capture
        f()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f, _, _ in calls:
            f()
    for o in outs:
        o.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    for o, e in zip(outs, eager):
        if not torch.equal(o.view(torch.int16), e.view(torch.int16)):
            raise RuntimeError(f"{what}: the replayed step differs from the eager calls")
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(steps):
        g.replay()
    e.record()
    e.synchronize()
    torch.cuda.synchronize()
    del g
    return s.elapsed_time(e) / steps


def layer_launches_in_graph(torch, wl, M, mode, steps, warmup):
    """The step's int4 GEMV launches alone (the 72 grouped launches of the 36
    layers, without the head), captured into one graph and replayed exactly as
    in the step: milliseconds per launch -- each launch's duration inside the
    replayed graph, dispatch gap included -- and the average algorithmic bytes
    per launch (weights + activations read + outputs written)."""
    calls = [c for c in wl.launches(M, mode) if c[2]]
    xs, ys, _, _ = wl.buffers(M)
    act = sum(ys[p].numel() * 2 for p in wl.order) + (2048 + 2048 + 8192) * M * 2   # per layer
    nbytes = (sum(b for _, b, _ in calls) + act * N_LAYERS) / len(calls)
    ms = graph_ms(torch, lambda: [f() for f, _, _ in calls], steps, warmup)
    return ms / len(calls), nbytes


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = self.ct.c_void_p()
        assert self.hip.hipEventCreate(self.ct.byref(ev)) == 0
        return ev

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        assert self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) == 0
        return ms.value

    def sync(self, e):
        assert self.hip.hipEventSynchronize(e) == 0

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def time_q4_launches(torch, q4, wl, M, mode, reps=3):
    """Average execution time of the int4 GEMV launches of one step.  Each
    launch records a pair of HIP events at its own start and end on the stream
    it runs on (q4gemv_time_next_launch), so host-side gaps between eager
    launches are not counted.  Returns (ms per launch, algorithmic bytes per
    launch: weights + activations read + outputs written)."""
    xs, ys, xin, yh = wl.buffers(M)
    calls = [c for c in wl.launches(M, mode) if c[2]]
    act = sum(ys[p].numel() * 2 for p in wl.order) + (2048 + 2048 + 8192) * M * 2   # per layer
    io_per_launch = act * N_LAYERS / len(calls)
    he = HipEvents()
    evs = [(he.create(), he.create()) for _ in calls]
    tot_ms, tot_bytes, n = 0.0, 0, 0
    for _ in range(reps):
        for (f, b, _), (a, z) in zip(calls, evs):
            q4.lib.q4gemv_time_next_launch(a, z)
            f()
        torch.cuda.synchronize()
        he.sync(evs[-1][1])
        for (f, b, _), (a, z) in zip(calls, evs):
            tot_ms += he.elapsed_ms(a, z)
            tot_bytes += b + io_per_launch
            n += 1
    for a, z in evs:
        he.destroy(a)
        he.destroy(z)
    return tot_ms / n, tot_bytes / n


def time_graph_nv(torch, nv, M, steps, warmup, mode):
    """The NVFP4 step captured into a hipGraph and replayed, checked once
    against the eager calls like time_graph.  Returns (ms per step, None)."""
    return replay_checked(torch, nv.launches(M, mode), nv.int4.outputs(M), steps, warmup, f"NVFP4 M={M} {mode}"), None


def nvfp4_launches_in_graph(torch, nv, M, steps, warmup):
    """The NVFP4 projections' own launches of the per-projection NVFP4 step
    (q, k, o, gate, up of the 36 layers: 180 launches), captured into one
    graph and replayed: milliseconds per launch inside the graph and the
    average algorithmic bytes per launch (weights + that projection's x and
    y)."""
    xs, ys, _, _ = nv.int4.buffers(M)
    calls, nbytes = [], 0
    all_calls = nv.launches(M)
    k = 0
    for li in range(N_LAYERS):
        for p in nv.order:
            f, b, is_nv = all_calls[k]
            k += 1
            if is_nv:
                calls.append(f)
                nbytes += b + xs[p].numel() * 2 + ys[p].numel() * 2
    ms = graph_ms(torch, lambda: [f() for f in calls], steps, warmup)
    return ms / len(calls), nbytes / len(calls)


def nvfp4_grouped_launches_in_graph(torch, nv, M, steps, warmup):
    """The grouped NVFP4 step's 72 layer launches (per layer the NVFP4 q, k,
    gate, up with the BF16 v, and the NVFP4 o with the BF16 down; the head
    left out), captured into one graph and replayed: milliseconds per launch
    and the average algorithmic bytes per launch (weights + activations read
    + outputs written)."""
    xs, ys, _, _ = nv.int4.buffers(M)
    calls = nv.launches(M, "grouped")[:-1]
    act = sum(ys[p].numel() * 2 for p in nv.order) + (2048 + 2048 + 8192) * M * 2   # per layer
    nbytes = (sum(b for _, b, _ in calls) + act * N_LAYERS) / len(calls)
    ms = graph_ms(torch, lambda: [f() for f, _, _ in calls], steps, warmup)
    return ms / len(calls), nbytes


def cpu_baseline(wl, budget_s=12.0):
    """The oracle (plain NumPy: dequantize to fp32, fp64 matrix product) on
    the step's own weights, on this host's cores.  Dequantization and the
    product are timed separately, per projection, for whole layers until
    about budget_s seconds of CPU time (the product at M = 1 and at M = 48),
    then one layer again on a single thread; the head's BF16 GEMV once.  The
    per-step figures extrapolate the per-layer means to the 36 layers plus
    the head (one step = one dequantization of every matrix and one product;
    the oracle has no cache of dequantized weights)."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count() or 1
    x = {(M, K): synth.bits16(synth.x_bf16(M, K, ("cpu-x", M, K))) for M in (1, 48) for K in (2048, 8192)}

    def layer(host):
        t = {"dequant": 0.0, "mm1": 0.0, "mm48": 0.0}
        for p in wl.order:
            N, K = wl.shapes[p]
            t0 = time.perf_counter()
            w32 = oracle.q4g128_dequant_f32(*host[p])
            t1 = time.perf_counter()
            oracle.gemv_f64(x[(1, K)], w32)
            t2 = time.perf_counter()
            oracle.gemv_f64(x[(48, K)], w32)
            t3 = time.perf_counter()
            t["dequant"] += t1 - t0
            t["mm1"] += t2 - t1
            t["mm48"] += t3 - t2
        return t

    def host_of(lay):
        return {p: (t[0].cpu().numpy(), synth.bits16(t[1]), synth.bits16(t[2])) for p, t in lay.items()}

    tot = {"dequant": 0.0, "mm1": 0.0, "mm48": 0.0}
    layers = 0
    for lay in wl.layers:
        t = layer(host_of(lay))
        for k in tot:
            tot[k] += t[k]
        layers += 1
        if sum(tot.values()) >= budget_s:
            break
    per = {k: v / layers for k, v in tot.items()}
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            one = layer(host_of(wl.layers[0]))
    # the head: BF16 widened to fp32, then the fp64 product
    hb = synth.bits16(wl.heads[wl.head_rows].cpu())
    t0 = time.perf_counter()
    hw = oracle.bf16_dequant_f32(hb)
    t1 = time.perf_counter()
    oracle.gemv_f64(x[(1, 2048)], hw)
    t2 = time.perf_counter()
    oracle.gemv_f64(x[(48, 2048)], hw)
    t3 = time.perf_counter()
    head = {"dequant": t1 - t0, "mm1": t2 - t1, "mm48": t3 - t2}
    step = {M: N_LAYERS * (per["dequant"] + per[f"mm{M}"]) + head["dequant"] + head[f"mm{M}"] for M in (1, 48)}
    b1, b48 = wl.step_bytes(1), wl.step_bytes(48)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    rec = {"value": round(b1 / step[1] / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{layers} of {N_LAYERS} int4 layers (7 projections each) + the {wl.head_rows}-row BF16 head, "
                     f"NumPy dequantization to fp32 and fp64 matrix product timed separately at M=1 and M=48 "
                     f"({sum(tot.values()) + sum(head.values()):.1f} s of CPU time); per-step figures extrapolate "
                     f"the per-layer means to {N_LAYERS} layers",
           "steps_per_s_M1": round(1.0 / step[1], 3), "steps_per_s_M48": round(1.0 / step[48], 3),
           "GB_s_M48": round(b48 / step[48] / 1e9, 4),
           "per_layer_s": {"dequant": round(per["dequant"], 4), "matmul_fp64_M1": round(per["mm1"], 4),
                           "matmul_fp64_M48": round(per["mm48"], 4)},
           "head_s": {k: round(v, 4) for k, v in head.items()},
           "cpu": model, "nproc": os.cpu_count()}
    if one is not None:
        rec["one_thread_per_layer_s"] = {"dequant": round(one["dequant"], 4), "matmul_fp64_M1": round(one["mm1"], 4),
                                         "matmul_fp64_M48": round(one["mm48"], 4)}
        rec["value_1_thread"] = round(b1 / (N_LAYERS * (one["dequant"] + one["mm1"]) + head["dequant"] + head["mm1"]) / 1e9, 4)
    return rec


# per batch size: the kernel the grouped int4 launches run, the sources it is
# built from, and the committed rocprofv3 traffic record for it
KERNELS = {
    1: ("gemv_stream_kernel<FmtQ4, 1, false>", ("common.h", "formats.h", "internal.h", "gemv_stream.hip"),
        os.path.join(ROOT, "profiles", "gemv_stream_q4_M1_grouped_traffic.json")),
    48: ("skinny_q4_kernel<3, R, 1>", ("common.h", "formats.h", "internal.h", "gemv_skinny.hip"),
         os.path.join(ROOT, "profiles", "skinny_q4_M48_grouped_traffic.json")),
}
# the NVFP4 step's grouped launches at M = 48 (NVFP4 with BF16 v / down)
NVFP4_KERNEL_M48 = ("skinny_q4_kernel<3, R, 6>", ("common.h", "formats.h", "internal.h", "gemv_skinny.hip"),
                    os.path.join(ROOT, "profiles", "skinny_nvfp4_bf16_M48_grouped_traffic.json"))


def _code_only(src):
    """C++ source with comments and blank space removed (string literals in
    these kernels hold no comment markers)."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


# the NVFP4 streaming kernel (M = 1, per-projection launches)
NVFP4_KERNEL = ("gemv_stream_kernel<FmtNvfp4, 1, false>", ("common.h", "formats.h", "internal.h", "gemv_stream.hip"),
                os.path.join(ROOT, "profiles", "gemv_stream_nvfp4_M1_traffic.json"))
# the NVFP4 step's grouped launches at M = 1 (one mixed-format streaming launch per stage)
NVFP4_KERNEL_M1_GROUPED = ("gemv_stream_mixed_kernel<1>", ("common.h", "formats.h", "internal.h", "gemv_stream.hip"),
                           os.path.join(ROOT, "profiles", "gemv_stream_mixed_nvfp4_M1_grouped_traffic.json"))


def csrc_digest(M):
    """sha256 over the code (comments and layout removed) of the sources of
    the kernel the grouped launches run at M."""
    return csrc_digest_of(KERNELS[M][1])


def csrc_digest_of(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_weight_only_q4g128_amd", "csrc", n)) as fh:
            h.update(n.encode())
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(M):
    """HBM bytes per grouped int4 launch at M from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE runs, or None if the kernel sources changed since
    those counters were taken."""
    return _traffic(KERNELS[M][2], KERNELS[M][1])


def measured_traffic_nvfp4(M=1, grouped=False):
    """The same for the NVFP4 step: the streaming kernel's per-projection
    launches at M = 1 (grouped: the mixed-format streaming launches of the
    grouped step), the grouped mixed-format skinny launches at M = 48."""
    k = NVFP4_KERNEL_M48 if M != 1 else (NVFP4_KERNEL_M1_GROUPED if grouped else NVFP4_KERNEL)
    return _traffic(k[2], k[1])


def _traffic(path, sources):
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("csrc_digest") != csrc_digest_of(sources):
        return None
    return rec.get("traffic_bytes_per_launch")


def counters_pass(q4, synth, torch, head_rows, M, nvfp4=False, grouped=False):
    """Workload for hardware-counter runs (no timing): the grouped step at M
    (int4, or with nvfp4 the NVFP4 step: per projection at M = 1 unless
    grouped, grouped at M = 48) three times, eagerly, then a 256 MiB
    device-to-device copy whose byte count is known (the reference that scales
    FETCH_SIZE / WRITE_SIZE)."""
    wl = Workload(q4, synth, torch, head_rows)
    if nvfp4:
        calls = Nvfp4Workload(q4, synth, torch, wl).launches(M, "plain" if M == 1 and not grouped else "grouped")
    else:
        calls = wl.launches(M, "grouped")
    for _ in range(3):
        for f, _, _ in calls:
            f()
    torch.cuda.synchronize()
    a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    kern = (NVFP4_KERNEL_M48 if M != 1 else NVFP4_KERNEL_M1_GROUPED if grouped else NVFP4_KERNEL) if nvfp4 else KERNELS[M]
    log(f"bench: counters pass at M={M}{' NVFP4' if nvfp4 else ''}{' grouped' if nvfp4 and grouped else ''} done "
        f"({len(calls)} launches per step, csrc digest {csrc_digest_of(kern[1])})")


def counters_prefill(q4, synth, torch):
    """Workload for hardware-counter runs of the prefill GEMM (no timing): the
    large-tile kernel on the 8192 x 2048 projection at M = 4096, five times."""
    N, K, M = 8192, 2048, 4096
    qd = tuple(t.cuda() for t in synth.q4_matrix(N, K, ("bench-prefill", N, K)))
    x = synth.x_bf16(M, K, ("bench-prefill-x", M, K), device="cuda")
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    for _ in range(5):
        q4.q4g128_gemm(x, *qd, out=y, variant=q4.VARIANT_GEMM)
    torch.cuda.synchronize()
    log(f"bench: prefill counters pass done (N={N} K={K} M={M}, 5 launches)")


def mode_key(k):
    M, mode = k
    return f"{M}_{mode}" if isinstance(M, str) else f"M{M}_{mode}"


def mode_record(k, r, int4_wbytes, ceil_ms):
    """One timed mode: step time and rates; the int4 modes also against the
    plain read of their weight buffers (the read ceiling)."""
    M, _ = k
    batch = int(M.split("_M")[1]) if isinstance(M, str) else M
    wb = r.get("wbytes", int4_wbytes)
    rec = {"ms_per_step": round(r["ms"], 5), "GB_s": round(r["gbs"], 1), "weight_GB_s": round(wb / (r["ms"] * 1e-3) / 1e9, 1),
           "pct_of_8TBps": round(100 * r["gbs"] / PEAK_GBS, 2), "steps_per_s": round(1e3 / r["ms"], 1),
           "tokens_per_s": round(batch * 1e3 / r["ms"], 1), "launches_per_step": r["launches"], "bytes_per_step": r["bytes"]}
    rec["head_rows"] = r.get("head_rows")
    rec["weight_bytes_per_step"] = wb
    if not isinstance(M, str) and wb == int4_wbytes:
        rec["pct_of_read_ceiling"] = round(100 * ceil_ms / r["ms"], 1)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--head", choices=("full", "slice"), default="full",
                    help="head of the headline step: the 16385-row audio head (default) or the 2049-row codebook slice")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counters", action="store_true", help="run the fixed workload for rocprofv3 --pmc passes; no timing")
    ap.add_argument("--counters-m", type=int, choices=(1, 48), default=1, help="batch size of the --counters workload")
    ap.add_argument("--counters-nvfp4", action="store_true", help="the --counters workload with the NVFP4 step instead")
    ap.add_argument("--counters-grouped", action="store_true",
                    help="with --counters-nvfp4 at M=1: the grouped mixed-format launches instead of one per projection")
    ap.add_argument("--counters-prefill", action="store_true",
                    help="run the prefill GEMM (8192 x 2048, M = 4096) five times for rocprofv3 --pmc passes; no timing")
    ap.add_argument("--modes", default="M1_grouped,M1_grouped_slice,M1_fused,M1_plain,M48_grouped,M48_grouped_slice,M48_fused,"
                                       "M48_plain,NVFP4_M1_grouped,NVFP4_M48_grouped,NVFP4_M1_plain,NVFP4_M48_plain",
                    help="comma list of timed modes; M1_grouped is always timed (it is the headline value)")
    ap.add_argument("--no-extras", action="store_true", help="skip the per-call records (fused calls, sampling, prefill, projections)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_weight_only_q4g128_amd as q4
    import synth

    assert torch.cuda.is_available(), "no GPU"
    torch.cuda.set_device(0)
    head_rows = synth.HEAD_FULL[0] if args.head == "full" else synth.HEAD_SLICE[0]
    if args.counters_prefill:
        counters_prefill(q4, synth, torch)
        return
    if args.counters:
        counters_pass(q4, synth, torch, head_rows, args.counters_m, args.counters_nvfp4, args.counters_grouped)
        return
    wl = Workload(q4, synth, torch, head_rows)
    other_head = synth.HEAD_SLICE[0] if head_rows == synth.HEAD_FULL[0] else synth.HEAD_FULL[0]

    modes = {"M1_grouped"} | set(m for m in args.modes.split(",") if m)
    res = {}
    for M in (1, 48):
        for mode in ("grouped", "grouped_slice", "plain", "fused"):
            if f"M{M}_{mode}" not in modes:
                continue
            base_mode = "grouped" if mode == "grouped_slice" else mode
            hr = other_head if mode == "grouped_slice" else head_rows
            ms = time_graph(torch, wl, M, args.steps, args.warmup, base_mode, hr)
            by = wl.step_bytes(M, base_mode, hr)
            # a fused call on the tiled kernel forms silu(gate) * up in a pass of its own
            extra = N_LAYERS if base_mode == "fused" and M > 4 else 0
            res[(M, mode)] = dict(ms=ms, bytes=by, gbs=by / (ms * 1e-3) / 1e9, launches=len(wl.launches(M, base_mode, hr)) + extra,
                                  head_rows=hr, wbytes=sum(b for _, b, _ in wl.launches(1, "plain", hr)))
            log(f"bench: M={M} {mode:13s} step {ms * 1e3:8.1f} us, {by / 1e6:.1f} MB, {res[(M, mode)]['gbs']:6.0f} GB/s, "
                f"{1e3 / ms:6.0f} steps/s, {res[(M, mode)]['launches']} launches, head {hr} rows")
    nv = None
    for M in (1, 48):
        for mode in ("grouped", "plain"):
            if f"NVFP4_M{M}_{mode}" not in modes:
                continue
            if nv is None:
                nv = Nvfp4Workload(q4, synth, torch, wl)
            ms, g = time_graph_nv(torch, nv, M, args.steps, args.warmup, mode)
            by = nv.step_bytes(M)
            calls = nv.launches(M, mode)
            r = res[(f"NVFP4_M{M}", mode)] = dict(ms=ms, bytes=by, gbs=by / (ms * 1e-3) / 1e9, launches=len(calls),
                                                  wbytes=sum(b for _, b, _ in calls), head_rows=head_rows)
            log(f"bench: NVFP4 M={M} {mode:7s} step {ms * 1e3:8.1f} us, {by / 1e6:.1f} MB, {r['gbs']:6.0f} GB/s, "
                f"{1e3 / ms:6.0f} steps/s, {r['launches']} launches")
    # the roofline of the dominant kernel: its launches inside the replayed
    # step (the step's graph without the head), per launch
    roof = {}
    for M in (1, 48):
        if M != 1 and f"M{M}_grouped" not in modes:
            continue
        kms, kbytes = layer_launches_in_graph(torch, wl, M, "grouped", args.steps, args.warmup)
        achieved = kbytes / (kms * 1e-3) / 1e9
        vname = q4.variant_name(q4.FMT_Q4G128, 0, M, 2048, 2048)
        step_us = res[(M, "grouped")]["ms"] * 1e3
        nl = 2 * N_LAYERS
        log(f"bench: int4 GEMV launches at M={M} ({vname}) inside the replayed step: {kms * 1e3:.2f} us per launch, "
            f"{kbytes / 1e6:.2f} MB/launch, {achieved:.0f} GB/s; {nl} launches = {nl * kms * 1e3:.1f} of {step_us:.1f} us per step")
        roof[M] = {"bound": "hbm", "kernel": f"{KERNELS[M][0]} ({vname}), M={M}: the {nl} grouped launches of the step",
                   "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                   "traffic": measured_traffic(M), "avg_launch_us": round(kms * 1e3, 3), "alg_bytes_per_launch": round(kbytes),
                   "timing": f"{nl} launches captured in one graph exactly as in the step (head left out), replayed; per-launch "
                             f"period including the dispatch gap",
                   "launches_x_avg_us": round(nl * kms * 1e3, 1), "step_us": round(step_us, 1)}
    fz = hs = pj = pf = None
    if not args.no_extras:
        fz = {f"M{M}": fused_calls(torch, q4, synth, wl, M) for M in (1, 48)}
        for k, r in fz.items():
            log(f"bench: fused calls {k}: " + ", ".join(f"{n} fused {v['fused_us']} us / unfused {v['unfused_us']} us / "
                                                         f"plain GEMV {v['plain_gemv_us']} us" for n, v in r.items()))
        hs = {f"M{M}": head_sample_calls(torch, q4, synth, M) for M in (1, 48)}
        for k, r in hs.items():
            log(f"bench: head + top-k sampling {k}: " + ", ".join(f"{n}: GEMV {v['gemv_us']} us, GEMV+sample {v['gemv_and_sample_us']} us, "
                                                                  f"one launch {v.get('gemv_and_sample_one_launch_us')} us, "
                                                                  f"sample alone {v['sample_only_us']} us" for n, v in r.items()))
        pj = projection_calls(torch, q4, wl)
        log("bench: projections alone (36-copy rotation): " + ", ".join(f"{k} {v['us']} us {v['GB_s']} GB/s" for k, v in pj.items()
                                                                        if k.startswith(("gate", "down"))))
        pf = prefill_calls(torch, q4, synth)
        log("bench: int4 prefill GEMM: " + ", ".join(f"{k} {v['int4_us']} us ({v['int4_TFLOP_s']} TFLOP/s; BF16 library on dequantized "
                                                      f"weights {v['bf16_library_on_dequantized_us']} us)" for k, v in pf.items()))
    head = res[(1, "grouped")]
    wbytes = weight_bytes(wl)
    ceil_ms, _ = read_ceiling(torch, q4, wl, args.steps, args.warmup)
    ceil_gbs = wbytes / (ceil_ms * 1e-3) / 1e9
    one_ms, one_gbs = single_launch_read(torch, q4, 20)
    log(f"bench: plain read of the step's weight buffers in the same 73 launches: {ceil_ms * 1e3:.1f} us, {ceil_gbs:.0f} GB/s; "
        f"one launch over 1 GiB: {one_ms * 1e3:.1f} us, {one_gbs:.0f} GB/s")
    # where the time of one M=1 layer launch goes
    layers_ms, layer_read_bytes = read_ceiling(torch, q4, wl, args.steps, args.warmup, head=False)
    floor_us = launch_floor(torch, q4, args.steps) * 1e3
    read_us = layers_ms * 1e3 / (2 * N_LAYERS)
    read_b = layer_read_bytes / (2 * N_LAYERS)
    g_us, g_b = roof[1]["avg_launch_us"], roof[1]["alg_bytes_per_launch"]
    breakdown = {
        "what": "one grouped M=1 layer launch, in-graph periods: an almost empty launch; the plain read of the same "
                "buffers in the step's 72 layer launches (its bytes at the 1 GiB single-launch rate, the rest its ramp "
                "and drain); what the GEMV adds over that read",
        "gemv_launch_us": g_us, "gemv_bytes": g_b,
        "plain_read_launch_us": round(read_us, 3), "plain_read_bytes": round(read_b),
        "empty_launch_us": round(floor_us, 3),
        "parts_us": {"empty_launch": round(floor_us, 3),
                     "read_bytes_at_single_launch_rate": round(read_b / one_gbs / 1e3, 3),
                     "read_ramp_and_drain": round(read_us - floor_us - read_b / one_gbs / 1e3, 3),
                     "gemv_over_plain_read": round(g_us - read_us, 3)},
    }
    log(f"bench: M=1 layer launch {g_us:.2f} us = empty launch {floor_us:.2f} + read at the 1 GiB rate "
        f"{read_b / one_gbs / 1e3:.2f} + read ramp/drain {read_us - floor_us - read_b / one_gbs / 1e3:.2f} + GEMV over plain read "
        f"{g_us - read_us:.2f}")

    out = {
        "metric": METRIC,
        "value": round(head["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"decode step: {N_LAYERS} int4 g128 layers (hidden 2048, ffn 8192) + bf16 head {head_rows}x2048, M=1, "
                        f"grouped launches (q,k,v,gate,up | o,down | head), hipGraph replay",
            "M": 1,
            "bytes_per_step": head["bytes"],
            "steps_per_s": round(1e3 / head["ms"], 1),
            "pct_of_8TBps": round(100 * head["gbs"] / PEAK_GBS, 2),
            "launches_per_step": head["launches"],
            "weight_bytes_per_step": wbytes,
            "read_ceiling": {"what": "diagnostic plain read of the same weight buffers in the same 73 launches, hipGraph",
                             "ms_per_step": round(ceil_ms, 5), "weight_GB_s": round(ceil_gbs, 1),
                             "pct_of_8TBps": round(100 * ceil_gbs / PEAK_GBS, 2),
                             "single_launch": {"what": "one diagnostic plain-read launch over one contiguous 1 GiB buffer, hipGraph",
                                               "us": round(one_ms * 1e3, 1), "GB_s": round(one_gbs, 1),
                                               "pct_of_8TBps": round(100 * one_gbs / PEAK_GBS, 2)},
                             "value_pct_of_single_launch": round(100 * head["gbs"] / one_gbs, 1),
                             "launch_breakdown_M1": breakdown},
            "modes": {mode_key(k): mode_record(k, r, wbytes, ceil_ms) for k, r in res.items()},
        },
        "roofline": roof[1],
    }
    for name, val in (("fused_calls", fz), ("head_sample", hs), ("prefill", pf), ("projections", pj)):
        if val is not None:
            out["config"][name] = val
    if 48 in roof:
        out["roofline_M48"] = roof[48]
    if nv is not None:
        kms, kbytes = nvfp4_launches_in_graph(torch, nv, 1, args.steps, args.warmup)
        achieved = kbytes / (kms * 1e-3) / 1e9
        vname = q4.variant_name(q4.FMT_NVFP4G16, 0, 1, 2048, 2048)
        log(f"bench: NVFP4 GEMV launches at M=1 ({vname}) inside a replayed graph: {kms * 1e3:.2f} us, {kbytes / 1e6:.2f} MB/launch, "
            f"{achieved:.0f} GB/s")
        out["roofline_nvfp4_M1"] = {"bound": "hbm", "kernel": f"gemv_stream_kernel<FmtNvfp4, 1, false> ({vname}), M=1: the 180 NVFP4 "
                                                              f"projection launches of the per-projection step",
                                    "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                                    "frac": round(achieved / PEAK_GBS, 4), "traffic": measured_traffic_nvfp4(),
                                    "avg_launch_us": round(kms * 1e3, 3), "alg_bytes_per_launch": round(kbytes)}
        kern = {1: "gemv_stream_mixed_kernel<1> (stream, NVFP4 and BF16 tasks)",
                48: "skinny_q4_kernel<3, R, 6> (skinny, NVFP4 and BF16 tasks)"}
        for M in (1, 48):
            if f"NVFP4_M{M}_grouped" not in modes:
                continue
            kms, kbytes = nvfp4_grouped_launches_in_graph(torch, nv, M, args.steps, args.warmup)
            achieved = kbytes / (kms * 1e-3) / 1e9
            log(f"bench: NVFP4 step launches at M={M} (NVFP4 with BF16 v / down) inside the replayed step graph: "
                f"{kms * 1e3:.2f} us, {kbytes / 1e6:.2f} MB/launch, {achieved:.0f} GB/s")
            out[f"roofline_nvfp4_M{M}_grouped"] = {
                "bound": "hbm", "kernel": f"{kern[M]}, M={M}: the 72 grouped mixed-format launches of the step",
                "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                "traffic": measured_traffic_nvfp4(M, grouped=True), "avg_launch_us": round(kms * 1e3, 3),
                "alg_bytes_per_launch": round(kbytes),
                "timing": "72 launches captured in one graph exactly as in the step (head left out), replayed; per-launch "
                          "period including the dispatch gap"}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
