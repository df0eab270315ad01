"""GPU parity of top-k sampling (q4_sample_topk, bf16_head_sample) through the
C ABI.

The selection is exact, so the top-k indices must equal the oracle's; the
probabilities are fp32 (oracle fp64) within a relative 2e-6; the token must
be the oracle's, except when u lies within 1e-5 of the oracle's cumulative
boundary between the two candidates (fp32 sums in another order may cross).
The head path is checked with one-hot activations, which make the GEMV exact
(logits = the weight column), so the oracle samples from logits it derives
itself.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_weight_only_q4g128_amd as m
    return m


def bits(t):
    return synth.bits16(t)


def check_sample(tok, ti, tp, logit_bits, T, k, u):
    o_tok, o_idx, o_prob = oracle.sample_topk(logit_bits, T, k, u)
    ti, tp, tok = ti.cpu().numpy(), tp.cpu().numpy(), tok.cpu().numpy()
    assert np.array_equal(ti, o_idx), "top-k indices differ"
    assert np.allclose(tp, o_prob, rtol=2e-6, atol=1e-30), float(np.max(np.abs(tp / o_prob - 1)))
    for m in range(len(tok)):
        if tok[m] == o_tok[m]:
            continue
        c = np.cumsum(o_prob[m])
        pos_g, pos_o = list(o_idx[m]).index(tok[m]), list(o_idx[m]).index(o_tok[m])
        assert abs(pos_g - pos_o) == 1, (m, pos_g, pos_o)
        assert abs(c[min(pos_g, pos_o)] - u[m]) < 1e-5, (m, c[min(pos_g, pos_o)], u[m])


def logits_with_ties(M, V, seed):
    g = synth.make_gen(("sample-logits", M, V, seed))
    x = torch.randn((M, V), generator=g, dtype=torch.float32) * 3
    x = torch.round(x * 4) / 4                         # many exact ties
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("M,V,k,T", [(1, 2049, 30, 0.8), (4, 2049, 30, 0.8), (48, 2049, 30, 0.8), (3, 16385, 30, 0.8),
                                     (2, 100, 64, 1.3), (5, 64, 64, 0.8), (1, 1, 1, 0.8), (7, 2049, 1, 0.8), (16, 513, 17, 0.05)])
def test_sample_topk_against_oracle(q4, M, V, k, T):
    lg = logits_with_ties(M, V, 0)
    rng = np.random.default_rng(M * 7 + V)
    u = rng.uniform(0, 1, M).astype(np.float32)
    u[0] = 0.0
    if M > 1:
        u[-1] = np.float32(0.99999994)
    tok, ti, tp = q4.sample_topk(gpu(lg), gpu(torch.from_numpy(u)), temperature=T, top_k=k, return_topk=True)
    check_sample(tok, ti, tp, bits(lg), T, k, u.astype(np.float64))


def test_sample_many_draws_one_row(q4):
    """1024 draws from one row: each token is the oracle's (up to boundary
    cases), and u = 0 picks the largest logit."""
    V, k = 2049, 30
    lg = logits_with_ties(1, V, 3).repeat(1024, 1)
    u = np.linspace(0, 1, 1024, endpoint=False).astype(np.float32)
    tok, ti, tp = q4.sample_topk(gpu(lg), gpu(torch.from_numpy(u)), return_topk=True)
    check_sample(tok, ti, tp, bits(lg), 0.8, k, u.astype(np.float64))
    assert int(tok[0]) == int(ti[0, 0])


@pytest.mark.parametrize("M,N", [(1, 2049), (4, 2049), (48, 2049), (1, 16385)])
def test_head_sample_one_hot(q4, M, N):
    K = 2048
    w = synth.bf16_matrix(N, K, ("head-sample", N), std=1.0)
    ks = np.random.default_rng(N + M).choice(K, size=M, replace=False)
    x = torch.zeros(M, K, dtype=torch.bfloat16)
    x[torch.arange(M), torch.from_numpy(ks)] = 1.0
    u = np.random.default_rng(M).uniform(0, 1, M).astype(np.float32)
    tok, ti, tp, lg = q4.bf16_head_sample(gpu(x), gpu(w), gpu(torch.from_numpy(u)), return_topk=True)
    want_logits = bits(w)[:, ks].T                     # one-hot rows: the weight columns, exactly
    assert np.array_equal(bits(lg), want_logits)
    check_sample(tok, ti, tp, want_logits, 0.8, 30, u.astype(np.float64))
    tok2, lg2 = q4.bf16_head_sample(gpu(x), gpu(w), gpu(torch.from_numpy(u)))
    assert torch.equal(tok2, tok) and torch.equal(lg2.view(torch.int16), lg.view(torch.int16))


def test_sample_signed_zero_ties(q4):
    """-0 and +0 are equal logits: ties go to the lower index."""
    lg = torch.full((1, 10), -5.0, dtype=torch.bfloat16)
    lg[0, 3] = -0.0
    lg[0, 1] = 0.0
    tok, ti, tp = q4.sample_topk(gpu(lg), gpu(torch.zeros(1)), top_k=2, return_topk=True)
    assert ti.cpu().tolist() == [[1, 3]] and int(tok[0]) == 1


def _head_inputs(M, N, K, seed, ties=False):
    """Random activations and a BF16 head; with ties, weights on a coarse grid
    and one-hot activations, so that many logits are exactly equal."""
    if ties:
        w = torch.round(synth.bf16_matrix(N, K, ("head-ties", N, K, seed), std=1.0).float() * 2) / 2
        w = w.to(torch.bfloat16)
        ks = np.random.default_rng(seed).choice(K, size=M, replace=False)
        x = torch.zeros(M, K, dtype=torch.bfloat16)
        x[torch.arange(M), torch.from_numpy(ks)] = 1.0
    else:
        w = synth.bf16_matrix(N, K, ("head-fused", N, K, seed), std=0.05)
        x = synth.x_bf16(M, K, ("head-fused-x", M, K, seed))
    u = np.random.default_rng(seed + 17).uniform(0, 1, M).astype(np.float32)
    u[0] = 0.0
    return x, w, u


FUSED = [(1, 2049, 2048, 30, False), (4, 2049, 2048, 30, False), (1, 16385, 2048, 30, False), (1, 16385, 2048, 64, False),
         (1, 30720, 2048, 64, False), (1, 3000, 1024, 1, False), (1, 5000, 512, 17, False), (1, 64, 2048, 64, False),
         (1, 4097, 4096, 30, False), (1, 2049, 8192, 30, False), (1, 2049, 2048, 30, True), (1, 16385, 2048, 64, True),
         (2, 2049, 2048, 30, True), (48, 16385, 2048, 30, False), (48, 2049, 2048, 30, False), (3, 30720, 2048, 64, False),
         (5, 1025, 2048, 30, False), (2, 1024, 2048, 30, False), (64, 16385, 2048, 64, True), (7, 4097, 4096, 1, True)]


@pytest.mark.parametrize("M,N,K,k,ties", FUSED)
def test_head_sample_one_launch(q4, M, N, K, k, ties):
    """The one-launch head sampling equals the two-launch path bitwise (logits,
    token, top-k indices and probabilities) and the oracle's sampling of its
    logits; repeated calls on the same workspace (never re-zeroed) give the
    same results and leave the arrival counters zero (for one row and a head
    of at most 3072 rows the whole workspace; for a batch, split sampling, the
    first M x 128 bytes)."""
    print(f"head sample one launch: M={M} N={N} K={K} k={k} ties={ties}", flush=True)
    x, w, u = _head_inputs(M, N, K, M * 131 + N + K, ties)
    need = q4.bf16_head_sample_workspace_bytes(M, N, K, k)
    assert (need > 0) == (M == 1 or N > 1024)  # a batch row of one block gains nothing from the split
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    xg, wg, ug = gpu(x), gpu(w), gpu(torch.from_numpy(u))
    ref = q4.bf16_head_sample(xg, wg, ug, top_k=k, return_topk=True)
    for rep in range(3):
        got = q4.bf16_head_sample(xg, wg, ug, top_k=k, return_topk=True, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got[3].view(torch.int16), ref[3].view(torch.int16)), "logits differ from the two-launch path"
        for a, b, name in zip(got[:3], ref[:3], ("token", "topk_index", "topk_prob")):
            assert torch.equal(a, b), f"{name} differs from the two-launch path (call {rep})"
        if M == 1 and N <= 3072:
            assert int(ws.count_nonzero()) == 0, "arrival counters not left at zero"
        elif M > 1:
            assert int(ws[:M * 128].count_nonzero()) == 0, "arrival counters not left at zero"
    check_sample(got[0], got[1], got[2], bits(got[3]), 0.8, k, u.astype(np.float64))
    if ties:
        # one-hot rows: the logits are weight columns, exactly, full of ties
        # (a -0 weight gives a +0 logit: compare with -0 read as +0)
        cols = [int(np.flatnonzero(x.float().numpy()[m])[0]) for m in range(M)]
        have, want = bits(got[3]).copy(), bits(w)[:, cols].T.copy()
        have[have == 0x8000] = 0
        want[want == 0x8000] = 0
        assert np.array_equal(have, want)


def _concentrated_head(M, N, K, pattern, seed):
    """One-hot activations (column m of the head for batch row m), so the logits
    are the head's columns exactly.  "lanes": the largest logits sit at rows
    t + 256 j (t < 16, j < 8) -- a few lanes of the selecting workgroup's first
    wave hold all of them, so the lane-maximum bound leaves more than 64
    candidates and the bit-by-bit threshold runs; "equal": every logit equal
    (entries differ only by index)."""
    w = synth.bf16_matrix(N, K, ("head-conc", N, K, seed), std=0.5)
    cols = list(range(M))
    if pattern == "lanes":
        rows = np.array([t + 256 * j for j in range(8) for t in range(16) if t + 256 * j < N])
        big = torch.from_numpy(np.random.default_rng(seed).permutation(len(rows)).astype(np.float32) * 0.125 + 40.0)
        for c in cols:
            w[torch.from_numpy(rows), c] = big.to(torch.bfloat16)
    else:
        w[:, cols] = 1.5
    x = torch.zeros(M, K, dtype=torch.bfloat16)
    x[torch.arange(M), torch.tensor(cols)] = 1.0
    u = np.random.default_rng(seed + 5).uniform(0, 1, M).astype(np.float32)
    return x, w, u


@pytest.mark.parametrize("M,N,pattern", [(1, 2049, "lanes"), (2, 2049, "lanes"), (48, 2049, "lanes"), (1, 16385, "lanes"),
                                         (3, 16385, "lanes"), (1, 2049, "equal"), (4, 4097, "equal")])
def test_head_sample_concentrated_candidates(q4, M, N, pattern):
    """Selections whose candidates crowd into a few lanes, or tie on every
    logit, in the one-launch and split samplers: equal bitwise to the
    two-launch path (a radix select) and to the oracle's sampling."""
    print(f"head sample concentrated: M={M} N={N} {pattern}", flush=True)
    K, k = 2048, 30
    x, w, u = _concentrated_head(M, N, K, pattern, M * 7 + N)
    ws = torch.zeros(max(q4.bf16_head_sample_workspace_bytes(M, N, K, k), 256), dtype=torch.uint8, device="cuda")
    xg, wg, ug = gpu(x), gpu(w), gpu(torch.from_numpy(u))
    ref = q4.bf16_head_sample(xg, wg, ug, top_k=k, return_topk=True)
    got = q4.bf16_head_sample(xg, wg, ug, top_k=k, return_topk=True, workspace=ws)
    torch.cuda.synchronize()
    for a, b, name in zip(got, ref, ("token", "topk_index", "topk_prob", "logits")):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{name} differs from the two-launch path"
    check_sample(got[0], got[1], got[2], bits(got[3]), 0.8, k, u.astype(np.float64))
    if pattern == "lanes":
        want = np.array(sorted(t + 256 * j for j in range(8) for t in range(16) if t + 256 * j < N))
        assert set(got[1].cpu().numpy()[0].tolist()) <= set(want.tolist())


@pytest.mark.parametrize("M", [1, 48])
def test_head_sample_one_launch_graph_replay(q4, M):
    """The workspace head sampling (one launch at M = 1, the split sampler for
    a batch) captured in a graph and replayed three times, outputs poisoned
    before each replay, equals the eager call."""
    N, K, k = 16385, 2048, 30
    x, w, u = _head_inputs(M, N, K, 5)
    ws = torch.zeros(q4.bf16_head_sample_workspace_bytes(M, N, K, k), dtype=torch.uint8, device="cuda")
    xg, wg, ug = gpu(x), gpu(w), gpu(torch.from_numpy(u))
    tok = torch.empty(M, dtype=torch.int32, device="cuda")
    lg = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    eager = q4.bf16_head_sample(xg, wg, ug, top_k=k, return_topk=True, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = q4.bf16_head_sample(xg, wg, ug, top_k=k, return_topk=True, workspace=ws, logits=lg)
    for r in range(3):
        for t in out[:3]:
            t.fill_(-1)
        lg.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, eager):
            assert a.dtype == b.dtype and torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {r}"
    del g
