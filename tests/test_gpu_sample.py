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
