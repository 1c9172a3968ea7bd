"""GPU speculative-sampling acceptance against the oracle.

The number of accepted drafts is decided exactly (u * q < p in binary64 on
both sides) and must match bit for bit.  The sampled token is an inverse-CDF
decision on binary64 running sums that the two sides associate differently;
it must match except where u * total lies within a few ulps of a running-sum
boundary, and there the GPU's token must still be a valid draw (positive
weight, boundary straddles the target within that bound).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_kv_gqa_02_amd as lib
    return lib


def say(msg):
    print(msg, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_sample(pa, c):
    say(f"[gpu sample] B={c.batch} K={c.num_drafts} V={c.vocab}")
    k = c.num_drafts
    tokens, acc = pa.paged_attn_rejection_sample(
        dev(c.p), dev(c.q) if k else None, dev(c.draft) if k else None,
        dev(c.u_accept) if k else None, dev(c.u_sample))
    torch.cuda.synchronize()
    return tokens.cpu().numpy(), acc.cpu().numpy()


def weights(c, b, r):
    p = c.p[b, r].astype(np.float64)
    if r == c.num_drafts:
        return p
    w = np.maximum(p - c.q[b, r].astype(np.float64), 0.0)
    return w if w.sum() > 0 else p


def valid_draw(w, u, j):
    """j is an inverse-CDF draw for uniform u up to binary64 summation error."""
    if j < 0 or j >= len(w) or w[j] <= 0:
        return False
    cdf = np.cumsum(w)
    total = cdf[-1]
    slack = 4 * len(w) * np.finfo(np.float64).eps * total
    target = float(u) * total
    lo = cdf[j - 1] if j > 0 else 0.0
    return lo <= target + slack and cdf[j] > target - slack


def check(c, got, want):
    (tg, ag), (tw, aw) = got, want
    assert (ag == aw).all(), f"accepted counts differ at {np.nonzero(ag != aw)[0][:8]}"
    k = c.num_drafts
    for b in np.nonzero((tg != tw).any(axis=1))[0]:
        r = aw[b]
        assert (tg[b, :r] == tw[b, :r]).all() and (tg[b, r + 1:] == -1).all()
        assert valid_draw(weights(c, b, r), c.u_sample[b], tg[b, r]), \
            f"sequence {b}: GPU token {tg[b, r]} vs oracle {tw[b, r]} is not a near tie"
    return int(((tg != tw).any(axis=1)).sum()) if k >= 0 else 0


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_matches_oracle_at_8b_vocab(pa, seed):
    c = W.sampler_inputs(16, 4, W.VOCAB_8B, seed)
    ties = check(c, gpu_sample(pa, c), oracle.rejection_sample(c.p, c.q, c.draft, c.u_accept,
                                                               c.u_sample))
    assert ties == 0


@pytest.mark.parametrize("batch", [64, 8])
def test_matches_oracle_at_the_bench_configurations(pa, batch):
    """The inputs bench.py --op sample times (same generator and seed)."""
    c = W.sampler_inputs(batch, 4, W.VOCAB_8B, 20261202)
    check(c, gpu_sample(pa, c), oracle.rejection_sample(c.p, c.q, c.draft, c.u_accept, c.u_sample))


@pytest.mark.parametrize("B,K,V", [(1, 0, 1), (3, 1, 7), (5, 4, 4095), (5, 4, 4096), (5, 4, 4097),
                                   (7, 3, 8193), (4, 64, 300), (9, 0, 50000), (2, 7, 1 << 20)])
def test_matches_oracle_at_edge_shapes(pa, B, K, V):
    c = W.sampler_inputs(B, K, V, 100 + K + V)
    check(c, gpu_sample(pa, c), oracle.rejection_sample(c.p, c.q, c.draft, c.u_accept,
                                                        c.u_sample))


def test_greedy_one_hot(pa):
    c = W.sampler_inputs(32, 4, 3000, 5, greedy=True)
    got = gpu_sample(pa, c)
    check(c, got, oracle.rejection_sample(c.p, c.q, c.draft, c.u_accept, c.u_sample))
    tokens, acc = got
    arg = c.p.argmax(axis=-1)
    for b in range(c.batch):
        assert tokens[b, acc[b]] == arg[b, acc[b]]


def test_all_accepted_all_rejected_and_empty_residual(pa):
    c = W.sampler_inputs(12, 4, 5000, 6)
    c.q[:4] = c.p[:4, :4]                        # q == p: every draft passes, bonus row used
    c.p[4:8, np.arange(4)[:, None], c.draft[4:8].T] = 0.0   # p = 0 on the drafts: first rejected
    c.q[8:] = c.p[8:, :4]                        # q == p and p = q = 0 on the draft:
    for b in range(8, 12):                       # rejected with an empty residual -> p
        c.p[b, 0, c.draft[b, 0]] = 0.0
        c.q[b, 0, c.draft[b, 0]] = 0.0
    got = gpu_sample(pa, c)
    want = oracle.rejection_sample(c.p, c.q, c.draft, c.u_accept, c.u_sample)
    check(c, got, want)
    assert (got[1][:4] == 4).all() and (got[1][4:] == 0).all()


def test_tokens_per_forward_closed_form_on_gpu(pa):
    """Drafts pass independently with rate 0.8 (q one-hot, p = 0.8 on the draft):
    tokens per target pass average (1 - 0.8^5) / (1 - 0.8) = 3.36."""
    n, gamma, alpha = 65535, 4, 0.8
    rng = np.random.default_rng(21)
    p = np.zeros((n, gamma + 1, 2), np.float32)
    p[:, :, 0], p[:, :, 1] = alpha, 1 - alpha
    q = np.zeros((n, gamma, 2), np.float32)
    q[:, :, 0] = 1.0
    c = W.SamplerCase(p=p, q=q, draft=np.zeros((n, gamma), np.int32),
                      u_accept=rng.random((n, gamma), dtype=np.float32),
                      u_sample=rng.random(n, dtype=np.float32))
    got = gpu_sample(pa, c)
    check(c, got, oracle.rejection_sample(c.p, c.q, c.draft, c.u_accept, c.u_sample))
    exact = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    assert abs((got[1] + 1).mean() - exact) < 0.02


def test_emitted_distribution_is_p_on_a_grid(pa):
    V, n = 5, 100
    rng = np.random.default_rng(22)
    prow = rng.dirichlet(np.ones(V)).astype(np.float32)
    qrow = rng.dirichlet(np.ones(V)).astype(np.float32)
    g = ((np.arange(n) + 0.5) / n).astype(np.float32)
    ua, us = np.meshgrid(g, g, indexing="ij")
    rows = V * n * n
    c = W.SamplerCase(p=np.ascontiguousarray(np.broadcast_to(np.stack([prow, prow]), (rows, 2, V))),
                      q=np.ascontiguousarray(np.broadcast_to(qrow, (rows, 1, V))),
                      draft=np.repeat(np.arange(V, dtype=np.int32), n * n)[:, None],
                      u_accept=np.tile(ua.ravel(), V)[:, None].astype(np.float32),
                      u_sample=np.tile(us.ravel(), V).astype(np.float32))
    got = gpu_sample(pa, c)
    check(c, got, oracle.rejection_sample(c.p, c.q, c.draft, c.u_accept, c.u_sample))
    w = np.repeat(qrow.astype(np.float64), n * n) / (n * n)
    emitted = np.bincount(got[0][:, 0], weights=w, minlength=V)
    assert np.abs(emitted - prow).max() <= 2.0 / n + 1e-6


def test_repeat_calls_are_identical(pa):
    c = W.sampler_inputs(8, 4, 20000, 7)
    a, b = gpu_sample(pa, c), gpu_sample(pa, c)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()
