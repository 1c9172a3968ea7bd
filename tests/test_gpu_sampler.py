"""GPU speculative-sampling acceptance against the oracle, bit for bit.

The number of accepted drafts is decided exactly (u * q < p in binary64 on
both sides).  The sampled token is the first j whose running sum of the
weights exceeds u * their total, which both sides decide exactly (integers in
units of 2^-149: multi-limb comparisons in the oracle, exact column sums in
the kernels), so tokens must be equal everywhere.
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


def check(c, got, want):
    (tg, ag), (tw, aw) = got, want
    assert (ag == aw).all(), f"accepted counts differ at {np.nonzero(ag != aw)[0][:8]}"
    bad = np.nonzero((tg != tw).any(axis=1))[0]
    assert len(bad) == 0, (f"tokens differ at sequences {bad[:8]}: GPU {tg[bad[:4]]} "
                           f"oracle {tw[bad[:4]]}")


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_matches_oracle_at_8b_vocab(pa, seed):
    c = W.sampler_inputs(16, 4, W.VOCAB_8B, seed)
    check(c, gpu_sample(pa, c), oracle.rejection_sample(c.p, c.q, c.draft, c.u_accept,
                                                        c.u_sample))


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


def no_drafts(p, u):
    B, _, V = p.shape
    return W.SamplerCase(p=np.ascontiguousarray(p, dtype=np.float32),
                         q=np.zeros((B, 0, V), np.float32), draft=np.zeros((B, 0), np.int32),
                         u_accept=np.zeros((B, 0), np.float32),
                         u_sample=np.asarray(u, dtype=np.float32))


def test_ties_at_running_sum_boundaries(pa):
    """u * total equal to a running sum: the draw moves on to the next positive weight."""
    p = np.broadcast_to(np.array([0.25, 0.0, 0.25, 0.5], np.float32), (4, 1, 4))
    c = no_drafts(p, [0.0, 0.25, 0.5, 0.75])
    got = gpu_sample(pa, c)
    check(c, got, oracle.rejection_sample(c.p, c.q, c.draft, c.u_accept, c.u_sample))
    assert list(got[0][:, 0]) == [0, 2, 3, 3]


@pytest.mark.parametrize("V,where", [(3, 1), (5000, 4095), (9000, 4096), (70000, 65536 + 63)])
def test_targets_inside_weights_binary64_cannot_hold(pa, V, where):
    """1/2 on token 0 and the last token, tiny weights (2^-90 .. 2^-60) in a run
    starting at `where` (across lane-run and chunk edges), u = 1/2: the target
    lies among the tiny weights, which binary64 running sums would not see."""
    rng = np.random.default_rng(V)
    B, n = 16, min(200, V - 2)
    where = min(where, V - 1 - n)
    p = np.zeros((B, 1, V), np.float32)
    p[:, 0, 0] = p[:, 0, -1] = 0.5
    mant = rng.integers(1 << 23, 1 << 24, size=(B, n)).astype(np.float64)
    p[:, 0, where:where + n] = np.ldexp(mant, rng.integers(-90, -60, size=(B, n)) - 23)
    c = no_drafts(p, np.full(B, 0.5))
    got = gpu_sample(pa, c)
    check(c, got, oracle.rejection_sample(c.p, c.q, c.draft, c.u_accept, c.u_sample))
    assert ((got[0][:, 0] >= where) & (got[0][:, 0] < where + n)).all()


def wide_rows(rng, shape):
    mant = rng.integers(1 << 23, 1 << 24, size=shape).astype(np.float64)
    expo = rng.choice([-170, -149, -140, -126, -100, -60, -30, -20, -10, -3, 0, 8],
                      size=shape) + rng.integers(-3, 4, size=shape)
    vals = np.ldexp(mant, expo - 23).astype(np.float32)
    vals[rng.random(shape) < 0.2] = 0.0
    return vals


@pytest.mark.parametrize("V", [24, 4100, 12289])
def test_wide_exponent_range_rows(pa, V):
    """Entries from subnormals to 2^8 (every exponent bucket of the kernel), p - q
    residuals, empty residuals, rows with no mass, and the extreme uniforms."""
    rng = np.random.default_rng(V + 5)
    B, K = 48, 3
    p = wide_rows(rng, (B, K + 1, V))
    q = wide_rows(rng, (B, K, V))
    draft = rng.integers(0, V, size=(B, K)).astype(np.int32)
    q[:12] = np.where(np.arange(V)[None, None, :] == draft[:12, :, None], 0.0, q[:12])
    q[12:16, 0] = p[12:16, 0]
    p[16:18] = 0.0
    us = rng.random(B, dtype=np.float32)
    us[:6] = 0.0
    us[6:12] = np.nextafter(np.float32(1), np.float32(0))
    c = W.SamplerCase(p=p, q=q, draft=draft, u_accept=rng.random((B, K), dtype=np.float32),
                      u_sample=us)
    check(c, gpu_sample(pa, c), oracle.rejection_sample(c.p, c.q, c.draft, c.u_accept,
                                                        c.u_sample))
