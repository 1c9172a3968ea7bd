"""Pins for the oracle's speculative-sampling acceptance (rejection sampler).

Values the pages print (tests/golden/spec_sampling.json, each with its
citation), the distribution identity min(q, p) + max(0, p - q) = p checked by
integrating the oracle's decisions over a grid of uniforms, the closed form for
tokens per target pass, the greedy and K = 0 special cases, and the invariant
that a zero-weight token is never drawn.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "spec_sampling.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def grid(n):
    """n midpoints of [0, 1) as float32: (k + 1/2) / n."""
    return ((np.arange(n, dtype=np.float64) + 0.5) / n).astype(np.float32)


def two_token(p0, q0):
    """Target / draft rows over a two-token vocabulary with mass p0 / q0 on token 0."""
    return (np.array([p0, 1 - p0], dtype=np.float32), np.array([q0, 1 - q0], dtype=np.float32))


@pytest.mark.parametrize("ex", golden()["accept_examples"], ids=lambda e: f"p{e['p']}_q{e['q']}")
def test_accept_probability_matches_the_pages(ex):
    n = 3000
    prow, qrow = two_token(ex["p"], ex["q"])
    u = grid(n)
    p = np.broadcast_to(np.stack([prow, prow]), (n, 2, 2))      # position 0 and the bonus row
    q = np.broadcast_to(qrow, (n, 1, 2))
    draft = np.zeros((n, 1), dtype=np.int32)
    tokens, acc = oracle.rejection_sample(p, q, draft, u[:, None], np.full(n, 0.5, np.float32))
    want = ex["accept_probability"][0] / ex["accept_probability"][1]
    assert abs(acc.mean() - want) <= 1.0 / n
    assert set(np.unique(acc)) <= {0, 1}
    assert (tokens[acc == 1, 0] == 0).all()


def test_residual_distribution_of_table_10_6_2():
    g = golden()["residual_table_10_6_2"]
    n = 4000
    prow = np.array(g["p"], dtype=np.float32)
    qrow = np.array(g["q"], dtype=np.float32)
    p = np.broadcast_to(np.stack([prow, prow]), (n, 2, 3))
    q = np.broadcast_to(qrow, (n, 1, 3))
    draft = np.full((n, 1), g["tokens"].index("today"), dtype=np.int32)
    u_acc = np.full((n, 1), 0.9, dtype=np.float32)                    # 0.9 >= 0.1 / 0.5: rejected
    tokens, acc = oracle.rejection_sample(p, q, draft, u_acc, grid(n))
    assert (acc == 0).all()
    freq = np.bincount(tokens[:, 0], minlength=3) / n
    assert np.abs(freq - np.array(g["residual_probability"])).max() <= 1.0 / n
    assert freq[2] == 0.0                                              # 'today' drops out
    assert (tokens[:, 1] == -1).all()


def round_inputs(u_last):
    """The Table 10.6.1 round: vocabulary [and, Machine, Learning, today, everyday,
    tomorrow]; the first three drafts have p >= q, 'today' has q = 0.5, p = 0.1."""
    V = 6
    p = np.zeros((1, 5, V), dtype=np.float32)
    q = np.zeros((1, 4, V), dtype=np.float32)
    for i in range(3):                       # p >= q on the drafted token: always passes
        q[0, i, i], q[0, i, 5] = 0.6, 0.4
        p[0, i, i], p[0, i, 5] = 0.8, 0.2
    q[0, 3, [4, 5, 3]] = [0.2, 0.3, 0.5]      # the rejected position, as in Table 10.6.2
    p[0, 3, [4, 5, 3]] = [0.5, 0.4, 0.1]
    p[0, 4, 4] = 1.0                         # the bonus row
    draft = np.array([[0, 1, 2, 3]], dtype=np.int32)
    u_acc = np.array([[0.99, 0.99, 0.99, u_last]], dtype=np.float32)
    return p, q, draft, u_acc


def test_worked_round_of_table_10_6_1():
    g = golden()["round_table_10_6_1"]
    vocab = ["and", "Machine", "Learning", "today", "everyday", "tomorrow"]
    p, q, draft, u_acc = round_inputs(0.5)                          # 0.5 >= 0.2: 'today' rejected
    tokens, acc = oracle.rejection_sample(p, q, draft, u_acc, np.array([0.3], np.float32))
    assert acc[0] == 3
    assert [vocab[t] for t in tokens[0, :4]] == g["emitted_on_rejection"]
    assert tokens[0, 4] == -1
    p, q, draft, u_acc = round_inputs(0.1)                          # 0.1 < 0.2: all four pass
    tokens, acc = oracle.rejection_sample(p, q, draft, u_acc, np.array([0.3], np.float32))
    assert acc[0] == 4 and (tokens[0] >= 0).sum() == g["tokens_if_all_accepted"]
    assert [vocab[t] for t in tokens[0, :4]] == g["drafts"]
    assert vocab[tokens[0, 4]] == "everyday"                        # the bonus row's only token


def test_acceptance_length_example_with_k3():
    g = golden()["acceptance_length_k3"]
    V = 4
    p = np.zeros((2, 4, V), dtype=np.float32)
    q = np.zeros((2, 3, V), dtype=np.float32)
    p[:, :, 0] = 0.5
    p[:, :, 1] = 0.5
    q[:, :, 0] = 1.0                         # the draft always offers token 0: accept rate 1/2
    draft = np.zeros((2, 3), dtype=np.int32)
    u_acc = np.array([[0.1, 0.2, 0.9], [0.1, 0.2, 0.3]], dtype=np.float32)
    tokens, acc = oracle.rejection_sample(p, q, draft, u_acc, np.array([0.7, 0.7], np.float32))
    assert list(acc) == g["accepted"]
    lengths = (tokens >= 0).sum(axis=1)
    assert list(lengths) == g["lengths"] and lengths.sum() == g["tokens"]
    assert Fraction(int(acc.sum()), 2 * 3) == Fraction(*g["acceptance_rate"])
    assert tokens[0, 2] == 1                 # residual of (0.5, 0.5) - (1, 0) is token 1 alone


def test_tokens_per_forward_closed_form():
    """Drafts pass independently with rate alpha (q one-hot, p = alpha on the draft)."""
    g = golden()["expected_tokens_per_forward"]
    alpha, gamma = g["alpha"], g["gamma"]
    exact = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    assert abs(exact - g["tokens_per_forward"]) < 1e-12
    n = 200_000
    rng = np.random.default_rng(7)
    p = np.zeros((n, gamma + 1, 2), dtype=np.float32)
    p[:, :, 0], p[:, :, 1] = alpha, 1 - alpha
    q = np.zeros((n, gamma, 2), dtype=np.float32)
    q[:, :, 0] = 1.0
    draft = np.zeros((n, gamma), dtype=np.int32)
    u_acc = rng.random((n, gamma), dtype=np.float32)
    tokens, acc = oracle.rejection_sample(p, q, draft, u_acc, rng.random(n, dtype=np.float32))
    per_forward = acc + 1
    # P(accepted = j) = alpha^j (1 - alpha) for j < gamma and alpha^gamma for j = gamma
    probs = np.array([alpha ** j * (1 - alpha) for j in range(gamma)] + [alpha ** gamma])
    sd = np.sqrt(((np.arange(gamma + 1) + 1) ** 2 * probs).sum() - exact ** 2)
    assert abs(per_forward.mean() - exact) < 5 * sd / np.sqrt(n)
    counts = np.bincount(acc, minlength=gamma + 1)
    chi2 = (((counts - n * probs) ** 2) / (n * probs)).sum()
    assert chi2 < 20.5                       # 4 degrees of freedom, p ~ 4e-4
    assert (tokens[acc < gamma, :][np.arange((acc < gamma).sum()), acc[acc < gamma]] == 1).all()


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_emitted_token_follows_p_exactly_on_a_grid(seed):
    """First emitted token: sum over draft tokens x~q and a grid of both uniforms.
    min(q, p) + max(0, p - q) = p means the result is p up to the grid's resolution."""
    rng = np.random.default_rng(seed)
    V, n = 5, 400
    prow = rng.dirichlet(np.ones(V)).astype(np.float32)
    qrow = rng.dirichlet(np.ones(V)).astype(np.float32)
    ua, us = np.meshgrid(grid(n), grid(n), indexing="ij")
    rows = V * n * n
    draft = np.repeat(np.arange(V, dtype=np.int32), n * n)[:, None]
    p = np.broadcast_to(np.stack([prow, prow]), (rows, 2, V))
    q = np.broadcast_to(qrow, (rows, 1, V))
    tokens, _ = oracle.rejection_sample(p, q, draft, np.tile(ua.ravel(), V)[:, None],
                                        np.tile(us.ravel(), V))
    weight = np.repeat(qrow.astype(np.float64), n * n) / (n * n)
    emitted = np.bincount(tokens[:, 0], weights=weight, minlength=V)
    assert np.abs(emitted - prow).max() <= 2.0 / n + 1e-6
    # the two paths separately: accepted mass min(q, p), residual mass max(0, p - q)
    accepted = tokens[:, 0] == draft[:, 0]
    acc_mass = np.bincount(draft[accepted, 0], weights=weight[accepted], minlength=V)
    assert np.abs(acc_mass - np.minimum(qrow, prow)).max() <= 1.0 / n + 1e-6


def test_greedy_one_hot_accepts_only_the_argmax():
    """Temperature 0: p and q one-hot; a draft passes iff it is the target's argmax,
    and a rejection emits the argmax."""
    rng = np.random.default_rng(11)
    B, K, V = 500, 4, 7
    arg = rng.integers(0, V, size=(B, K + 1))
    draft = np.where(rng.random((B, K)) < 0.7, arg[:, :K], rng.integers(0, V, size=(B, K)))
    p = np.zeros((B, K + 1, V), np.float32)
    np.put_along_axis(p, arg[:, :, None], 1.0, axis=2)
    q = np.zeros((B, K, V), np.float32)
    np.put_along_axis(q, draft[:, :, None], 1.0, axis=2)
    tokens, acc = oracle.rejection_sample(p, q, draft.astype(np.int32),
                                          rng.random((B, K), dtype=np.float32),
                                          rng.random(B, dtype=np.float32))
    match = draft == arg[:, :K]
    want = np.where(match.all(axis=1), K, np.argmin(match, axis=1))
    assert (acc == want).all()
    for b in range(B):
        r = acc[b]
        assert (tokens[b, :r] == draft[b, :r]).all() and tokens[b, r] == arg[b, r]


def test_k_zero_is_inverse_cdf_sampling():
    """No drafts: the one token is an inverse-CDF draw from p, which numpy's
    searchsorted over the float64 cumulative sum gives too."""
    rng = np.random.default_rng(12)
    B, V = 2000, 50
    p = rng.dirichlet(np.ones(V), size=B).astype(np.float32)
    p[:, rng.integers(0, V, size=10)] = 0.0
    u = rng.random(B, dtype=np.float32)
    tokens, acc = oracle.rejection_sample(p[:, None, :], np.zeros((B, 0, V), np.float32),
                                          np.zeros((B, 0), np.int32), np.zeros((B, 0), np.float32), u)
    cdf = np.cumsum(p.astype(np.float64), axis=1)
    ref = np.array([np.searchsorted(cdf[b], u[b] * cdf[b, -1], side="right") for b in range(B)])
    assert (acc == 0).all() and (tokens[:, 0] == ref).all()


def test_zero_weight_tokens_are_never_drawn_and_the_extremes():
    V = 8
    p = np.array([[[0, 0, 0.25, 0, 0.5, 0, 0.25, 0], [0, 0.5, 0, 0, 0, 0, 0.5, 0]]], np.float32)
    q = np.array([[[0, 0, 0.5, 0, 0.25, 0, 0.25, 0]]], np.float32)
    draft = np.array([[2]], np.int32)
    top = np.float32(np.nextafter(np.float32(1), np.float32(0)))
    for u_s, want in ((0.0, 4), (top, 4)):              # residual = token 4 alone
        tokens, acc = oracle.rejection_sample(p, q, draft, np.array([[0.75]], np.float32),
                                              np.array([u_s], np.float32))
        assert acc[0] == 0 and tokens[0, 0] == want
    for u_s, want in ((0.0, 1), (top, 6)):              # bonus row: first and last positive
        tokens, acc = oracle.rejection_sample(p, q, draft, np.array([[0.25]], np.float32),
                                              np.array([u_s], np.float32))
        assert acc[0] == 1 and tokens[0, 1] == want
    # p >= q: accepted even for the largest uniform below 1
    tokens, acc = oracle.rejection_sample(p, p[:, :1], draft, np.array([[top]], np.float32),
                                          np.array([0.5], np.float32))
    assert acc[0] == 1


def test_no_residual_mass_falls_back_to_p():
    """p == q at a rejected position (only possible when p(x) = 0 = q(x) style ties):
    the residual is empty and the token is drawn from p."""
    p = np.array([[[0.0, 0.5, 0.5], [1, 0, 0]]], np.float32)
    q = p[:, :1].copy()
    tokens, acc = oracle.rejection_sample(p, q, np.array([[0]], np.int32),
                                          np.array([[0.5]], np.float32), np.array([0.75], np.float32))
    assert acc[0] == 0 and tokens[0, 0] == 2


def test_rejects_out_of_range_drafts():
    p = np.full((1, 2, 3), 1 / 3, np.float32)
    with pytest.raises(ValueError):
        oracle.rejection_sample(p, p[:, :1], np.array([[3]], np.int32),
                                np.array([[0.5]], np.float32), np.array([0.5], np.float32))


# ----------------------------------------------------------------------------
# the draw is exact: pinned against rational arithmetic (Python's fractions)
# ----------------------------------------------------------------------------
def fraction_reference(p, q, draft, u_accept, u_sample):
    """The acceptance step written out over exact rationals: the draft tests
    u * q(x) < p(x), then the first j whose running sum of the weights exceeds
    u * (their total), with p, q and u taken at their exact float32 values."""
    B, k1, V = p.shape
    K = k1 - 1
    tokens = np.full((B, k1), -1, dtype=np.int64)
    acc = np.zeros(B, dtype=np.int64)

    def inverse_cdf(w, u):
        total = sum(w, Fraction(0))
        if total == 0:
            return -1
        target = Fraction(float(u)) * total
        run = Fraction(0)
        for j, wj in enumerate(w):
            run += wj
            if run > target:
                return j
        raise AssertionError("running sum never passed the target")

    for b in range(B):
        r = 0
        while r < K:
            x = int(draft[b, r])
            if not Fraction(float(u_accept[b, r])) * Fraction(float(q[b, r, x])) < \
                    Fraction(float(p[b, r, x])):
                break
            tokens[b, r] = x
            r += 1
        acc[b] = r
        prow = [Fraction(float(v)) for v in p[b, r]]
        if r < K:
            qrow = [Fraction(float(v)) for v in q[b, r]]
            tok = inverse_cdf([max(Fraction(0), a - c) for a, c in zip(prow, qrow)], u_sample[b])
            if tok < 0:
                tok = inverse_cdf(prow, u_sample[b])
        else:
            tok = inverse_cdf(prow, u_sample[b])
        tokens[b, r] = tok
    return tokens, acc


def wide_range_rows(rng, shape):
    """float32 values spread over the whole non-negative range below 2^22:
    subnormals, tiny normals, ordinary probabilities and large values, zeros."""
    mant = rng.integers(1 << 23, 1 << 24, size=shape).astype(np.float64)
    expo = rng.choice([-170, -149, -140, -126, -100, -60, -30, -20, -10, -3, 0, 8],
                      size=shape) + rng.integers(-3, 4, size=shape)
    vals = np.ldexp(mant, expo - 23).astype(np.float32)
    vals[rng.random(shape) < 0.2] = 0.0
    return vals


@pytest.mark.parametrize("seed", [21, 22, 23, 24])
def test_draw_equals_rational_reference(seed):
    rng = np.random.default_rng(seed)
    B, K, V = 200, 3, 24
    p = wide_range_rows(rng, (B, K + 1, V))
    q = wide_range_rows(rng, (B, K, V))
    draft = rng.integers(0, V, size=(B, K)).astype(np.int32)
    # some drafts pass for sure (q = 0 at the draft) and some rows have an empty residual
    q[:B // 4, :, :] = np.where(np.arange(V)[None, None, :] == draft[:B // 4, :, None], 0.0,
                                q[:B // 4])
    q[B // 4:B // 4 + 10, 0] = p[B // 4:B // 4 + 10, 0]
    p[B // 4 + 10:B // 4 + 15] = 0.0                         # no mass at all: -1
    ua = rng.random((B, K), dtype=np.float32)
    us = rng.random(B, dtype=np.float32)
    us[:20] = np.float32(0.0)
    us[20:40] = np.float32(np.nextafter(np.float32(1), np.float32(0)))
    tokens, acc = oracle.rejection_sample(p, q, draft, ua, us)
    want_t, want_a = fraction_reference(p, q, draft, ua, us)
    assert (acc == want_a).all()
    assert (tokens == want_t).all()


def test_ties_at_running_sum_boundaries():
    """u * total equal to a running sum: that entry is not drawn (the sum must
    exceed the target), the next positive one is."""
    p = np.array([[[0.25, 0.0, 0.25, 0.5]]], np.float32)
    none = np.zeros((1, 0, 4), np.float32)
    for u, want in ((0.0, 0), (0.25, 2), (0.5, 3), (0.75, 3)):
        tokens, _ = oracle.rejection_sample(p, none, np.zeros((1, 0), np.int32),
                                            np.zeros((1, 0), np.float32), np.array([u], np.float32))
        assert tokens[0, 0] == want, (u, tokens)


def test_draw_keeps_weights_that_binary64_sums_lose():
    """Weights 1/2, 2^-80, 1/2 with u = 1/2: the target is 1/2 + 2^-81, which the
    first running sum (1/2) does not exceed and the second (1/2 + 2^-80) does.
    Summed in binary64, 1/2 + 2^-80 rounds to 1/2 and the third token comes out."""
    p = np.array([[[0.5, 2.0 ** -80, 0.5]]], np.float32)
    none = np.zeros((1, 0, 3), np.float32)
    tokens, _ = oracle.rejection_sample(p, none, np.zeros((1, 0), np.int32),
                                        np.zeros((1, 0), np.float32), np.array([0.5], np.float32))
    assert tokens[0, 0] == 1
    cdf = np.cumsum(p[0, 0].astype(np.float64))
    assert np.searchsorted(cdf, 0.5 * cdf[-1], side="right") == 2     # what binary64 gives


def test_residual_is_exact_below_binary64_resolution():
    """p - q formed exactly: p = 1 + 2^-23 and q = 2^-140 at token 0, p = 2^-130 at
    token 1 (q = 0).  With u = 2^-1 the target is far inside token 0; with u the
    largest float32 below 1 it still is (token 0's share is 1 - 2^-130ish)."""
    p = np.array([[[np.float32(1 + 2.0 ** -23), np.float32(2.0 ** -130)], [1.0, 0.0]]], np.float32)
    q = np.array([[[np.float32(2.0 ** -140), 0.0]]], np.float32)
    draft = np.array([[0]], np.int32)
    top = np.float32(np.nextafter(np.float32(1), np.float32(0)))
    for u in (np.float32(0.5), top):
        tokens, acc = oracle.rejection_sample(p, q, draft, np.array([[top]], np.float32),
                                              np.array([u], np.float32))
        want_t, want_a = fraction_reference(p, q, draft, np.array([[top]], np.float32),
                                            np.array([u], np.float32))
        assert acc[0] == want_a[0] and tokens[0, 0] == want_t[0, 0]


def test_rejects_negative_or_nonfinite_probabilities():
    p = np.full((1, 2, 3), 1 / 3, np.float32)
    for bad in (-0.1, np.inf, np.nan):
        pb = p.copy()
        pb[0, 1, 2] = bad
        with pytest.raises(ValueError):
            oracle.rejection_sample(pb, p[:, :1], np.array([[0]], np.int32),
                                    np.array([[0.5]], np.float32), np.array([0.5], np.float32))


@pytest.mark.parametrize("seed", [31, 32])
def test_targets_inside_weights_binary64_cannot_hold(seed):
    """Rows 1/2, t_1, ..., t_n, 1/2 with tiny t_i (2^-90 .. 2^-60) and u = 1/2: the
    target 1/2 + (t_1 + ... + t_n) / 2 falls among the tiny tokens, where the
    rational reference and the oracle agree; binary64 running sums never leave 1/2
    there and would give the last token."""
    rng = np.random.default_rng(seed)
    B, n = 64, 30
    V = n + 2
    p = np.zeros((B, 1, V), np.float32)
    p[:, 0, 0] = p[:, 0, -1] = 0.5
    mant = rng.integers(1 << 23, 1 << 24, size=(B, n)).astype(np.float64)
    p[:, 0, 1:-1] = np.ldexp(mant, rng.integers(-90, -60, size=(B, n)) - 23).astype(np.float32)
    none = np.zeros((B, 0, V), np.float32)
    us = np.full(B, 0.5, np.float32)
    tokens, _ = oracle.rejection_sample(p, none, np.zeros((B, 0), np.int32),
                                        np.zeros((B, 0), np.float32), us)
    want, _ = fraction_reference(p, none, np.zeros((B, 0), np.int32), np.zeros((B, 0)), us)
    assert (tokens == want).all()
    assert ((tokens[:, 0] >= 1) & (tokens[:, 0] <= n)).all()
