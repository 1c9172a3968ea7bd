"""Pins for the CPU oracle: closed forms, invariants, spec values, printed figures.

Each test checks the oracle against something other than itself, chosen so
that a plausible slip (a dropped term, a wrong index, a transposed operand, an
off-by-one in the causal limit, a wrong head mapping) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------
# element decoders
# ----------------------------------------------------------------------------
def test_bf16_decoder_spec_values():
    assert oracle.bf16_value(0x3F80) == 1.0
    assert oracle.bf16_value(0xC000) == -2.0
    assert oracle.bf16_value(0x0001) == 2.0 ** -133          # smallest subnormal
    assert oracle.bf16_value(0x0080) == 2.0 ** -126          # smallest normal
    assert oracle.bf16_value(0x7F7F) == (2 - 2 ** -7) * 2.0 ** 127
    assert math.isinf(oracle.bf16_value(0x7F80))
    assert math.isnan(oracle.bf16_value(0x7FC0))


def test_bf16_decoder_matches_torch_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    ours = np.array([oracle.bf16_value(int(b)) for b in bits])
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_e4m3_decoder_spec_values():
    # OCP OFP8 E4M3: bias 7, subnormals m/8 * 2^-6, max 448, S.1111.111 = NaN
    assert oracle.e4m3_value(0x00) == 0.0
    assert math.copysign(1.0, oracle.e4m3_value(0x80)) == -1.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x40) == 2.0
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0xFE) == -448.0
    assert math.isnan(oracle.e4m3_value(0x7F))
    assert math.isnan(oracle.e4m3_value(0xFF))
    vals = [oracle.e4m3_value(b) for b in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))         # strictly increasing


def test_e4m3_decoder_matches_torch_all_bytes():
    byts = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(byts).view(torch.float8_e4m3fn).double().numpy()
    ours = np.array([oracle.e4m3_value(int(b)) for b in byts])
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


# ----------------------------------------------------------------------------
# input encoders (workloads) checked against the oracle's decoders and torch
# ----------------------------------------------------------------------------
def test_e4m3_encoder_round_trips_every_finite_byte():
    finite = [b for b in range(256) if b not in (0x7F, 0xFF)]
    vals = np.array([oracle.e4m3_value(b) for b in finite])
    assert (W.e4m3_bytes(vals) == np.array(finite, dtype=np.uint8)).all()


def test_e4m3_encoder_ties_to_even_and_saturates():
    # midpoint between 1.0 (0x38) and 1.125 (0x39) -> even mantissa 0x38
    assert W.e4m3_bytes(np.array([1.0625]))[0] == 0x38
    # midpoint between 1.125 (0x39) and 1.25 (0x3A) -> 0x3A
    assert W.e4m3_bytes(np.array([1.1875]))[0] == 0x3A
    # subnormal midpoint 1.5 * 2^-9 -> 2 * 2^-9 (even)
    assert W.e4m3_bytes(np.array([1.5 * 2.0 ** -9]))[0] == 0x02
    assert W.e4m3_bytes(np.array([500.0, -1e9, 448.0]))[0] == 0x7E
    assert W.e4m3_bytes(np.array([-1e9]))[0] == 0xFE


def _e4m3_table():
    codes = np.array([b for b in range(256) if b not in (0x7F, 0xFF)])
    return codes, np.array([oracle.e4m3_value(int(b)) for b in codes])


def test_e4m3_encoder_is_nearest_value_ties_to_even():
    # brute force: the encoded byte decodes to the finite E4M3 value nearest x;
    # on an exact tie the even code wins
    codes, vals = _e4m3_table()
    x = np.concatenate([_rng(1).standard_normal(20000) * 60,
                        _rng(2).standard_normal(5000) * 0.01,
                        (vals[1:] + vals[:-1]) / 2])               # every midpoint
    x = x[np.abs(x) <= 448]
    enc = W.e4m3_bytes(x)
    dec = np.array([oracle.e4m3_value(int(b)) for b in enc])
    dist = np.abs(x[:, None] - vals[None, :])
    best = dist.min(axis=1)
    assert (np.abs(x - dec) == best).all()
    tie = (dist == best[:, None]).sum(axis=1) > 1
    tie_codes = enc[tie]
    nonzero = np.array([oracle.e4m3_value(int(b)) != 0 for b in tie_codes])
    assert (tie_codes[nonzero] % 2 == 0).all()


def test_bf16_rounding_is_nearest_ties_to_even():
    x = _rng(2).standard_normal(200000).astype(np.float32)
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000], dtype=np.uint32).view(np.float32)
    bits = W.bf16_bits(np.concatenate([x, ties]))
    dec = np.array([oracle.bf16_value(int(b)) for b in bits[-3:]])
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: the even pattern 0x3F80 wins
    assert list(bits[-3:]) == [0x3F80, 0x3F82, 0xBF80]
    assert dec[0] == 1.0
    # every other value is within half a bf16 ulp
    vals = (bits[:-3].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(np.abs(x))[1] - 8)
    assert (np.abs(vals - x) <= ulp / 2).all()
    assert (W.bf16_bits(np.array([np.nan], dtype=np.float32)) == 0x7FC0).all()


# ----------------------------------------------------------------------------
# attention closed forms
# ----------------------------------------------------------------------------
def _rand_qkv(seed, L, n, hq, hkv, d):
    r = _rng(seed)
    return (r.standard_normal((n, hq, d)), r.standard_normal((L, hkv, d)),
            r.standard_normal((L, hkv, d)))


def test_two_key_hand_example():
    # D = 1, scale = 1: z = (0, ln 3) -> weights 1/4, 3/4
    q = np.array([[[1.0]]])
    k = np.array([[[0.0]], [[math.log(3.0)]]])
    v = np.array([[[2.0]], [[6.0]]])
    out = oracle.attention(q, k, v, 1.0)
    assert abs(out[0, 0, 0] - (0.25 * 2 + 0.75 * 6)) < 1e-15


@pytest.mark.parametrize("n", [1, 3])
def test_identical_keys_give_mean_of_visible_values(n):
    L, hq, hkv, d = 37, 6, 2, 16
    q, _, v = _rand_qkv(3, L, n, hq, hkv, d)
    k = np.broadcast_to(_rng(4).standard_normal((1, hkv, d)), (L, hkv, d))
    out = oracle.attention(q, k, v, 0.3)
    g = hq // hkv
    for i in range(n):
        vis = L - n + i + 1
        for h in range(hq):
            np.testing.assert_allclose(out[i, h], v[:vis, h // g].mean(axis=0),
                                       rtol=0, atol=1e-13)


def test_zero_scale_gives_mean():
    q, k, v = _rand_qkv(5, 29, 2, 4, 4, 8)
    out = oracle.attention(q, k, v, 0.0)
    np.testing.assert_allclose(out[0], v[:28].mean(axis=0), atol=1e-13)
    np.testing.assert_allclose(out[1], v[:29].mean(axis=0), atol=1e-13)


def test_single_key_returns_its_value():
    q, k, v = _rand_qkv(6, 1, 1, 8, 2, 128)
    out = oracle.attention(q, k, v, 1 / math.sqrt(128))
    for h in range(8):
        assert (out[0, h] == v[0, h // 4]).all()


def test_one_hot_logit_selects_value_row():
    L, hq, hkv, d = 300, 4, 1, 64
    r = _rng(7)
    u = r.standard_normal(d)
    q = np.broadcast_to(u, (1, hq, d)).copy()
    k = np.zeros((L, hkv, d))
    jstar = 123
    s = 1 / math.sqrt(d)
    lam = (30 + math.log(L)) / (s * (u @ u))
    k[jstar, 0] = lam * u
    v = r.standard_normal((L, hkv, d))
    out = oracle.attention(q, k, v, s)
    for h in range(hq):
        np.testing.assert_allclose(out[0, h], v[jstar, 0], atol=1e-11)


def test_linear_in_values():
    q, k, v1 = _rand_qkv(8, 50, 2, 8, 2, 32)
    v2 = _rng(9).standard_normal(v1.shape)
    a, b = 0.7, -1.9
    lhs = oracle.attention(q, k, a * v1 + b * v2, 0.2)
    rhs = a * oracle.attention(q, k, v1, 0.2) + b * oracle.attention(q, k, v2, 0.2)
    np.testing.assert_allclose(lhs, rhs, atol=1e-12)


def test_invariant_under_common_key_shift():
    q, k, v = _rand_qkv(10, 64, 1, 8, 2, 32)
    c = _rng(11).standard_normal((1, 2, 32))
    np.testing.assert_allclose(oracle.attention(q, k + c, v, 0.25),
                               oracle.attention(q, k, v, 0.25), atol=1e-12)


def test_gqa_head_mapping_is_floor_h_over_g():
    L, hq, hkv, d = 40, 12, 3, 16
    q, k, _ = _rand_qkv(12, L, 2, hq, hkv, d)
    v = np.zeros((L, hkv, d))
    for hk in range(hkv):
        v[:, hk, :] = hk
    out = oracle.attention(q, k, v, 0.5)
    for h in range(hq):
        assert np.all(out[:, h] == h // (hq // hkv))


def test_gqa_is_per_group_single_head_attention():
    L, hq, hkv, d = 33, 8, 2, 16
    q, k, v = _rand_qkv(13, L, 3, hq, hkv, d)
    out = oracle.attention(q, k, v, 0.4)
    g = hq // hkv
    for h in range(hq):
        one = oracle.attention(q[:, h:h + 1], k[:, h // g:h // g + 1],
                               v[:, h // g:h // g + 1], 0.4)
        assert (one[:, 0] == out[:, h]).all()


def test_verify_row_equals_decode_at_its_position():
    L, n, hq, hkv, d = 70, 5, 8, 2, 32
    q, k, v = _rand_qkv(14, L, n, hq, hkv, d)
    out = oracle.attention(q, k, v, 0.3)
    for i in range(n):
        lp = L - n + i + 1
        dec = oracle.attention(q[i:i + 1], k[:lp], v[:lp], 0.3)
        assert (dec[0] == out[i]).all()


def test_verify_rows_do_not_see_later_drafts():
    L, n, hq, hkv, d = 50, 5, 4, 2, 16
    q, k, v = _rand_qkv(15, L, n, hq, hkv, d)
    base = oracle.attention(q, k, v, 0.3)
    j = 3                                    # perturb the key/value of draft row j
    k2, v2 = k.copy(), v.copy()
    k2[L - n + j] += 5.0
    v2[L - n + j] -= 7.0
    pert = oracle.attention(q, k2, v2, 0.3)
    assert (pert[:j] == base[:j]).all()
    assert not np.allclose(pert[j:], base[j:])


def test_rejects_bad_arguments():
    q, k, v = _rand_qkv(16, 4, 5, 4, 2, 8)   # n = 5 > L = 4
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, 1.0)


# ----------------------------------------------------------------------------
# paged lookup
# ----------------------------------------------------------------------------
def _scatter(kc, vc, tables, num_pages, fill=np.nan):
    """Place each sequence's contiguous K/V [L][Hkv][D] at its table's pages."""
    hkv, d = kc[0].shape[1:]
    kp = np.full((num_pages, hkv, 16, d), fill, dtype=np.float32)
    vp = np.full((num_pages, hkv, 16, d), fill, dtype=np.float32)
    for kk, vv, tab in zip(kc, vc, tables):
        for t in range(kk.shape[0]):
            kp[tab[t // 16], :, t % 16] = kk[t]
            vp[tab[t // 16], :, t % 16] = vv[t]
    return W.k_to_pool(kp), vp


def _table(tabs):
    width = max(len(t) for t in tabs)
    out = np.full((len(tabs), width), -1, dtype=np.int32)
    for b, t in enumerate(tabs):
        out[b, :len(t)] = t
    return out


def test_paged_lookup_follows_figure_10_4_2():
    fix = json.load(open(os.path.join(GOLDEN, "block_table_fig_10_4_2.json")))
    tab = fix["logical_to_physical"]
    L, hq, hkv, d = 40, 4, 2, 16                      # 3 pages, the last partial
    r = _rng(17)
    kc = r.standard_normal((L, hkv, d)).astype(np.float32)
    vc = r.standard_normal((L, hkv, d)).astype(np.float32)
    q = r.standard_normal((1, 1, hq, d)).astype(np.float32)
    kp, vp = _scatter([kc], [vc], [tab], 16)          # every other slot is NaN
    got = oracle.paged_attention(kp, vp, "f32", q, "f32", _table([tab]), [L], 1, 0.3)
    want = oracle.attention(q[0], kc, vc, 0.3)
    assert (got[0] == want).all()


def test_paged_lookup_shared_pool_figure_10_12_2():
    fix = json.load(open(os.path.join(GOLDEN, "shared_pool_fig_10_12_2.json")))
    tabs = [[x - 1 for x in fix["tables"][k]] for k in ("A", "B", "C")]
    lens = [16 * len(t) - 3 for t in tabs]
    hq, hkv, d = 4, 1, 8
    r = _rng(18)
    kc = [r.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    vc = [r.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    q = r.standard_normal((3, 1, hq, d)).astype(np.float32)
    kp, vp = _scatter(kc, vc, tabs, fix["pool_blocks"])
    got = oracle.paged_attention(kp, vp, "f32", q, "f32", _table(tabs), lens, 1, 0.5)
    for b in range(3):
        assert (got[b] == oracle.attention(q[b], kc[b], vc[b], 0.5)).all()
    free = [x - 1 for x in fix["free"]]
    assert np.isnan(kp[free]).all()                   # free blocks were never read


def test_shared_prefix_blocks_figure_10_12_2b():
    fix = json.load(open(os.path.join(GOLDEN, "shared_pool_fig_10_12_2.json")))["shared_prefix"]
    common = [x - 1 for x in fix["common"]]
    tabs = [common + [fix[k][0] - 1] for k in ("A", "B", "C")]
    hq, hkv, d, L = 4, 2, 8, 40
    r = _rng(19)
    pre_k = r.standard_normal((32, hkv, d)).astype(np.float32)
    pre_v = r.standard_normal((32, hkv, d)).astype(np.float32)
    kc = [np.concatenate([pre_k, r.standard_normal((8, hkv, d)).astype(np.float32)]) for _ in tabs]
    vc = [np.concatenate([pre_v, r.standard_normal((8, hkv, d)).astype(np.float32)]) for _ in tabs]
    kp, vp = _scatter(kc, vc, tabs, 9)
    q = np.broadcast_to(r.standard_normal((1, 1, hq, d)), (3, 1, hq, d)).astype(np.float32)
    got = oracle.paged_attention(kp, vp, "f32", q, "f32", _table(tabs), [L] * 3, 1, 0.5)
    for b in range(3):
        assert (got[b] == oracle.attention(q[b], kc[b], vc[b], 0.5)).all()
    # two sequences with the same table and query give the same output
    same = oracle.paged_attention(kp, vp, "f32", q[:2], "f32", _table([tabs[0], tabs[0]]),
                                  [L, L], 1, 0.5)
    assert (same[0] == same[1]).all()


def test_page_permutation_invariance():
    case = W.make_case("perm", batch=3, q_per_seq=2, num_q_heads=8, num_kv_heads=2,
                       seq_lens=[17, 64, 45], kv_dtype="f32", q_dtype="f32", seed=20,
                       num_pages=20)
    base = oracle.paged_attention(case.k_pool, case.v_pool, "f32", case.q, "f32",
                                  case.block_table, case.seq_lens, 2, case.scale)
    perm = _rng(21).permutation(case.num_pages)      # new id of old page p = perm[p]
    kp = np.empty_like(case.k_pool)
    vp = np.empty_like(case.v_pool)
    kp[perm] = case.k_pool
    vp[perm] = case.v_pool
    tab = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)], -1)
    moved = oracle.paged_attention(kp, vp, "f32", case.q, "f32", tab, case.seq_lens, 2,
                                   case.scale)
    assert (moved == base).all()
    assert np.isfinite(base).all()                    # poisoned slots were never read


def test_bf16_pool_reads_same_values_as_f32_pool():
    case = W.make_case("bf", batch=2, q_per_seq=1, num_q_heads=4, num_kv_heads=2,
                       seq_lens=[30, 7], kv_dtype="bf16", q_dtype="bf16", seed=22)
    as_f32 = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    a = oracle.paged_attention(case.k_pool, case.v_pool, "bf16", case.q, "bf16",
                               case.block_table, case.seq_lens, 1, case.scale)
    k32 = W.k_to_pool(as_f32(W.k_from_pool(case.k_pool)))
    b = oracle.paged_attention(k32, as_f32(case.v_pool), "f32",
                               as_f32(case.q), "f32", case.block_table, case.seq_lens, 1,
                               case.scale)
    assert (a == b).all()


def test_fp8_scales_enter_as_temperature_and_value_gain():
    case = W.make_case("f8", batch=2, q_per_seq=1, num_q_heads=8, num_kv_heads=2,
                       seq_lens=[40, 23], kv_dtype="fp8", q_dtype="bf16", seed=23)
    args = (case.k_pool, case.v_pool, "fp8", case.q, "bf16", case.block_table,
            case.seq_lens, 1)
    base = oracle.paged_attention(*args, case.scale, k_scale=case.k_scale,
                                  v_scale=case.v_scale)
    # doubling every K scale is the same as doubling the softmax scale
    a = oracle.paged_attention(*args, case.scale, k_scale=case.k_scale * 2,
                               v_scale=case.v_scale)
    b = oracle.paged_attention(*args, case.scale * 2, k_scale=case.k_scale,
                               v_scale=case.v_scale)
    np.testing.assert_allclose(a, b, atol=1e-12)
    # doubling every V scale doubles the output exactly
    c = oracle.paged_attention(*args, case.scale, k_scale=case.k_scale,
                               v_scale=case.v_scale * 2)
    assert (c == 2 * base).all()
    assert np.isfinite(base).all()


def test_fp8_identical_pages_give_mean_value():
    # every visible K row identical -> output is the mean of the dequantised V rows
    L, hkv, d, hq = 48, 2, 16, 4
    tab = [[2, 0, 1]]
    kbyte = W.e4m3_bytes(_rng(24).standard_normal((hkv, d)))
    vbyte = W.e4m3_bytes(_rng(25).standard_normal((3, hkv, 16, d)))
    kp = W.k_to_pool(np.broadcast_to(kbyte[None, :, None, :], (3, hkv, 16, d)).copy())
    vp = vbyte
    ks = np.full((3, hkv), 0.5, dtype=np.float32)
    vs = np.array([[0.25, 2.0], [1.0, 0.5], [4.0, 0.125]], dtype=np.float32)
    q = W.bf16_bits(_rng(26).standard_normal((1, 1, hq, d)).astype(np.float32))
    got = oracle.paged_attention(kp, vp, "fp8", q, "bf16", _table(tab), [L], 1, 0.1,
                                 k_scale=ks, v_scale=vs)
    dec = np.vectorize(oracle.e4m3_value)(vp).astype(np.float64) * vs[:, :, None, None]
    logical = np.concatenate([dec[p] for p in tab[0]], axis=1)          # [hkv][48][d]
    for h in range(hq):
        np.testing.assert_allclose(got[0, 0, h], logical[h // 2].mean(axis=0), atol=1e-13)


def test_chunked_k_layout_index_formula():
    # element d of token t of a slab sits at ((d / x) * 16 + t) * x + d % x
    for dt, x in ((np.float32, 4), (np.uint16, 8), (np.uint8, 16)):
        tok = np.arange(16 * 128).reshape(16, 128).astype(dt)
        pool = W.k_to_pool(tok).reshape(-1)
        t, d = 5, 77
        assert pool[((d // x) * 16 + t) * x + d % x] == tok[t, d]
        assert (W.k_from_pool(W.k_to_pool(tok)) == tok).all()


def test_paged_rejects_out_of_range_page():
    case = W.make_case("bad", batch=1, q_per_seq=1, num_q_heads=2, num_kv_heads=1,
                       seq_lens=[20], kv_dtype="f32", q_dtype="f32", seed=27)
    tab = case.block_table.copy()
    tab[0, 1] = case.num_pages
    with pytest.raises(ValueError):
        oracle.paged_attention(case.k_pool, case.v_pool, "f32", case.q, "f32", tab,
                               case.seq_lens, 1, 1.0)


# ----------------------------------------------------------------------------
# draft-tree verification
# ----------------------------------------------------------------------------
def test_chain_tree_is_the_causal_verify():
    L, n, hq, hkv, d = 60, 6, 8, 2, 16
    q, k, v = _rand_qkv(40, L, n, hq, hkv, d)
    assert (oracle.attention_tree(q, k, v, 0.3, W.chain_tree(n)) ==
            oracle.attention(q, k, v, 0.3)).all()


@pytest.mark.parametrize("n", [2, 7, 16, 64])
def test_tree_node_equals_decode_along_its_path(n):
    """Each node's output is plain decode over the context plus its ancestor path."""
    L, hq, hkv, d = 40 + n, 4, 2, 16
    rng = _rng(41 + n)
    q, k, v = _rand_qkv(42 + n, L, n, hq, hkv, d)
    _, masks = W.random_tree(rng, n)
    out = oracle.attention_tree(q, k, v, 0.25, masks)
    ctx = L - n
    for i in range(n):
        path = list(range(ctx)) + [ctx + j for j in W.ancestors(masks, i)]
        dec = oracle.attention(q[i:i + 1], k[path], v[path], 0.25)
        assert (dec[0] == out[i]).all()


def test_star_tree_rows_see_root_and_self():
    L, n, hq, hkv, d = 30, 5, 2, 1, 8
    q, k, v = _rand_qkv(43, L, n, hq, hkv, d)
    masks = np.array([1] + [1 | (1 << i) for i in range(1, n)], dtype=np.uint64)
    out = oracle.attention_tree(q, k, v, 0.5, masks)
    for i in range(1, n):
        path = list(range(L - n)) + [L - n, L - n + i]
        assert (oracle.attention(q[i:i + 1], k[path], v[path], 0.5)[0] == out[i]).all()


def test_tree_rejects_too_many_nodes_and_blind_rows():
    q, k, v = _rand_qkv(44, 70, 65, 2, 1, 8)
    with pytest.raises(ValueError):
        oracle.attention_tree(q, k, v, 1.0, np.ones(65, dtype=np.uint64))
    q, k, v = _rand_qkv(45, 3, 3, 2, 1, 8)            # no context: row 1 sees nothing
    with pytest.raises(ValueError):
        oracle.attention_tree(q, k, v, 1.0, np.array([1, 0, 4], dtype=np.uint64))


def test_paged_tree_matches_contiguous_tree():
    n = 9
    rng = _rng(46)
    lens = [50, 9, 80]
    hq, hkv, d = 8, 2, 16
    kc = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    vc = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    tabs = [[3, 0, 7, 1], [5], [2, 4, 6, 8, 9]]
    kp, vp = _scatter(kc, vc, tabs, 10)
    q = rng.standard_normal((3, n, hq, d)).astype(np.float32)
    masks = np.stack([W.random_tree(rng, n)[1] for _ in range(3)])
    got = oracle.paged_attention(kp, vp, "f32", q, "f32", _table(tabs), lens, n, 0.3,
                                 tree_mask=masks)
    for b in range(3):
        assert (got[b] == oracle.attention_tree(q[b], kc[b], vc[b], 0.3, masks[b])).all()


# ----------------------------------------------------------------------------
# KV append (quantize-on-write)
# ----------------------------------------------------------------------------
def test_e4m3_encode_is_nearest_with_ties_to_even():
    codes, vals = _e4m3_table()
    for x in [0.0, 1.0625, 1.1875, 447.9, 448.0, 470.0, 1e9, 2.0 ** -10, 0.75 * 2.0 ** -9]:
        for sgn in (1, -1):
            byte = oracle.e4m3_encode(sgn * x)
            assert byte == W.e4m3_bytes(np.array([sgn * x]))[0]
    assert oracle.e4m3_encode(float("nan")) == 0x7F


def _append_case(kv, lens, n_new, seed, src="f32", num_pages=None):
    qd = "f32" if kv == "f32" else "bf16"
    case = W.make_case("app", batch=len(lens), q_per_seq=1, num_q_heads=4, num_kv_heads=2,
                       seq_lens=lens, kv_dtype=kv, q_dtype=qd, seed=seed,
                       num_pages=num_pages)
    kn, vn = W.append_inputs(case, n_new, src, seed + 1)
    return case, kn, vn


def _append(case, kn, vn, src, n_new):
    return oracle.append_kv(case.k_pool, case.v_pool, case.kv_dtype, kn, vn, src,
                            case.block_table, case.seq_lens, n_new, case.k_scale, case.v_scale)


@pytest.mark.parametrize("kv,src", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16")])
def test_append_writes_rounded_values_where_attention_reads_them(kv, src):
    lens, n_new = [37, 16, 5], 5
    case, kn, vn = _append_case(kv, lens, n_new, 50, src)
    kp, vp, _, _ = _append(case, kn, vn, src, n_new)
    ktok = W.k_from_pool(kp)
    srcf = lambda a: a if src == "f32" else (a.astype(np.uint32) << 16).view(np.float32)
    want = lambda a: srcf(a) if kv == "f32" else W.bf16_bits(srcf(a))
    for b, L in enumerate(lens):
        for j in range(n_new):
            t = L - n_new + j
            page, slot = case.block_table[b, t // 16], t % 16
            assert (ktok[page, :, slot] == want(kn[b, j])).all()
            assert (vp[page, :, slot] == want(vn[b, j])).all()
    # older tokens and other pages untouched
    for b, L in enumerate(lens):
        for t in range(L - n_new):
            page, slot = case.block_table[b, t // 16], t % 16
            assert (vp[page, :, slot] == case.v_pool[page, :, slot]).all() or np.isnan(
                case.v_pool[page, :, slot]).all() if kv == "f32" else True


def test_append_into_fresh_fp8_page_spans_the_range():
    # a page whose first slot is new: scale = absmax / 448 and the largest value codes 448
    lens, n_new = [16, 32], 16
    case, kn, vn = _append_case("fp8", lens, n_new, 51, "f32")
    kp, vp, ks, vs = _append(case, kn, vn, "f32", n_new)
    for b in range(2):
        page = case.block_table[b, lens[b] // 16 - 1]
        for hk in range(2):
            amax = np.abs(kn[b, :, hk]).max()
            assert ks[page, hk] == np.float32(amax) / np.float32(448)
            slab = W.k_from_pool(kp)[page, hk]
            assert (slab & 0x7F).max() == 0x7E
            dec = np.vectorize(oracle.e4m3_value)(slab) * float(ks[page, hk])
            step = np.abs(kn[b, :, hk]) * 2.0 ** -4 + float(ks[page, hk]) * 2.0 ** -10
            assert (np.abs(dec - kn[b, :, hk]) <= step).all()   # RNE: half an E4M3 step


def test_append_one_at_a_time_equals_bulk_when_the_first_token_holds_the_max():
    lens, n_new = [16], 16
    case, kn, vn = _append_case("fp8", lens, n_new, 52, "f32")
    kn[:, 0] *= 10.0                                  # token 0 holds each head's absmax
    vn[:, 0] *= 10.0
    bulk = _append(case, kn, vn, "f32", n_new)
    state = (case.k_pool, case.v_pool, case.k_scale, case.v_scale)
    for j in range(n_new):
        state = oracle.append_kv(state[0], state[1], "fp8", kn[:, j:j + 1], vn[:, j:j + 1],
                                 "f32", case.block_table, np.array([j + 1], np.int32), 1,
                                 state[2], state[3])
    for a, b2 in zip(bulk, state):
        assert (a == b2).all()


def test_append_requantizes_older_tokens_when_the_scale_grows():
    lens, n_new = [20], 3                             # page 1 holds tokens 16..19
    case, kn, vn = _append_case("fp8", lens, n_new, 53, "f32")
    page = case.block_table[0, 1]
    old_scale = case.k_scale[page, 0]
    old_byte = W.k_from_pool(case.k_pool)[page, 0, 0]      # token 16: live, not rewritten
    kn[0, 0, 0] = 1000.0 * old_scale                        # new absmax >> old range
    kp, _, ks, _ = _append(case, kn, vn, "f32", n_new)
    new_scale = ks[page, 0]
    assert new_scale == np.float32(np.abs(kn[0, :, 0]).max()) / np.float32(448)
    for d in (0, 5, 127):
        val = np.float32(oracle.e4m3_value(old_byte[d])) * old_scale
        assert W.k_from_pool(kp)[page, 0, 0, d] == oracle.e4m3_encode(float(val / new_scale))
    # a smaller new token leaves the scale and the older bytes alone
    case2, kn2, vn2 = _append_case("fp8", lens, n_new, 54, "f32")
    kn2 *= 0.0
    kp2, _, ks2, _ = _append(case2, kn2, vn2, "f32", n_new)
    assert (ks2[page] == case2.k_scale[page]).all()
    assert (W.k_from_pool(kp2)[page, :, 0] == W.k_from_pool(case2.k_pool)[page, :, 0]).all()


def test_append_then_attention_equals_attention_on_the_source_values():
    lens, n_new = [40, 18], 6
    case, kn, vn = _append_case("f32", lens, n_new, 55, "f32")
    kp, vp, _, _ = _append(case, kn, vn, "f32", n_new)
    full = oracle.paged_attention(kp, vp, "f32", case.q, "f32", case.block_table,
                                  case.seq_lens, 1, case.scale)
    ktok = W.k_from_pool(case.k_pool)
    for b, L in enumerate(lens):
        kc = np.stack([ktok[case.block_table[b, t // 16], :, t % 16] for t in range(L)])
        vc = np.stack([case.v_pool[case.block_table[b, t // 16], :, t % 16] for t in range(L)])
        kc[L - n_new:] = kn[b]
        vc[L - n_new:] = vn[b]
        assert (oracle.attention(case.q[b], kc, vc, case.scale) == full[b]).all()
