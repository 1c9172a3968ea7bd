"""GPU KV append (quantize-on-write) against the oracle: pool bytes and fp8
scales must match bit for bit (this is byte work)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads.device import tensor, to_device, to_numpy_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_kv_gqa_02_amd as lib
    return lib


def say(msg):
    print(msg, flush=True)


def gpu_append(pa, case, kn, vn, n_new):
    say(f"[gpu append] kv={case.kv_dtype} src={kn.dtype} B={case.batch} n_new={n_new} "
        f"lens={list(case.seq_lens)[:6]} seed={case.seed}")
    d = to_device(case)
    pool = pa.paged_attn_create_pool(d.k, d.v, d.k_scale, d.v_scale)
    pa.paged_attn_append_kv(pool, tensor(kn, "cuda"), tensor(vn, "cuda"), d.block_table,
                            d.seq_lens)
    torch.cuda.synchronize()
    as_np = lambda t, like: None if t is None else (
        t.view(torch.int16).cpu().numpy().view(np.uint16) if like.dtype == np.uint16
        else t.cpu().numpy())
    return (as_np(d.k, case.k_pool), as_np(d.v, case.v_pool),
            None if d.k_scale is None else d.k_scale.cpu().numpy(),
            None if d.v_scale is None else d.v_scale.cpu().numpy())


def oracle_append(case, kn, vn, src, n_new):
    return oracle.append_kv(case.k_pool, case.v_pool, case.kv_dtype, kn, vn, src,
                            case.block_table, case.seq_lens, n_new, case.k_scale, case.v_scale)


def same_bits(a, b):
    if a.dtype == np.float32:
        return (a.view(np.uint32) == b.view(np.uint32)).all()
    return (a == b).all()


def assert_pools_equal(got, want):
    for name, g, w in zip(("k", "v", "k_scale", "v_scale"), got, want):
        if w is None:
            continue
        bad = ~((g == w) | (np.isnan(g.astype(np.float64)) & np.isnan(w.astype(np.float64))))
        assert not bad.any(), f"{name}: {int(bad.sum())} elements differ"


COMBOS = [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16"), ("fp8", "f32"), ("fp8", "bf16")]


@pytest.mark.parametrize("kv,src", COMBOS)
@pytest.mark.parametrize("n_new", [1, 5, 20])
def test_append_matches_oracle(pa, kv, src, n_new):
    lens = [n_new, n_new + 17, 33, 300, 16 * 3]
    qd = "f32" if kv == "f32" else "bf16"
    case = W.make_case("append", batch=len(lens), q_per_seq=1, num_q_heads=8, num_kv_heads=2,
                       seq_lens=lens, kv_dtype=kv, q_dtype=qd, seed=400 + n_new,
                       num_pages=sum(W.pages_for(x) for x in lens) + 4)
    kn, vn = W.append_inputs(case, n_new, src, 500 + n_new)
    assert_pools_equal(gpu_append(pa, case, kn, vn, n_new),
                       oracle_append(case, kn, vn, src, n_new))


def test_append_requantizes_like_the_oracle(pa):
    lens, n_new = [20, 35, 50], 3
    case = W.make_case("requant", batch=3, q_per_seq=1, num_q_heads=4, num_kv_heads=2,
                       seq_lens=lens, kv_dtype="fp8", q_dtype="bf16", seed=410)
    kn, vn = W.append_inputs(case, n_new, "f32", 411, spread=50.0)   # beats the old scales
    kn[1] *= 0.0                                                    # and one that does not
    assert_pools_equal(gpu_append(pa, case, kn, vn, n_new),
                       oracle_append(case, kn, vn, "f32", n_new))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_append_then_attention(pa, kv):
    """GPU append followed by GPU decode equals GPU decode on the oracle-appended pool."""
    lens, n_new = [100, 257, 16], 1
    case = W.make_case("chain", batch=3, q_per_seq=1, num_q_heads=32, num_kv_heads=8,
                       seq_lens=lens, kv_dtype=kv, q_dtype="bf16", seed=420)
    kn, vn = W.append_inputs(case, n_new, "bf16", 421)
    d = to_device(case)
    pool = pa.paged_attn_create_pool(d.k, d.v, d.k_scale, d.v_scale)
    pa.paged_attn_append_kv(pool, tensor(kn, "cuda"), tensor(vn, "cuda"), d.block_table,
                            d.seq_lens)
    out = torch.empty_like(d.q)
    ws = pa.workspace_for(pool, d.q, case.max_seq_len)
    pa.paged_attn_decode(pool, d.q, out, d.block_table, d.seq_lens, case.max_seq_len,
                         case.scale, ws)
    torch.cuda.synchronize()
    kp, vp, ks, vs = oracle_append(case, kn, vn, "bf16", n_new)
    ref = oracle.paged_attention(kp, vp, kv, case.q, "bf16", case.block_table, case.seq_lens, 1,
                                 case.scale, k_scale=ks, v_scale=vs)
    err = float(np.abs(to_numpy_f64(out) - ref).max())
    say(f"    append then decode: max_abs={err:.3e}")
    assert err <= (1.5e-2 if kv == "bf16" else 5e-2)


@pytest.mark.parametrize("name,n_new,src", [("decode8b", 1, "bf16"), ("verify", 5, "bf16"),
                                            ("fp8long", 1, "f32"), ("decode8b", 256, "bf16"),
                                            ("fp8long", 256, "bf16")])
def test_append_workloads(pa, name, n_new, src):
    case = W.workload(name)
    kn, vn = W.append_inputs(case, n_new, src, 20261202)     # the inputs bench.py --op append times
    assert_pools_equal(gpu_append(pa, case, kn, vn, n_new),
                       oracle_append(case, kn, vn, src, n_new))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_append_prefill_chunk(pa, kv):
    """A prefill chunk: 256 new tokens per sequence, starting mid-page, 17 pages each."""
    lens = [256 + 7, 1000, 256, 777, 300, 512 + 15, 999, 260]
    case = W.make_case("chunk", batch=len(lens), q_per_seq=1, num_q_heads=32, num_kv_heads=8,
                       seq_lens=lens, kv_dtype=kv, q_dtype="bf16", seed=450)
    kn, vn = W.append_inputs(case, 256, "bf16", 451)
    assert_pools_equal(gpu_append(pa, case, kn, vn, 256),
                       oracle_append(case, kn, vn, "bf16", 256))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_append_is_invariant_to_page_placement(pa, kv):
    """Renumbering the physical pages (data moved with them) renumbers the result."""
    lens, n_new = [70, 33, 129], 20
    case = W.make_case("perm", batch=3, q_per_seq=1, num_q_heads=4, num_kv_heads=2,
                       seq_lens=lens, kv_dtype=kv, q_dtype="bf16", seed=460)
    kn, vn = W.append_inputs(case, n_new, "bf16", 461)
    base = gpu_append(pa, case, kn, vn, n_new)
    perm = np.random.default_rng(462).permutation(case.num_pages)    # new id of page j
    moved = W.Case(**{**case.__dict__})
    inv = np.argsort(perm)
    moved.k_pool, moved.v_pool = case.k_pool[inv], case.v_pool[inv]
    if case.k_scale is not None:
        moved.k_scale, moved.v_scale = case.k_scale[inv], case.v_scale[inv]
    moved.block_table = perm[case.block_table].astype(np.int32)
    got = gpu_append(pa, moved, kn, vn, n_new)
    for g, w in zip(got, base):
        if w is not None:
            assert same_bits(np.ascontiguousarray(g[perm]), w)


def test_append_rejects_bad_arguments(pa):
    case = W.make_case("bad", batch=1, q_per_seq=1, num_q_heads=2, num_kv_heads=1,
                       seq_lens=[20], kv_dtype="f32", q_dtype="f32", seed=440)
    d = to_device(case)
    pool = pa.paged_attn_create_pool(d.k, d.v)
    kb = torch.zeros((1, 1, 1, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pa.PagedAttnError):      # f32 pool takes f32 values
        pa.paged_attn_append_kv(pool, kb, kb, d.block_table, d.seq_lens)
