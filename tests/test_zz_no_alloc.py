"""paged_attn_verify_noalloc (split-K partials in the library's static scratch)
against paged_attn_verify with a caller workspace: bit for bit, on two calls in
a row, the second with a smaller input, both taking the split plan."""
import numpy as np
import pytest
import torch

import workloads as W
from workloads.device import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_kv_gqa_02_amd as lib
    return lib


def both(pa, case, kv):
    print(f"[gpu no-alloc] {case.name} kv={kv} B={case.batch} n={case.q_per_seq} "
          f"lens={list(case.seq_lens)} seed={case.seed}", flush=True)
    d = to_device(case)
    pool = pa.paged_attn_create_pool(d.k, d.v, d.k_scale, d.v_scale)
    plan = pa.paged_attn_plan(pool, case.batch, case.q_per_seq, case.num_q_heads,
                              case.max_seq_len)
    assert plan["reduce"] == 1, plan                 # the scratch is really used
    ws = pa.workspace_for(pool, d.q, case.max_seq_len)
    want = torch.empty_like(d.q)
    pa.paged_attn_verify(pool, d.q, want, d.block_table, d.seq_lens, case.max_seq_len,
                         case.scale, ws)
    got = torch.full_like(d.q, float("nan"))
    pa.paged_attn_verify_noalloc(pool, d.q, got, d.block_table, d.seq_lens, case.max_seq_len,
                                 case.scale)
    torch.cuda.synchronize()
    return want, got


@pytest.mark.parametrize("kv", ["bf16", "f32", "fp8"])
def test_noalloc_matches_workspace_call_twice(pa, kv):
    qd = "f32" if kv == "f32" else "bf16"
    big = W.make_case("noalloc-big", batch=8, q_per_seq=5, num_q_heads=32, num_kv_heads=8,
                      seq_lens=[4101, 3000, 4101, 17, 2222, 4101, 900, 4096], kv_dtype=kv,
                      q_dtype=qd, seed=5151)
    small = W.make_case("noalloc-small", batch=2, q_per_seq=5, num_q_heads=32, num_kv_heads=8,
                        seq_lens=[1000, 333], kv_dtype=kv, q_dtype=qd, seed=5152)
    for case in (big, small):
        want, got = both(pa, case, kv)
        view = torch.int32 if kv == "f32" else torch.int16
        same = torch.equal(want.view(view), got.view(view))
        print(f"    {case.name}: bitwise equal {same}", flush=True)
        assert same


def test_noalloc_unsplit_call_needs_no_scratch(pa):
    case = W.make_case("noalloc-unsplit", batch=64, q_per_seq=1, num_q_heads=32, num_kv_heads=8,
                       seq_lens=[600] * 64, kv_dtype="bf16", q_dtype="bf16", seed=5153)
    d = to_device(case)
    pool = pa.paged_attn_create_pool(d.k, d.v)
    assert pa.paged_attn_workspace_bytes(pool, 64, 1, 32, case.max_seq_len) == 0
    want, got = torch.empty_like(d.q), torch.empty_like(d.q)
    pa.paged_attn_verify(pool, d.q, want, d.block_table, d.seq_lens, case.max_seq_len, case.scale)
    pa.paged_attn_verify_noalloc(pool, d.q, got, d.block_table, d.seq_lens, case.max_seq_len,
                                 case.scale)
    torch.cuda.synchronize()
    assert torch.equal(want.view(torch.int16), got.view(torch.int16))
