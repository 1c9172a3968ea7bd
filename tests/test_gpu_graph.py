"""Graph capture: one speculative step (append the new tokens' K/V, score them
with verify and with verify_noalloc, accept or reject the drafts), and one
chunked-prefill call, captured into a HIP graph through torch and replayed.

The entry points launch kernels only (no memset, copy or allocation inside a
call), so they capture as plain kernel nodes on torch's capture stream.  Each
replay must equal the same calls made eagerly, bit for bit: new inputs are
written into the captured tensors before every replay, the outputs are
poisoned first, and the program's own eager work and synchronisations run
between the replays."""
import numpy as np
import pytest
import torch

import workloads as W
from workloads.device import to_device

pytestmark = pytest.mark.gpu

ROUNDS = 3


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_kv_gqa_02_amd as lib
    return lib


def say(msg):
    print(msg, flush=True)


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def capture(step):
    """Warm up on a side stream (first launches, the no-alloc scratch lookup),
    then capture `step` into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def eager_noise(pa, pool, d, case):
    """Unrelated eager work between replays: a verify call into its own buffers
    and a torch reduction, then a synchronisation."""
    out = torch.empty_like(d.q)
    ws = pa.workspace_for(pool, d.q, case.max_seq_len)
    pa.paged_attn_verify(pool, d.q * 0.5, out, d.block_table, d.seq_lens, case.max_seq_len,
                         case.scale, ws)
    torch.ones(1 << 20, device="cuda").sum()
    torch.cuda.synchronize()


def test_speculative_step_graph_replays_match_eager(pa):
    B, K, Hq, Hkv, V = 8, 4, 32, 8, 32000
    lens = [4101, 700, 1500, 64, 2048, 333, 900, 3001]     # already count the K + 1 new tokens
    case = W.make_case("graph-step", batch=B, q_per_seq=K + 1, num_q_heads=Hq, num_kv_heads=Hkv,
                       seq_lens=lens, kv_dtype="bf16", q_dtype="bf16", seed=6161)
    say(f"[gpu graph] speculative step B={B} K={K} Hq={Hq} Hkv={Hkv} V={V} lens={lens}")
    d = to_device(case)
    pool = pa.paged_attn_create_pool(d.k, d.v)
    plan = pa.paged_attn_plan(pool, B, K + 1, Hq, case.max_seq_len)
    assert plan["reduce"] == 1, plan                     # the split-K reduce is captured too
    ws = pa.workspace_for(pool, d.q, case.max_seq_len)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    rng = np.random.default_rng(6162)

    def new_tokens():
        x = rng.standard_normal((B, K + 1, Hkv, 128), dtype=np.float32)
        return torch.from_numpy(x).to(torch.bfloat16).cuda()

    k_new, v_new = new_tokens(), new_tokens()
    s0 = W.sampler_inputs(B, K, V, 6163)
    p, qd, draft = dev(s0.p), dev(s0.q), dev(s0.draft)
    ua, us = dev(s0.u_accept), dev(s0.u_sample)
    out = torch.empty_like(d.q)
    out_na = torch.empty_like(d.q)
    tokens = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
    acc = torch.empty((B,), dtype=torch.int32, device="cuda")
    sws = torch.empty(pa.paged_attn_rejection_sample_workspace_bytes(B, V), dtype=torch.uint8,
                      device="cuda")

    def step():
        pa.paged_attn_append_kv(pool, k_new, v_new, d.block_table, d.seq_lens)
        pa.paged_attn_verify(pool, d.q, out, d.block_table, d.seq_lens, case.max_seq_len,
                             case.scale, ws)
        pa.paged_attn_verify_noalloc(pool, d.q, out_na, d.block_table, d.seq_lens,
                                     case.max_seq_len, case.scale)
        pa.paged_attn_rejection_sample(p, qd, draft, ua, us, tokens=tokens, num_accepted=acc,
                                       workspace=sws)

    g = capture(step)
    for r in range(ROUNDS):
        # new inputs in the captured tensors
        d.q.copy_(torch.from_numpy(rng.standard_normal(tuple(d.q.shape), dtype=np.float32))
                  .to(torch.bfloat16))
        k_new.copy_(new_tokens())
        v_new.copy_(new_tokens())
        s = W.sampler_inputs(B, K, V, 6200 + r)
        for t, a in ((p, s.p), (qd, s.q), (draft, s.draft), (ua, s.u_accept), (us, s.u_sample)):
            t.copy_(dev(a))
        torch.cuda.synchronize()
        step()                                           # eager reference
        torch.cuda.synchronize()
        want = [x.clone() for x in (out, out_na, tokens, acc, d.k, d.v)]
        out.fill_(float("nan"))
        out_na.fill_(float("nan"))
        tokens.fill_(-7)
        acc.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (out, out_na, tokens, acc, d.k, d.v)
        same = [torch.equal(bits(a), bits(b)) for a, b in zip(want, got)]
        say(f"    replay {r}: bitwise equal (out, out_noalloc, tokens, accepted, K pool, V pool) "
            f"{same}; accepted {acc.tolist()}")
        assert all(same)
        assert torch.equal(bits(out), bits(out_na))
        eager_noise(pa, pool, d, case)


def test_chunked_prefill_graph_replays_match_eager(pa):
    B, n, Hq, Hkv = 2, 256, 32, 8
    lens = [256 + 1000, 256]
    case = W.make_case("graph-prefill", batch=B, q_per_seq=n, num_q_heads=Hq, num_kv_heads=Hkv,
                       seq_lens=lens, kv_dtype="bf16", q_dtype="bf16", seed=6171)
    say(f"[gpu graph] chunked prefill B={B} n={n} Hq={Hq} Hkv={Hkv} lens={lens}")
    d = to_device(case)
    pool = pa.paged_attn_create_pool(d.k, d.v)
    plan = pa.paged_attn_plan(pool, B, n, Hq, case.max_seq_len)
    assert plan["kernel"] == 1, plan                     # the LDS-staged kernel
    ws = pa.workspace_for(pool, d.q, case.max_seq_len)
    out = torch.empty_like(d.q)
    rng = np.random.default_rng(6172)

    def step():
        pa.paged_attn_verify(pool, d.q, out, d.block_table, d.seq_lens, case.max_seq_len,
                             case.scale, ws)

    g = capture(step)
    for r in range(ROUNDS):
        d.q.copy_(torch.from_numpy(rng.standard_normal(tuple(d.q.shape), dtype=np.float32))
                  .to(torch.bfloat16))
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        want = out.clone()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(bits(want), bits(out))
        say(f"    replay {r}: bitwise equal {same}")
        assert same
        eager_noise(pa, pool, d, case)
