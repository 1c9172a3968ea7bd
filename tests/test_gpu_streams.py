"""Concurrent calls: two pools, each with its own workspace, driven on two HIP
streams at once from two host threads (ctypes releases the interpreter lock
during each call, so both threads are inside the library together).  Every
output must equal, bit for bit, the same call made alone; calls are
deterministic for a fixed plan, so concurrency may change nothing."""
import threading

import pytest
import torch

import workloads as W
from workloads.device import to_device

pytestmark = pytest.mark.gpu

ITERS = 20


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_kv_gqa_02_amd as lib
    return lib


def setup(pa, case):
    d = to_device(case)
    pool = pa.paged_attn_create_pool(d.k, d.v, d.k_scale, d.v_scale)
    ws = pa.workspace_for(pool, d.q, case.max_seq_len)
    return d, pool, ws


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_two_streams_from_two_threads_match_solo_calls(pa):
    cases = [
        W.make_case("streams-a", batch=16, q_per_seq=5, num_q_heads=32, num_kv_heads=8,
                    seq_lens=[4101, 900, 2222, 64, 3000, 17, 1500, 4000] * 2, kv_dtype="bf16",
                    q_dtype="bf16", seed=7171),
        W.make_case("streams-b", batch=4, q_per_seq=1, num_q_heads=64, num_kv_heads=8,
                    seq_lens=[8192, 5000, 8000, 333], kv_dtype="fp8", q_dtype="bf16", seed=7172),
    ]
    print(f"[gpu streams] {[c.name for c in cases]}", flush=True)
    state = [setup(pa, c) for c in cases]
    want = []
    for c, (d, pool, ws) in zip(cases, state):
        out = torch.empty_like(d.q)
        pa.paged_attn_verify(pool, d.q, out, d.block_table, d.seq_lens, c.max_seq_len, c.scale, ws)
        torch.cuda.synchronize()
        want.append(out.clone())
    streams = [torch.cuda.Stream() for _ in cases]
    outs = [[torch.full_like(d.q, float("nan")) for _ in range(ITERS)] for d, _, _ in state]
    barrier = threading.Barrier(len(cases))
    errors = []

    def worker(k):
        c, (d, pool, ws), s = cases[k], state[k], streams[k]
        try:
            barrier.wait()
            for it in range(ITERS):
                pa.paged_attn_verify(pool, d.q, outs[k][it], d.block_table, d.seq_lens,
                                     c.max_seq_len, c.scale, ws, stream=s)
        except Exception as e:          # reported below, on the main thread
            errors.append(repr(e))

    torch.cuda.synchronize()
    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k, c in enumerate(cases):
        same = [torch.equal(bits(o), bits(want[k])) for o in outs[k]]
        print(f"    {c.name}: {sum(same)}/{ITERS} calls bitwise equal to the solo call", flush=True)
        assert all(same)
