"""Reentrancy of the host half (CPU, no device memory touched): eight threads
call the C ABI at the same time (ctypes releases the interpreter lock for the
duration of each call), creating and destroying pools, planning, sizing
workspaces and provoking argument errors.  Every plan must equal the one
computed alone beforehand, and each thread must read back its own last-error
message (the message is per thread)."""
import ctypes
import threading

import numpy as np

from paged_kv_gqa_02_amd import binding as B

LIB = B.library()
THREADS = 8
ITERS = 400
FAKE_K, FAKE_V = 0x10000, 0x20000          # never dereferenced by these calls


def make_pool(kv_dtype, hkv, partition_pages=0, waves=0, prefetch=0):
    d = B.pa_pool_desc(num_pages=4096, page_size=16, num_kv_heads=hkv, head_dim=128,
                       kv_dtype=kv_dtype, k=FAKE_K, v=FAKE_V,
                       k_scale=0x30000 if kv_dtype == B.PA_FP8_E4M3 else None,
                       v_scale=0x40000 if kv_dtype == B.PA_FP8_E4M3 else None,
                       partition_pages=partition_pages, waves=waves, prefetch=prefetch,
                       staged_from=0)
    h = ctypes.c_void_p()
    assert LIB.paged_attn_create_pool(ctypes.byref(d), ctypes.byref(h)) == 0
    return h


def plan_of(h, shape):
    pl = B.pa_plan()
    st = LIB.paged_attn_plan(h, *shape, ctypes.byref(pl))
    return st, tuple(getattr(pl, f) for f, _ in B.pa_plan._fields_)


def workspace_of(h, shape):
    n = ctypes.c_size_t()
    st = LIB.paged_attn_workspace_bytes(h, *shape, ctypes.byref(n))
    return st, n.value


POOLS = [(B.PA_BF16, 8, 0, 0, 0), (B.PA_FP8_E4M3, 8, 0, 0, 0), (B.PA_F32, 2, 0, 0, 0),
         (B.PA_BF16, 8, 33, 8, 3), (B.PA_BF16, 1, 1000, 4, 0)]
SHAPES = [(64, 1, 32, 2048), (8, 5, 32, 4101), (4, 512, 32, 2048), (240, 1, 32, 1424),
          (4, 1, 64, 32768), (1, 1, 8, 270000), (8, 16, 32, 4112), (3, 7, 24, 999)]


def test_concurrent_host_calls_match_serial_results():
    # serial reference
    ref = {}
    for pi, p in enumerate(POOLS):
        h = make_pool(*p)
        for si, s in enumerate(SHAPES):
            if s[2] % p[1]:
                continue
            ref[pi, si] = (plan_of(h, s), workspace_of(h, s))
        LIB.paged_attn_destroy_pool(h)
    assert len(ref) > 30

    barrier = threading.Barrier(THREADS)
    problems = []

    def worker(tid):
        rng = np.random.default_rng(100 + tid)
        keys = list(ref)
        barrier.wait()
        for it in range(ITERS):
            pi, si = keys[int(rng.integers(len(keys)))]
            h = make_pool(*POOLS[pi])
            got = (plan_of(h, SHAPES[si]), workspace_of(h, SHAPES[si]))
            if got != ref[pi, si]:
                problems.append(f"thread {tid} iter {it}: {got} != {ref[pi, si]}")
            # an argument error of this thread's own kind, then its message
            if tid % 2:
                st = LIB.paged_attn_plan(h, 0, 1, 32, 100, ctypes.byref(B.pa_plan()))
                want = b"batch, q_per_seq, num_q_heads and max_seq_len must be >= 1"
            else:
                st = LIB.paged_attn_plan(h, 1, 200, 64, 100, ctypes.byref(B.pa_plan()))
                want = b"max_seq_len < q_per_seq"
            msg = LIB.paged_attn_last_error()
            if st != B.PA_ERR_INVALID_ARG or msg != want:
                problems.append(f"thread {tid} iter {it}: status {st}, message {msg!r}")
            LIB.paged_attn_destroy_pool(h)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(THREADS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not problems, problems[:5]
