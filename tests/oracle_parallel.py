"""The float64 oracle over whole workloads, spread across host threads.

Attention is independent per (sequence, KV head): query heads kh * G ..
kh * G + G - 1 read only KV head kh.  So the oracle is called once per
(sequence, KV head) on a one-KV-head view of the pool (the pool's slice for
that head, its G query heads), and the calls run on a thread pool (the
oracle's C entry point releases the GIL).  Nothing here computes attention
itself: every number comes from ``oracle.paged_attention``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import oracle


def host_threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(int(n or 1), 16))


def oracle_all(case, seqs=None, threads=None) -> np.ndarray:
    """oracle.paged_attention(case) for `seqs` (default: every sequence), as
    [len(seqs)][n][Hq][D] float64."""
    seqs = list(range(case.batch)) if seqs is None else [int(s) for s in seqs]
    hkv = case.num_kv_heads
    g = case.num_q_heads // hkv
    # one contiguous copy of each KV head's slice of the pool
    kp = [np.ascontiguousarray(case.k_pool[:, kh:kh + 1]) for kh in range(hkv)]
    vp = [np.ascontiguousarray(case.v_pool[:, kh:kh + 1]) for kh in range(hkv)]
    ks = vs = [None] * hkv
    if case.kv_dtype == "fp8":
        ks = [np.ascontiguousarray(case.k_scale[:, kh:kh + 1]) for kh in range(hkv)]
        vs = [np.ascontiguousarray(case.v_scale[:, kh:kh + 1]) for kh in range(hkv)]
    qh = [np.ascontiguousarray(case.q[:, :, kh * g:(kh + 1) * g]) for kh in range(hkv)]
    out = np.empty((len(seqs), case.q_per_seq, case.num_q_heads, case.head_dim), np.float64)

    def one(item):
        i, kh = item
        out[i, :, kh * g:(kh + 1) * g] = oracle.paged_attention(
            kp[kh], vp[kh], case.kv_dtype, qh[kh], case.q_dtype, case.block_table,
            case.seq_lens, case.q_per_seq, case.scale, seqs=[seqs[i]], k_scale=ks[kh],
            v_scale=vs[kh], tree_mask=case.tree_mask)[0]

    items = [(i, kh) for i in range(len(seqs)) for kh in range(hkv)]
    with cf.ThreadPoolExecutor(max_workers=threads or host_threads()) as ex:
        list(ex.map(one, items))
    return out
