"""Chunked-prefill attention over the paged cache: hundreds of query rows per
sequence, each attending to the earlier chunks' keys and causally within its
own chunk.  Every case runs through the chunked-prefill kernel (the automatic
choice from 128 rows per sequence) and through the partition kernel
(staged_from = -1), against the oracle; at the full workload also against the
pin that prefill row i is the decode of the same query at length L - n + i + 1.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle_parallel import oracle_all
from workloads.device import to_device, to_numpy_f64
from test_gpu_parity import MAX_ABS, check, run_oracle, say, small_case

pytestmark = pytest.mark.gpu

KERNELS = {"prefill": 0, "partition": -1}      # pool staged_from


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_kv_gqa_02_amd as lib
    return lib


def run(pa, case, kernel, dev=None, partition_pages=0):
    d = dev if dev is not None else to_device(case)
    pool = pa.paged_attn_create_pool(d.k, d.v, d.k_scale, d.v_scale, partition_pages,
                                     staged_from=KERNELS[kernel])
    plan = pa.paged_attn_plan(pool, case.batch, case.q_per_seq, case.num_q_heads,
                              case.max_seq_len)
    say(f"[gpu prefill] {case.name} kernel={kernel} (plan {plan['kernel']}, "
        f"{plan['num_splits']} splits) kv={case.kv_dtype} "
        f"B={case.batch} n={case.q_per_seq} Hq={case.num_q_heads} Hkv={case.num_kv_heads} "
        f"lens={list(case.seq_lens)} seed={case.seed}")
    want = 1 if kernel == "prefill" and case.kv_dtype != "f32" else 0
    assert plan["kernel"] == want
    out = torch.empty_like(d.q)
    ws = pa.workspace_for(pool, d.q, case.max_seq_len)
    pa.paged_attn_verify(pool, d.q, out, d.block_table, d.seq_lens, case.max_seq_len,
                         case.scale, ws)
    torch.cuda.synchronize()
    return to_numpy_f64(out)


@pytest.mark.parametrize("kernel", ["prefill", "partition"])
@pytest.mark.parametrize("kv,heads", [("bf16", (32, 8)), ("f32", (8, 2)), ("fp8", (16, 2))])
def test_prefill_chunk_matches_oracle(pa, kernel, kv, heads):
    # a first chunk (no context), a chunk after a ragged context, a chunk ending mid-page
    n = 256
    case = small_case(kv, n, heads[0], heads[1], [n, n + 300, n + 17 + 16 * 20], seed=900)
    check(run(pa, case, kernel), run_oracle(case), kv, f"prefill n={n} {kv} {kernel}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("n,heads,lens", [
    (130, (32, 8), [130, 131, 400, 1000]),      # 520 rows: a partial last block of 8
    (128, (64, 8), [128, 129 + 16 * 7, 600]),   # G = 8 (1024 rows)
    (200, (8, 8), [200, 215, 777]),             # G = 1 (MHA): 200 rows, one partial block
    (160, (4, 1), [160, 161, 2000]),            # MQA, an odd page count, a long context
])
def test_prefill_kernel_edge_shapes(pa, kv, n, heads, lens):
    case = small_case(kv, n, heads[0], heads[1], lens, seed=910 + n)
    check(run(pa, case, "prefill"), run_oracle(case), kv, f"prefill edge n={n} {heads} {kv}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_prefill_sequences_ranked_by_length(pa, kv):
    # the kernel orders row blocks by the sequences' lengths (longest first, ties
    # by index): unsorted lengths with a tie and a first chunk of its own
    n = 128
    case = small_case(kv, n, 8, 2, [n + 100, n + 700, n, n + 700, n + 333], seed=940)
    check(run(pa, case, "prefill"), run_oracle(case), kv, f"prefill ranked {kv}")


def test_prefill_many_sequences_in_index_order(pa):
    # more than 64 sequences are taken in index order (one wave ranks up to 64)
    n = 128
    rng = np.random.default_rng(941)
    lens = [int(x) for x in rng.integers(n, n + 90, size=66)]
    case = small_case("bf16", n, 1, 1, lens, seed=941)
    check(run(pa, case, "prefill"), run_oracle(case), "bf16", "prefill B=66")


def test_prefill_items_in_several_rounds(pa):
    # 40 sequences x 8 kv heads x 2 row blocks = 640 items over one workgroup
    # per CU: a forward round, a reversed round and a partial third one
    n = 128
    rng = np.random.default_rng(942)
    lens = [int(x) for x in rng.integers(n, n + 64, size=40)]
    case = small_case("bf16", n, 16, 8, lens, seed=942)
    check(run(pa, case, "prefill"), run_oracle(case), "bf16", "prefill 640 items")


def test_prefill_workload_structure_in_fp32(pa):
    """Same shape in fp32 (1e-5 gate; the partition kernel), every sequence: the
    chunks after 1536, 1024 and 512 earlier tokens and the first chunk."""
    case = W.workload("prefill", kv_dtype="f32", q_dtype="f32")
    gpu = run(pa, case, "partition")
    check(gpu, oracle_all(case), "f32", "prefill fp32, all 4 chunks")


@pytest.mark.parametrize("kernel", ["prefill", "partition"])
def test_prefill_workload_native(pa, kernel):
    case = W.workload("prefill")
    gpu = run(pa, case, kernel)
    ref = oracle_all(case)
    for b in range(case.batch):
        ctx = int(case.seq_lens[b]) - case.q_per_seq
        check(gpu[b:b + 1], ref[b:b + 1], "bf16", f"prefill bf16 seq {b} ({ctx} earlier) {kernel}")


def test_prefill_kernels_agree_at_the_workload(pa):
    case = W.workload("prefill")
    d = to_device(case)
    a, b = run(pa, case, "prefill", dev=d), run(pa, case, "partition", dev=d)
    err = float(np.abs(a - b).max())
    say(f"    prefill vs partition kernel: max_abs={err:.3e}")
    assert err <= MAX_ABS["bf16"]


def test_prefill_kernel_is_deterministic(pa):
    case = W.workload("prefill")
    d = to_device(case)
    a, b = run(pa, case, "prefill", dev=d), run(pa, case, "prefill", dev=d)
    assert np.array_equal(a, b)


def test_prefill_rows_are_stacked_decodes(pa):
    """Row i of a chunk equals the decode of its query over the first L - n + i + 1 keys."""
    case = W.workload("prefill")
    d = to_device(case)
    full = run(pa, case, "prefill", dev=d)
    pool = pa.paged_attn_create_pool(d.k, d.v, d.k_scale, d.v_scale)
    n = case.q_per_seq
    rows = [0, 1, 15, 16, 255, 383, n - 2, n - 1]
    worst = 0.0
    for b in range(case.batch):
        L = int(case.seq_lens[b])
        q = d.q[b, rows].unsqueeze(1).contiguous()                  # [rows][1][Hq][D]
        lens = torch.tensor([L - n + i + 1 for i in rows], dtype=torch.int32, device="cuda")
        bt = d.block_table[b:b + 1].expand(len(rows), -1).contiguous()
        out = torch.empty_like(q)
        ws = pa.workspace_for(pool, q, L)
        pa.paged_attn_decode(pool, q, out, bt, lens, L, case.scale, ws)
        torch.cuda.synchronize()
        diff = np.abs(to_numpy_f64(out)[:, 0] - full[b, rows]).max()
        worst = max(worst, float(diff))
    say(f"    prefill rows vs decode: max_abs={worst:.3e}")
    assert worst <= MAX_ABS["bf16"]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("part", [3, 8])
def test_prefill_kernel_split_partitions(pa, kv, part):
    """Shorter partitions asked through the pool: the staged kernel writes split-K
    partials (odd partition lengths reach one page into the next partition, and
    row blocks whose causal limit ends before a partition write empty partials),
    and the reduce merges them."""
    n = 200
    case = small_case(kv, n, 32, 8, [n, n + 333, n + 16 * 9 + 5], seed=930 + part)
    check(run(pa, case, "prefill", partition_pages=part), run_oracle(case), kv,
          f"prefill split part={part} {kv}")
