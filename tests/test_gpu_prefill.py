"""Chunked-prefill attention over the paged cache: hundreds of query rows per
sequence, each attending to the earlier chunks' keys and causally within its
own chunk.  Checked against the oracle, and (at the full workload) against the
pin that prefill row i is the decode of the same query at length L - n + i + 1.
"""
import numpy as np
import pytest
import torch

import workloads as W
from workloads.device import to_device, to_numpy_f64
from test_gpu_parity import MAX_ABS, check, run_gpu, run_oracle, say, small_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_kv_gqa_02_amd as lib
    return lib


@pytest.mark.parametrize("kv,heads", [("bf16", (32, 8)), ("f32", (8, 2)), ("fp8", (16, 2))])
def test_prefill_chunk_matches_oracle(pa, kv, heads):
    # a first chunk (no context), a chunk after a ragged context, a chunk ending mid-page
    n = 256
    case = small_case(kv, n, heads[0], heads[1], [n, n + 300, n + 17 + 16 * 20], seed=900)
    check(run_gpu(pa, case), run_oracle(case), kv, f"prefill n={n} {kv}")


def test_prefill_workload_structure_in_fp32(pa):
    """Same shape in fp32 (1e-5 gate): the first chunk, fully causal."""
    case = W.workload("prefill", kv_dtype="f32", q_dtype="f32")
    gpu = run_gpu(pa, case, label="fp32 structure")
    check(gpu[3:4], run_oracle(case, seqs=[3]), "f32", "prefill fp32 seq 3")


def test_prefill_workload_native(pa):
    case = W.workload("prefill")
    gpu = run_gpu(pa, case, label="native")
    check(gpu[3:4], run_oracle(case, seqs=[3]), "bf16", "prefill bf16 seq 3")


def test_prefill_rows_are_stacked_decodes(pa):
    """Row i of a chunk equals the decode of its query over the first L - n + i + 1 keys."""
    case = W.workload("prefill")
    d = to_device(case)
    full = run_gpu(pa, case, dev=d, label="rows vs decode")
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
