"""The threaded per-(sequence, KV head) oracle runner equals the oracle's own
whole-batch call bit for bit (CPU)."""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle_parallel import oracle_all


@pytest.mark.parametrize("kv,n,heads,tree", [("f32", 1, (8, 2), False), ("bf16", 5, (32, 8), False),
                                             ("fp8", 3, (16, 2), False), ("bf16", 6, (8, 4), True)])
def test_threaded_runner_equals_whole_batch_call(kv, n, heads, tree):
    lens = [n, 17, 100, 333 + n]
    case = W.make_case("par", batch=len(lens), q_per_seq=n, num_q_heads=heads[0],
                       num_kv_heads=heads[1], seq_lens=lens, kv_dtype=kv,
                       q_dtype="f32" if kv == "f32" else "bf16", seed=71 + n)
    if tree:
        rng = np.random.default_rng(72)
        case.tree_mask = np.stack([W.random_tree(rng, n)[1] for _ in range(case.batch)])
    whole = oracle.paged_attention(case.k_pool, case.v_pool, case.kv_dtype, case.q, case.q_dtype,
                                   case.block_table, case.seq_lens, case.q_per_seq, case.scale,
                                   k_scale=case.k_scale, v_scale=case.v_scale,
                                   tree_mask=case.tree_mask)
    assert np.array_equal(oracle_all(case, threads=3), whole)
    assert np.array_equal(oracle_all(case, seqs=[2, 0], threads=2), whole[[2, 0]])
