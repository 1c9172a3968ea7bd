"""Seeded shape sweep: random (but fixed) combinations of dtype, GQA layout,
query rows, draft trees, lengths, page-pool layout and launch knobs, each run
through the C ABI and compared with the float64 oracle at the standard gates.

Every case is small enough for the oracle to finish in well under a second;
together they cross the paths the planner chooses between (partition kernel
with one to four row tiles, the LDS-staged kernel for trees and chunked
prefill, split-K with the reduce, odd partitions) with lengths that end
mid-page, one-token sequences next to long ones, and fragmented pools.
"""
import numpy as np
import pytest
import torch

import workloads as W
from workloads.device import to_device
from test_gpu_parity import check, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu

NUM_CASES = 100


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_kv_gqa_02_amd as lib
    return lib


def fuzz_case(seed):
    rng = np.random.default_rng(5000 + seed)
    kv = ["f32", "bf16", "fp8"][int(rng.integers(0, 3))]
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 8]))
    mode = ["decode", "verify", "tree", "prefill"][int(rng.integers(0, 4))]
    if mode == "decode":
        n = 1
    elif mode == "verify":
        n = int(rng.integers(2, 9))
    elif mode == "tree":
        n = int(rng.integers(2, 33))
    else:
        n = int(rng.integers(128, 181))
    batch = int(rng.integers(1, 5))
    longest = 2500
    if mode == "prefill":               # keep the oracle's work (rows x keys x heads) small
        batch, longest = min(batch, 2), 700
        hkv, group = min(hkv, 2), min(group, 4)
    lens = [int(rng.integers(n, longest + 1)) for _ in range(batch)]
    lens[int(rng.integers(0, batch))] = n if rng.random() < 0.5 else lens[0]
    layout = "fragmented" if rng.random() < 0.3 else "shuffled"
    qd = "f32" if kv == "f32" else "bf16"
    need = sum(W.pages_for(x) for x in lens)
    kw = {} if layout == "fragmented" else {"num_pages": need + int(rng.integers(0, 9))}
    case = W.make_case(f"fuzz{seed}", batch=batch, q_per_seq=n, num_q_heads=hkv * group,
                       num_kv_heads=hkv, seq_lens=lens, kv_dtype=kv, q_dtype=qd,
                       seed=6000 + seed, layout=layout, **kw)
    if mode == "tree":
        case.tree_mask = np.stack([W.random_tree(rng, n)[1] for _ in range(batch)])
    part = int(rng.choice([0, 0, 1, 2, 3, 5, 8, 17]))
    staged_from = int(rng.choice([0, 0, -1]))
    return case, mode, part, staged_from


@pytest.mark.parametrize("seed", range(NUM_CASES))
def test_fuzz_against_oracle(pa, seed):
    case, mode, part, staged_from = fuzz_case(seed)
    say(f"[fuzz {seed}] mode={mode} kv={case.kv_dtype} B={case.batch} n={case.q_per_seq} "
        f"Hq={case.num_q_heads} Hkv={case.num_kv_heads} lens={list(case.seq_lens)} "
        f"part={part} staged_from={staged_from}")
    gpu = run_gpu(pa, case, part, label=f"fuzz {mode}", staged_from=staged_from)
    check(gpu, run_oracle(case), case.kv_dtype, f"fuzz {seed} {mode}")
