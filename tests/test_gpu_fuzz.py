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


# ----------------------------------------------------------------------------
# long sequences whose waves take their page ids in several rounds of 64
# ----------------------------------------------------------------------------
NUM_ROUND_CASES = 20


def rounds_case(seed):
    rng = np.random.default_rng(7000 + seed)
    kv = ["f32", "bf16", "fp8"][int(rng.integers(0, 3))]
    hkv = int(rng.choice([1, 2]))
    group = int(rng.choice([1, 2, 4]))
    n = int(rng.choice([1, 1, 3, 5]))
    batch = int(rng.integers(1, 4))
    lens = [int(rng.integers(max(n, 3000), 22000)) for _ in range(batch)]
    waves = int(rng.choice([4, 8]))
    part = int(rng.choice([300, 513, 1000, 1400]))     # > 64 ids per wave: two or more rounds
    qd = "f32" if kv == "f32" else "bf16"
    need = sum(W.pages_for(x) for x in lens)
    case = W.make_case(f"rounds{seed}", batch=batch, q_per_seq=n, num_q_heads=hkv * group,
                       num_kv_heads=hkv, seq_lens=lens, kv_dtype=kv, q_dtype=qd,
                       seed=8000 + seed, num_pages=need + int(rng.integers(0, 9)))
    return case, part, waves


@pytest.mark.parametrize("seed", range(NUM_ROUND_CASES))
def test_page_id_rounds_against_oracle(pa, seed):
    case, part, waves = rounds_case(seed)
    say(f"[rounds {seed}] kv={case.kv_dtype} B={case.batch} n={case.q_per_seq} "
        f"Hq={case.num_q_heads} Hkv={case.num_kv_heads} lens={list(case.seq_lens)} "
        f"part={part} waves={waves}")
    gpu = run_gpu(pa, case, part, label="rounds", waves=waves, staged_from=-1)
    check(gpu, run_oracle(case), case.kv_dtype, f"rounds {seed}")


# ----------------------------------------------------------------------------
# acceptance: random shapes and value ranges, tokens bit for bit
# ----------------------------------------------------------------------------
NUM_SAMPLER_CASES = 30


@pytest.mark.parametrize("seed", range(NUM_SAMPLER_CASES))
def test_sampler_fuzz_bit_exact(pa, seed):
    import oracle
    rng = np.random.default_rng(9000 + seed)
    B = int(rng.integers(1, 40))
    K = int(rng.choice([0, 1, 3, 4, 7, 64]))
    V = int(rng.choice([1, 5, 63, 4095, 4096, 4097, 9000, 20000]))
    if K >= 7:
        V = min(V, 4097)                 # keep [B][K + 1][V] small
    if rng.random() < 0.5:
        c = W.sampler_inputs(B, K, V, 9100 + seed)
        p, q = c.p, c.q
    else:
        # entries spread from subnormals to 2^11, zeros, empty residuals
        def wide(shape):
            mant = rng.integers(1 << 23, 1 << 24, size=shape).astype(np.float64)
            expo = rng.integers(-160, 12, size=shape)
            v = np.ldexp(mant, expo - 23).astype(np.float32)
            v[rng.random(shape) < 0.3] = 0.0
            return v
        p, q = wide((B, K + 1, V)), wide((B, K, V))
        if K and B > 1:
            q[0, 0] = p[0, 0]
    draft = rng.integers(0, V, size=(B, K)).astype(np.int32)
    ua = rng.random((B, K), dtype=np.float32)
    us = rng.random(B, dtype=np.float32)
    say(f"[sampler fuzz {seed}] B={B} K={K} V={V}")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    tokens, acc = pa.paged_attn_rejection_sample(dev(p), dev(q) if K else None,
                                                 dev(draft) if K else None,
                                                 dev(ua) if K else None, dev(us))
    torch.cuda.synchronize()
    want_t, want_a = oracle.rejection_sample(p, q, draft, ua, us)
    assert (acc.cpu().numpy() == want_a).all()
    assert (tokens.cpu().numpy() == want_t).all()
