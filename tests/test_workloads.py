"""Host-side checks of the seeded input generators (no GPU, no oracle arithmetic)."""
import json
import os

import numpy as np

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_block_accounting_matches_section_10_12_2():
    fix = json.load(open(os.path.join(GOLDEN, "block_accounting_10_12_2.json")))
    blocks = [W.pages_for(x) for x in fix["lengths"]]
    assert blocks == fix["blocks"]
    assert sum(blocks) == fix["total_blocks"]
    assert sum(blocks) * fix["page_size"] == fix["slots"]
    assert fix["slots"] - sum(fix["lengths"]) == fix["wasted"]


def _check_table(case):
    used = []
    for b, length in enumerate(case.seq_lens):
        c = W.pages_for(length)
        row = case.block_table[b]
        assert (row[:c] >= 0).all() and (row[:c] < case.num_pages).all()
        assert (row[c:] == -1).all()
        used.extend(row[:c].tolist())
    assert len(used) == len(set(used))          # no page handed out twice


def test_named_workload_shapes_and_bytes():
    tiny = W.workload("tiny")
    assert tiny.num_pages == 16 and tiny.block_table.shape == (1, 4)
    assert tiny.algorithmic_bytes() == 139264
    _check_table(tiny)


def test_shuffled_tables_are_deterministic_and_scattered():
    rng = np.random.default_rng(5)
    a = W.shuffled_tables(rng, [2048] * 4, 512)
    b = W.shuffled_tables(np.random.default_rng(5), [2048] * 4, 512)
    assert (a == b).all()
    assert sorted(a.reshape(-1).tolist()) == list(range(512))
    assert (np.diff(a[0]) != 1).mean() > 0.9      # not laid out contiguously


def test_fragmented_tables_interleave_alloc_and_free():
    rng = np.random.default_rng(7)
    lens = W.ragged_lengths(rng, 40)
    table, num_pages = W.fragmented_tables(np.random.default_rng(8), lens)
    need = sum(W.pages_for(x) for x in lens)
    assert num_pages == int(np.ceil(1.25 * need))
    used = [p for b, x in enumerate(lens) for p in table[b, :W.pages_for(x)]]
    assert len(used) == len(set(used)) == need
    assert all(0 <= p < num_pages for p in used)
    # the free pages are spread through the pool, not one contiguous tail
    free = sorted(set(range(num_pages)) - set(used))
    assert free[0] < num_pages // 2


def test_ragged_lengths_recipe():
    lens = W.ragged_lengths(np.random.default_rng(3), 2000)
    assert lens.min() >= 128 + 50 and lens.max() <= 1024 + 400
    # mean of U{128..1024} is 576 and of {50, 400} is 225
    assert abs(lens.mean() - 801) < 20


def test_poison_marks_unused_slots():
    case = W.make_case("p", batch=2, q_per_seq=1, num_q_heads=4, num_kv_heads=2,
                       seq_lens=[20, 3], kv_dtype="bf16", q_dtype="bf16", seed=1,
                       num_pages=5)
    _check_table(case)
    p_last0 = case.block_table[0, 1]
    k_tok = W.k_from_pool(case.k_pool)
    assert (k_tok[p_last0, :, 4:] == W.BF16_NAN).all()
    assert (k_tok[p_last0, :, :4] != W.BF16_NAN).all()
    unused = sorted(set(range(5)) - set(case.block_table[case.block_table >= 0].tolist()))
    assert unused and (case.v_pool[unused] == W.BF16_NAN).all()


def test_fp8_scales_are_absmax_over_448():
    case = W.make_case("s", batch=1, q_per_seq=1, num_q_heads=2, num_kv_heads=1,
                       seq_lens=[40], kv_dtype="fp8", q_dtype="bf16", seed=2)
    # the largest byte of each live slab encodes +-448 (absmax / scale = 448)
    for p in case.block_table[0, :3]:
        live = 16 if p != case.block_table[0, 2] else 8
        slab = W.k_from_pool(case.k_pool)[p, 0, :live]
        assert (slab & 0x7F).max() == 0x7E
    assert np.isfinite(case.k_scale).all() and (case.k_scale > 0).all()
