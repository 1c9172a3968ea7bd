"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Gates (max |GPU - oracle| over every compared output): 1e-5 for fp32 inputs,
1.5e-2 for bf16 inputs with fp32 accumulation, 5e-2 for fp8-e4m3 KV; plus a
relative L2 gate, because with N(0, 1) data the outputs shrink like
sqrt(e / L) and a max-abs gate alone gets loose at long contexts.  The
relative gate is 1e-2 for bf16 and fp8: a kernel that dropped one 16-token
page of a 32768-token sequence would be off by about sqrt(16 / 32768) = 2.2e-2
there, and correct kernels stay near 3e-3 at most.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle_parallel import oracle_all
from workloads.device import to_device, to_numpy_f64

pytestmark = pytest.mark.gpu

MAX_ABS = {"f32": 1e-5, "bf16": 1.5e-2, "fp8": 5e-2}
REL_L2 = {"f32": 1e-5, "bf16": 1e-2, "fp8": 1e-2}


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_kv_gqa_02_amd as lib
    return lib


def say(msg):
    print(msg, flush=True)


def run_gpu(pa, case, partition_pages=0, dev=None, label="", waves=0, prefetch=0,
            staged_from=0):
    say(f"[gpu] {case.name} {label} kv={case.kv_dtype} B={case.batch} n={case.q_per_seq} "
        f"Hq={case.num_q_heads} Hkv={case.num_kv_heads} maxL={case.max_seq_len} "
        f"part={partition_pages} waves={waves} prefetch={prefetch} staged_from={staged_from} "
        f"seed={case.seed}")
    d = dev if dev is not None else to_device(case)
    pool = pa.paged_attn_create_pool(d.k, d.v, d.k_scale, d.v_scale, partition_pages, waves,
                                     prefetch, staged_from)
    out = torch.empty_like(d.q)
    ws = pa.workspace_for(pool, d.q, case.max_seq_len)
    pa.paged_attn_verify(pool, d.q, out, d.block_table, d.seq_lens, case.max_seq_len,
                         case.scale, ws, tree_mask=d.tree_mask)
    torch.cuda.synchronize()
    return to_numpy_f64(out)


def run_oracle(case, seqs=None):
    return oracle.paged_attention(case.k_pool, case.v_pool, case.kv_dtype, case.q, case.q_dtype,
                                  case.block_table, case.seq_lens, case.q_per_seq, case.scale,
                                  seqs=seqs, k_scale=case.k_scale, v_scale=case.v_scale,
                                  tree_mask=case.tree_mask)


def check(gpu, ref, kv_dtype, what):
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    err = float(np.abs(gpu - ref).max())
    rel = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300))
    say(f"    {what}: max_abs={err:.3e} rel_l2={rel:.3e}")
    assert err <= MAX_ABS[kv_dtype], f"{what}: max abs error {err}"
    assert rel <= REL_L2[kv_dtype], f"{what}: relative L2 error {rel}"
    return err, rel


def small_case(kv, n, hq, hkv, lens, seed, layout="shuffled", extra=3):
    qd = "f32" if kv == "f32" else "bf16"
    need = sum(W.pages_for(x) for x in lens)
    kw = {} if layout == "fragmented" else {"num_pages": need + extra}
    return W.make_case(f"small-{kv}", batch=len(lens), q_per_seq=n, num_q_heads=hq,
                       num_kv_heads=hkv, seq_lens=lens, kv_dtype=kv, q_dtype=qd, seed=seed,
                       layout=layout, **kw)


# ----------------------------------------------------------------------------
# small cases: every dtype, head layout, row count and split size
# ----------------------------------------------------------------------------
def test_tiny_workload(pa):
    case = W.workload("tiny")
    ref = run_oracle(case)
    for part in (0, 1, 2, 3):
        check(run_gpu(pa, case, part), ref, "f32", f"tiny part={part}")


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("n", [1, 5])
@pytest.mark.parametrize("heads", [(8, 2), (4, 4), (8, 1), (16, 2)])
def test_small_cases(pa, kv, n, heads):
    hq, hkv = heads
    lens = [max(n, 1), 17, 100, 333, 16, 48 + n]
    case = small_case(kv, n, hq, hkv, lens, seed=1000 + 7 * n + hq + 3 * hkv)
    ref = run_oracle(case)
    dev = to_device(case)
    for part in (0, 1, 3, 8):
        check(run_gpu(pa, case, part, dev=dev), ref, kv, f"part={part}")


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
def test_many_rows_span_several_workgroups(pa, kv):
    # G = 8, n = 12 -> 96 rows: two row chunks of 64
    case = small_case(kv, 12, 16, 2, [40, 200, 12], seed=77)
    ref = run_oracle(case)
    dev = to_device(case)
    for part in (0, 2):
        check(run_gpu(pa, case, part, dev=dev), ref, kv, f"rows=96 part={part}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("n", [1, 5])
def test_tuning_variants(pa, kv, n):
    """Every (waves, prefetch) instantiation, unsplit and split, against the oracle."""
    case = small_case(kv, n, 32, 8, [513, 100, 17, 2048, 64], seed=31 + n)
    ref = run_oracle(case)
    dev = to_device(case)
    for waves in (4, 8):
        for prefetch in (2, 3, 4, 5, 6):
            if waves == 8 and prefetch > 4:
                continue
            for part in (0, 7):
                check(run_gpu(pa, case, part, dev=dev, waves=waves, prefetch=prefetch), ref, kv,
                      f"waves={waves} prefetch={prefetch} part={part}")


def test_fragmented_pool(pa):
    lens = W.ragged_lengths(np.random.default_rng(5), 24)
    case = small_case("bf16", 1, 32, 8, lens, seed=55, layout="fragmented")
    check(run_gpu(pa, case), run_oracle(case), "bf16", "fragmented")


# ----------------------------------------------------------------------------
# exactness checks with closed forms
# ----------------------------------------------------------------------------
def test_fp8_bytes_decode_exactly(pa):
    """Single visible key: the output is that key's value row, for every finite byte."""
    finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)
    case = small_case("fp8", 1, 4, 2, [1, 1], seed=3, extra=0)
    vals = np.resize(finite, (2, 2, 128))                   # [seq][kv head][d]
    vscale = np.float32(0.5)
    for b in range(2):
        page = case.block_table[b, 0]
        case.v_pool[page, :, 0, :] = vals[b]
        case.v_scale[page, :] = vscale
    gpu = run_gpu(pa, case)
    dec = np.vectorize(oracle.e4m3_value)(vals) * float(vscale)
    for b in range(2):
        for h in range(4):
            assert (gpu[b, 0, h] == dec[b, h // 2]).all()


def one_hot(case, rng):
    """Make key j* of every (sequence, kv head) dominate: the output becomes V[j*]."""
    g = case.num_q_heads // case.num_kv_heads
    d = case.head_dim
    u = rng.standard_normal((case.batch, case.num_kv_heads, d)).astype(np.float32)
    u = np.round(u * 8) / 8                                  # exact in bf16 and e4m3
    q = np.repeat(u[:, None, :, None, :], g, axis=3).reshape(case.batch, 1, case.num_q_heads, d)
    q = np.broadcast_to(q, case.q.shape).astype(np.float32)
    case.q = W.bf16_bits(q) if case.q_dtype == "bf16" else q
    jstar = []
    lam_min = (30 + math.log(case.max_seq_len)) * 2
    for b in range(case.batch):
        L = int(case.seq_lens[b])
        js = rng.integers(0, L - case.q_per_seq + 1, size=case.num_kv_heads)
        jstar.append(js)
        for kh in range(case.num_kv_heads):
            uu = float(u[b, kh] @ u[b, kh])
            lam = lam_min / (case.scale * uu)
            pages = case.block_table[b, :W.pages_for(L)]
            case.k_pool[pages, kh] = 0
            if case.kv_dtype == "fp8":
                case.k_scale[pages, kh] = 1.0
            p, slot = pages[js[kh] // 16], js[kh] % 16
            row = (lam * u[b, kh]).astype(np.float32)
            if case.kv_dtype == "bf16":
                W.set_k_token(case.k_pool, p, kh, slot, W.bf16_bits(row))
            elif case.kv_dtype == "fp8":
                W.set_k_token(case.k_pool, p, kh, slot, W.e4m3_bytes(row))
            else:
                W.set_k_token(case.k_pool, p, kh, slot, row)
    return jstar


def check_one_hot(pa, case, label):
    """Outputs are O(1) here, so the dtype gates are tight relative to them."""
    rng = np.random.default_rng(case.seed + 1)
    jstar = one_hot(case, rng)
    gpu = run_gpu(pa, case, label=label + " one-hot")
    seqs = [0, case.batch - 1]
    check(gpu[seqs], run_oracle(case, seqs), case.kv_dtype, f"{label} one-hot vs oracle")
    g = case.num_q_heads // case.num_kv_heads
    for b in seqs:
        for kh in range(case.num_kv_heads):
            j = int(jstar[b][kh])
            page, slot = case.block_table[b, j // 16], j % 16
            raw = case.v_pool[page, kh, slot]
            if case.kv_dtype == "bf16":
                vrow = (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            elif case.kv_dtype == "fp8":
                vrow = np.vectorize(oracle.e4m3_value)(raw) * float(case.v_scale[page, kh])
            else:
                vrow = raw.astype(np.float64)
            got = gpu[b, :, kh * g:(kh + 1) * g]
            err = np.abs(got - vrow).max()
            assert err <= MAX_ABS[case.kv_dtype], f"{label}: b={b} kh={kh} off by {err}"


# ----------------------------------------------------------------------------
# invariants of the paged gather
# ----------------------------------------------------------------------------
def test_page_permutation_is_bitwise_invariant(pa):
    case = small_case("bf16", 3, 8, 2, [30, 129, 64, 7], seed=91, extra=10)
    base = run_gpu(pa, case, 2)
    perm = np.random.default_rng(92).permutation(case.num_pages)
    moved = W.Case(**{**case.__dict__})
    moved.k_pool = np.empty_like(case.k_pool)
    moved.v_pool = np.empty_like(case.v_pool)
    moved.k_pool[perm] = case.k_pool
    moved.v_pool[perm] = case.v_pool
    moved.block_table = np.where(case.block_table >= 0,
                                 perm[np.maximum(case.block_table, 0)], -1).astype(np.int32)
    assert (run_gpu(pa, moved, 2, label="permuted") == base).all()


def test_repeat_calls_are_bitwise_identical(pa):
    case = small_case("bf16", 1, 32, 8, [2048, 999], seed=93)
    dev = to_device(case)
    a = run_gpu(pa, case, dev=dev)
    b = run_gpu(pa, case, dev=dev)
    assert (a == b).all()


def test_aliased_pages_give_identical_rows(pa):
    case = small_case("bf16", 2, 8, 2, [70, 70, 33], seed=94)
    case.block_table[1] = case.block_table[0]
    case.q[1] = case.q[0]
    out = run_gpu(pa, case, 1)
    assert (out[0] == out[1]).all()
    check(out, run_oracle(case), "bf16", "aliased")


def test_verify_rows_match_prefix_decode(pa):
    n = 5
    case = small_case("bf16", n, 32, 8, [4101, 700, 90], seed=95)
    ver = run_gpu(pa, case)
    for i in range(n):
        pref = W.Case(**{**case.__dict__})
        pref.q_per_seq = 1
        pref.q = np.ascontiguousarray(case.q[:, i:i + 1])
        pref.seq_lens = (case.seq_lens - n + i + 1).astype(np.int32)
        dec = run_gpu(pa, pref, label=f"prefix row {i}")
        check(ver[:, i:i + 1], dec, "bf16", f"verify row {i} vs decode")


def test_split_sizes_agree(pa):
    case = small_case("f32", 5, 32, 8, [1000, 257, 5], seed=96)
    dev = to_device(case)
    ref = run_gpu(pa, case, 0, dev=dev)
    for part in (1, 2, 5, 16, 63):
        check(run_gpu(pa, case, part, dev=dev), ref, "f32", f"part={part} vs auto")


def test_workspace_reuse_and_partition_merge(pa):
    """One workspace serves repeated split calls (bit for bit the same output)
    and then a call of another shape: the partition kernel writes every partial
    the reduce reads, so nothing from an earlier call leaks into a later one."""
    big = small_case("bf16", 5, 32, 8, [4101, 700, 90], seed=61)
    d = to_device(big)
    pool = pa.paged_attn_create_pool(d.k, d.v, None, None, 7)
    plan = pa.paged_attn_plan(pool, big.batch, 5, 32, big.max_seq_len)
    assert plan["reduce"] == 1 and plan["num_splits"] > 1
    ws = pa.workspace_for(pool, d.q, big.max_seq_len)
    outs = []
    for _ in range(3):
        o = torch.empty_like(d.q)
        pa.paged_attn_verify(pool, d.q, o, d.block_table, d.seq_lens, big.max_seq_len,
                             big.scale, ws)
        outs.append(o)
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    check(to_numpy_f64(outs[0]), run_oracle(big), "bf16", "reused workspace")
    small = small_case("bf16", 1, 32, 8, [1000, 33], seed=62)
    ds = to_device(small)
    pool2 = pa.paged_attn_create_pool(ds.k, ds.v, None, None, 3)
    assert pa.paged_attn_workspace_bytes(pool2, 2, 1, 32, small.max_seq_len) <= ws.numel()
    o2 = torch.empty_like(ds.q)
    pa.paged_attn_verify(pool2, ds.q, o2, ds.block_table, ds.seq_lens, small.max_seq_len,
                         small.scale, ws)
    torch.cuda.synchronize()
    check(to_numpy_f64(o2), run_oracle(small), "bf16", "second shape, same workspace")


def test_sixty_four_partitions(pa):
    case = small_case("f32", 1, 8, 2, [16 * 64 * 3, 100], seed=63)
    check(run_gpu(pa, case, 1), run_oracle(case), "f32", "64 partitions of 3 pages")


def test_decode_entry_point_matches_verify(pa):
    case = small_case("bf16", 1, 32, 8, [300, 2048, 17], seed=97)
    d = to_device(case)
    pool = pa.paged_attn_create_pool(d.k, d.v)
    o1 = torch.empty_like(d.q)
    o2 = torch.empty_like(d.q)
    ws = pa.workspace_for(pool, d.q, case.max_seq_len)
    pa.paged_attn_decode(pool, d.q, o1, d.block_table, d.seq_lens, case.max_seq_len,
                         case.scale, ws)
    pa.paged_attn_verify(pool, d.q, o2, d.block_table, d.seq_lens, case.max_seq_len,
                         case.scale, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_validate_reports_bad_tables(pa):
    case = small_case("bf16", 1, 8, 2, [40, 20], seed=98)
    d = to_device(case)
    pool = pa.paged_attn_create_pool(d.k, d.v)
    pa.paged_attn_validate(pool, d.block_table, d.seq_lens, case.max_seq_len, 1)
    bad = d.block_table.clone()
    bad[1, 0] = case.num_pages
    with pytest.raises(pa.PagedAttnError):
        pa.paged_attn_validate(pool, bad, d.seq_lens, case.max_seq_len, 1)


# ----------------------------------------------------------------------------
# draft-tree verification
# ----------------------------------------------------------------------------
def with_tree(case, seed):
    rng = np.random.default_rng(seed)
    case.tree_mask = np.stack([W.random_tree(rng, case.q_per_seq)[1] for _ in range(case.batch)])
    return case


@pytest.mark.parametrize("kernel", ["staged", "partition"])
@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("n", [5, 16, 64])
def test_tree_verify_matches_oracle(pa, kernel, kv, n):
    # bf16 / fp8 trees take the LDS-staged kernel unless staged_from = -1; f32 never
    case = with_tree(small_case(kv, n, 32, 8, [n, n + 17, 300, 1000], seed=200 + n), 300 + n)
    ref = run_oracle(case)
    dev = to_device(case)
    sf = 0 if kernel == "staged" else -1
    for part in (0, 3, 4):      # odd and even partition lengths
        check(run_gpu(pa, case, part, dev=dev, label=f"tree {kernel}", staged_from=sf), ref, kv,
              f"tree n={n} part={part} {kernel}")


@pytest.mark.parametrize("n", [5, 16])
def test_chain_tree_equals_causal_verify_bitwise(pa, n):
    """On one kernel (the partition kernel takes both), a chain tree is the causal mask."""
    case = small_case("bf16", n, 32, 8, [4101, 77, n], seed=210 + n)
    dev = to_device(case)
    causal = run_gpu(pa, case, dev=dev, label="causal", staged_from=-1)
    case.tree_mask = np.stack([W.chain_tree(n)] * case.batch)
    chain = run_gpu(pa, case, label="chain tree", staged_from=-1)
    assert (chain == causal).all()


@pytest.mark.parametrize("n", [5, 16, 64])
def test_staged_chain_tree_equals_causal_verify(pa, n):
    """The LDS-staged tree kernel on a chain tree against the causal verify."""
    case = small_case("bf16", n, 32, 8, [4101, 77, n], seed=230 + n)
    dev = to_device(case)
    causal = run_gpu(pa, case, dev=dev, label="causal", staged_from=-1)
    case.tree_mask = np.stack([W.chain_tree(n)] * case.batch)
    for part in (0, 5):
        chain = run_gpu(pa, case, part, label="staged chain tree")
        # two kernels, two fp32 accumulation orders, each rounded to bf16, so
        # the same bf16 gate each of them meets against the oracle (outputs
        # here reach O(1), where one bf16 ulp is 2^-7)
        check(chain, causal, "bf16", f"staged chain tree vs causal part={part}")


def test_tree_entry_point_and_limits(pa):
    case = with_tree(small_case("bf16", 7, 8, 2, [100, 40], seed=220), 221)
    d = to_device(case)
    pool = pa.paged_attn_create_pool(d.k, d.v)
    out = torch.empty_like(d.q)
    ws = pa.workspace_for(pool, d.q, case.max_seq_len)
    pa.paged_attn_verify_tree(pool, d.q, out, d.block_table, d.seq_lens, case.max_seq_len,
                              case.scale, d.tree_mask, ws)
    torch.cuda.synchronize()
    check(to_numpy_f64(out), run_oracle(case), "bf16", "verify_tree entry point")
    big = small_case("bf16", 65, 8, 2, [100], seed=222)
    db = to_device(big)
    with pytest.raises(pa.PagedAttnError):
        pa.paged_attn_verify_tree(pool, db.q, torch.empty_like(db.q), db.block_table,
                                  db.seq_lens, big.max_seq_len, big.scale,
                                  torch.zeros((1, 65), dtype=torch.int64, device="cuda"))


# ----------------------------------------------------------------------------
# the named workloads at full size, every sequence against the oracle
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["decode8b", "ragged", "verify", "fp8long", "tree"])
def test_workload_native_dtype(pa, name):
    case = W.workload(name)
    gpu = run_gpu(pa, case)
    check(gpu, oracle_all(case), case.kv_dtype, f"{name}, all {case.batch} sequences")


@pytest.mark.parametrize("name", ["decode8b", "ragged", "verify", "fp8long", "tree"])
def test_workload_fp32_structure(pa, name):
    """Same shapes and layout in fp32: pins gather, masks and splits at 1e-5."""
    case = W.workload(name, kv_dtype="f32", q_dtype="f32")
    gpu = run_gpu(pa, case, label="fp32")
    check(gpu, oracle_all(case), "f32", f"{name} fp32, all {case.batch} sequences")


@pytest.mark.parametrize("kv", ["f32", "bf16"])
def test_context_past_64_page_ids_per_wave(pa, kv):
    """A context of 270,000 tokens (16,875 pages) in one sequence, one KV head
    and one query head: the automatic plan caps the partitions at 64, so each
    of a workgroup's four waves walks 66 pages and takes its page ids in two
    rounds."""
    case = W.make_case(f"long-{kv}", batch=1, q_per_seq=1, num_q_heads=1, num_kv_heads=1,
                       seq_lens=[270000], kv_dtype=kv, q_dtype=kv, seed=4242)
    d = to_device(case)
    pool = pa.paged_attn_create_pool(d.k, d.v)
    plan = pa.paged_attn_plan(pool, 1, 1, 1, case.max_seq_len)
    assert plan["num_splits"] == 64 and plan["partition_pages"] > 64 * plan["waves"], plan
    check(run_gpu(pa, case, dev=d), run_oracle(case), kv, f"L=270000 {kv} plan {plan}")


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("n", [1, 5])
def test_partition_of_many_page_id_rounds(pa, kv, n):
    """A pool asking for 1,000-page partitions: a wave of four walks up to 250
    pages in four rounds of page ids (the last round partial), unsplit and
    split, with ragged lengths around the round edges."""
    lens = [4000 * 16 + 5, 257 * 16, 64 * 4 * 16 + 1, 1000 * 16 + 3, 33]
    case = small_case(kv, n, 8, 2, lens, seed=4300 + n)
    ref = run_oracle(case)
    dev = to_device(case)
    for part in (1000, 257, 256):
        check(run_gpu(pa, case, part, dev=dev), ref, kv, f"part={part}")


@pytest.mark.parametrize("name", ["decode8b", "verify", "fp8long"])
def test_workload_one_hot(pa, name):
    case = W.workload(name, poison=True)
    check_one_hot(pa, case, name)


@pytest.mark.parametrize("kind", ["partition", "staged tree", "split partition"])
def test_timed_call_same_output_and_kernel_time(pa, kind):
    """paged_attn_verify_timed: the same bits as the untimed call, and the
    events attached to the attention kernel's dispatch give its execution time,
    which lies inside the time of events recorded around the whole call."""
    n = 16 if kind == "staged tree" else 1
    case = small_case("bf16", n, 32, 8, [1500, 700, 33], seed=77)
    if kind == "staged tree":
        rng = np.random.default_rng(78)
        case.tree_mask = np.stack([W.random_tree(rng, n)[1] for _ in range(case.batch)])
    d = to_device(case)
    part = 16 if kind == "split partition" else 0
    pool = pa.paged_attn_create_pool(d.k, d.v, d.k_scale, d.v_scale, part)
    ws = pa.workspace_for(pool, d.q, case.max_seq_len)
    plain = torch.empty_like(d.q)
    pa.paged_attn_verify(pool, d.q, plain, d.block_table, d.seq_lens, case.max_seq_len,
                         case.scale, ws, tree_mask=d.tree_mask)
    timed = torch.empty_like(d.q)
    stream = torch.cuda.current_stream()
    c0, c1, k0, k1 = (pa.HipEvent() for _ in range(4))
    c0.record(stream)
    pa.paged_attn_verify(pool, d.q, timed, d.block_table, d.seq_lens, case.max_seq_len,
                         case.scale, ws, ev_begin=k0, ev_end=k1, tree_mask=d.tree_mask)
    c1.record(stream)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), timed.view(torch.int16))
    kern, call = k0.elapsed_ms(k1), c0.elapsed_ms(c1)
    say(f"    {kind}: kernel {kern * 1e3:.2f} us inside call {call * 1e3:.2f} us")
    assert 0 < kern <= call



def test_tree_call_with_low_staged_from(pa):
    """A pool whose staged_from (16) is below the tree size (20 nodes): the causal
    plan of the shape is the chunked-prefill one, the tree call must still take
    the split tree path with the workspace the library reports."""
    n = 20
    case = small_case("bf16", n, 32, 8, [3000, 900, 41], seed=321)
    rng = np.random.default_rng(322)
    case.tree_mask = np.stack([W.random_tree(rng, n)[1] for _ in range(case.batch)])
    check(run_gpu(pa, case, label="tree, staged_from 16", staged_from=16), run_oracle(case),
          "bf16", "tree staged_from=16")


def _perturb_token(case, b, t, rng):
    """Give token t of sequence b new K and V rows (every kv head), in place."""
    page = int(case.block_table[b, t // W.PAGE_SIZE])
    slot = t % W.PAGE_SIZE
    for kh in range(case.num_kv_heads):
        k = rng.standard_normal(case.head_dim).astype(np.float32) * 3
        v = rng.standard_normal(case.head_dim).astype(np.float32) * 3
        if case.kv_dtype == "bf16":
            k, v = W.bf16_bits(k), W.bf16_bits(v)
        W.set_k_token(case.k_pool, page, kh, slot, k)
        case.v_pool[page, kh, slot, :] = v


@pytest.mark.parametrize("kind", ["verify", "prefill", "tree"])
def test_causality_under_perturbation(pa, kind):
    """New K/V for token j leave every row that does not see j bitwise unchanged
    (and change the rows that do): the causal limit, the chunked-prefill kernel's
    limit and the tree's ancestor masks, each on its own kernel."""
    rng = np.random.default_rng(880)
    n = {"verify": 5, "prefill": 160, "tree": 16}[kind]
    case = small_case("bf16", n, 32, 8, [700, n + 3, 1300], seed=881)
    if kind == "tree":
        case.tree_mask = np.stack([W.random_tree(rng, n)[1] for _ in range(case.batch)])
    before = run_gpu(pa, case, label=f"{kind} before")
    j = {"verify": 3, "prefill": 100, "tree": 9}[kind]
    for b in range(case.batch):
        _perturb_token(case, b, int(case.seq_lens[b]) - n + j, rng)
    after = run_gpu(pa, case, label=f"{kind} after")
    for b in range(case.batch):
        for i in range(n):
            sees = (int(case.tree_mask[b, i]) >> j) & 1 if kind == "tree" else i >= j
            same = np.array_equal(before[b, i], after[b, i])
            assert same != bool(sees), f"{kind}: b={b} row {i} {'changed' if not same else 'unchanged'}"


@pytest.mark.parametrize("kv,n", [("bf16", 1), ("bf16", 5), ("f32", 5), ("bf16", 16)])
def test_gqa_mapping_with_constant_values(pa, kv, n):
    """V of kv head k equal to k everywhere: query head h must return h // G, whatever
    the keys and queries (the head grouping, on the decode, verify and tree paths)."""
    hq, hkv = 32, 4
    case = small_case(kv, n, hq, hkv, [300, 57, 1000], seed=890)
    for kh in range(hkv):
        val = np.full(case.v_pool[:, kh].shape, float(kh), dtype=np.float32)
        case.v_pool[:, kh] = W.bf16_bits(val) if kv == "bf16" else val
    if n == 16:
        rng = np.random.default_rng(891)
        case.tree_mask = np.stack([W.random_tree(rng, n)[1] for _ in range(case.batch)])
    out = run_gpu(pa, case, label="constant V")
    want = (np.arange(hq) // (hq // hkv)).astype(np.float64)
    err = float(np.abs(out - want[None, None, :, None]).max())
    say(f"    GQA mapping {kv} n={n}: max_abs={err:.3e}")
    assert err <= (1e-5 if kv == "f32" else 1e-6)


@pytest.mark.parametrize("name,batch,n,hq,hkv,kv,lo,hi", [
    ("decode", 2048, 1, 32, 8, "bf16", 1, 300),
    ("verify", 1024, 5, 32, 8, "bf16", 5, 700),
])
def test_large_batches(pa, name, batch, n, hq, hkv, kv, lo, hi):
    """Serving-sized batches of short ragged sequences (grids of 8,192 to 16,384
    workgroups), every sequence against the oracle."""
    rng = np.random.default_rng(300 + batch)
    lens = [int(x) for x in rng.integers(lo, hi + 1, size=batch)]
    case = W.make_case(f"large-{name}", batch=batch, q_per_seq=n, num_q_heads=hq,
                       num_kv_heads=hkv, seq_lens=lens, kv_dtype=kv, q_dtype="bf16",
                       seed=400 + batch)
    gpu = run_gpu(pa, case, label="large batch")
    check(gpu, oracle_all(case), kv, f"{name}, batch {batch}, all sequences")
