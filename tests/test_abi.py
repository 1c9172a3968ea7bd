"""C-ABI checks that need no GPU: exports, host-side validation, launch plans."""
import ctypes
import re

import pytest

import paged_kv_gqa_02_amd as pa
from paged_kv_gqa_02_amd import binding as B

LIB = B.library()
FAKE_K, FAKE_V, FAKE_S = 0x10000, 0x20000, 0x30000   # never dereferenced by these calls


def test_every_declared_symbol_is_exported():
    names = pa.declared_symbols()
    assert len(names) >= 11
    for name in names:
        assert hasattr(LIB, name), name


def test_header_and_binding_agree_on_names():
    text = open(B.HEADER).read()
    for name in re.findall(r"\b(paged_attn_\w+)\s*\(", text):
        if name not in ("paged_attn_status_str", "paged_attn_last_error"):
            assert hasattr(pa, name), name


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert LIB.paged_attn_status_str(code)
    assert LIB.paged_attn_status_str(-99) == b"unknown status"


def _desc(**kw):
    d = dict(num_pages=64, page_size=16, num_kv_heads=8, head_dim=128, kv_dtype=B.PA_BF16,
             k=FAKE_K, v=FAKE_V, k_scale=None, v_scale=None, partition_pages=0, waves=0,
             prefetch=0, staged_from=0)
    d.update(kw)
    return B.pa_pool_desc(**d)


def _create(**kw):
    h = ctypes.c_void_p()
    st = LIB.paged_attn_create_pool(ctypes.byref(_desc(**kw)), ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("kw,status", [
    (dict(page_size=8), B.PA_ERR_UNSUPPORTED),
    (dict(head_dim=64), B.PA_ERR_UNSUPPORTED),
    (dict(kv_dtype=7), B.PA_ERR_UNSUPPORTED),
    (dict(num_pages=0), B.PA_ERR_INVALID_ARG),
    (dict(num_kv_heads=0), B.PA_ERR_INVALID_ARG),
    (dict(k=None), B.PA_ERR_INVALID_ARG),
    (dict(kv_dtype=B.PA_FP8_E4M3), B.PA_ERR_INVALID_ARG),      # fp8 without scales
    (dict(partition_pages=-1), B.PA_ERR_INVALID_ARG),
    (dict(waves=6), B.PA_ERR_UNSUPPORTED),
    (dict(prefetch=9), B.PA_ERR_UNSUPPORTED),
    (dict(waves=8, prefetch=5), B.PA_ERR_UNSUPPORTED),
    (dict(staged_from=-2), B.PA_ERR_INVALID_ARG),
])
def test_create_pool_rejects(kw, status):
    st, h = _create(**kw)
    assert st == status and not h.value
    assert LIB.paged_attn_last_error()


def test_pool_bytes():
    kb, vb = pa.paged_attn_pool_bytes(8192, 8, B.PA_BF16)
    assert kb == vb == 8192 * 8 * 16 * 128 * 2
    kb, _ = pa.paged_attn_pool_bytes(8192, 8, B.PA_FP8_E4M3)
    assert kb == 8192 * 8 * 16 * 128


def _plan(h, batch, n, hq, maxlen):
    pl = B.pa_plan()
    assert LIB.paged_attn_plan(h, batch, n, hq, maxlen, ctypes.byref(pl)) == 0
    return pl


def test_plans_for_named_workloads():
    st, h = _create(num_pages=8192)
    assert st == 0
    one = _plan(h, 64, 1, 32, 2048)                  # 512 (seq, kv head) units: no split
    assert one.num_splits == 1 and one.reduce == 0 and one.grid == 512 and one.row_tiles == 1
    ver = _plan(h, 8, 5, 32, 4101)                   # 20 rows -> two 16-row tiles, split
    assert ver.row_tiles == 2 and ver.row_chunks == 1 and ver.reduce == 1
    assert ver.num_splits * ver.partition_pages >= 257
    big = _plan(h, 1, 20, 32, 4096)                  # 80 rows -> two 64-row chunks
    assert big.row_tiles == 4 and big.row_chunks == 2
    assert one.kernel == ver.kernel == big.kernel == 0
    LIB.paged_attn_destroy_pool(h)


def test_prefill_plans():
    st, h = _create(num_pages=8192)
    pre = _plan(h, 4, 512, 32, 2048)                 # 2048 rows -> 8 blocks of 256, no split
    assert pre.kernel == 1 and pre.row_chunks == 16 and pre.grid == 4 * 8 * 16
    assert pre.reduce == 0 and pre.num_splits == 1
    assert _plan(h, 4, 127, 32, 2048).kernel == 0    # below 128 rows per sequence
    assert _plan(h, 1, 130, 32, 2048).row_chunks == 5    # 520 rows: the last block partial
    assert _plan(h, 1, 128, 32, 2048 * 16 + 16).kernel == 0   # past the page-id table
    ws = ctypes.c_size_t(1)
    assert LIB.paged_attn_workspace_bytes(h, 4, 512, 32, 2048, ctypes.byref(ws)) == 0
    assert ws.value == 0
    LIB.paged_attn_destroy_pool(h)
    st, h = _create(num_pages=8192, staged_from=-1)  # never
    assert _plan(h, 4, 512, 32, 2048).kernel == 0
    LIB.paged_attn_destroy_pool(h)
    st, h = _create(num_pages=8192, staged_from=16)
    assert _plan(h, 4, 16, 32, 2048).kernel == 1
    LIB.paged_attn_destroy_pool(h)
    st, h = _create(num_pages=8192, kv_dtype=B.PA_F32)   # fp32 stays on the partition kernel
    assert _plan(h, 4, 512, 32, 2048).kernel == 0
    LIB.paged_attn_destroy_pool(h)


def test_split_count_is_capped():
    st, h = _create(num_pages=8192, partition_pages=1)
    pl = _plan(h, 1, 1, 8, 32768)                    # 2048 pages, asked 1 page each
    assert pl.num_splits <= 64 and pl.num_splits * pl.partition_pages >= 2048
    LIB.paged_attn_destroy_pool(h)


def test_workspace_sizes():
    st, h = _create(num_pages=8192)
    n = ctypes.c_size_t()
    assert LIB.paged_attn_workspace_bytes(h, 64, 1, 32, 2048, ctypes.byref(n)) == 0
    assert n.value == 0
    assert LIB.paged_attn_workspace_bytes(h, 8, 5, 32, 4101, ctypes.byref(n)) == 0
    pl = _plan(h, 8, 5, 32, 4101)
    rows = 8 * 5 * 32 * pl.num_splits
    acc = (rows * 128 * 4 + 255) // 256 * 256
    assert n.value == acc + rows * 2 * 4
    LIB.paged_attn_destroy_pool(h)


def _verify(h, **kw):
    a = dict(q=0x40000, q_dtype=B.PA_BF16, out=0x50000, bt=0x60000, max_pages=128,
             lens=0x70000, max_len=2048, batch=64, n=1, hq=32, scale=0.088, ws=None,
             ws_bytes=0)
    a.update(kw)
    return LIB.paged_attn_verify(h, a["q"], a["q_dtype"], a["out"], a["bt"], a["max_pages"],
                                 a["lens"], a["max_len"], a["batch"], a["n"], a["hq"],
                                 a["scale"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), B.PA_ERR_INVALID_ARG),
    (dict(bt=None), B.PA_ERR_INVALID_ARG),
    (dict(q_dtype=B.PA_F32), B.PA_ERR_UNSUPPORTED),              # bf16 pool, f32 q
    (dict(q_dtype=9), B.PA_ERR_INVALID_ARG),
    (dict(batch=0), B.PA_ERR_INVALID_ARG),
    (dict(n=0), B.PA_ERR_INVALID_ARG),
    (dict(hq=12), B.PA_ERR_INVALID_ARG),                         # not a multiple of 8
    (dict(max_len=4000), B.PA_ERR_INVALID_ARG),                  # > 16 * max_pages
    (dict(max_len=3, n=5), B.PA_ERR_INVALID_ARG),                # max_seq_len < q_per_seq
    (dict(scale=float("nan")), B.PA_ERR_INVALID_ARG),
    (dict(q=0x40008), B.PA_ERR_INVALID_ARG),                     # misaligned q
    (dict(batch=8, n=5, max_len=4101, max_pages=257), B.PA_ERR_WORKSPACE),   # split, no ws
    (dict(batch=8, n=5, max_len=4101, max_pages=257, ws=0x80000, ws_bytes=16),
     B.PA_ERR_WORKSPACE),
    (dict(batch=8, n=5, max_len=4101, max_pages=257, ws=0x80010, ws_bytes=1 << 30),
     B.PA_ERR_WORKSPACE),                                        # misaligned workspace
])
def test_verify_rejects_before_launch(kw, status):
    st, h = _create(num_pages=8192)
    assert _verify(h, **kw) == status
    assert LIB.paged_attn_last_error()
    LIB.paged_attn_destroy_pool(h)


def test_null_pool_rejected():
    assert _verify(None) == B.PA_ERR_INVALID_ARG


# ----------------------------------------------------------------------------
# speculative-sampling acceptance: host-side checks (return before any launch)
# ----------------------------------------------------------------------------
def _sample(p=0x40000, q=0x50000, draft=0x60000, ua=0x70000, us=0x80000, batch=4, k=4,
            vocab=128256, tokens=0x90000, acc=0xA0000, ws=0xB0000, ws_bytes=1 << 20):
    return LIB.paged_attn_rejection_sample(p, q, draft, ua, us, batch, k, vocab, tokens, acc, ws,
                                           ws_bytes, None)


def test_sample_workspace_bytes():
    # two exact sums (six uint32 columns each) per 4096-entry chunk, then one
    # int32 per sequence
    assert pa.paged_attn_rejection_sample_workspace_bytes(64, 128256) == 64 * 32 * 48 + 64 * 4
    assert pa.paged_attn_rejection_sample_workspace_bytes(1, 4096) == 48 + 4
    assert pa.paged_attn_rejection_sample_workspace_bytes(1, 4097) == 96 + 4
    assert pa.paged_attn_rejection_sample_workspace_bytes(0, 10) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(p=None), B.PA_ERR_INVALID_ARG),
    (dict(us=None), B.PA_ERR_INVALID_ARG),
    (dict(tokens=None), B.PA_ERR_INVALID_ARG),
    (dict(q=None), B.PA_ERR_INVALID_ARG),                        # drafts but no q
    (dict(batch=0), B.PA_ERR_INVALID_ARG),
    (dict(vocab=0), B.PA_ERR_INVALID_ARG),
    (dict(k=-1), B.PA_ERR_INVALID_ARG),
    (dict(k=65), B.PA_ERR_UNSUPPORTED),
    (dict(vocab=(1 << 20) + 1), B.PA_ERR_UNSUPPORTED),
    (dict(batch=65536), B.PA_ERR_UNSUPPORTED),
    (dict(ws=None), B.PA_ERR_WORKSPACE),
    (dict(ws_bytes=64 * 32 * 48 - 1, batch=64), B.PA_ERR_WORKSPACE),
    (dict(ws=0xB0002), B.PA_ERR_INVALID_ARG),                    # misaligned workspace
])
def test_sample_rejects_before_launch(kw, status):
    assert _sample(**kw) == status
    assert LIB.paged_attn_last_error()


def test_workspace_covers_tree_calls_when_prefill_plan_is_reported():
    """staged_from = 16: a 20-row shape reports the chunked-prefill plan (no
    workspace), but a draft-tree call of that shape runs the split plan, so the
    reported workspace must cover that plan too."""
    st, h = _create(num_pages=8192, staged_from=16)
    assert st == 0
    pl = _plan(h, 2, 20, 32, 4096)
    assert pl.kernel == 1 and pl.reduce == 0
    ws = ctypes.c_size_t()
    assert LIB.paged_attn_workspace_bytes(h, 2, 20, 32, 4096, ctypes.byref(ws)) == 0
    st2, h2 = _create(num_pages=8192, staged_from=-1)      # the split plan itself
    tree = _plan(h2, 2, 20, 32, 4096)
    assert tree.kernel == 0 and tree.reduce == 1
    need = ctypes.c_size_t()
    assert LIB.paged_attn_workspace_bytes(h2, 2, 20, 32, 4096, ctypes.byref(need)) == 0
    assert ws.value >= need.value > 0
    LIB.paged_attn_destroy_pool(h)
    LIB.paged_attn_destroy_pool(h2)


@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("max_len", [262160, 524304, 1 << 20])
def test_long_context_plans_take_page_id_rounds(waves, max_len):
    """Past 64 * W * 64 pages the automatic plan stays at 64 partitions, so a
    wave walks more than 64 pages and the partition kernel takes its page ids in
    rounds of 64 (checked against the oracle on the GPU at 270,000 tokens)."""
    st, h = _create(num_pages=1 << 16, waves=waves)
    assert st == 0
    pl = _plan(h, 1, 1, 32, max_len)
    pages = (max_len + 15) // 16
    assert pl.num_splits == 64 and pl.num_splits * pl.partition_pages >= pages
    assert pl.kernel == 0 and pl.waves == waves
    assert pl.partition_pages > 64 * waves or pages <= 64 * 64 * waves
    LIB.paged_attn_destroy_pool(h)


def test_pool_partition_request_is_kept():
    """A partition length the pool asks for is used as given, also above 64
    pages per wave (the kernel then takes its page ids in rounds)."""
    st, h = _create(num_pages=8192, partition_pages=1000)
    pl = _plan(h, 2, 1, 32, 16 * 4001)
    assert pl.partition_pages == 1000 and pl.num_splits == 5
    LIB.paged_attn_destroy_pool(h)


def test_noalloc_rejects_partials_past_its_scratch():
    """The no-allocation call checks its 16 MiB limit on the host before any HIP call."""
    st, h = _create(num_pages=8192, partition_pages=1)       # 52 splits of 5 pages
    need = ctypes.c_size_t()
    assert LIB.paged_attn_workspace_bytes(h, 8, 5, 32, 4101, ctypes.byref(need)) == 0
    assert need.value > 16 << 20
    st = LIB.paged_attn_verify_noalloc(h, 0x40000, B.PA_BF16, 0x50000, 0x60000, 257, 0x70000,
                                       4101, 8, 5, 32, 0.088, None)
    assert st == B.PA_ERR_WORKSPACE and b"16 MiB" in LIB.paged_attn_last_error()
    assert LIB.paged_attn_verify_noalloc(None, 0x40000, B.PA_BF16, 0x50000, 0x60000, 257,
                                         0x70000, 4101, 8, 5, 32, 0.088, None) == B.PA_ERR_INVALID_ARG
    LIB.paged_attn_destroy_pool(h)
