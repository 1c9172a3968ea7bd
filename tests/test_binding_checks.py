"""The binding rejects tensors whose extents the library cannot check through
raw pointers (CPU: every check raises before a pointer is taken)."""
import pytest
import torch

import paged_kv_gqa_02_amd as pa
from paged_kv_gqa_02_amd import binding as B


def pool(hkv=8, pages=64, kv=B.PA_BF16):
    return B.Pool(None, (), pages, hkv, kv)


def tables(batch, pages=4, bt_dtype=torch.int32, len_dtype=torch.int32):
    return torch.zeros((batch, pages), dtype=bt_dtype), torch.ones(batch, dtype=len_dtype)


@pytest.mark.parametrize("shape,match", [
    ((2, 1, 32, 64), "128"),              # head dim other than 128
    ((2, 1, 12, 128), "multiple"),        # 12 query heads over 8 KV heads
    ((2, 32, 128), r"\[batch\]"),         # not 4-d
])
def test_verify_rejects_q_extents(shape, match):
    q = torch.zeros(shape, dtype=torch.bfloat16)
    bt, lens = tables(2)
    with pytest.raises(ValueError, match=match):
        pa.paged_attn_verify(pool(), q, torch.empty_like(q), bt, lens, 16, 0.1)


@pytest.mark.parametrize("bt_dtype,len_dtype", [(torch.int64, torch.int32),
                                                 (torch.int32, torch.int64)])
def test_verify_rejects_table_dtypes(bt_dtype, len_dtype):
    q = torch.zeros((2, 1, 32, 128), dtype=torch.bfloat16)
    bt, lens = tables(2, bt_dtype=bt_dtype, len_dtype=len_dtype)
    with pytest.raises(ValueError, match="int32"):
        pa.paged_attn_verify(pool(), q, torch.empty_like(q), bt, lens, 16, 0.1)


def test_decode_rejects_head_dim():
    q = torch.zeros((2, 1, 32, 96), dtype=torch.bfloat16)
    bt, lens = tables(2)
    with pytest.raises(ValueError, match="128"):
        pa.paged_attn_decode(pool(), q, torch.empty_like(q), bt, lens, 16, 0.1)


def test_tree_rejects_head_dim():
    q = torch.zeros((2, 4, 32, 64), dtype=torch.bfloat16)
    bt, lens = tables(2)
    with pytest.raises(ValueError, match="128"):
        pa.paged_attn_verify_tree(pool(), q, torch.empty_like(q), bt, lens, 16, 0.1,
                                  torch.zeros((2, 4), dtype=torch.int64))


@pytest.mark.parametrize("shape,match", [
    ((2, 1, 4, 128), "Hkv"),              # 4 KV heads into an 8-head pool
    ((2, 1, 8, 64), "128"),
])
def test_append_rejects_source_extents(shape, match):
    k = torch.zeros(shape, dtype=torch.float32)
    bt, lens = tables(2)
    with pytest.raises(ValueError, match=match):
        pa.paged_attn_append_kv(pool(), k, k.clone(), bt, lens)


@pytest.mark.parametrize("bt_dtype,len_dtype", [(torch.int64, torch.int32),
                                                 (torch.int32, torch.int16)])
def test_append_rejects_table_dtypes(bt_dtype, len_dtype):
    k = torch.zeros((2, 1, 8, 128), dtype=torch.float32)
    bt, lens = tables(2, bt_dtype=bt_dtype, len_dtype=len_dtype)
    with pytest.raises(ValueError, match="int32"):
        pa.paged_attn_append_kv(pool(), k, k.clone(), bt, lens)


@pytest.mark.parametrize("which,numel,dtype", [("k_scale", 63 * 8, torch.float32),
                                               ("v_scale", 64 * 8, torch.float16),
                                               ("k_scale", None, None)])
def test_fp8_pool_rejects_scale_sizes(which, numel, dtype):
    v = torch.zeros((64, 8, 16, 128), dtype=torch.uint8)
    k = torch.zeros((64, 8, 8, 16, 16), dtype=torch.uint8)
    good = torch.ones(64 * 8, dtype=torch.float32)
    bad = None if numel is None else torch.ones(numel, dtype=dtype)
    ks, vs = (bad, good) if which == "k_scale" else (good, bad)
    with pytest.raises(ValueError, match=which):
        pa.paged_attn_create_pool(k, v, ks, vs)


def test_sampler_rejects_output_shapes():
    p = torch.zeros((2, 3, 10), dtype=torch.float32)
    q = torch.zeros((2, 2, 10), dtype=torch.float32)
    d = torch.zeros((2, 2), dtype=torch.int32)
    ua = torch.zeros((2, 2), dtype=torch.float32)
    us = torch.zeros(2, dtype=torch.float32)
    with pytest.raises(ValueError, match="tokens"):
        pa.paged_attn_rejection_sample(p, q, d, ua, us, tokens=torch.zeros((2, 2), dtype=torch.int32))
    with pytest.raises(ValueError, match="num_accepted"):
        pa.paged_attn_rejection_sample(p, q, d, ua, us,
                                       num_accepted=torch.zeros(2, dtype=torch.int64))


def test_import_fails_loudly_without_the_library(tmp_path):
    """No fallback: with the HIP library absent, importing the package raises."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PAGED_ATTN_LIB=str(tmp_path / "absent" / "libpaged_attn.so"))
    res = subprocess.run([sys.executable, "-c", "import paged_kv_gqa_02_amd"], cwd=root, env=env,
                         capture_output=True, text=True, timeout=300)
    assert res.returncode != 0
    assert "ImportError" in res.stderr and "is missing" in res.stderr, res.stderr[-2000:]
