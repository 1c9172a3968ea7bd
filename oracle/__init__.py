"""CPU oracle for paged GQA decode / verify attention (float64, plain C).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the GPU library in ``paged_kv_gqa_02_amd`` and never imports it.

The arithmetic lives in ``oracle.c`` (sources cited in ``oracle.h``); this
module only builds that file with gcc and marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
# ORACLE_LIB names another build of oracle.c to load (the sanitizer test's)
LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

F32, BF16, E4M3 = 0, 1, 2
_CODES = {"f32": F32, "bf16": BF16, "fp8": E4M3}

_lib = None


GCC_FLAGS = ["-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-fno-fast-math"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (strict IEEE, no fast-math)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-O2", *GCC_FLAGS, SOURCE, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def build_sanitized(path: str) -> str:
    """oracle.c built with AddressSanitizer and UndefinedBehaviorSanitizer (host
    code, gcc), every finding fatal; load it by running the tests with
    ORACLE_LIB=path and gcc's libasan preloaded."""
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", *GCC_FLAGS, SOURCE, "-o", path, "-lm"],
                   check=True)
    return path


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(LIB_PATH)
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        vp = ctypes.c_void_p
        i = ctypes.c_int
        lib.oracle_attention.restype = i
        lib.oracle_attention.argtypes = [vp, vp, vp, i, i, i, i, i, ctypes.c_double, vp]
        lib.oracle_attention_tree.restype = i
        lib.oracle_attention_tree.argtypes = [vp, vp, vp, i, i, i, i, i, ctypes.c_double, vp, vp]
        lib.oracle_paged_attention_tree.restype = i
        lib.oracle_paged_attention_tree.argtypes = [vp, vp, i, vp, vp, i, i, i, i, vp, i, vp, i,
                                                    vp, i, i, i, ctypes.c_double, vp, vp, i, vp]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        lib.oracle_append_kv.restype = i
        lib.oracle_append_kv.argtypes = [vp, vp, i, vp, vp, i, i, i, i, vp, vp, i, vp, i, vp,
                                         i, i]
        lib.oracle_rejection_sample.restype = i
        lib.oracle_rejection_sample.argtypes = [vp, vp, vp, vp, vp, i, i, i, vp, vp]
        lib.oracle_paged_attention.restype = i
        lib.oracle_paged_attention.argtypes = [vp, vp, i, vp, vp, i, i, i, i, vp, i, vp, i,
                                               vp, i, i, i, ctypes.c_double, vp, i, vp]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(int(bits))


def e4m3_value(byte: int) -> float:
    return _load().oracle_e4m3_value(int(byte))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Plain attention for one sequence.

    q [n][Hq][D], k and v [L][Hkv][D] (any float dtype, converted to float64).
    Returns [n][Hq][D] float64; row i sees keys 0 .. L - n + i.
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    n, hq, d = q.shape
    length, hkv, d2 = k.shape
    if v.shape != k.shape or d2 != d:
        raise ValueError("shape mismatch")
    out = np.empty((n, hq, d), dtype=np.float64)
    rc = _load().oracle_attention(_ptr(q), _ptr(k), _ptr(v), length, n, hq, hkv, d,
                                  float(scale), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_attention rejected its arguments (code {rc})")
    return out


def attention_tree(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   tree_mask) -> np.ndarray:
    """Tree verification for one sequence: row i sees every context key and
    the tree keys whose bit is set in tree_mask[i] (uint64, n <= 64)."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    mask = np.ascontiguousarray(tree_mask, dtype=np.uint64)
    n, hq, d = q.shape
    length, hkv, d2 = k.shape
    if v.shape != k.shape or d2 != d or mask.shape != (n,):
        raise ValueError("shape mismatch")
    out = np.empty((n, hq, d), dtype=np.float64)
    rc = _load().oracle_attention_tree(_ptr(q), _ptr(k), _ptr(v), length, n, hq, hkv, d,
                                       float(scale), _ptr(mask), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_attention_tree rejected its arguments (code {rc})")
    return out


def paged_attention(k_pool, v_pool, kv_dtype: str, q, q_dtype: str, block_table,
                    seq_lens, q_per_seq: int, scale: float, seqs=None,
                    k_scale=None, v_scale=None, tree_mask=None) -> np.ndarray:
    """Paged attention read straight from the pool, for the listed sequences.

    v_pool: [num_pages][Hkv][page_size][D] as float32 (``f32``), uint16 bf16
    bits (``bf16``) or uint8 E4M3 bytes (``fp8``); k_pool: the same elements in
    the chunked K layout [num_pages][Hkv][D/x][page_size][x], x = 16 bytes /
    element size.
    q: [batch][n][Hq][D] float32 or uint16 bf16 bits.  Returns
    [len(seqs)][n][Hq][D] float64.  tree_mask: optional [batch][n] uint64
    ancestor masks (draft-tree verification); None = the causal chain.
    """
    k_pool = np.ascontiguousarray(k_pool)
    v_pool = np.ascontiguousarray(v_pool)
    q = np.ascontiguousarray(q)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    num_pages, hkv, page_size, d = v_pool.shape
    batch, n, hq, dq = q.shape
    x = 16 // v_pool.dtype.itemsize
    if (n != q_per_seq or dq != d or k_pool.dtype != v_pool.dtype
            or k_pool.shape != (num_pages, hkv, d // x, page_size, x)):
        raise ValueError("shape mismatch")
    if bt.ndim != 2 or bt.shape[0] != batch or lens.shape != (batch,):
        raise ValueError("block_table / seq_lens must have one row per sequence")
    if seqs is None:
        seqs = np.arange(batch, dtype=np.int32)
    seqs = np.ascontiguousarray(seqs, dtype=np.int32)
    ks = vs = None
    if kv_dtype == "fp8":
        ks = np.ascontiguousarray(k_scale, dtype=np.float32)
        vs = np.ascontiguousarray(v_scale, dtype=np.float32)
    mask = None
    if tree_mask is not None:
        mask = np.ascontiguousarray(tree_mask, dtype=np.uint64)
        if mask.shape != (batch, n):
            raise ValueError("tree_mask must be [batch][q_per_seq]")
    out = np.empty((len(seqs), n, hq, d), dtype=np.float64)
    rc = _load().oracle_paged_attention_tree(
        _ptr(k_pool), _ptr(v_pool), _CODES[kv_dtype], _ptr(ks), _ptr(vs),
        num_pages, hkv, page_size, d, _ptr(q), _CODES[q_dtype], _ptr(bt), bt.shape[1],
        _ptr(lens), batch, n, hq, float(scale), _ptr(mask), _ptr(seqs), len(seqs), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_paged_attention rejected its arguments (code {rc})")
    return out


def e4m3_encode(x: float) -> int:
    """Nearest E4M3 byte (ties to the even code, saturating at 448)."""
    return int(_load().oracle_e4m3_encode(float(x)))


def append_kv(k_pool, v_pool, kv_dtype: str, k_new, v_new, src_dtype: str, block_table,
              seq_lens, n_new: int, k_scale=None, v_scale=None):
    """KV append / quantize-on-write (see oracle_append_kv in oracle.h).

    Works on copies: returns (k_pool, v_pool, k_scale, v_scale) after the
    append.  k_new / v_new: [batch][n_new][Hkv][D] float32 or bf16 bits.
    """
    kp = np.array(k_pool, copy=True, order="C")
    vp = np.array(v_pool, copy=True, order="C")
    ks = vs = None
    if kv_dtype == "fp8":
        ks = np.array(k_scale, dtype=np.float32, copy=True)
        vs = np.array(v_scale, dtype=np.float32, copy=True)
    kn = np.ascontiguousarray(k_new)
    vn = np.ascontiguousarray(v_new)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    num_pages, hkv, page_size, d = vp.shape
    batch = lens.shape[0]
    if kn.shape != (batch, n_new, hkv, d) or vn.shape != kn.shape or bt.shape[0] != batch:
        raise ValueError("shape mismatch")
    rc = _load().oracle_append_kv(_ptr(kp), _ptr(vp), _CODES[kv_dtype], _ptr(ks), _ptr(vs),
                                  num_pages, hkv, page_size, d, _ptr(kn), _ptr(vn),
                                  _CODES[src_dtype], _ptr(bt), bt.shape[1], _ptr(lens), batch,
                                  n_new)
    if rc != 0:
        raise ValueError(f"oracle_append_kv rejected its arguments (code {rc})")
    return kp, vp, ks, vs


def rejection_sample(p, q, draft, u_accept, u_sample):
    """Speculative-sampling acceptance (see oracle_rejection_sample in oracle.h).

    p [B][K+1][V], q [B][K][V] float32; draft [B][K] int32; u_accept [B][K],
    u_sample [B] float32 in [0, 1).  Returns (tokens [B][K+1] int32 with -1
    after the sampled token, accepted [B] int32).
    """
    p = np.ascontiguousarray(p, dtype=np.float32)
    batch, k1, vocab = p.shape
    k = k1 - 1
    q = np.ascontiguousarray(q, dtype=np.float32).reshape(batch, k, vocab)
    draft = np.ascontiguousarray(draft, dtype=np.int32).reshape(batch, k)
    ua = np.ascontiguousarray(u_accept, dtype=np.float32).reshape(batch, k)
    us = np.ascontiguousarray(u_sample, dtype=np.float32).reshape(batch)
    tokens = np.empty((batch, k + 1), dtype=np.int32)
    accepted = np.empty(batch, dtype=np.int32)
    rc = _load().oracle_rejection_sample(_ptr(p), _ptr(q), _ptr(draft), _ptr(ua), _ptr(us),
                                         batch, k, vocab, _ptr(tokens), _ptr(accepted))
    if rc != 0:
        raise ValueError(f"oracle_rejection_sample rejected its arguments (code {rc})")
    return tokens, accepted
