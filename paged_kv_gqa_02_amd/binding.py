"""ctypes binding of libpaged_attn.so (argument marshalling only).

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: it turns torch tensors into device pointers and sizes,
passes torch's current HIP stream, and raises on a non-zero status.  All work
on the device runs in the library's HIP kernels.  If the library has not been
built the import fails loudly; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
# PAGED_ATTN_LIB names another build of the same sources to load (the host
# sanitizer test's); by default the in-tree library
LIB_PATH = os.environ.get("PAGED_ATTN_LIB") or os.path.join(PKG, "libpaged_attn.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "paged_attn.h")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_CONTRACT = \
    0, -1, -2, -3, -4, -5
PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        super().__init__(f"{fn}: status {status} ({detail})")
        self.status = status


class pa_pool_desc(ctypes.Structure):
    _fields_ = [
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("partition_pages", ctypes.c_int32),
        ("waves", ctypes.c_int32),
        ("prefetch", ctypes.c_int32),
        ("staged_from", ctypes.c_int32),
    ]


class pa_plan(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in
                ("partition_pages", "num_splits", "row_tiles", "row_chunks", "waves", "grid",
                 "reduce", "kernel")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python paged_kv_gqa_02_amd/build.py` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    st = ctypes.c_int
    sig = {
        "paged_attn_pool_bytes": (st, [i32, i32, i32, i32, ctypes.c_int,
                                       ctypes.POINTER(sz), ctypes.POINTER(sz)]),
        "paged_attn_create_pool": (st, [ctypes.POINTER(pa_pool_desc), ctypes.POINTER(vp)]),
        "paged_attn_destroy_pool": (None, [vp]),
        "paged_attn_plan": (st, [vp, i32, i32, i32, i32, ctypes.POINTER(pa_plan)]),
        "paged_attn_workspace_bytes": (st, [vp, i32, i32, i32, i32, ctypes.POINTER(sz)]),
        "paged_attn_decode": (st, [vp, vp, ctypes.c_int, vp, vp, i32, vp, i32, i32, i32,
                                   ctypes.c_float, vp, sz, vp]),
        "paged_attn_verify": (st, [vp, vp, ctypes.c_int, vp, vp, i32, vp, i32, i32, i32, i32,
                                   ctypes.c_float, vp, sz, vp]),
        "paged_attn_verify_timed": (st, [vp, vp, ctypes.c_int, vp, vp, i32, vp, i32, i32, i32,
                                         i32, ctypes.c_float, vp, vp, sz, vp, vp, vp]),
        "paged_attn_verify_noalloc": (st, [vp, vp, ctypes.c_int, vp, vp, i32, vp, i32, i32, i32,
                                           i32, ctypes.c_float, vp]),
        "paged_attn_verify_tree": (st, [vp, vp, ctypes.c_int, vp, vp, i32, vp, i32, i32, i32,
                                        i32, ctypes.c_float, vp, vp, sz, vp]),
        "paged_attn_append_kv": (st, [vp, vp, vp, ctypes.c_int, vp, i32, vp, i32, i32, vp]),
        "paged_attn_validate": (st, [vp, vp, i32, vp, i32, i32, i32, vp]),
        "paged_attn_rejection_sample_workspace_bytes": (sz, [i32, i32]),
        "paged_attn_rejection_sample": (st, [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, sz,
                                             vp]),
        "paged_attn_status_str": (ctypes.c_char_p, [st]),
        "paged_attn_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def declared_symbols() -> list:
    """Entry points declared in include/paged_attn.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(paged_attn_\w+)\s*\(", text)))


def library():
    return _lib


def _check(status: int, fn: str):
    if status != PA_OK:
        detail = _lib.paged_attn_status_str(status).decode()
        last = _lib.paged_attn_last_error().decode()
        raise PagedAttnError(status, fn, f"{detail}: {last}" if last else detail)


def _dptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _kv_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PA_FP8_E4M3
    raise ValueError(f"unsupported kv dtype {t.dtype}")


def _q_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise ValueError(f"unsupported q dtype {t.dtype}")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Pool:
    """Handle of a page pool; keeps the pool tensors alive while it lives."""

    def __init__(self, handle, tensors, num_pages, num_kv_heads, kv_dtype):
        self.handle = handle
        self._tensors = tensors
        self.num_pages = num_pages
        self.num_kv_heads = num_kv_heads
        self.kv_dtype = kv_dtype

    def close(self):
        if self.handle:
            _lib.paged_attn_destroy_pool(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def paged_attn_pool_bytes(num_pages: int, num_kv_heads: int, kv_dtype: int,
                          page_size: int = 16, head_dim: int = 128):
    kb, vb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib.paged_attn_pool_bytes(num_pages, page_size, num_kv_heads, head_dim, kv_dtype,
                                      ctypes.byref(kb), ctypes.byref(vb)),
           "paged_attn_pool_bytes")
    return kb.value, vb.value


def paged_attn_create_pool(k: torch.Tensor, v: torch.Tensor, k_scale=None, v_scale=None,
                           partition_pages: int = 0, waves: int = 0, prefetch: int = 0,
                           staged_from: int = 0) -> Pool:
    """v: [num_pages][Hkv][16][128]; k: the same elements in the chunked K layout
    [num_pages][Hkv][128/x][16][x], x = 16 bytes / element size (device tensors of
    float32, bfloat16 or fp8 bytes)."""
    if v.dim() != 4 or k.dtype != v.dtype or k.numel() != v.numel() or k.shape[:2] != v.shape[:2]:
        raise ValueError("v must be [num_pages][Hkv][16][128] and k the same elements, chunked")
    if _kv_code(k) == PA_FP8_E4M3:
        for name, sc in (("k_scale", k_scale), ("v_scale", v_scale)):
            if sc is None or sc.dtype != torch.float32 or sc.numel() != v.shape[0] * v.shape[1]:
                raise ValueError(f"{name} must be float32 with num_pages * Hkv entries")
    desc = pa_pool_desc(num_pages=v.shape[0], page_size=v.shape[2], num_kv_heads=v.shape[1],
                        head_dim=v.shape[3], kv_dtype=_kv_code(k), k=_dptr(k), v=_dptr(v),
                        k_scale=_dptr(k_scale), v_scale=_dptr(v_scale),
                        partition_pages=partition_pages, waves=waves, prefetch=prefetch,
                        staged_from=staged_from)
    h = ctypes.c_void_p()
    _check(_lib.paged_attn_create_pool(ctypes.byref(desc), ctypes.byref(h)),
           "paged_attn_create_pool")
    return Pool(h, (k, v, k_scale, v_scale), v.shape[0], v.shape[1], _kv_code(k))


def paged_attn_destroy_pool(pool: Pool):
    pool.close()


def paged_attn_plan(pool: Pool, batch: int, q_per_seq: int, num_q_heads: int,
                    max_seq_len: int) -> dict:
    pl = pa_plan()
    _check(_lib.paged_attn_plan(pool.handle, batch, q_per_seq, num_q_heads, max_seq_len,
                                ctypes.byref(pl)), "paged_attn_plan")
    return {name: getattr(pl, name) for name, _ in pa_plan._fields_}


def paged_attn_workspace_bytes(pool: Pool, batch: int, q_per_seq: int, num_q_heads: int,
                               max_seq_len: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.paged_attn_workspace_bytes(pool.handle, batch, q_per_seq, num_q_heads,
                                           max_seq_len, ctypes.byref(n)),
           "paged_attn_workspace_bytes")
    return n.value


def workspace_for(pool: Pool, q: torch.Tensor, max_seq_len: int) -> Optional[torch.Tensor]:
    """A workspace tensor of the size the library asks for (None if it needs none)."""
    batch, n, hq, _ = q.shape
    nbytes = paged_attn_workspace_bytes(pool, batch, n, hq, max_seq_len)
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=q.device)


HEAD_DIM = 128


def _tables(batch, block_table, seq_lens):
    if block_table.dim() != 2 or block_table.shape[0] != batch or block_table.dtype != torch.int32:
        raise ValueError("block_table must be int32 [batch][max_pages]")
    if seq_lens.shape != (batch,) or seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32 [batch]")


def _shapes(pool, q, block_table, seq_lens):
    """Checks what the library reads through raw pointers and cannot check itself:
    the tensors' extents (head dim, query heads) and the table dtypes."""
    if q.dim() != 4 or q.shape[3] != HEAD_DIM:
        raise ValueError("q must be [batch][q_per_seq][Hq][128]")
    if q.shape[2] % pool.num_kv_heads != 0:
        raise ValueError("the query heads must be a multiple of the pool's KV heads")
    batch = q.shape[0]
    _tables(batch, block_table, seq_lens)
    return batch


def paged_attn_verify(pool: Pool, q: torch.Tensor, out: torch.Tensor, block_table: torch.Tensor,
                      seq_lens: torch.Tensor, max_seq_len: int, scale: float,
                      workspace: Optional[torch.Tensor] = None, stream=None,
                      ev_begin=None, ev_end=None, tree_mask: Optional[torch.Tensor] = None
                      ) -> torch.Tensor:
    """q, out: [batch][q_per_seq][Hq][128]; returns out.  With events (HipEvent)
    or a tree mask this goes through paged_attn_verify_timed."""
    batch = _shapes(pool, q, block_table, seq_lens)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if tree_mask is not None and (tree_mask.shape != (batch, q.shape[1])
                                  or tree_mask.element_size() != 8):
        raise ValueError("tree_mask must be 64-bit [batch][q_per_seq]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    head = (pool.handle, _dptr(q), _q_code(q), _dptr(out), _dptr(block_table),
            block_table.shape[1], _dptr(seq_lens), int(max_seq_len), batch, q.shape[1],
            q.shape[2], float(scale))
    if ev_begin is None and ev_end is None and tree_mask is None:
        _check(_lib.paged_attn_verify(*head, _dptr(workspace), ws_bytes, _stream(stream)),
               "paged_attn_verify")
    else:
        hb = ev_begin.handle if ev_begin is not None else None
        he = ev_end.handle if ev_end is not None else None
        _check(_lib.paged_attn_verify_timed(*head, _dptr(tree_mask), _dptr(workspace), ws_bytes,
                                            _stream(stream), hb, he),
               "paged_attn_verify_timed")
    return out


def paged_attn_verify_noalloc(pool: Pool, q: torch.Tensor, out: torch.Tensor,
                              block_table: torch.Tensor, seq_lens: torch.Tensor,
                              max_seq_len: int, scale: float, stream=None) -> torch.Tensor:
    """paged_attn_verify with the library's static split-K scratch (no workspace,
    nothing allocated); calls that overlap on one GPU race.  Returns out."""
    batch = _shapes(pool, q, block_table, seq_lens)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    _check(_lib.paged_attn_verify_noalloc(pool.handle, _dptr(q), _q_code(q), _dptr(out),
                                          _dptr(block_table), block_table.shape[1],
                                          _dptr(seq_lens), int(max_seq_len), batch, q.shape[1],
                                          q.shape[2], float(scale), _stream(stream)),
           "paged_attn_verify_noalloc")
    return out


def paged_attn_verify_tree(pool: Pool, q: torch.Tensor, out: torch.Tensor,
                           block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                           scale: float, tree_mask: torch.Tensor,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Draft-tree verification; tree_mask: [batch][q_per_seq] uint64 ancestor masks
    (a torch.int64 / torch.uint64 device tensor holding the bit patterns)."""
    batch = _shapes(pool, q, block_table, seq_lens)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if tree_mask.shape != (batch, q.shape[1]) or tree_mask.element_size() != 8:
        raise ValueError("tree_mask must be 64-bit [batch][q_per_seq]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.paged_attn_verify_tree(pool.handle, _dptr(q), _q_code(q), _dptr(out),
                                       _dptr(block_table), block_table.shape[1], _dptr(seq_lens),
                                       int(max_seq_len), batch, q.shape[1], q.shape[2],
                                       float(scale), _dptr(tree_mask), _dptr(workspace),
                                       ws_bytes, _stream(stream)),
           "paged_attn_verify_tree")
    return out


def paged_attn_verify_timed(pool, q, out, block_table, seq_lens, max_seq_len, scale,
                            ev_begin, ev_end, workspace=None, stream=None, tree_mask=None):
    return paged_attn_verify(pool, q, out, block_table, seq_lens, max_seq_len, scale,
                             workspace=workspace, stream=stream, ev_begin=ev_begin,
                             ev_end=ev_end, tree_mask=tree_mask)


def paged_attn_decode(pool: Pool, q: torch.Tensor, out: torch.Tensor, block_table: torch.Tensor,
                      seq_lens: torch.Tensor, max_seq_len: int, scale: float,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q, out: [batch][1][Hq][128] (or [batch][Hq][128]); returns out."""
    q4 = q if q.dim() == 4 else q.unsqueeze(1)
    o4 = out if out.dim() == 4 else out.unsqueeze(1)
    if q4.shape[1] != 1:
        raise ValueError("decode takes one query row per sequence")
    batch = _shapes(pool, q4, block_table, seq_lens)
    if o4.shape != q4.shape or o4.dtype != q4.dtype:
        raise ValueError("out must match q in shape and dtype")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.paged_attn_decode(pool.handle, _dptr(q4), _q_code(q4), _dptr(o4),
                                  _dptr(block_table), block_table.shape[1], _dptr(seq_lens),
                                  int(max_seq_len), batch, q4.shape[2], float(scale),
                                  _dptr(workspace), ws_bytes, _stream(stream)),
           "paged_attn_decode")
    return out


def paged_attn_append_kv(pool: Pool, k_new: torch.Tensor, v_new: torch.Tensor,
                         block_table: torch.Tensor, seq_lens: torch.Tensor, stream=None):
    """Write the n_new newest tokens ([batch][n_new][Hkv][128], float32 or bfloat16)
    of every sequence into the pool (fp8 pools: quantize-on-write)."""
    if (k_new.shape != v_new.shape or k_new.dim() != 4 or k_new.dtype != v_new.dtype
            or k_new.shape[2] != pool.num_kv_heads or k_new.shape[3] != HEAD_DIM):
        raise ValueError("k_new and v_new must both be [batch][n_new][Hkv][128], Hkv the pool's")
    batch, n_new = k_new.shape[0], k_new.shape[1]
    _tables(batch, block_table, seq_lens)
    _check(_lib.paged_attn_append_kv(pool.handle, _dptr(k_new), _dptr(v_new), _q_code(k_new),
                                     _dptr(block_table), block_table.shape[1], _dptr(seq_lens),
                                     batch, n_new, _stream(stream)),
           "paged_attn_append_kv")


def paged_attn_validate(pool: Pool, block_table: torch.Tensor, seq_lens: torch.Tensor,
                        max_seq_len: int, q_per_seq: int, stream=None):
    batch = seq_lens.shape[0]
    _check(_lib.paged_attn_validate(pool.handle, _dptr(block_table), block_table.shape[1],
                                    _dptr(seq_lens), int(max_seq_len), batch, q_per_seq,
                                    _stream(stream)), "paged_attn_validate")


def paged_attn_rejection_sample_workspace_bytes(batch: int, vocab: int) -> int:
    return int(_lib.paged_attn_rejection_sample_workspace_bytes(int(batch), int(vocab)))


def paged_attn_rejection_sample(p: torch.Tensor, q: Optional[torch.Tensor],
                                draft: Optional[torch.Tensor], u_accept: Optional[torch.Tensor],
                                u_sample: torch.Tensor, tokens: Optional[torch.Tensor] = None,
                                num_accepted: Optional[torch.Tensor] = None, workspace=None,
                                stream=None):
    """Speculative-sampling acceptance.  p [B][K+1][V], q [B][K][V] float32; draft
    [B][K] int32; u_accept [B][K], u_sample [B] float32.  Returns (tokens [B][K+1],
    num_accepted [B]) int32 device tensors (allocated here unless passed in)."""
    if p.dim() != 3 or p.dtype != torch.float32:
        raise ValueError("p must be float32 [batch][K+1][vocab]")
    batch, k1, vocab = p.shape
    k = k1 - 1
    if k > 0:
        if q is None or q.shape != (batch, k, vocab) or q.dtype != torch.float32:
            raise ValueError("q must be float32 [batch][K][vocab]")
        if draft is None or draft.shape != (batch, k) or draft.dtype != torch.int32:
            raise ValueError("draft must be int32 [batch][K]")
        if u_accept is None or u_accept.shape != (batch, k) or u_accept.dtype != torch.float32:
            raise ValueError("u_accept must be float32 [batch][K]")
    if u_sample.shape != (batch,) or u_sample.dtype != torch.float32:
        raise ValueError("u_sample must be float32 [batch]")
    if tokens is None:
        tokens = torch.empty((batch, k1), dtype=torch.int32, device=p.device)
    if num_accepted is None:
        num_accepted = torch.empty((batch,), dtype=torch.int32, device=p.device)
    if tokens.shape != (batch, k1) or tokens.dtype != torch.int32:
        raise ValueError("tokens must be int32 [batch][K+1]")
    if num_accepted.shape != (batch,) or num_accepted.dtype != torch.int32:
        raise ValueError("num_accepted must be int32 [batch]")
    ws_bytes = paged_attn_rejection_sample_workspace_bytes(batch, vocab)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=p.device)
    kk = k > 0
    _check(_lib.paged_attn_rejection_sample(
        _dptr(p), _dptr(q) if kk else None, _dptr(draft) if kk else None,
        _dptr(u_accept) if kk else None, _dptr(u_sample), batch, k, vocab, _dptr(tokens),
        _dptr(num_accepted), _dptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)), "paged_attn_rejection_sample")
    return tokens, num_accepted


# ---------------------------------------------------------------------------
# HIP events (plumbing for timing one kernel on the stream it runs on)
# ---------------------------------------------------------------------------
_hip = None


def _hip_rt():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                             ctypes.c_void_p]
    return _hip


class HipEvent:
    def __init__(self):
        self.handle = ctypes.c_void_p()
        rc = _hip_rt().hipEventCreate(ctypes.byref(self.handle))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")

    def record(self, stream=None):
        rc = _hip_rt().hipEventRecord(self.handle, _stream(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, end: "HipEvent") -> float:
        rt = _hip_rt()
        if rt.hipEventSynchronize(end.handle) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        ms = ctypes.c_float()
        rc = rt.hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        try:
            if self.handle:
                _hip_rt().hipEventDestroy(self.handle)
        except Exception:
            pass
