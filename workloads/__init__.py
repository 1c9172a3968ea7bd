"""Seeded synthetic inputs for paged GQA decode / verify attention.

This module builds the inputs that BOTH the CPU oracle and the GPU library
consume: page pools, block tables, sequence lengths and queries.  It holds
none of the attention arithmetic (no dot products, softmax or gathers); it
only draws random numbers, rounds them to the storage formats and lays them
out in the documented pool layout.

Layouts (shared contract, documented in ``include/paged_attn.h``):
  V pool          [num_pages][Hkv][page_size=16][D]   (token-major slabs)
  K pool          [num_pages][Hkv][D/x][16][x], x = 16 bytes / element size
                  (the head dimension cut into 16-byte chunks, each chunk
                  holding the 16 tokens in turn); ``k_to_pool`` /
                  ``k_from_pool`` convert from / to token-major slabs
  k_scale/v_scale [num_pages][Hkv] float32           (fp8 pools only)
  Q               [batch][q_per_seq][Hq][D]
  block_table     [batch][max_pages] int32, -1 past a sequence's last page
  seq_lens        [batch] int32

Random numbers: numpy's PCG64 ``Generator`` seeded per case; values are
N(0, 1) drawn as float32, then rounded to the storage format.  Draw order per
case: lengths (ragged only), page layout, K pool, V pool, Q.

Where the sources describe the allocation pattern: a request gets one 16-token
block when it starts and one more from anywhere in the pool each time the
previous one fills; all its blocks are freed when it ends ("Latency and cost
in production" §10.12.2; "Batching, speculative decoding, paged attention"
§5.3.7).  Unused slots and pages are poisoned with NaN so that any read of
them shows up in the result.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

PAGE_SIZE = 16
HEAD_DIM = 128
E4M3_MAX = 448.0
BASE_SEED = 20261202

BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)


# ----------------------------------------------------------------------------
# storage-format rounding (input preparation only)
# ----------------------------------------------------------------------------
def bf16_bits(x) -> np.ndarray:
    """Round to bfloat16 (round to nearest, ties to even); the 16-bit patterns as uint16.

    NaN becomes the canonical quiet NaN 0x7FC0.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    r = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    r = r.copy()
    nan = np.isnan(f)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def e4m3_bytes(x) -> np.ndarray:
    """Encode as OCP E4M3 bytes: round to nearest even, saturate at +-448, NaN -> 0x7F.

    E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
    holds subnormals m/8 * 2^-6; S.1111.111 is NaN; the largest finite
    magnitude is 448 (code 0x7E).
    """
    a = np.asarray(x)
    if a.dtype not in (np.float32, np.float64):
        a = a.astype(np.float64)
    a = np.ascontiguousarray(np.clip(a, -E4M3_MAX, E4M3_MAX))
    r = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    nan = np.isnan(a)
    if nan.any():
        r[nan] = E4M3_NAN
    return r


def k_to_pool(k_tokens: np.ndarray) -> np.ndarray:
    """Token-major K slabs [..., 16, D] -> the pool's chunked K layout [..., D/x, 16, x]."""
    x = 16 // k_tokens.dtype.itemsize
    sh = k_tokens.shape
    a = k_tokens.reshape(sh[:-1] + (sh[-1] // x, x))          # [..., 16, D/x, x]
    return np.ascontiguousarray(np.swapaxes(a, -3, -2))        # [..., D/x, 16, x]


def k_from_pool(k_pool: np.ndarray) -> np.ndarray:
    """The pool's chunked K layout [..., D/x, 16, x] -> token-major slabs [..., 16, D]."""
    a = np.swapaxes(k_pool, -3, -2)                             # [..., 16, D/x, x]
    return np.ascontiguousarray(a).reshape(a.shape[:-2] + (-1,))


def set_k_token(k_pool: np.ndarray, page: int, kv_head: int, slot: int, row) -> None:
    """Write one token's K row (already in the storage dtype) into the chunked pool."""
    c, _, x = k_pool.shape[-3:]
    k_pool[page, kv_head, :, slot, :] = np.asarray(row, dtype=k_pool.dtype).reshape(c, x)


def pages_for(length: int) -> int:
    """Number of 16-token pages a sequence of `length` tokens occupies."""
    return -(-int(length) // PAGE_SIZE)


# ----------------------------------------------------------------------------
# block tables
# ----------------------------------------------------------------------------
def shuffled_tables(rng: np.random.Generator, seq_lens, num_pages: int):
    """Hand out pages of one seeded permutation of the pool in order."""
    need = [pages_for(x) for x in seq_lens]
    if sum(need) > num_pages:
        raise ValueError("pool too small")
    perm = rng.permutation(num_pages).astype(np.int32)
    width = max(need)
    table = np.full((len(need), width), -1, dtype=np.int32)
    pos = 0
    for b, c in enumerate(need):
        table[b, :c] = perm[pos:pos + c]
        pos += c
    return table


def fragmented_tables(rng: np.random.Generator, seq_lens, slack: float = 1.25,
                      ghosts: Optional[int] = None):
    """Block tables after an interleaved allocate / free history.

    The pool holds ceil(slack * sum of pages needed) pages and its free list
    starts as a seeded permutation.  The survivors (one per sequence) and as
    many short-lived "ghost" requests grow round-robin, one page per active
    request per round, in a seeded order each round, taking the page at the
    head of the free list.  A ghost starts at a seeded round, and when it
    reaches its own seeded length it ends and pushes its pages back onto the
    head of the free list (last allocated on top).  Stops when every survivor
    holds its pages.  Returns (table, num_pages).
    """
    need = np.array([pages_for(x) for x in seq_lens], dtype=np.int64)
    nsurv = len(need)
    nghost = nsurv if ghosts is None else ghosts
    num_pages = int(math.ceil(slack * need.sum()))
    free = list(rng.permutation(num_pages).astype(np.int64)[::-1])  # head = end of list
    ghost_need = np.array([pages_for(x) for x in rng.choice(seq_lens, size=nghost)],
                          dtype=np.int64) if nghost else np.zeros(0, np.int64)
    ghost_start = rng.integers(0, max(1, int(need.max())), size=nghost)
    target = np.concatenate([need, ghost_need])
    held = [[] for _ in range(nsurv + nghost)]
    done = np.zeros(nsurv + nghost, dtype=bool)

    def finish(r):
        for p in held[r]:
            free.append(p)          # last allocated ends on top of the head
        held[r] = []
        done[r] = True

    rnd = 0
    while not all(len(held[b]) == need[b] for b in range(nsurv)):
        order = rng.permutation(nsurv + nghost)
        for r in order:
            if done[r] or len(held[r]) >= target[r]:
                continue
            if r >= nsurv and rnd < ghost_start[r - nsurv]:
                continue
            if not free:
                live = [g for g in range(nsurv, nsurv + nghost) if held[g] and not done[g]]
                if not live:
                    raise RuntimeError("pool exhausted")
                finish(max(live, key=lambda g: len(held[g])))
            held[r].append(free.pop())
            if r >= nsurv and len(held[r]) == target[r]:
                finish(r)
        rnd += 1
    width = int(need.max())
    table = np.full((nsurv, width), -1, dtype=np.int32)
    for b in range(nsurv):
        table[b, :need[b]] = held[b]
    return table, num_pages


# ----------------------------------------------------------------------------
# draft trees
# ----------------------------------------------------------------------------
def chain_tree(n: int) -> np.ndarray:
    """Ancestor masks of a chain of n drafts (the causal verify): row i sees rows 0..i."""
    return np.array([(1 << (i + 1)) - 1 for i in range(n)], dtype=np.uint64)


def random_tree(rng: np.random.Generator, n: int):
    """A seeded random draft tree in topological order.

    Node 0 is the root (the last accepted token); node i >= 1 hangs under a
    parent drawn uniformly from 0 .. i-1.  Returns (parents, masks) with
    masks[i] = the ancestors of node i and node i itself, as bits.
    """
    if not 1 <= n <= 64:
        raise ValueError("trees of 1..64 nodes")
    parents = np.full(n, -1, dtype=np.int64)
    masks = np.zeros(n, dtype=np.uint64)
    masks[0] = 1
    for i in range(1, n):
        p = int(rng.integers(0, i))
        parents[i] = p
        masks[i] = masks[p] | np.uint64(1 << i)
    return parents, masks


def ancestors(masks: np.ndarray, i: int):
    """Indices of the tree rows node i sees, in row order."""
    m = int(masks[i])
    return [j for j in range(64) if (m >> j) & 1]


# ----------------------------------------------------------------------------
# cases
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Case:
    """One seeded input set.  Arrays are numpy, in the documented layouts."""
    name: str
    kv_dtype: str           # "f32" | "bf16" | "fp8"
    q_dtype: str            # "f32" | "bf16"
    batch: int
    q_per_seq: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    seq_lens: np.ndarray    # [B] int32
    block_table: np.ndarray  # [B][max_pages] int32
    num_pages: int
    k_pool: np.ndarray      # chunked K layout; float32 | uint16 (bf16 bits) | uint8 (E4M3)
    v_pool: np.ndarray      # token-major V layout, same dtype
    q: np.ndarray           # float32 | uint16
    k_scale: Optional[np.ndarray] = None   # [num_pages][Hkv] float32 (fp8)
    v_scale: Optional[np.ndarray] = None
    seed: int = 0
    tree_mask: Optional[np.ndarray] = None  # [B][q_per_seq] uint64 draft-tree ancestor masks

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max())

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def kv_bytes(self, seqs=None) -> int:
        """Bytes of K and V for every token of every sequence (or of the
        sequences `seqs`), + fp8 scales."""
        lens = self.seq_lens if seqs is None else self.seq_lens[list(seqs)]
        esz = {"f32": 4, "bf16": 2, "fp8": 1}[self.kv_dtype]
        toks = int(lens.astype(np.int64).sum())
        b = 2 * toks * self.num_kv_heads * self.head_dim * esz
        if self.kv_dtype == "fp8":
            pages = sum(pages_for(x) for x in lens)
            b += 2 * pages * self.num_kv_heads * 4
        return b

    def q_bytes(self, seqs=None) -> int:
        esz = {"f32": 4, "bf16": 2}[self.q_dtype]
        nseq = self.batch if seqs is None else len(list(seqs))
        return nseq * self.q_per_seq * self.num_q_heads * self.head_dim * esz

    def algorithmic_bytes(self, seqs=None) -> int:
        """KV (+ scales) read once per (sequence, kv head), Q read once, O written
        once: for the whole batch, or for the sequences `seqs`."""
        return self.kv_bytes(seqs) + 2 * self.q_bytes(seqs)


def _valid_slots(block_table, seq_lens, num_pages):
    """Number of live slots of every physical page (max over sequences using it)."""
    valid = np.zeros(num_pages, dtype=np.int64)
    for b, length in enumerate(seq_lens):
        c = pages_for(length)
        ids = block_table[b, :c].astype(np.int64)
        cnt = np.full(c, PAGE_SIZE, dtype=np.int64)
        cnt[-1] = int(length) - PAGE_SIZE * (c - 1)
        np.maximum.at(valid, ids, cnt)
    return valid


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_case(name: str, *, batch: int, q_per_seq: int, num_q_heads: int,
              num_kv_heads: int, seq_lens, kv_dtype: str, q_dtype: str, seed: int,
              layout: str = "shuffled", num_pages: Optional[int] = None,
              poison: bool = True, head_dim: int = HEAD_DIM,
              scale: Optional[float] = None, block_table=None) -> Case:
    """Build one case.

    layout: "shuffled" (pages of one seeded permutation handed out in order),
    "fragmented" (the allocate/free history of ``fragmented_tables``), or
    "given" (use ``block_table`` as passed).
    """
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    if seq_lens.shape != (batch,):
        raise ValueError("seq_lens must have one entry per sequence")
    if layout == "shuffled":
        need = sum(pages_for(x) for x in seq_lens)
        num_pages = need if num_pages is None else num_pages
        table = shuffled_tables(rng, seq_lens, num_pages)
    elif layout == "fragmented":
        table, num_pages = fragmented_tables(rng, seq_lens)
    elif layout == "given":
        table = np.ascontiguousarray(block_table, dtype=np.int32)
        if num_pages is None:
            raise ValueError("num_pages required with a given table")
    else:
        raise ValueError(layout)

    shape = (num_pages, num_kv_heads, PAGE_SIZE, head_dim)
    k = _normal(rng, shape)
    v = _normal(rng, shape)
    q = _normal(rng, (batch, q_per_seq, num_q_heads, head_dim))

    valid = _valid_slots(table, seq_lens, num_pages)
    dead = np.arange(PAGE_SIZE)[None, :] >= valid[:, None]          # [pages][slot]
    dead4 = np.broadcast_to(dead[:, None, :, None], shape)

    k_scale = v_scale = None
    if kv_dtype == "fp8":
        def quant(x):
            live = np.abs(x)
            live[dead4] = 0.0
            amax = live.max(axis=(2, 3))                             # [pages][Hkv]
            del live
            sc = np.where(amax > 0, amax / np.float32(E4M3_MAX),
                          np.float32(1.0)).astype(np.float32)
            x = x / np.where(valid[:, None] == 0, np.float32(1.0), sc)[:, :, None, None]
            if poison:
                sc[valid == 0] = np.nan
            byt = e4m3_bytes(x)
            if poison:
                byt[dead4] = E4M3_NAN
            return byt, sc
        k_pool, k_scale = quant(k)
        v_pool, v_scale = quant(v)
    elif kv_dtype == "bf16":
        if poison:
            k[dead4] = np.nan
            v[dead4] = np.nan
        k_pool, v_pool = bf16_bits(k), bf16_bits(v)
    elif kv_dtype == "f32":
        if poison:
            k[dead4] = np.nan
            v[dead4] = np.nan
        k_pool, v_pool = k, v
    else:
        raise ValueError(kv_dtype)

    k_pool = k_to_pool(k_pool)

    if q_dtype == "bf16":
        qa = bf16_bits(q)
    elif q_dtype == "f32":
        qa = q
    else:
        raise ValueError(q_dtype)

    return Case(name=name, kv_dtype=kv_dtype, q_dtype=q_dtype, batch=batch,
                q_per_seq=q_per_seq, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                head_dim=head_dim,
                scale=(1.0 / math.sqrt(head_dim)) if scale is None else float(scale),
                seq_lens=seq_lens, block_table=table, num_pages=num_pages,
                k_pool=k_pool, v_pool=v_pool, q=qa, k_scale=k_scale, v_scale=v_scale,
                seed=seed)


# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------
def ragged_lengths(rng: np.random.Generator, batch: int = 240) -> np.ndarray:
    """Prompt length U{128..1024} plus a generated length of 50 or 400 (p = 1/2 each)."""
    prompt = rng.integers(128, 1025, size=batch)
    gen = np.where(rng.random(batch) < 0.5, 50, 400)
    return (prompt + gen).astype(np.int32)


WORKLOADS = ("tiny", "decode8b", "ragged", "verify", "fp8long", "tree", "prefill", "verify_decode")


def workload(name: str, kv_dtype: Optional[str] = None, q_dtype: Optional[str] = None,
             seed: Optional[int] = None, poison: bool = True) -> Case:
    """The named workloads; dtype overrides give same-shape structural runs.

    tiny      B1, 8/2 heads, ctx 64, 16-page pool (4 pages used), fp32
    decode8b  B64, 32/8 heads, ctx 2048, 8192-page pool, bf16
    ragged    B240, 32/8 heads, ctx = U{128..1024} + {50|400}, fragmented pool, bf16
    verify    B8, 5 query rows (K = 4 drafts), 32/8 heads, ctx 4096 + 5, bf16
    fp8long   B4, 64/8 heads, ctx 32768, E4M3 K/V with per-(page, head) scales, bf16 Q
    tree      B8, 32/8 heads, a seeded random 16-node draft tree per sequence after a
              4096-token context (draft-tree verification), bf16
    prefill   B4, 32/8 heads, one 512-token prefill chunk per sequence after 1536, 1024,
              512 and 0 earlier tokens (a 2048-token prompt in four chunks), bf16
    verify_decode  verify's shape and seed with one query row per sequence (decode at
              the same context: the verify / decode time comparison)
    """
    idx = WORKLOADS.index(name)
    s = BASE_SEED + idx if seed is None else seed
    if name == "tiny":
        kv, qd = kv_dtype or "f32", q_dtype or "f32"
        return make_case(name, batch=1, q_per_seq=1, num_q_heads=8, num_kv_heads=2,
                         seq_lens=[64], kv_dtype=kv, q_dtype=qd, seed=s, num_pages=16,
                         poison=poison)
    if name == "decode8b":
        kv, qd = kv_dtype or "bf16", q_dtype or "bf16"
        return make_case(name, batch=64, q_per_seq=1, num_q_heads=32, num_kv_heads=8,
                         seq_lens=[2048] * 64, kv_dtype=kv, q_dtype=qd, seed=s,
                         poison=poison)
    if name == "ragged":
        kv, qd = kv_dtype or "bf16", q_dtype or "bf16"
        rng = np.random.default_rng(s)
        lens = ragged_lengths(rng)
        return make_case(name, batch=240, q_per_seq=1, num_q_heads=32, num_kv_heads=8,
                         seq_lens=lens, kv_dtype=kv, q_dtype=qd,
                         seed=int(rng.integers(0, 2**31)), layout="fragmented",
                         poison=poison)
    if name == "verify":
        kv, qd = kv_dtype or "bf16", q_dtype or "bf16"
        return make_case(name, batch=8, q_per_seq=5, num_q_heads=32, num_kv_heads=8,
                         seq_lens=[4096 + 5] * 8, kv_dtype=kv, q_dtype=qd, seed=s,
                         poison=poison)
    if name == "verify_decode":
        # the verify workload's pool and lengths with one query row per sequence:
        # decode at the same context, for the verify / decode time ratio
        kv, qd = kv_dtype or "bf16", q_dtype or "bf16"
        s = BASE_SEED + WORKLOADS.index("verify") if seed is None else seed
        return make_case(name, batch=8, q_per_seq=1, num_q_heads=32, num_kv_heads=8,
                         seq_lens=[4096 + 5] * 8, kv_dtype=kv, q_dtype=qd, seed=s,
                         poison=poison)
    if name == "fp8long":
        kv = kv_dtype or "fp8"
        qd = q_dtype or ("bf16" if kv != "f32" else "f32")
        return make_case(name, batch=4, q_per_seq=1, num_q_heads=64, num_kv_heads=8,
                         seq_lens=[32768] * 4, kv_dtype=kv, q_dtype=qd, seed=s,
                         poison=poison)
    if name == "tree":
        kv, qd = kv_dtype or "bf16", q_dtype or "bf16"
        n = 16
        case = make_case(name, batch=8, q_per_seq=n, num_q_heads=32, num_kv_heads=8,
                         seq_lens=[4096 + n] * 8, kv_dtype=kv, q_dtype=qd, seed=s,
                         poison=poison)
        rng = np.random.default_rng(s + 1)
        case.tree_mask = np.stack([random_tree(rng, n)[1] for _ in range(case.batch)])
        return case
    if name == "prefill":
        kv, qd = kv_dtype or "bf16", q_dtype or "bf16"
        n = 512
        return make_case(name, batch=4, q_per_seq=n, num_q_heads=32, num_kv_heads=8,
                         seq_lens=[1536 + n, 1024 + n, 512 + n, n], kv_dtype=kv, q_dtype=qd,
                         seed=s, poison=poison)
    raise ValueError(name)


# ----------------------------------------------------------------------------
# KV append inputs
# ----------------------------------------------------------------------------
def append_inputs(case: Case, n_new: int, src_dtype: str, seed: int, spread: float = 1.0):
    """Source K/V for the n_new newest tokens of every sequence of `case`:
    [batch][n_new][Hkv][D], N(0, spread^2) as float32 or bf16 bits."""
    rng = np.random.default_rng(seed)
    shape = (case.batch, n_new, case.num_kv_heads, case.head_dim)
    k = (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(spread))
    v = (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(spread))
    if src_dtype == "bf16":
        return bf16_bits(k), bf16_bits(v)
    return k, v


# ----------------------------------------------------------------------------
# speculative-sampling acceptance inputs
# ----------------------------------------------------------------------------
VOCAB_8B = 128256        # vocabulary of an 8B-class GQA model (the pages fix none)


@dataclasses.dataclass
class SamplerCase:
    """Inputs of one acceptance call: p [B][K+1][V], q [B][K][V] float32 rows,
    draft [B][K] int32 drawn from q, uniforms u_accept [B][K], u_sample [B]."""
    p: np.ndarray
    q: np.ndarray
    draft: np.ndarray
    u_accept: np.ndarray
    u_sample: np.ndarray

    @property
    def batch(self) -> int:
        return self.p.shape[0]

    @property
    def num_drafts(self) -> int:
        return self.p.shape[1] - 1

    @property
    def vocab(self) -> int:
        return self.p.shape[2]


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def _draw_rows(rows: np.ndarray, u: np.ndarray) -> np.ndarray:
    """One index per row of probabilities (the draft model's own sampling)."""
    cdf = np.cumsum(rows.astype(np.float64), axis=-1)
    idx = (cdf < (u * cdf[..., -1])[..., None]).sum(axis=-1)
    return np.minimum(idx, rows.shape[-1] - 1).astype(np.int32)


def sampler_inputs(batch: int, num_drafts: int, vocab: int, seed: int,
                   temperature_logit_sd: float = 3.0, draft_noise_sd: float = 0.5,
                   greedy: bool = False) -> SamplerCase:
    """Target logits N(0, sd^2) per row; the draft's logits are the target's
    plus N(0, noise^2) (a close but imperfect draft: at the defaults a draft
    passes about 80 % of the time); p, q = softmax; draft
    token i is drawn from q row i; uniforms in [0, 1) as float32.  greedy:
    one-hot rows at the logits' argmax instead (temperature 0)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((batch, num_drafts + 1, vocab), dtype=np.float32) * \
        np.float32(temperature_logit_sd)
    zq = z[:, :num_drafts] + rng.standard_normal((batch, num_drafts, vocab),
                                                 dtype=np.float32) * np.float32(draft_noise_sd)
    if greedy:
        p = np.zeros_like(z)
        np.put_along_axis(p, z.argmax(axis=-1)[..., None], 1.0, axis=-1)
        q = np.zeros_like(zq)
        np.put_along_axis(q, zq.argmax(axis=-1)[..., None], 1.0, axis=-1)
    else:
        p = _softmax_rows(z.astype(np.float64))
        q = _softmax_rows(zq.astype(np.float64))
    del z, zq
    draft = _draw_rows(q, rng.random((batch, num_drafts)))
    return SamplerCase(p=p, q=q.astype(np.float32), draft=draft,
                       u_accept=rng.random((batch, num_drafts), dtype=np.float32),
                       u_sample=rng.random(batch, dtype=np.float32))
