"""Benchmark of the paged GQA decode / verify attention hot path on one MI355X.

Default: the 8B-GQA decode layer (batch 64, one query row, 32 query heads / 8
KV heads, head_dim 128, context 2048, page size 16, bf16 K/V/Q, block tables
from a seeded shuffled free list).  One step = one paged_attn_verify call
(partition kernel, plus the split-K reduce when the plan splits) over the
whole batch; inputs are resident in HBM and a 1 GiB buffer is read before
every step so that no K/V byte is served from L2 or the MALL.  The flush
reads rather than writes: a written buffer leaves dirty lines in the MALL
whose write-back would then compete with the timed kernel for HBM.

Prints ONE JSON line (rank 0).  `value` is effective HBM GB/s: (K + V bytes of
every token of every sequence, fp8 scales, Q, O) / mean call time, the call
bracketed by two HIP events on its stream.  `roofline.achieved` divides the
same bytes by the attention kernel's own execution time, from events the
library attaches to that kernel's dispatch (paged_attn_verify_timed).
`copy_gbs` is the box's own device-copy bandwidth (bytes read + written by a
512 MiB copy, timed the same way), and `pct_of_copy` / `roofline.frac_of_copy`
the call's and the kernel's rates against it: a second denominator next to
the 8 TB/s data-sheet peak.

`--op append` instead times paged_attn_append_kv, the step before attention:
the n_new newest tokens of every sequence of the workload (default: its query
rows; `--n-new 256` is a prefill chunk) are written into the pool, quantised
on write for fp8.  Its bytes are the source K/V read, the pool bytes written
and, for fp8, every touched page scale read and written.

`--op sample` times paged_attn_rejection_sample, the step after the verify
pass: speculative-sampling acceptance for `--batch` sequences (default 64)
with `--drafts` drafts (4) over a `--vocab` (128,256) vocabulary.  Its bytes
are the probabilities the method must read given the outcome (the drafted
tokens' p and q up to the first rejection, then the residual's p and q rows,
or the bonus p row), the draft tokens and uniforms, and the outputs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

import workloads as W

METRIC = "decode attention effective HBM GB/s (% of peak) + tokens/s, B=64 ctx=2048"
PEAK_HBM_GBS = 8000.0
FLUSH_BYTES = 1 << 30
HOST_THREADS_PER_GPU = 16


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode8b", choices=W.WORKLOADS)
    ap.add_argument("--kv-dtype", default=None, choices=("bf16", "fp8", "f32"),
                    help="K/V pool dtype in place of the workload's own (same shape)")
    ap.add_argument("--partition-pages", type=int, default=0)
    ap.add_argument("--waves", type=int, default=0, help="pool knob: waves per workgroup")
    ap.add_argument("--prefetch", type=int, default=0, help="pool knob: pages in flight per wave")
    ap.add_argument("--staged-from", type=int, default=0,
                    help="pool knob: rows per sequence from which causal calls take the "
                         "LDS-staged kernel (0 = library default, -1 = never)")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=5)
    ap.add_argument("--op", default="attention", choices=("attention", "append", "sample"))
    ap.add_argument("--batch", type=int, default=64, help="sample: sequences")
    ap.add_argument("--drafts", type=int, default=4, help="sample: drafts per sequence")
    ap.add_argument("--vocab", type=int, default=W.VOCAB_8B, help="sample: vocabulary size")
    ap.add_argument("--n-new", type=int, default=0, help="append: tokens per sequence")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a torch copy of 512 MiB ten times (scale for HBM counters)")
    return ap.parse_args()


PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "fp8": 2500.0, "f32": 157.3}   # dense; fp8 KV runs bf16 MFMA
MFMA_RIDGE = 2500.0e12 / 8000.0e9                                  # FLOP per HBM byte, bf16


def attention_flops(case):
    """4 * head_dim multiply-adds-as-two-flops per (query head, visible key):
    q.k and p * v.  Row i of a sequence sees L - n + i + 1 keys (draft trees:
    the context plus the row's ancestors)."""
    n = case.q_per_seq
    keys = 0
    for b, L in enumerate(case.seq_lens.astype(np.int64)):
        if case.tree_mask is not None:
            anc = sum(bin(int(m)).count("1") for m in case.tree_mask[b])
            keys += n * (L - n) + anc
        else:
            keys += n * (L - n) + n * (n + 1) // 2
    return 4 * case.head_dim * case.num_q_heads * int(keys)


def code_digest(path):
    """sha256 of a C / HIP source with its comments and whitespace removed: it
    changes when the code does, not when a comment does."""
    import hashlib
    import re
    text = open(path, encoding="utf-8").read()
    # string and character literals are kept; comments are dropped
    token = re.compile(r'"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|//[^\n]*|/\*.*?\*/', re.S)
    code = token.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", text)
    return hashlib.sha256(" ".join(code.split()).encode()).hexdigest()


def measured_traffic(key):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter runs (profiles/traffic.json), if they were taken on the kernel
    code as it is now (else None)."""
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        rec = json.load(open(os.path.join(root, "profiles", "traffic.json"))).get(key)
        if not rec:
            return None
        digest = code_digest(os.path.join(root, rec["source"]))
    except (OSError, ValueError, KeyError):
        return None
    if rec.get("code_sha256") != digest:
        return None
    return int(round(rec["traffic_bytes"]))


def add_speedup(result):
    """The GPU rate over the oracle's (same unit, same byte or FLOP formula) as
    cpu_baseline.gpu_speedup: a stated ratio, not a measure of kernel quality."""
    cpu = result.get("cpu_baseline")
    if cpu and cpu.get("unit") == result["unit"] and cpu["value"] > 0:
        cpu["gpu_speedup"] = round(result["value"] / cpu["value"], 1)


def cpu_baseline(case, reps):
    """The float64 oracle, as it is, over the whole batch on every host core."""
    import concurrent.futures as cf
    import oracle

    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    # the host share that goes with one GPU on the MI355X boxes is 16 threads,
    # whatever os.cpu_count() reports; a larger pool is not allowed there
    cores = max(1, min(affinity, HOST_THREADS_PER_GPU))

    def one(b):
        oracle.paged_attention(case.k_pool, case.v_pool, case.kv_dtype, case.q, case.q_dtype,
                               case.block_table, case.seq_lens, case.q_per_seq, case.scale,
                               seqs=[b], k_scale=case.k_scale, v_scale=case.v_scale,
                               tree_mask=case.tree_mask)

    times = []
    with cf.ThreadPoolExecutor(max_workers=cores) as ex:
        for r in range(reps):
            t0 = time.perf_counter()
            list(ex.map(one, range(case.batch)))
            times.append(time.perf_counter() - t0)
            log(f"cpu baseline rep {r}: {times[-1]:.2f} s")
    t = float(np.median(times))
    used = min(cores, case.batch)             # one sequence per thread
    # the same oracle on one thread, over the first sequences that fit a few seconds
    t1 = time.perf_counter()
    one(0)
    t1 = time.perf_counter() - t1
    k = int(max(1, min(case.batch, 4.0 / max(t1, 1e-6))))
    if k > 1:
        t1 = time.perf_counter()
        for b in range(k):
            one(b)
        t1 = time.perf_counter() - t1
    log(f"cpu baseline, one thread: {k} sequences in {t1:.2f} s")
    return {"value": case.algorithmic_bytes() / t / 1e9, "unit": "GB/s", "cores": used,
            "kind": "oracle",
            "sample": f"whole batch ({case.batch} sequences, every head and row) x {reps} reps, "
                      f"median {t:.3f} s, float64 C oracle, one sequence per thread",
            "tokens_per_s": case.batch * case.q_per_seq / t,
            "cpu_model": cpu_model(),
            "host_cpus": {"os_cpu_count": os.cpu_count(), "affinity": affinity,
                          "threads_allowed": HOST_THREADS_PER_GPU},
            "single_thread": {"value": case.algorithmic_bytes(seqs=range(k)) / t1 / 1e9,
                              "unit": "GB/s", "cores": 1,
                              "sample": f"sequences 0..{k - 1} of {case.batch}, once, {t1:.2f} s"}}


def cpu_model():
    """The host CPU as /proc/cpuinfo names it: model name, family, model and
    stepping (a virtual machine may report only the vendor's family name), or
    None."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            key, _, val = line.partition(":")
            key = key.strip()
            if key in ("model name", "cpu family", "model", "stepping") and key not in fields:
                fields[key] = val.strip()
            if not line.strip() and fields:
                break
    except OSError:
        return None
    if not fields:
        return None
    ident = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields)
    return f"{fields.get('model name', '?')} ({ident})" if ident else fields.get("model name")


def append_bytes(case, n_new, src_dtype, seq_lens=None):
    """Source K/V read + pool bytes written (+ fp8 scales of touched pages, read and
    written) for the sequences with lengths `seq_lens` (default: the whole batch)."""
    lens = (case.seq_lens if seq_lens is None else seq_lens).astype(np.int64)
    esz = {"f32": 4, "bf16": 2, "fp8": 1}
    elems = len(lens) * n_new * case.num_kv_heads * case.head_dim
    nbytes = 2 * elems * (esz[src_dtype] + esz[case.kv_dtype])
    if case.kv_dtype == "fp8":
        pages = (lens - 1) // W.PAGE_SIZE - (lens - n_new) // W.PAGE_SIZE + 1
        nbytes += 2 * 2 * 4 * int(pages.sum()) * case.num_kv_heads
    return nbytes


def cpu_append_baseline(case, kn, vn, src, n_new, budget_s=10.0):
    """The oracle's append over a bounded prefix of the batch, one thread."""
    import oracle

    def run(k):
        t0 = time.perf_counter()
        oracle.append_kv(case.k_pool, case.v_pool, case.kv_dtype, kn[:k], vn[:k], src,
                         case.block_table[:k], case.seq_lens[:k], n_new, case.k_scale,
                         case.v_scale)
        return time.perf_counter() - t0

    t1 = run(1)
    k = int(max(1, min(case.batch, budget_s / max(t1, 1e-6))))
    t = run(k) if k > 1 else t1
    log(f"cpu append baseline: {k} sequences in {t:.2f} s")
    return {"value": append_bytes(case, n_new, src, case.seq_lens[:k]) / t / 1e9, "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{k} of {case.batch} sequences, n_new={n_new}, one call of the C oracle "
                      f"(which also copies the pool), {t:.2f} s",
            "tokens_per_s": k * n_new / t}


def bench_append(args, torch, pa, case, dev, pool, flush_caches, stream):
    from workloads.device import tensor

    n_new = args.n_new or case.q_per_seq
    if n_new > int(case.seq_lens.min()):
        sys.exit(f"bench.py: n_new={n_new} exceeds the shortest sequence of {case.name}")
    src = "f32" if case.kv_dtype == "f32" else "bf16"
    kn, vn = W.append_inputs(case, n_new, src, 20261202)
    dk, dv = tensor(kn, "cuda"), tensor(vn, "cuda")

    def call():
        pa.paged_attn_append_kv(pool, dk, dv, dev.block_table, dev.seq_lens)

    for _ in range(args.warmup):
        flush_caches()
        call()
    torch.cuda.synchronize()
    # The flush kernel in front of every call keeps the queue busy while the
    # host enqueues the begin event and the launch, so the events bracket the
    # append kernel and its dispatch.
    evs = [(pa.HipEvent(), pa.HipEvent()) for _ in range(args.steps)]
    for e0, e1 in evs:
        flush_caches()
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = np.array([e0.elapsed_ms(e1) for e0, e1 in evs])
    nbytes = append_bytes(case, n_new, src)
    sec = float(ms.mean()) / 1e3
    gbs = nbytes / sec / 1e9
    log(f"append: {ms.mean() * 1e3:.2f} us per call, {gbs:.1f} GB/s")
    result = {
        "metric": "KV append (quantize-on-write) effective HBM GB/s",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(float(ms.mean()), 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8-e4m3 kv / bf16 source", "f32": "f32"}[case.kv_dtype],
        "data": "synthetic (seeded N(0,1) sources, shuffled page pool)",
        "config": {"workload": f"append into {case.name}", "batch": case.batch, "n_new": n_new,
                   "num_kv_heads": case.num_kv_heads, "head_dim": case.head_dim,
                   "kv_dtype": case.kv_dtype, "src_dtype": src, "bytes_per_call": nbytes},
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(case.batch * n_new / sec, 1),
        "call_us": {"mean": round(float(ms.mean()) * 1e3, 2),
                    "p10": round(float(np.percentile(ms, 10)) * 1e3, 2),
                    "p50": round(float(np.percentile(ms, 50)) * 1e3, 2),
                    "p90": round(float(np.percentile(ms, 90)) * 1e3, 2)},
        "roofline": {"bound": "hbm", "kernel": "paged_attn_append", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(f"append:{case.name}:{n_new}"), "kernel_us_mean": round(sec * 1e6, 2),
                     "algorithmic_bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_append_baseline(case, kn, vn, src, n_new)
    add_speedup(result)
    print(json.dumps(result), flush=True)


def sample_bytes(case, accepted):
    """Bytes the acceptance must touch given the outcome (see the module doc)."""
    k, v = case.num_drafts, case.vocab
    acc = accepted.astype(np.int64)
    tests = np.minimum(acc + 1, k)                     # acceptance tests actually run
    rows = np.where(acc < k, 2 * v * 4, v * 4)         # residual p and q rows, or the bonus row
    return int((tests * 16 + rows + 4 + (k + 1) * 4 + 4).sum())


def bench_sample(args, torch, pa, flush_caches, stream):
    log(f"generating sampler inputs B={args.batch} K={args.drafts} V={args.vocab}")
    case = W.sampler_inputs(args.batch, args.drafts, args.vocab, 20261202)
    k = case.num_drafts
    dp = torch.from_numpy(case.p).cuda()
    dq = torch.from_numpy(case.q).cuda() if k else None
    dd = torch.from_numpy(case.draft).cuda() if k else None
    dua = torch.from_numpy(case.u_accept).cuda() if k else None
    dus = torch.from_numpy(case.u_sample).cuda()
    tokens = torch.empty((case.batch, k + 1), dtype=torch.int32, device="cuda")
    acc = torch.empty(case.batch, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, pa.paged_attn_rejection_sample_workspace_bytes(case.batch, case.vocab)),
                     dtype=torch.uint8, device="cuda")

    def call():
        pa.paged_attn_rejection_sample(dp, dq, dd, dua, dus, tokens, acc, ws)

    for _ in range(args.warmup):
        flush_caches()
        call()
    torch.cuda.synchronize()
    evs = [(pa.HipEvent(), pa.HipEvent()) for _ in range(args.steps)]
    for e0, e1 in evs:
        flush_caches()
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = np.array([e0.elapsed_ms(e1) for e0, e1 in evs])
    accepted = acc.cpu().numpy()
    nbytes = sample_bytes(case, accepted)
    sec = float(ms.mean()) / 1e3
    gbs = nbytes / sec / 1e9
    log(f"sample: {ms.mean() * 1e3:.2f} us per call, {gbs:.1f} GB/s, "
        f"mean accepted {accepted.mean():.2f}")
    result = {
        "metric": "speculative-sampling acceptance effective HBM GB/s",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(float(ms.mean()), 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 probabilities, f64 sums",
        "data": "synthetic (seeded N(0, 3^2) target logits, draft = target + N(0, 0.5^2))",
        "config": {"workload": f"acceptance B={case.batch} K={k} V={case.vocab}",
                   "batch": case.batch, "num_drafts": k, "vocab": case.vocab,
                   "mean_accepted": round(float(accepted.mean()), 4), "bytes_per_call": nbytes},
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(float((accepted + 1).sum()) / sec, 1),
        "call_us": {"mean": round(float(ms.mean()) * 1e3, 2),
                    "p10": round(float(np.percentile(ms, 10)) * 1e3, 2),
                    "p50": round(float(np.percentile(ms, 50)) * 1e3, 2),
                    "p90": round(float(np.percentile(ms, 90)) * 1e3, 2)},
        "roofline": {"bound": "hbm", "kernel": "spec_sample_chunks + spec_sample_pick",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": (measured_traffic(f"sample:{case.batch}")
                                 if (k, case.vocab) == (4, W.VOCAB_8B) else None),
                     "traffic_kernel": "spec_sample_chunks",
                     "kernel_us_mean": round(sec * 1e6, 2), "algorithmic_bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        import oracle
        times = []
        for _ in range(max(3, args.cpu_reps)):
            t0 = time.perf_counter()
            oracle.rejection_sample(case.p, case.q, case.draft, case.u_accept, case.u_sample)
            times.append(time.perf_counter() - t0)
        t = float(np.median(times))
        result["cpu_baseline"] = {
            "value": nbytes / t / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"whole batch, {len(times)} reps, median {t * 1e3:.2f} ms, one thread",
            "tokens_per_s": float((accepted + 1).sum()) / t}
    add_speedup(result)
    print(json.dumps(result), flush=True)


def copy_calibration(torch):
    """A plain device copy of known size: reads and writes 512 MiB per launch."""
    n = 512 << 20
    x = torch.ones(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    for _ in range(10):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": 10}), flush=True)


def measure_copy_gbs(torch, stream):
    """The box's device-copy bandwidth, (bytes read + bytes written) / time, over
    ten 512 MiB copies on `stream` bracketed by HIP events: a secondary
    denominator for the HBM-bound lines, next to the 8 TB/s data-sheet peak."""
    n = 512 << 20
    x = torch.ones(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    with torch.cuda.stream(stream):
        for _ in range(3):
            y.copy_(x)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            y.copy_(x)
        e1.record(stream)
    torch.cuda.synchronize()
    gbs = 2 * n * 10 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    return gbs


def measure_read_gbs(torch, stream, flush_caches):
    """The box's read-stream bandwidth in the same run: the bench's own 1 GiB
    cache-flush read (torch's float64 sum over it), timed with HIP events on
    `stream`, best of ten.  A read-only denominator next to the copy rate (a
    copy mixes reads and writes and runs slower); a reduction kernel of
    torch's, so a lower bound of what a plain read stream reaches."""
    best = None
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        flush_caches()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    return FLUSH_BYTES / (best / 1e3) / 1e9


def measure_read_us(torch, stream, flush_caches, nbytes):
    """Time of one plain read of `nbytes` from HBM (torch's float64 sum over a
    buffer of that size, the caches flushed first), median of ten, with HIP
    events on `stream`."""
    buf = torch.ones(max(nbytes // 8, 1), dtype=torch.float64, device="cuda")
    times = []
    for _ in range(10):
        flush_caches()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        buf.sum()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    del buf
    torch.cuda.empty_cache()
    return float(np.median(times))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this benchmark runs on one GPU only (there is no multi-GPU path); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import paged_kv_gqa_02_amd as pa
    from workloads.device import to_device

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)
        return

    flush = None
    if not args.no_flush:
        flush = torch.ones(FLUSH_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def flush_caches():
        # a read of the whole 1 GiB buffer (as float64: a quarter of the elements
        # of its bf16 view, so the reduction keeps up with HBM)
        if flush is not None:
            flush.view(torch.float64).sum()

    if args.op == "sample":
        bench_sample(args, torch, pa, flush_caches, stream)
        return

    log(f"generating {args.workload}")
    case = W.workload(args.workload, kv_dtype=args.kv_dtype)
    dev = to_device(case)
    pool = pa.paged_attn_create_pool(dev.k, dev.v, dev.k_scale, dev.v_scale,
                                     args.partition_pages, args.waves, args.prefetch,
                                     staged_from=args.staged_from)
    plan = pa.paged_attn_plan(pool, case.batch, case.q_per_seq, case.num_q_heads,
                              case.max_seq_len)
    out = torch.empty_like(dev.q)
    ws = pa.workspace_for(pool, dev.q, case.max_seq_len)

    def call(ev_begin=None, ev_end=None):
        pa.paged_attn_verify(pool, dev.q, out, dev.block_table, dev.seq_lens, case.max_seq_len,
                             case.scale, ws, ev_begin=ev_begin, ev_end=ev_end,
                             tree_mask=dev.tree_mask)

    if args.op == "append":
        bench_append(args, torch, pa, case, dev, pool, flush_caches, stream)
        return

    log(f"plan {plan}; warmup {args.warmup}")
    for _ in range(args.warmup):
        flush_caches()
        call()
    torch.cuda.synchronize()

    # Timed region: K steps, each = cache flush + one call bracketed by HIP
    # events recorded on the stream the kernels run on (the events' own
    # latency counts against the call).  A second pass of the same length
    # times the attention kernel alone: the library attaches the events to
    # that kernel's dispatch, so they hold its start and end times.
    evs = [(pa.HipEvent(), pa.HipEvent()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        flush_caches()
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = np.array([e0.elapsed_ms(e1) for e0, e1 in evs])
    kevs = [(pa.HipEvent(), pa.HipEvent()) for _ in range(args.steps)]
    for e0, e1 in kevs:
        flush_caches()
        call(e0, e1)
    torch.cuda.synchronize()
    kern_ms = np.array([e0.elapsed_ms(e1) for e0, e1 in kevs])
    log(f"timed {args.steps} steps: call {call_ms.mean() * 1e3:.1f} us, "
        f"attention kernel {kern_ms.mean() * 1e3:.1f} us")

    # chunked prefill, and draft trees on bf16 / fp8 pools, run the LDS-staged kernel
    staged = plan.get("kernel") == 1 or (case.tree_mask is not None and case.kv_dtype != "f32"
                                         and args.staged_from != -1)
    kernel_name = "paged_attn_staged" if staged else "paged_attn_partition"
    nbytes = case.algorithmic_bytes()
    flops = attention_flops(case)
    call_s = float(call_ms.mean()) / 1e3
    kern_s = float(kern_ms.mean()) / 1e3
    gbs = nbytes / call_s / 1e9
    achieved = nbytes / kern_s / 1e9
    rows = case.batch * case.q_per_seq
    mfma_bound = flops / nbytes > MFMA_RIDGE
    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(float(call_ms.mean()), 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8-e4m3 kv / bf16 q", "f32": "f32"}[case.kv_dtype],
        "data": "synthetic (seeded N(0,1), shuffled page pool)",
        "config": {"workload": case.name, "batch": case.batch, "q_per_seq": case.q_per_seq,
                   "num_q_heads": case.num_q_heads, "num_kv_heads": case.num_kv_heads,
                   "head_dim": case.head_dim, "seq_len_max": case.max_seq_len,
                   "seq_len_mean": float(case.seq_lens.mean()), "page_size": W.PAGE_SIZE,
                   "kv_dtype": case.kv_dtype, "bytes_per_call": nbytes},
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(rows / call_s, 1),
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
        "call_us": {"mean": round(float(call_ms.mean()) * 1e3, 2),
                    "p10": round(float(np.percentile(call_ms, 10)) * 1e3, 2),
                    "p50": round(float(np.percentile(call_ms, 50)) * 1e3, 2),
                    "p90": round(float(np.percentile(call_ms, 90)) * 1e3, 2)},
        "plan": plan,
        "roofline": {"bound": "hbm",
                     "kernel": kernel_name,
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(case.name),
                     "kernel_us_mean": round(kern_s * 1e6, 2),
                     "algorithmic_bytes_per_launch": nbytes,
                     "flops_per_launch": flops},
    }
    if mfma_bound:
        # above the MFMA ridge (chunked prefill): the contraction bounds the kernel
        peak = PEAK_MFMA_TFLOPS[case.kv_dtype]
        tflops = flops / kern_s / 1e12
        result.update({
            "metric": "chunked-prefill attention TFLOP/s (MFMA-bound)",
            "value": round(flops / call_s / 1e12, 2), "unit": "TFLOP/s",
            "pct_of_peak": round(100 * flops / call_s / 1e12 / peak, 2)})
        result["roofline"].update({"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                                   "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                                   "hbm_gbs": round(achieved, 1)})
    copy_gbs = measure_copy_gbs(torch, stream)
    result["copy_gbs"] = round(copy_gbs, 1)
    if not mfma_bound:
        result["pct_of_copy"] = round(100 * gbs / copy_gbs, 2)
        result["roofline"]["frac_of_copy"] = round(achieved / copy_gbs, 4)
    if flush is not None:
        read_gbs = measure_read_gbs(torch, stream, flush_caches)
        result["read_gbs"] = round(read_gbs, 1)
        if not mfma_bound:
            result["pct_of_read"] = round(100 * gbs / read_gbs, 2)
            result["roofline"]["frac_of_read"] = round(achieved / read_gbs, 4)
            # the same number of bytes read as one plain stream, from HBM, with its
            # own launch and ramp: what a call of this size costs at the least
            same_us = measure_read_us(torch, stream, flush_caches, nbytes)
            result["read_same_bytes_us"] = round(same_us, 2)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(case, args.cpu_reps)
        if mfma_bound:
            sec = case.algorithmic_bytes() / (cpu["value"] * 1e9)
            cpu.update({"value": flops / sec / 1e12, "unit": "TFLOP/s"})
        result["cpu_baseline"] = cpu
    add_speedup(result)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
