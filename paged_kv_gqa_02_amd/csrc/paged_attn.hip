// paged_attn.hip -- host side of the library for MI355X: argument checks, the
// launch plan, launches and the C ABI of include/paged_attn.h.  The kernels
// live in decode.hip (partition kernel, split-K reduce), staged.hip (LDS-staged
// kernel for chunked prefill and draft trees), append.hip (KV append) and
// spec_sample.hip (speculative-sampling acceptance).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "decode.h"
#include "paged_attn.h"
#include "staged.h"
#include "status.h"

#define PA_API extern "C" __attribute__((visibility("default")))

namespace {

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
pa_status fail(pa_status st, const char* what) { return pa_record_error(st, what); }

pa_status hip_fail(hipError_t e, const char* where) { return pa_record_hip_error(e, where); }

int cu_count()
{
    static std::mutex mu;
    static std::vector<int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 256;
    }
    std::lock_guard<std::mutex> lock(mu);
    if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess || cus <= 0) {
            (void)hipGetLastError();
            cus = 256;
        }
        cache[dev] = cus;
    }
    return cache[dev];
}

// Defaults measured on MI355X (bf16 8B-GQA decode, B64 ctx 2048): four waves
// per workgroup (kDefaultWaves) and a three-page register pipeline for one row
// tile; two pages when the query tile (two row tiles, or fp8 conversion) needs
// the registers.
// query rows per sequence from which bf16 / fp8 causal calls take the LDS-staged
// (chunked-prefill) kernel
constexpr int kStagedFromRows = 128;
constexpr int default_prefetch(pa_dtype kv, int row_tiles)
{
    return (row_tiles == 1 && kv != PA_FP8_E4M3) ? 3 : 2;
}

size_t elem_size(pa_dtype t)
{
    return t == PA_F32 ? 4 : t == PA_BF16 ? 2 : 1;
}

bool dtype_known(pa_dtype t) { return t == PA_F32 || t == PA_BF16 || t == PA_FP8_E4M3; }

}  // namespace

struct pa_pool {
    pa_pool_desc d;
};

namespace {

pa_status make_plan(const pa_pool* pool, int32_t batch, int32_t n, int32_t hq, int32_t max_len,
                    pa_plan* pl, bool allow_prefill = true)
{
    if (!pool || !pl) return fail(PA_ERR_INVALID_ARG, "null pool or plan");
    const pa_pool_desc& d = pool->d;
    if (batch < 1 || n < 1 || hq < 1 || max_len < 1)
        return fail(PA_ERR_INVALID_ARG, "batch, q_per_seq, num_q_heads and max_seq_len must be >= 1");
    if (hq < d.num_kv_heads || hq % d.num_kv_heads != 0)
        return fail(PA_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
    if (max_len < n) return fail(PA_ERR_INVALID_ARG, "max_seq_len < q_per_seq");
    const int64_t rows = (int64_t)(hq / d.num_kv_heads) * n;
    if (rows > INT32_MAX / 2) return fail(PA_ERR_UNSUPPORTED, "too many query rows");
    // chunked prefill: many rows per sequence make the call a dense contraction
    const int staged_from = d.staged_from == 0 ? kStagedFromRows : d.staged_from;
    if (allow_prefill && d.kv_dtype != PA_F32 && staged_from > 0 && n >= staged_from &&
        (max_len + kPage - 1) / kPage <= kStagedMaxPages) {
        const int64_t row_blocks = (rows + kStagedPrefillRows - 1) / kStagedPrefillRows;
        const int max_pages = (max_len + kPage - 1) / kPage;
        int part = max_pages;
        if (d.partition_pages > 0) part = std::min(d.partition_pages, max_pages);
        part = std::max(part, (max_pages + kMaxSplits - 1) / kMaxSplits);
        const int64_t ns = (max_pages + part - 1) / part;
        const int64_t grid = (int64_t)batch * d.num_kv_heads * row_blocks * ns;
        if (grid > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "grid too large");
        pl->partition_pages = part;
        pl->num_splits = (int32_t)ns;
        pl->row_tiles = kStagedPrefillRows / 16;
        pl->row_chunks = (int32_t)row_blocks;
        pl->waves = 4;
        pl->grid = (int32_t)grid;
        pl->reduce = ns > 1 ? 1 : 0;
        pl->kernel = 1;
        return PA_OK;
    }
    const int nt = (int)std::min<int64_t>(kMaxRowTiles, (rows + 15) / 16);
    const int64_t row_chunks = (rows + 16 * nt - 1) / (16 * nt);
    const int max_pages = (max_len + kPage - 1) / kPage;
    const int64_t units = (int64_t)batch * d.num_kv_heads * row_chunks;
    const int waves = d.waves > 0 ? d.waves : kDefaultWaves;
    int part;
    if (d.partition_pages > 0) {
        part = std::min(d.partition_pages, max_pages);
    } else {
        // two workgroups per CU for one row tile; one for wider query tiles,
        // whose workgroups already fill the register file (MI355X sweep)
        const int64_t target = (nt == 1 ? 2LL : 1LL) * cu_count();
        int64_t ns = (target + units - 1) / units;
        const int64_t ns_cap = std::max<int64_t>(1, max_pages / (2 * waves));
        ns = std::max<int64_t>(1, std::min(ns, ns_cap));
        part = (int)((max_pages + ns - 1) / ns);
        // a wave takes its page ids 64 at a time: keep automatic partitions to
        // one round per wave while the split count allows
        part = std::min(part, 64 * waves);
    }
    // at most kMaxSplits partitions: longer sequences (more than 64 * W *
    // kMaxSplits pages) and partitions the pool asks for give a wave more than
    // 64 pages, which the partition kernel takes in several rounds of ids
    part = std::max(part, (max_pages + kMaxSplits - 1) / kMaxSplits);
    const int64_t ns = (max_pages + part - 1) / part;
    const int64_t grid = units * ns;
    if (grid > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "grid too large");
    pl->partition_pages = part;
    pl->num_splits = (int32_t)ns;
    pl->row_tiles = nt;
    pl->row_chunks = (int32_t)row_chunks;
    pl->waves = waves;
    pl->grid = (int32_t)grid;
    pl->reduce = ns > 1 ? 1 : 0;
    pl->kernel = 0;
    return PA_OK;
}

size_t workspace_for(const pa_plan& pl, int32_t batch, int32_t n, int32_t hq)
{
    if (!pl.reduce) return 0;
    const size_t rows = (size_t)batch * n * hq * pl.num_splits;
    const size_t acc = rows * kHeadDim * sizeof(float);
    const size_t acc_aligned = (acc + 255) & ~size_t(255);
    return acc_aligned + rows * 2 * sizeof(float);
}

pa_status run(const pa_pool* pool, const void* q, pa_dtype q_dtype, void* out,
              const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
              int32_t max_seq_len, int32_t batch, int32_t n, int32_t hq, float scale,
              const uint64_t* tree_mask, void* workspace, size_t workspace_bytes, void* stream,
              void* ev_begin, void* ev_end)
{
    if (!pool) return fail(PA_ERR_INVALID_ARG, "null pool");
    if (!q || !out || !block_table || !seq_lens)
        return fail(PA_ERR_INVALID_ARG, "null q, out, block_table or seq_lens");
    const pa_pool_desc& d = pool->d;
    const bool combo_ok = (d.kv_dtype == PA_F32 && q_dtype == PA_F32) ||
                          (d.kv_dtype == PA_BF16 && q_dtype == PA_BF16) ||
                          (d.kv_dtype == PA_FP8_E4M3 && q_dtype == PA_BF16);
    if (!dtype_known(q_dtype)) return fail(PA_ERR_INVALID_ARG, "unknown q dtype");
    if (!combo_ok)
        return fail(PA_ERR_UNSUPPORTED,
                    "supported (kv, q) dtypes: (f32, f32), (bf16, bf16), (fp8, bf16)");
    if (max_pages_per_seq < 1) return fail(PA_ERR_INVALID_ARG, "max_pages_per_seq must be >= 1");
    if (max_seq_len > (int64_t)kPage * max_pages_per_seq)
        return fail(PA_ERR_INVALID_ARG, "max_seq_len exceeds 16 * max_pages_per_seq");
    if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
    pa_plan pl;
    // the LDS-staged kernel writes O in 8- and 16-byte pieces; draft trees
    // never take the chunked-prefill plan (they have their own staged path)
    const bool out16 = reinterpret_cast<uintptr_t>(out) % 16 == 0;
    pa_status stt = make_plan(pool, batch, n, hq, max_seq_len, &pl, out16 && !tree_mask);
    if (stt != PA_OK) return stt;
    const size_t need = workspace_for(pl, batch, n, hq);
    if (need > 0) {
        if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace required for a split call");
        if (workspace_bytes < need) return fail(PA_ERR_WORKSPACE, "workspace too small");
        if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
            return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    }
    if (reinterpret_cast<uintptr_t>(q) % 16 || reinterpret_cast<uintptr_t>(d.k) % 16 ||
        reinterpret_cast<uintptr_t>(d.v) % 16)
        return fail(PA_ERR_INVALID_ARG, "q, k and v must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(out) % elem_size(q_dtype))
        return fail(PA_ERR_INVALID_ARG, "out must be aligned to its element size");

    DecodeArgs a;
    a.k = d.k;
    a.v = d.v;
    a.k_scale = d.k_scale;
    a.v_scale = d.v_scale;
    a.q = q;
    a.out = out;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.tree_mask = tree_mask;
    a.part_acc = static_cast<float*>(workspace);
    a.part_ml = need ? reinterpret_cast<float*>(
                           static_cast<char*>(workspace) +
                           (((size_t)batch * n * hq * pl.num_splits * kHeadDim * sizeof(float) +
                             255) & ~size_t(255)))
                     : nullptr;
    a.page_stride = (int64_t)d.num_kv_heads * kSlab;
    a.num_pages = d.num_pages;
    a.max_pages = max_pages_per_seq;
    a.n = n;
    a.hq = hq;
    a.hkv = d.num_kv_heads;
    a.group = hq / d.num_kv_heads;
    a.rows = a.group * n;
    a.row_chunks = pl.row_chunks;
    a.num_splits = pl.num_splits;
    a.part_pages = pl.partition_pages;
    a.scale_log2 = scale * kLog2e;

    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    // draft trees on bf16 / fp8 pools: the LDS-staged kernel, 64 rows per
    // workgroup, under the same split plan (and workspace) as the partition kernel
    const bool staged_tree = tree_mask && d.kv_dtype != PA_F32 && d.staged_from != -1 && out16 &&
                             pl.partition_pages <= kStagedTreeMaxPages;
    const hipEvent_t e0 = static_cast<hipEvent_t>(ev_begin), e1 = static_cast<hipEvent_t>(ev_end);
    if (pl.kernel == 1 || staged_tree) {
        StagedArgs sa;
        sa.k = d.k;
        sa.v = d.v;
        sa.k_scale = d.k_scale;
        sa.v_scale = d.v_scale;
        sa.q = static_cast<const uint16_t*>(q);
        sa.out = static_cast<uint16_t*>(out);
        sa.block_table = block_table;
        sa.seq_lens = seq_lens;
        sa.tree_mask = tree_mask;
        sa.part_acc = a.part_acc;
        sa.part_ml = a.part_ml;
        sa.page_stride = a.page_stride;
        sa.num_pages = d.num_pages;
        sa.max_pages = max_pages_per_seq;
        sa.batch = batch;
        sa.n = n;
        sa.hq = hq;
        sa.hkv = d.num_kv_heads;
        sa.group = a.group;
        sa.rows = a.rows;
        sa.row_blocks = staged_tree ? (a.rows + kStagedTreeRows - 1) / kStagedTreeRows : pl.row_chunks;
        sa.num_splits = pl.num_splits;
        sa.part_pages = pl.partition_pages;
        sa.scale_log2 = a.scale_log2;
        const int64_t items = (int64_t)batch * d.num_kv_heads * sa.row_blocks * sa.num_splits;
        if (items < 1 || items > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "grid too large");
        // chunked prefill: one workgroup per CU (its LDS ring fills the CU), each
        // taking its share of the row blocks in turn; draft trees: one per item
        sa.workgroups = staged_tree ? (int32_t)items : (int32_t)std::min<int64_t>(items, cu_count());
        if ((e = launch_staged(sa, d.kv_dtype == PA_FP8_E4M3, staged_tree, st, e0, e1)) != hipSuccess)
            return hip_fail(e, "staged kernel launch");
    } else {
        // the partition kernel decodes blockIdx as (sequence, kv head, row chunk,
        // partition): only its own plan may reach it
        if (pl.kernel != 0 || pl.row_tiles < 1 || pl.row_tiles > kMaxRowTiles ||
            (int64_t)pl.grid != (int64_t)batch * d.num_kv_heads * pl.row_chunks * pl.num_splits)
            return fail(PA_ERR_INVALID_ARG, "internal: plan does not fit the partition kernel");
        const int pf = d.prefetch > 0 ? d.prefetch : default_prefetch(d.kv_dtype, pl.row_tiles);
        if ((e = launch_partition(a, d.kv_dtype, pl.row_tiles, pl.waves, pf, pl.grid, st, e0, e1)) !=
            hipSuccess)
            return hip_fail(e, "partition kernel launch");
    }
    if (pl.reduce) {
        const unsigned rows_out = (unsigned)((int64_t)batch * n * hq);
        if ((e = launch_reduce(a, q_dtype == PA_F32, rows_out, st)) != hipSuccess)
            return hip_fail(e, "reduce kernel launch");
    }
    return PA_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
PA_API pa_status paged_attn_pool_bytes(int32_t num_pages, int32_t page_size, int32_t num_kv_heads,
                                       int32_t head_dim, pa_dtype kv_dtype, size_t* k_bytes,
                                       size_t* v_bytes)
{
    if (!k_bytes || !v_bytes) return fail(PA_ERR_INVALID_ARG, "null output pointer");
    if (num_pages < 1 || page_size < 1 || num_kv_heads < 1 || head_dim < 1)
        return fail(PA_ERR_INVALID_ARG, "counts must be >= 1");
    if (!dtype_known(kv_dtype)) return fail(PA_ERR_UNSUPPORTED, "unknown kv dtype");
    const size_t b = (size_t)num_pages * num_kv_heads * page_size * head_dim * elem_size(kv_dtype);
    *k_bytes = b;
    *v_bytes = b;
    return PA_OK;
}

PA_API pa_status paged_attn_create_pool(const pa_pool_desc* desc, pa_pool** out)
{
    if (!out) return fail(PA_ERR_INVALID_ARG, "null output handle");
    *out = nullptr;
    if (!desc) return fail(PA_ERR_INVALID_ARG, "null descriptor");
    if (desc->num_pages < 1 || desc->num_kv_heads < 1)
        return fail(PA_ERR_INVALID_ARG, "num_pages and num_kv_heads must be >= 1");
    if (!desc->k || !desc->v) return fail(PA_ERR_INVALID_ARG, "null k or v pool");
    if (desc->page_size != kPage) return fail(PA_ERR_UNSUPPORTED, "page_size must be 16");
    if (desc->head_dim != kHeadDim) return fail(PA_ERR_UNSUPPORTED, "head_dim must be 128");
    if (!dtype_known(desc->kv_dtype)) return fail(PA_ERR_UNSUPPORTED, "unknown kv dtype");
    if (desc->kv_dtype == PA_FP8_E4M3 && (!desc->k_scale || !desc->v_scale))
        return fail(PA_ERR_INVALID_ARG, "fp8 pools need k_scale and v_scale");
    if (desc->partition_pages < 0) return fail(PA_ERR_INVALID_ARG, "partition_pages must be >= 0");
    if (desc->waves != 0 && desc->waves != 4 && desc->waves != 8)
        return fail(PA_ERR_UNSUPPORTED, "waves must be 0, 4 or 8");
    if (desc->prefetch != 0 && (desc->prefetch < 2 || desc->prefetch > 6 ||
                                (desc->waves == 8 && desc->prefetch > 4)))
        return fail(PA_ERR_UNSUPPORTED, "prefetch must be 0, 2..6 (2..4 with 8 waves)");
    if (desc->staged_from < -1) return fail(PA_ERR_INVALID_ARG, "staged_from must be >= -1");
    pa_pool* p = new (std::nothrow) pa_pool;
    if (!p) return fail(PA_ERR_INVALID_ARG, "out of host memory");
    p->d = *desc;
    *out = p;
    return PA_OK;
}

PA_API void paged_attn_destroy_pool(pa_pool* pool) { delete pool; }

PA_API pa_status paged_attn_plan(const pa_pool* pool, int32_t batch, int32_t q_per_seq,
                                 int32_t num_q_heads, int32_t max_seq_len, pa_plan* plan)
{
    return make_plan(pool, batch, q_per_seq, num_q_heads, max_seq_len, plan);
}

PA_API pa_status paged_attn_workspace_bytes(const pa_pool* pool, int32_t batch, int32_t q_per_seq,
                                            int32_t num_q_heads, int32_t max_seq_len,
                                            size_t* bytes)
{
    if (!bytes) return fail(PA_ERR_INVALID_ARG, "null output pointer");
    // enough for the causal call of this shape and for the draft-tree call,
    // which never takes the chunked-prefill plan
    pa_plan pl, tree;
    pa_status st = make_plan(pool, batch, q_per_seq, num_q_heads, max_seq_len, &pl);
    if (st != PA_OK) return st;
    st = make_plan(pool, batch, q_per_seq, num_q_heads, max_seq_len, &tree, false);
    if (st != PA_OK) return st;
    *bytes = std::max(workspace_for(pl, batch, q_per_seq, num_q_heads),
                      workspace_for(tree, batch, q_per_seq, num_q_heads));
    return PA_OK;
}

PA_API pa_status paged_attn_decode(const pa_pool* pool, const void* q, pa_dtype q_dtype, void* out,
                                   const int32_t* block_table, int32_t max_pages_per_seq,
                                   const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                                   int32_t num_q_heads, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream)
{
    return run(pool, q, q_dtype, out, block_table, max_pages_per_seq, seq_lens, max_seq_len, batch,
               1, num_q_heads, scale, nullptr, workspace, workspace_bytes, stream, nullptr,
               nullptr);
}

PA_API pa_status paged_attn_verify(const pa_pool* pool, const void* q, pa_dtype q_dtype, void* out,
                                   const int32_t* block_table, int32_t max_pages_per_seq,
                                   const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                                   int32_t q_per_seq, int32_t num_q_heads, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream)
{
    return run(pool, q, q_dtype, out, block_table, max_pages_per_seq, seq_lens, max_seq_len, batch,
               q_per_seq, num_q_heads, scale, nullptr, workspace, workspace_bytes, stream, nullptr,
               nullptr);
}

PA_API pa_status paged_attn_verify_timed(const pa_pool* pool, const void* q, pa_dtype q_dtype,
                                         void* out, const int32_t* block_table,
                                         int32_t max_pages_per_seq, const int32_t* seq_lens,
                                         int32_t max_seq_len, int32_t batch, int32_t q_per_seq,
                                         int32_t num_q_heads, float scale,
                                         const uint64_t* tree_mask, void* workspace,
                                         size_t workspace_bytes, void* stream, void* ev_begin,
                                         void* ev_end)
{
    if (tree_mask && q_per_seq > 64)
        return fail(PA_ERR_UNSUPPORTED, "draft trees have at most 64 nodes");
    return run(pool, q, q_dtype, out, block_table, max_pages_per_seq, seq_lens, max_seq_len, batch,
               q_per_seq, num_q_heads, scale, tree_mask, workspace, workspace_bytes, stream,
               ev_begin, ev_end);
}

PA_API pa_status paged_attn_verify_tree(const pa_pool* pool, const void* q, pa_dtype q_dtype,
                                        void* out, const int32_t* block_table,
                                        int32_t max_pages_per_seq, const int32_t* seq_lens,
                                        int32_t max_seq_len, int32_t batch, int32_t q_per_seq,
                                        int32_t num_q_heads, float scale,
                                        const uint64_t* tree_mask, void* workspace,
                                        size_t workspace_bytes, void* stream)
{
    if (!tree_mask) return fail(PA_ERR_INVALID_ARG, "null tree_mask");
    if (q_per_seq > 64) return fail(PA_ERR_UNSUPPORTED, "draft trees have at most 64 nodes");
    return run(pool, q, q_dtype, out, block_table, max_pages_per_seq, seq_lens, max_seq_len, batch,
               q_per_seq, num_q_heads, scale, tree_mask, workspace, workspace_bytes, stream,
               nullptr, nullptr);
}

// ---------------------------------------------------------------------------
// paged_attn_verify_noalloc: the split-K partials in a static device array
// ---------------------------------------------------------------------------
// One copy per GPU the library runs on, held until the process ends.  In host
// code `scratch` names a host-side stand-in: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

pa_status scratch_address(void** out)
{
    static std::mutex mu;
    static std::vector<void*> addr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(mu);
    if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
    if (!addr[dev]) {
        void* p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess)
            return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
        addr[dev] = p;
    }
    *out = addr[dev];
    return PA_OK;
}

}  // namespace

PA_API pa_status paged_attn_verify_noalloc(const pa_pool* pool, const void* q, pa_dtype q_dtype,
                                           void* out, const int32_t* block_table,
                                           int32_t max_pages_per_seq, const int32_t* seq_lens,
                                           int32_t max_seq_len, int32_t batch, int32_t q_per_seq,
                                           int32_t num_q_heads, float scale, void* stream)
{
    // the partials the call's plan needs must fit the array; this is decided
    // on the host before any HIP call
    size_t need = 0;
    pa_status st = paged_attn_workspace_bytes(pool, batch, q_per_seq, num_q_heads, max_seq_len,
                                              &need);
    if (st != PA_OK) return st;
    if (need > kScratchBytes)
        return fail(PA_ERR_WORKSPACE,
                    "split-K partials exceed the 16 MiB static scratch; call paged_attn_verify "
                    "with a workspace");
    void* ws = nullptr;
    if (need > 0 && (st = scratch_address(&ws)) != PA_OK) return st;
    return run(pool, q, q_dtype, out, block_table, max_pages_per_seq, seq_lens, max_seq_len, batch,
               q_per_seq, num_q_heads, scale, nullptr, ws, need > 0 ? kScratchBytes : 0, stream,
               nullptr, nullptr);
}

PA_API pa_status paged_attn_append_kv(const pa_pool* pool, const void* k_new, const void* v_new,
                                      pa_dtype src_dtype, const int32_t* block_table,
                                      int32_t max_pages_per_seq, const int32_t* seq_lens,
                                      int32_t batch, int32_t n_new, void* stream)
{
    if (!pool) return fail(PA_ERR_INVALID_ARG, "null pool");
    if (!k_new || !v_new || !block_table || !seq_lens)
        return fail(PA_ERR_INVALID_ARG, "null k_new, v_new, block_table or seq_lens");
    if (batch < 1 || n_new < 1 || max_pages_per_seq < 1)
        return fail(PA_ERR_INVALID_ARG, "batch, n_new and max_pages_per_seq must be >= 1");
    if (n_new > (int64_t)kPage * max_pages_per_seq)
        return fail(PA_ERR_INVALID_ARG, "n_new exceeds 16 * max_pages_per_seq");
    if (src_dtype != PA_F32 && src_dtype != PA_BF16)
        return fail(PA_ERR_INVALID_ARG, "source values must be f32 or bf16");
    const pa_pool_desc& d = pool->d;
    if (d.kv_dtype == PA_F32 && src_dtype != PA_F32)
        return fail(PA_ERR_UNSUPPORTED, "an f32 pool takes f32 source values");
    if (reinterpret_cast<uintptr_t>(k_new) % 16 || reinterpret_cast<uintptr_t>(v_new) % 16)
        return fail(PA_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
    const int64_t span = (n_new + kPage - 2) / kPage + 1;   // most pages n_new tokens touch
    if ((int64_t)batch * d.num_kv_heads * 2 > INT32_MAX || span > 65535)
        return fail(PA_ERR_UNSUPPORTED, "grid too large");
    AppendArgs a;
    a.k = d.k;
    a.v = d.v;
    a.k_scale = d.k_scale;
    a.v_scale = d.v_scale;
    a.k_new = k_new;
    a.v_new = v_new;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.page_stride = (int64_t)d.num_kv_heads * kSlab;
    a.num_pages = d.num_pages;
    a.max_pages = max_pages_per_seq;
    a.hkv = d.num_kv_heads;
    a.n_new = n_new;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)(batch * d.num_kv_heads * 2), (unsigned)span);
    const hipError_t e = launch_append(a, d.kv_dtype, src_dtype == PA_BF16, grid, st);
    if (e != hipSuccess) return hip_fail(e, "append kernel launch");
    return PA_OK;
}

PA_API pa_status paged_attn_validate(const pa_pool* pool, const int32_t* block_table,
                                     int32_t max_pages_per_seq, const int32_t* seq_lens,
                                     int32_t max_seq_len, int32_t batch, int32_t q_per_seq,
                                     void* stream)
{
    if (!pool || !block_table || !seq_lens) return fail(PA_ERR_INVALID_ARG, "null argument");
    if (batch < 1 || max_pages_per_seq < 1 || q_per_seq < 1)
        return fail(PA_ERR_INVALID_ARG, "counts must be >= 1");
    std::vector<int32_t> lens(batch), tab((size_t)batch * max_pages_per_seq);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if ((e = hipMemcpyAsync(lens.data(), seq_lens, lens.size() * 4, hipMemcpyDeviceToHost, st)) !=
        hipSuccess)
        return hip_fail(e, "hipMemcpyAsync(seq_lens)");
    if ((e = hipMemcpyAsync(tab.data(), block_table, tab.size() * 4, hipMemcpyDeviceToHost, st)) !=
        hipSuccess)
        return hip_fail(e, "hipMemcpyAsync(block_table)");
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    for (int b = 0; b < batch; ++b) {
        const int L = lens[b];
        if (L < q_per_seq || L > max_seq_len || L > (int64_t)kPage * max_pages_per_seq) {
            char msg[128];
            snprintf(msg, sizeof msg, "seq_lens[%d] = %d out of range", b, L);
            return fail(PA_ERR_CONTRACT, msg);
        }
        const int np = (L + kPage - 1) / kPage;
        for (int p = 0; p < np; ++p) {
            const int id = tab[(size_t)b * max_pages_per_seq + p];
            if (id < 0 || id >= pool->d.num_pages) {
                char msg[128];
                snprintf(msg, sizeof msg, "block_table[%d][%d] = %d out of range", b, p, id);
                return fail(PA_ERR_CONTRACT, msg);
            }
        }
    }
    return PA_OK;
}

PA_API const char* paged_attn_status_str(pa_status status)
{
    switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_CONTRACT: return "device array violates the contract";
    default: return "unknown status";
    }
}

static thread_local std::string g_last_error;

pa_status pa_record_error(pa_status st, const char* what)
{
    g_last_error = what;
    return st;
}

pa_status pa_record_hip_error(hipError_t e, const char* where)
{
    g_last_error = std::string(where) + ": " + hipGetErrorString(e);
    return PA_ERR_HIP;
}

PA_API const char* paged_attn_last_error(void) { return g_last_error.c_str(); }
