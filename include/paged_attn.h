/*
 * paged_attn.h -- C ABI of libpaged_attn: paged GQA decode and speculative
 * verify attention for AMD Instinct MI355X (gfx950).
 *
 * What it computes (sources: "Latency and cost in production" ch. 10,
 * §10.3.1, §10.1.2, §10.4.2; "Batching, speculative decoding, paged
 * attention" §5.3.7; "Speculative decoding principles" 7.2.1, "the four
 * steps of one iteration"):
 *
 *   For sequence b with L = seq_lens[b] tokens already in the pool and n
 *   query rows (n = 1 for decode, K + 1 for verify), row i (0 <= i < n) is
 *   token L - n + i and attends to keys t = 0 .. L - n + i (itself and every
 *   earlier token; later draft rows are masked).  Query head h reads
 *   key/value head floor(h / G), G = num_q_heads / num_kv_heads.  Token t
 *   lives in slot t % 16 of physical page block_table[b][t / 16].
 *
 *     out[b][i][h] = sum_t softmax_t(scale * q[b][i][h] . K_t) * V_t
 *
 *   fp8 pools store OCP E4M3 bytes; the value of a key/value element is
 *   value(byte) * scale[page][kv_head] (symmetric, zero-point 0:
 *   "Latency and cost in production" §10.8.2-§10.8.3).
 *
 * Layouts (all row-major, all device memory unless noted):
 *   V pool           [num_pages][num_kv_heads][16][128] elements of kv_dtype
 *                    (token-major: one 128-element row per token)
 *   K pool           [num_pages][num_kv_heads][128 / x][16][x], x = 16 bytes /
 *                    element size (4 for f32, 8 for bf16, 16 for fp8): the head
 *                    dimension of a (page, head) slab is cut into 16-byte
 *                    chunks and each chunk holds the 16 tokens one after
 *                    another.  Element d of token t is at slab index
 *                    ((d / x) * 16 + t) * x + d % x.
 *   k_scale, v_scale [num_pages][num_kv_heads] float32 (fp8 pools only)
 *   q, out           [batch][q_per_seq][num_q_heads][128] elements of q_dtype
 *                    (out has the dtype of q)
 *   block_table      [batch][max_pages_per_seq] int32
 *   seq_lens         [batch] int32
 *   workspace        paged_attn_workspace_bytes() bytes, 256-byte aligned
 *
 * Supported element types: (kv f32, q f32), (kv bf16, q bf16),
 * (kv fp8-e4m3, q bf16).  page_size must be 16 and head_dim 128.
 *
 * Ownership: every buffer belongs to the caller.  The library allocates no
 * device memory (paged_attn_verify_noalloc uses a static array of the
 * library's code object instead of a workspace); a pool handle only records
 * the descriptor (a few dozen bytes of host memory) and never frees the
 * caller's arrays.
 *
 * Calls: asynchronous on the given stream (a hipStream_t; NULL = the null
 * stream of the current device) on the current HIP device.  Argument checks
 * run on the host before anything is launched and return an error without
 * launching.  Calls are reentrant; a pool handle is read-only after
 * creation and may be shared across threads.  Apart from paged_attn_validate,
 * which copies to the host and synchronises, a call only enqueues kernels on
 * `stream` (no memset, copy, allocation or synchronisation), so it may be
 * captured into a HIP graph and replayed; the graph then reads whatever the
 * captured buffers hold at each replay.
 *
 * Batch order: sequences are taken in index order.  On a mix of lengths a
 * batch ordered longest first finishes sooner (no long sequence is left for
 * the end of the grid); results do not depend on the order.
 *
 * Device-array contract (not checked on the fast path; paged_attn_validate
 * checks it): for every b, n <= seq_lens[b] <= max_seq_len <=
 * 16 * max_pages_per_seq, and block_table[b][p] lies in [0, num_pages) for
 * p < ceil(seq_lens[b] / 16).  Entries past a sequence's last page, slots
 * past its last token and pages no table names are never read and may hold
 * anything (NaN included).  Two tables may name the same page.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = -1,  /* null pointer, bad size or count */
    PA_ERR_UNSUPPORTED = -2,  /* valid request outside what the kernels handle */
    PA_ERR_WORKSPACE = -3,    /* workspace missing, too small or misaligned */
    PA_ERR_HIP = -4,          /* a HIP runtime call failed; see paged_attn_last_error() */
    PA_ERR_CONTRACT = -5,     /* paged_attn_validate found a bad device array */
    /* not a status: makes every int32 value a value of the type, so an arbitrary
       code a caller passes (paged_attn_status_str) is well defined */
    PA_STATUS_INT32_RANGE = 0x7fffffff
} pa_status;

typedef enum pa_dtype {
    PA_F32 = 0,
    PA_BF16 = 1,
    PA_FP8_E4M3 = 2,
    /* not a dtype: makes every int32 value a value of the type, so an unknown
       code is rejected (PA_ERR_UNSUPPORTED / PA_ERR_INVALID_ARG), not undefined */
    PA_DTYPE_INT32_RANGE = 0x7fffffff
} pa_dtype;

/* Description of a page pool.  All pointers are device pointers. */
typedef struct pa_pool_desc {
    int32_t num_pages;
    int32_t page_size;        /* must be 16 */
    int32_t num_kv_heads;
    int32_t head_dim;         /* must be 128 */
    pa_dtype kv_dtype;
    /* pool arrays: read by the attention calls, written only by paged_attn_append_kv */
    void* k;                  /* [num_pages][num_kv_heads][128/x][16][x], x = 16 / elem size */
    void* v;                  /* [num_pages][num_kv_heads][16][128] */
    float* k_scale;           /* [num_pages][num_kv_heads], fp8 only, else NULL */
    float* v_scale;           /* [num_pages][num_kv_heads], fp8 only, else NULL */
    int32_t partition_pages;  /* split-K partition length in pages; 0 = chosen per call */
    int32_t waves;            /* tuning: waves per workgroup (4 or 8); 0 = automatic */
    int32_t prefetch;         /* tuning: pages held in registers per wave (2..6, at most 4 with
                                 8 waves); 0 = automatic */
    int32_t staged_from;      /* the LDS-staged kernel (pages staged once per workgroup and
                                 shared by its waves): a bf16 / fp8 causal call with at
                                 least this many query rows per sequence takes it
                                 (0 = automatic: 128), and so does every bf16 / fp8 draft-
                                 tree call; -1 = never */
} pa_pool_desc;

typedef struct pa_pool pa_pool;

/* How one call is split across the GPU (for reporting and tests). */
typedef struct pa_plan {
    int32_t partition_pages;  /* pages per context partition */
    int32_t num_splits;       /* partitions of the longest sequence */
    int32_t row_tiles;        /* 16-row MFMA tiles per workgroup */
    int32_t row_chunks;       /* workgroups needed to cover the G * n rows */
    int32_t waves;            /* waves per workgroup */
    int32_t grid;             /* work items: workgroups of the partition kernel (and of the
                                 LDS-staged kernel on draft trees); the chunked-prefill
                                 kernel runs min(grid, CUs) workgroups that take them in
                                 turn, heaviest first */
    int32_t reduce;           /* 1 if the split-K reduce kernel runs */
    int32_t kernel;           /* 0: partition kernel (+ reduce); 1: LDS-staged kernel for
                                 chunked prefill (128 rows of one sequence and kv head per
                                 workgroup; one partition per sequence and no workspace,
                                 unless the pool's partition_pages asks for shorter
                                 partitions, which then take the reduce).  Draft-tree calls on
                                 bf16 / fp8 pools run the LDS-staged kernel with 64 rows per
                                 workgroup under the split plan reported here. */
} pa_plan;

/* Bytes of the K and V pool arrays for a pool of this shape (host only). */
pa_status paged_attn_pool_bytes(int32_t num_pages, int32_t page_size,
                                int32_t num_kv_heads, int32_t head_dim,
                                pa_dtype kv_dtype, size_t* k_bytes, size_t* v_bytes);

/* Checks the descriptor and returns a handle recording it (host only, no HIP call).
 * The pool is the shared set of equal-size 16-token blocks that every
 * sequence's block table points into ("Batching, speculative decoding, paged
 * attention" §5.3.7; "Latency and cost in production" §10.12.2: blocks are
 * taken from one pool on demand and returned when a request ends).
 * PA_ERR_INVALID_ARG for null pointers or counts < 1, PA_ERR_UNSUPPORTED for
 * page_size != 16, head_dim != 128 or an unknown dtype; *out is NULL on error. */
pa_status paged_attn_create_pool(const pa_pool_desc* desc, pa_pool** out);

/* Frees the handle only; the pool arrays stay with the caller.  NULL is a no-op. */
void paged_attn_destroy_pool(pa_pool* pool);

/* The split the library will use for a causal call of this shape (host only).
 * A draft-tree call never takes the chunked-prefill plan (kernel = 1): where
 * this reports it (q_per_seq at or above a pool's staged_from of 64 or less),
 * the tree call runs the split plan computed without it. */
pa_status paged_attn_plan(const pa_pool* pool, int32_t batch, int32_t q_per_seq,
                          int32_t num_q_heads, int32_t max_seq_len, pa_plan* plan);

/* Workspace bytes a call of this shape needs (0 when it runs unsplit); the
 * same buffer serves the causal and the draft-tree call of the shape. */
pa_status paged_attn_workspace_bytes(const pa_pool* pool, int32_t batch,
                                     int32_t q_per_seq, int32_t num_q_heads,
                                     int32_t max_seq_len, size_t* bytes);

/* Decode: one query row per sequence (q_per_seq = 1), attending to every key
 * of its sequence through the block table ("Latency and cost in production"
 * §10.3.1: the new token's query is compared with every earlier key; "Batching,
 * speculative decoding, paged attention" §5.3.1 and §5.3.7: a decode step reads
 * each request's whole KV cache, gathered block by block).  The newest token's
 * K/V must already be in the pool (seq_lens counts it).  max_seq_len is a
 * host-side upper bound of seq_lens used to size the split.  Errors as
 * paged_attn_verify. */
pa_status paged_attn_decode(const pa_pool* pool, const void* q, pa_dtype q_dtype,
                            void* out, const int32_t* block_table,
                            int32_t max_pages_per_seq, const int32_t* seq_lens,
                            int32_t max_seq_len, int32_t batch, int32_t num_q_heads,
                            float scale, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Verify: q_per_seq = K + 1 query rows per sequence (the last accepted token
 * and the K drafts, whose K/V are already appended), scored in one call under
 * the causal mask described at the top of this file ("Speculative decoding
 * principles" 7.2.1, "the four steps of one iteration": the target scores the
 * context and the K drafts in one forward, each position seeing only itself
 * and earlier positions).  Returns PA_ERR_INVALID_ARG for null pointers, counts
 * < 1, num_q_heads not a multiple of the pool's KV heads, max_seq_len <
 * q_per_seq or > 16 * max_pages_per_seq, a non-finite scale or misaligned q / k
 * / v (16 bytes) or out (element size); PA_ERR_UNSUPPORTED for a (kv, q) dtype
 * pair outside the three supported; PA_ERR_WORKSPACE when the plan splits and
 * the workspace is missing, smaller than paged_attn_workspace_bytes() or not
 * 256-byte aligned; PA_ERR_HIP if a launch fails.  Nothing is launched on an
 * error. */
pa_status paged_attn_verify(const pa_pool* pool, const void* q, pa_dtype q_dtype,
                            void* out, const int32_t* block_table,
                            int32_t max_pages_per_seq, const int32_t* seq_lens,
                            int32_t max_seq_len, int32_t batch, int32_t q_per_seq,
                            int32_t num_q_heads, float scale, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Tree verification (Medusa / EAGLE style draft trees; "Batching, speculative
 * decoding, paged attention" §5.3.13: a tree of candidate branches is verified
 * in one forward with tree attention).  The q_per_seq <= 64 query rows are the
 * tree's nodes in topological order, stored as the last q_per_seq tokens of
 * each sequence (row i is token L - q_per_seq + i, node 0 the root).  Row i
 * attends to every context token t < L - q_per_seq and to tree token j iff bit
 * j of tree_mask[b][i] is set: its ancestors and itself.  tree_mask is a device
 * array [batch][q_per_seq] of uint64; bits >= q_per_seq are ignored.  The chain
 * mask tree_mask[b][i] = 2^(i+1) - 1 gives exactly paged_attn_verify.  Every
 * row must see at least one key.  PA_ERR_INVALID_ARG for a null mask,
 * PA_ERR_UNSUPPORTED for q_per_seq > 64; otherwise as paged_attn_verify. */
pa_status paged_attn_verify_tree(const pa_pool* pool, const void* q, pa_dtype q_dtype,
                                 void* out, const int32_t* block_table,
                                 int32_t max_pages_per_seq, const int32_t* seq_lens,
                                 int32_t max_seq_len, int32_t batch, int32_t q_per_seq,
                                 int32_t num_q_heads, float scale, const uint64_t* tree_mask,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* paged_attn_verify (tree_mask NULL) or paged_attn_verify_tree (tree_mask set)
 * that also times the attention kernel (partition or LDS-staged; not the
 * split-K reduce): the events are attached to that kernel's own dispatch and
 * take the times at which it starts and ends, so hipEventElapsedTime gives its
 * execution time with no marker overhead.  The events are hipEvent_t handles
 * created by the caller; either may be NULL. */
pa_status paged_attn_verify_timed(const pa_pool* pool, const void* q, pa_dtype q_dtype,
                                  void* out, const int32_t* block_table,
                                  int32_t max_pages_per_seq, const int32_t* seq_lens,
                                  int32_t max_seq_len, int32_t batch, int32_t q_per_seq,
                                  int32_t num_q_heads, float scale, const uint64_t* tree_mask,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  void* ev_begin, void* ev_end);

/* paged_attn_verify for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument.  Split-K partials go to a static device
 * array of the library, 16 MiB per GPU, held until the process ends; a shape
 * whose partials need more (paged_attn_workspace_bytes) returns
 * PA_ERR_WORKSPACE before anything runs.  The call allocates nothing; the
 * first call on a device looks up the array's address there.  Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (on different
 * streams, or from several threads) race and give wrong results.  Otherwise
 * as paged_attn_verify (causal mask; q_per_seq = 1 is a decode). */
pa_status paged_attn_verify_noalloc(const pa_pool* pool, const void* q, pa_dtype q_dtype,
                                    void* out, const int32_t* block_table,
                                    int32_t max_pages_per_seq, const int32_t* seq_lens,
                                    int32_t max_seq_len, int32_t batch, int32_t q_per_seq,
                                    int32_t num_q_heads, float scale, void* stream);

/* KV append (quantize-on-write), the step before attention in a decode or
 * verify pass: writes the n_new newest tokens of each sequence (positions
 * L - n_new .. L - 1, L = seq_lens[b], which counts them) into the pool, in its
 * layouts.  k_new, v_new: device [batch][n_new][num_kv_heads][128] of src_dtype
 * (PA_F32 or PA_BF16; an f32 pool takes f32), 16-byte aligned.
 *   f32 / bf16 pools: the value rounded to the pool format (nearest even).
 *   fp8 pools, per (page, kv head), K and V separately, in binary32
 *   ("Latency and cost in production" §10.8.2-§10.8.3: q = round(x / scale),
 *   zero-point 0):
 *     a page none of whose earlier slots are live takes
 *       scale = absmax(its new values) / 448 (1 if that absmax is 0);
 *     otherwise scale = max(old scale, absmax / 448), and when it grows every
 *       earlier live byte b is re-encoded as encode(value(b) * old / scale);
 *     each new value x is stored as encode(x / scale): the nearest E4M3 value,
 *     ties to even, saturating at +-448.
 * The pages for the new positions must be in the block table.  Calls that
 * touch the same pages must not overlap. */
pa_status paged_attn_append_kv(const pa_pool* pool, const void* k_new, const void* v_new,
                               pa_dtype src_dtype, const int32_t* block_table,
                               int32_t max_pages_per_seq, const int32_t* seq_lens,
                               int32_t batch, int32_t n_new, void* stream);

/* Speculative-sampling acceptance (rejection sampling), the step after the
 * verify pass ("Latency and cost in production" §10.6.2; "Speculative
 * decoding principles" 7.2.1, acceptance rule and residual distribution).
 * All arrays are device memory owned by the caller:
 *   p            [batch][num_drafts + 1][vocab] float32 target probabilities
 *                (row r scores position r; the last row gives the bonus token)
 *   q            [batch][num_drafts][vocab] float32 draft probabilities
 *   draft        [batch][num_drafts] int32 draft tokens, in [0, vocab)
 *   u_accept     [batch][num_drafts] float32 uniforms in [0, 1)
 *   u_sample     [batch] float32 uniforms in [0, 1)
 *   tokens       [batch][num_drafts + 1] int32 out: the accepted drafts, then
 *                the sampled token, then -1
 *   num_accepted [batch] int32 out
 * Draft i (x = draft[b][i]) passes iff u_accept[b][i] * q[b][i][x] <
 * p[b][i][x], evaluated exactly in binary64, i.e. with probability
 * min(1, p/q); tests run in order and stop at the first rejection, at r.
 * One token is then drawn with u = u_sample[b] from the weights
 *   w = max(0, p[b][r] - q[b][r]) after a rejection (p[b][r] itself when that
 *       residual is all zero), or w = p[b][num_drafts] when all drafts pass,
 * as the first j with w[0] + ... + w[j] > u * (w[0] + ... + w[vocab - 1]),
 * decided exactly: every float32 is an integer multiple of 2^-149, and the
 * weights, their running sums and floor(u * total) are formed as integers
 * (192 bits), with no rounding, so the token does not depend on how the sums
 * are associated.  The running sum rises only on positive weights: a
 * zero-weight token is never drawn.  A row with no mass gives token -1.
 * Entries of p and q must be finite, >= 0 and below 2^22 (probabilities are);
 * other values, or a draft token outside [0, vocab) (clamped), leave the
 * result unspecified but never make an access outside the arrays.
 * Limits: num_drafts <= 64, vocab <= 1,048,576, batch <= 65535.  Workspace:
 * paged_attn_rejection_sample_workspace_bytes(batch, vocab) bytes (per
 * 4096-entry chunk of a row, the exact sums of the weights and of p as twelve
 * uint32; then one int32 per sequence), 4-byte aligned, no initial contents.
 * Two kernels on `stream`; asynchronous. */
size_t paged_attn_rejection_sample_workspace_bytes(int32_t batch, int32_t vocab);
pa_status paged_attn_rejection_sample(const float* p, const float* q, const int32_t* draft,
                                      const float* u_accept, const float* u_sample,
                                      int32_t batch, int32_t num_drafts, int32_t vocab,
                                      int32_t* tokens, int32_t* num_accepted,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Debug check of the device-array contract: copies block_table and seq_lens
 * to the host (synchronously, on `stream`) and returns PA_ERR_CONTRACT if a
 * length or a needed page id is out of range. */
pa_status paged_attn_validate(const pa_pool* pool, const int32_t* block_table,
                              int32_t max_pages_per_seq, const int32_t* seq_lens,
                              int32_t max_seq_len, int32_t batch, int32_t q_per_seq,
                              void* stream);

/* Static description of a status code. */
const char* paged_attn_status_str(pa_status status);

/* Text of the last error recorded on the calling thread ("" if none). */
const char* paged_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
