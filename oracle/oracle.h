/*
 * oracle.h -- CPU reference for paged GQA decode / verify attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, obviously-correct float64
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header, table or constant with the GPU library, and the
 * product path never calls it.
 *
 * Sources (the three web pages this work follows):
 *  - "Latency and cost in production" (ch. 10), §10.3.1: the current token's
 *    query is compared with the key of every earlier token to get scores,
 *    and the values of the high-scoring tokens are gathered.
 *  - same page, §10.1.2: softmax over the scores; GQA splits the query heads
 *    into groups, each group sharing one key/value head.
 *  - same page, §10.4.2 (Fig. 10.4.2) and "Batching, speculative decoding,
 *    paged attention" §5.3.7: a per-request block table maps logical block i
 *    to a physical block of 16 tokens anywhere in a shared pool.
 *  - "Speculative decoding principles" (7.2.1), "the four steps of one
 *    iteration": the target scores the context plus K draft tokens in one
 *    forward; each row attends only to itself and earlier positions.
 *  - "Latency and cost in production" §10.8.2-§10.8.3: real ~= (q - zp) *
 *    scale, symmetric quantisation has zp = 0.
 *
 * Readings where the pages are silent:
 *  - softmax uses the natural exponential of scale * q.k;
 *  - seq_lens[b] counts every key already in the pool, including the n new
 *    query tokens; row i (0 <= i < n) sees keys 0 .. L - n + i inclusive;
 *  - query head h uses key/value head floor(h / (Hq / Hkv));
 *  - fp8 is OCP E4M3 (bias 7, max 448, S.1111.111 is NaN), dequantised as
 *    value(byte) * scale[page][kv_head] with zero-point 0.
 */
#ifndef PAGED_ATTN_ORACLE_H
#define PAGED_ATTN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element codes of the oracle's own decoder */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_E4M3 = 2 };

/* return codes */
enum { ORACLE_OK = 0, ORACLE_BAD_ARG = -1, ORACLE_BAD_TABLE = -2, ORACLE_NO_MEMORY = -3 };

/* Exact value of a bfloat16 bit pattern (the top 16 bits of an IEEE binary32). */
double oracle_bf16_value(uint16_t bits);

/* Exact value of an OCP E4M3 byte; NaN for 0x7F and 0xFF. */
double oracle_e4m3_value(uint8_t byte);

/*
 * Plain attention for ONE sequence over contiguous keys and values.
 *   q   [n][Hq][D]     query rows (row i is the (L - n + i)-th token)
 *   k,v [L][Hkv][D]    every key / value of the sequence in logical order
 *   out [n][Hq][D]
 * Row i, head h: z_t = scale * sum_d q[i][h][d] * k[t][h/G][d] for
 * t = 0 .. L - n + i; out = sum_t exp(z_t - max z) v_t / sum_t exp(z_t - max z).
 * Returns ORACLE_BAD_ARG unless 1 <= n <= L, Hkv >= 1, Hq % Hkv == 0, D >= 1.
 */
int oracle_attention(const double* q, const double* k, const double* v,
                     int L, int n, int Hq, int Hkv, int D, double scale,
                     double* out);

/*
 * Tree verification: the n query rows are the nodes of a draft tree stored in
 * the last n slots of the sequence (row i is token L - n + i).  Row i sees
 * every context token t < L - n and tree token j (token L - n + j) iff bit j
 * of tree_mask[i] is set (its ancestors and itself).  Source: "Batching,
 * speculative decoding, paged attention" §5.3.13 (Medusa and its relatives
 * verify a tree of candidate branches in one forward with tree attention).
 * The chain tree tree_mask[i] = 2^(i+1) - 1 is the causal verify above.
 * Returns ORACLE_BAD_ARG if n > 64 or a row sees no key at all.
 */
int oracle_attention_tree(const double* q, const double* k, const double* v,
                          int L, int n, int Hq, int Hkv, int D, double scale,
                          const uint64_t* tree_mask, double* out);

/*
 * Paged attention for the listed sequences, read straight from the pool.
 *   v_pool          [num_pages][Hkv][page_size][D] elements of kv_dtype
 *                   (float32, bfloat16 bits, or E4M3 bytes), token-major
 *   k_pool          [num_pages][Hkv][D / x][page_size][x] with x = 16 bytes /
 *                   element size: the library's documented K layout, in which
 *                   the head dimension of a slab is cut into 16-byte chunks
 *                   that each hold every token of the page in turn
 *   k_scale,v_scale [num_pages][Hkv] float32, used only for E4M3
 *   q               [batch][n][Hq][D] elements of q_dtype (float32 or bf16)
 *   block_table     [batch][max_pages] int32
 *   seq_lens        [batch] int32
 *   seqs            [nseqs] sequence indices to evaluate
 *   out             [nseqs][n][Hq][D] float64
 * Token t of sequence b is slot t % page_size of physical page
 * block_table[b][t / page_size].  Returns ORACLE_BAD_TABLE when a page id
 * the sequence needs lies outside [0, num_pages) or L is outside [n,
 * page_size * max_pages].
 */
int oracle_paged_attention(const void* k_pool, const void* v_pool, int kv_dtype,
                           const float* k_scale, const float* v_scale,
                           int num_pages, int Hkv, int page_size, int D,
                           const void* q, int q_dtype,
                           const int32_t* block_table, int max_pages,
                           const int32_t* seq_lens, int batch, int n, int Hq,
                           double scale, const int32_t* seqs, int nseqs,
                           double* out);

/* As oracle_paged_attention, with a draft tree per sequence:
 * tree_mask [batch][n] (NULL = the causal chain). */
int oracle_paged_attention_tree(const void* k_pool, const void* v_pool, int kv_dtype,
                                const float* k_scale, const float* v_scale,
                                int num_pages, int Hkv, int page_size, int D,
                                const void* q, int q_dtype,
                                const int32_t* block_table, int max_pages,
                                const int32_t* seq_lens, int batch, int n, int Hq,
                                double scale, const uint64_t* tree_mask,
                                const int32_t* seqs, int nseqs, double* out);

/* Nearest E4M3 byte to x (ties to the even code), saturating at +-448; the
 * search runs over every finite code.  NaN gives 0x7F. */
uint8_t oracle_e4m3_encode(double x);

/*
 * KV append (quantize-on-write), the step before attention in a decode loop:
 * writes the n_new newest tokens of every sequence (positions L - n_new .. L-1,
 * L = seq_lens[b], which counts them) into the pool, in its layouts (K chunked,
 * V token-major; see oracle_paged_attention).
 *   k_new, v_new [batch][n_new][Hkv][D] source values, float32 or bf16 bits
 *   f32 / bf16 pools: the value rounded to the pool format (round to nearest even)
 *   E4M3 pools, per (page, kv head), K and V separately, all arithmetic in
 *   binary32 (the precision the quantised code is decided in):
 *     a page none of whose earlier slots are live gets
 *       scale = absmax(new values in it) / 448   (1 if that absmax is 0);
 *     otherwise scale = max(old scale, absmax / 448), and if it grew every
 *       earlier live byte b becomes encode(value(b) * old / scale);
 *     each new value x becomes encode(x / scale).
 * Sources: "Latency and cost in production" §10.8.2 (q = round(x / scale) +
 * zp, zp = 0 when symmetric, §10.8.3), §10.12.2 and "Batching, speculative
 * decoding, paged attention" §5.3.7 (a request's blocks fill one token at a
 * time, a new block when the last is full).
 * Returns ORACLE_BAD_TABLE for a needed page id out of range or L < n_new.
 */
int oracle_append_kv(void* k_pool, void* v_pool, int kv_dtype, float* k_scale, float* v_scale,
                     int num_pages, int Hkv, int page_size, int D,
                     const void* k_new, const void* v_new, int src_dtype,
                     const int32_t* block_table, int max_pages, const int32_t* seq_lens,
                     int batch, int n_new);

/*
 * Speculative-sampling acceptance (rejection sampling), the step after the
 * verify pass, for each sequence b of a batch:
 *   p         [batch][K+1][V] target probabilities (float32), one row per
 *             verify position (rows need not sum to exactly 1)
 *   q         [batch][K][V]   draft probabilities (float32)
 *   draft     [batch][K]      the draft tokens, in [0, V)
 *   u_accept  [batch][K]      uniforms in [0, 1), one per acceptance test
 *   u_sample  [batch]         a uniform in [0, 1) for the one token sampled
 *   tokens    [batch][K+1]    out: accepted drafts, the sampled token, then -1
 *   accepted  [batch]         out: number of accepted drafts (0 .. K)
 * Draft i (x = draft[b][i]) is accepted with probability min(1, p(x)/q(x)):
 * iff u_accept[b][i] * q[b][i][x] < p[b][i][x] (exact in binary64, because
 * both factors have 24-bit significands).  Tests run i = 0, 1, ... and stop
 * at the first rejection, at position r.  The one sampled token comes from
 *   w = max(0, p[b][r] - q[b][r])   after a rejection at r (the residual;
 *       if it sums to 0, w = p[b][r]),
 *   w = p[b][K]                     when all K drafts are accepted (the bonus),
 * by inverse CDF: the smallest j with w_0 + ... + w_j > u_sample[b] * sum(w),
 * decided exactly: every float32 is an integer multiple of 2^-149, so the
 * weights, their sums and u * sum(w) are compared as integers (multi-limb,
 * no rounding).  A row with no mass gives -1.
 * Sources: "Latency and cost in production" §10.6.2 (accept if p >= q, else
 * with probability p/q; on rejection sample from norm(max(0, p - q)); bonus
 * token when every draft passes) and "Speculative decoding principles"
 * (7.2.1), acceptance rule (a uniform u is drawn and the draft passes iff
 * u < p/q) and residual distribution.
 * Returns ORACLE_BAD_ARG for K < 0, V < 1, a draft token outside [0, V), or
 * an entry of p or q that is negative, infinite or NaN.
 */
int oracle_rejection_sample(const float* p, const float* q, const int32_t* draft,
                            const float* u_accept, const float* u_sample,
                            int batch, int K, int V, int32_t* tokens, int32_t* accepted);

#ifdef __cplusplus
}
#endif

#endif
