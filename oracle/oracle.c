/*
 * oracle.c -- float64 CPU reference for paged GQA decode / verify attention.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * CPU-baseline leg of the benchmark; never by the product path.  Every step
 * is the plain definition (full softmax, no tiling, no reordering); the
 * sources for each function are listed in oracle.h.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* bfloat16 is the upper half of an IEEE binary32: widen and reinterpret. */
double oracle_bf16_value(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/*
 * OCP 8-bit floating point, E4M3 variant: 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
 * (mantissa/8 * 2^-6); there are no infinities and S.1111.111 is NaN.
 */
double oracle_e4m3_value(uint8_t byte)
{
    int sign = (byte >> 7) & 1;
    int e = (byte >> 3) & 0xF;
    int m = byte & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* is key t visible to row i?  (mask == NULL: the causal chain) */
static int visible(int t, int i, int L, int n, const uint64_t* tree_mask)
{
    const int first_new = L - n;            /* the n query rows are the last n tokens */
    if (t < first_new)
        return 1;
    if (!tree_mask)
        return t <= first_new + i;
    return (int)((tree_mask[i] >> (t - first_new)) & 1u);
}

static int attention_rows(const double* q, const double* k, const double* v,
                          int L, int n, int Hq, int Hkv, int D, double scale,
                          const uint64_t* tree_mask, double* out)
{
    if (n < 1 || L < n || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || D < 1)
        return ORACLE_BAD_ARG;
    if (tree_mask && n > 64)
        return ORACLE_BAD_ARG;
    const int G = Hq / Hkv;
    double* z = (double*)malloc(sizeof(double) * (size_t)L);
    int* vis = (int*)malloc(sizeof(int) * (size_t)L);
    if (!z || !vis) {
        free(z); free(vis);
        return ORACLE_NO_MEMORY;
    }

    int rc = ORACLE_OK;
    for (int i = 0; i < n && rc == ORACLE_OK; ++i) {
        int count = 0;
        for (int t = 0; t < L; ++t) {
            vis[t] = visible(t, i, L, n, tree_mask);
            count += vis[t];
        }
        if (count == 0) {
            rc = ORACLE_BAD_ARG;
            break;
        }
        for (int h = 0; h < Hq; ++h) {
            const int hk = h / G;
            const double* qr = q + ((size_t)i * Hq + h) * D;
            double zmax = -INFINITY;
            for (int t = 0; t < L; ++t) {
                if (!vis[t])
                    continue;
                const double* kt = k + ((size_t)t * Hkv + hk) * D;
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += qr[d] * kt[d];
                z[t] = scale * dot;
                if (z[t] > zmax)
                    zmax = z[t];
            }
            double denom = 0.0;
            for (int t = 0; t < L; ++t) {
                if (!vis[t])
                    continue;
                z[t] = exp(z[t] - zmax);
                denom += z[t];
            }
            double* o = out + ((size_t)i * Hq + h) * D;
            for (int d = 0; d < D; ++d) {
                double acc = 0.0;
                for (int t = 0; t < L; ++t)
                    if (vis[t])
                        acc += z[t] * v[((size_t)t * Hkv + hk) * D + d];
                o[d] = acc / denom;
            }
        }
    }
    free(z);
    free(vis);
    return rc;
}

int oracle_attention(const double* q, const double* k, const double* v,
                     int L, int n, int Hq, int Hkv, int D, double scale,
                     double* out)
{
    /* row i is token L - n + i and sees itself and every earlier key */
    return attention_rows(q, k, v, L, n, Hq, Hkv, D, scale, NULL, out);
}

int oracle_attention_tree(const double* q, const double* k, const double* v,
                          int L, int n, int Hq, int Hkv, int D, double scale,
                          const uint64_t* tree_mask, double* out)
{
    if (!tree_mask)
        return ORACLE_BAD_ARG;
    return attention_rows(q, k, v, L, n, Hq, Hkv, D, scale, tree_mask, out);
}

/* bytes of one element of the given code */
static int element_bytes(int code)
{
    return code == ORACLE_F32 ? 4 : code == ORACLE_BF16 ? 2 : 1;
}

/* value of element `idx` of an array of the given element code */
static double element(const void* base, int code, size_t idx)
{
    switch (code) {
    case ORACLE_F32:
        return (double)((const float*)base)[idx];
    case ORACLE_BF16:
        return oracle_bf16_value(((const uint16_t*)base)[idx]);
    case ORACLE_E4M3:
        return oracle_e4m3_value(((const uint8_t*)base)[idx]);
    default:
        return NAN;
    }
}

int oracle_paged_attention_tree(const void* k_pool, const void* v_pool, int kv_dtype,
                                const float* k_scale, const float* v_scale,
                                int num_pages, int Hkv, int page_size, int D,
                                const void* q, int q_dtype,
                                const int32_t* block_table, int max_pages,
                                const int32_t* seq_lens, int batch, int n, int Hq,
                                double scale, const uint64_t* tree_mask,
                                const int32_t* seqs, int nseqs, double* out)
{
    if (!k_pool || !v_pool || !q || !block_table || !seq_lens || !out || !seqs)
        return ORACLE_BAD_ARG;
    if (kv_dtype != ORACLE_F32 && kv_dtype != ORACLE_BF16 && kv_dtype != ORACLE_E4M3)
        return ORACLE_BAD_ARG;
    if (q_dtype != ORACLE_F32 && q_dtype != ORACLE_BF16)
        return ORACLE_BAD_ARG;
    if (kv_dtype == ORACLE_E4M3 && (!k_scale || !v_scale))
        return ORACLE_BAD_ARG;
    if (num_pages < 1 || Hkv < 1 || page_size < 1 || D < 1 || max_pages < 1 ||
        batch < 1 || n < 1 || Hq < Hkv || Hq % Hkv != 0 || nseqs < 0)
        return ORACLE_BAD_ARG;
    /* K slabs hold the head dimension in chunks of 16 bytes = x elements */
    const int x = 16 / element_bytes(kv_dtype);
    if (D % x != 0)
        return ORACLE_BAD_ARG;

    for (int s = 0; s < nseqs; ++s) {
        const int b = seqs[s];
        if (b < 0 || b >= batch)
            return ORACLE_BAD_ARG;
        const int L = seq_lens[b];
        if (L < n || L > page_size * max_pages)
            return ORACLE_BAD_TABLE;

        double* kc = (double*)malloc(sizeof(double) * (size_t)L * Hkv * D);
        double* vc = (double*)malloc(sizeof(double) * (size_t)L * Hkv * D);
        double* qc = (double*)malloc(sizeof(double) * (size_t)n * Hq * D);
        if (!kc || !vc || !qc) {
            free(kc); free(vc); free(qc);
            return ORACLE_NO_MEMORY;
        }

        /* follow the block table: logical token t -> (page, slot) */
        int bad = 0;
        for (int t = 0; t < L && !bad; ++t) {
            const int page = block_table[(size_t)b * max_pages + t / page_size];
            const int slot = t % page_size;
            if (page < 0 || page >= num_pages) {
                bad = 1;
                break;
            }
            for (int hk = 0; hk < Hkv; ++hk) {
                double ks = 1.0, vs = 1.0;
                if (kv_dtype == ORACLE_E4M3) {
                    ks = (double)k_scale[(size_t)page * Hkv + hk];
                    vs = (double)v_scale[(size_t)page * Hkv + hk];
                }
                const size_t slab = ((size_t)page * Hkv + hk) * page_size * D;
                const size_t vrow = slab + (size_t)slot * D;
                const size_t dst = ((size_t)t * Hkv + hk) * D;
                for (int d = 0; d < D; ++d) {
                    const size_t kidx = slab + ((size_t)(d / x) * page_size + slot) * x + d % x;
                    kc[dst + d] = element(k_pool, kv_dtype, kidx) * ks;
                    vc[dst + d] = element(v_pool, kv_dtype, vrow + d) * vs;
                }
            }
        }
        for (size_t e = 0; e < (size_t)n * Hq * D; ++e)
            qc[e] = element(q, q_dtype, (size_t)b * n * Hq * D + e);

        int rc = bad ? ORACLE_BAD_TABLE
                     : attention_rows(qc, kc, vc, L, n, Hq, Hkv, D, scale,
                                      tree_mask ? tree_mask + (size_t)b * n : NULL,
                                      out + (size_t)s * n * Hq * D);
        free(kc); free(vc); free(qc);
        if (rc != ORACLE_OK)
            return rc;
    }
    return ORACLE_OK;
}

int oracle_paged_attention(const void* k_pool, const void* v_pool, int kv_dtype,
                           const float* k_scale, const float* v_scale,
                           int num_pages, int Hkv, int page_size, int D,
                           const void* q, int q_dtype,
                           const int32_t* block_table, int max_pages,
                           const int32_t* seq_lens, int batch, int n, int Hq,
                           double scale, const int32_t* seqs, int nseqs,
                           double* out)
{
    return oracle_paged_attention_tree(k_pool, v_pool, kv_dtype, k_scale, v_scale, num_pages,
                                       Hkv, page_size, D, q, q_dtype, block_table, max_pages,
                                       seq_lens, batch, n, Hq, scale, NULL, seqs, nseqs, out);
}

/* ------------------------------------------------------------------------ */
/* KV append                                                                  */
/* ------------------------------------------------------------------------ */

uint8_t oracle_e4m3_encode(double x)
{
    if (isnan(x))
        return 0x7F;
    const double a = fabs(x);
    int best = 0;
    double best_err = INFINITY;
    for (int code = 0; code <= 0x7E; ++code) {       /* every finite magnitude */
        const double err = fabs(oracle_e4m3_value((uint8_t)code) - a);
        if (err < best_err || (err == best_err && (code & 1) == 0)) {
            best = code;
            best_err = err;
        }
    }
    return (uint8_t)(best | (signbit(x) ? 0x80 : 0));
}

/* bfloat16 bits nearest to a binary32 value (ties to even); NaN -> 0x7FC0 */
static uint16_t to_bf16(float f)
{
    if (isnan(f))
        return 0x7FC0;
    /* candidates: truncate toward zero and the next pattern up in magnitude */
    uint32_t w;
    memcpy(&w, &f, sizeof w);
    const uint16_t lo = (uint16_t)(w >> 16);
    const uint16_t hi = (uint16_t)(lo + 1);
    const double dl = fabs(oracle_bf16_value(lo) - (double)f);
    const double dh = fabs(oracle_bf16_value(hi) - (double)f);
    if (dl < dh || (dl == dh && (lo & 1) == 0))
        return lo;
    return hi;
}

static float source_value(const void* base, int code, size_t idx)
{
    return (float)element(base, code, idx);
}

int oracle_append_kv(void* k_pool, void* v_pool, int kv_dtype, float* k_scale, float* v_scale,
                     int num_pages, int Hkv, int page_size, int D,
                     const void* k_new, const void* v_new, int src_dtype,
                     const int32_t* block_table, int max_pages, const int32_t* seq_lens,
                     int batch, int n_new)
{
    if (!k_pool || !v_pool || !k_new || !v_new || !block_table || !seq_lens)
        return ORACLE_BAD_ARG;
    if (kv_dtype != ORACLE_F32 && kv_dtype != ORACLE_BF16 && kv_dtype != ORACLE_E4M3)
        return ORACLE_BAD_ARG;
    if (src_dtype != ORACLE_F32 && src_dtype != ORACLE_BF16)
        return ORACLE_BAD_ARG;
    if (kv_dtype == ORACLE_F32 && src_dtype != ORACLE_F32)
        return ORACLE_BAD_ARG;
    if (kv_dtype == ORACLE_E4M3 && (!k_scale || !v_scale))
        return ORACLE_BAD_ARG;
    if (num_pages < 1 || Hkv < 1 || page_size < 1 || D < 1 || max_pages < 1 || batch < 1 ||
        n_new < 1)
        return ORACLE_BAD_ARG;
    const int x = 16 / element_bytes(kv_dtype);
    if (D % x != 0)
        return ORACLE_BAD_ARG;

    for (int b = 0; b < batch; ++b) {
        const int L = seq_lens[b];
        if (L < n_new || L > page_size * max_pages)
            return ORACLE_BAD_TABLE;
        const int first = L - n_new;
        for (int p = first / page_size; p <= (L - 1) / page_size; ++p) {
            const int page = block_table[(size_t)b * max_pages + p];
            if (page < 0 || page >= num_pages)
                return ORACLE_BAD_TABLE;
            const int s0 = p * page_size;                         /* first token of the page */
            const int lo = first > s0 ? first - s0 : 0;           /* first new slot */
            const int hi = (L - s0 < page_size) ? L - s0 : page_size;   /* one past the last */
            for (int hk = 0; hk < Hkv; ++hk) {
                const size_t slab = ((size_t)page * Hkv + hk) * page_size * D;
                for (int which = 0; which < 2; ++which) {          /* 0: K, 1: V */
                    void* pool = which ? v_pool : k_pool;
                    const void* src = which ? v_new : k_new;
                    float* scales = which ? v_scale : k_scale;
                    /* slab index of (slot, d) */
                    #define IDX(slot, d) (which ? slab + (size_t)(slot) * D + (d) \
                        : slab + ((size_t)((d) / x) * page_size + (slot)) * x + (d) % x)
                    #define SRC(slot, d) ((((size_t)b * n_new + (s0 + (slot) - first)) * Hkv + hk) \
                        * D + (d))
                    if (kv_dtype != ORACLE_E4M3) {
                        for (int slot = lo; slot < hi; ++slot)
                            for (int d = 0; d < D; ++d) {
                                const float v = source_value(src, src_dtype, SRC(slot, d));
                                if (kv_dtype == ORACLE_F32)
                                    ((float*)pool)[IDX(slot, d)] = v;
                                else
                                    ((uint16_t*)pool)[IDX(slot, d)] = to_bf16(v);
                            }
                        continue;
                    }
                    uint8_t* bytes = (uint8_t*)pool;
                    float amax = 0.0f;
                    for (int slot = lo; slot < hi; ++slot)
                        for (int d = 0; d < D; ++d) {
                            const float v = fabsf(source_value(src, src_dtype, SRC(slot, d)));
                            if (v > amax)
                                amax = v;
                        }
                    const float cand = amax / 448.0f;
                    float* sc = &scales[(size_t)page * Hkv + hk];
                    float scale;
                    if (lo == 0) {                                  /* no earlier live slot */
                        scale = amax > 0.0f ? cand : 1.0f;
                    } else {
                        const float old = *sc;
                        scale = cand > old ? cand : old;
                        if (scale != old)
                            for (int slot = 0; slot < lo; ++slot)
                                for (int d = 0; d < D; ++d) {
                                    const size_t i = IDX(slot, d);
                                    const float val = (float)oracle_e4m3_value(bytes[i]) * old;
                                    bytes[i] = oracle_e4m3_encode((double)(val / scale));
                                }
                    }
                    for (int slot = lo; slot < hi; ++slot)
                        for (int d = 0; d < D; ++d) {
                            const float v = source_value(src, src_dtype, SRC(slot, d));
                            bytes[IDX(slot, d)] = oracle_e4m3_encode((double)(v / scale));
                        }
                    *sc = scale;
                    #undef IDX
                    #undef SRC
                }
            }
        }
    }
    return ORACLE_OK;
}

/* ---- exact integers for the draw --------------------------------------
 * Every float32 is an integer multiple of 2^-149, below 2^128.  A weight,
 * a running sum of up to 2^20 weights, and the products compared below all
 * fit in 16 little-endian 32-bit limbs (512 bits). */
#define BIG_LIMBS 16
typedef struct { uint32_t d[BIG_LIMBS]; } big;

static void big_zero(big* a) { memset(a, 0, sizeof *a); }

static int big_is_zero(const big* a)
{
    for (int i = 0; i < BIG_LIMBS; ++i)
        if (a->d[i]) return 0;
    return 1;
}

/* a = |x| / 2^-149 (x finite); the bits of x give it exactly: significand
 * (with the hidden bit for normal numbers) times 2^(exponent field - 1) */
static void big_from_f32(big* a, float x)
{
    uint32_t bits;
    memcpy(&bits, &x, sizeof bits);
    const uint32_t e = (bits >> 23) & 0xffu;
    const uint64_t m = (bits & 0x7fffffu) | (e ? 0x800000u : 0u);
    const uint32_t s = e ? e - 1 : 0;
    big_zero(a);
    const uint64_t shifted = m << (s % 32);          /* at most 55 bits */
    a->d[s / 32] = (uint32_t)shifted;
    if (s / 32 + 1 < BIG_LIMBS) a->d[s / 32 + 1] = (uint32_t)(shifted >> 32);
}

static int big_cmp(const big* a, const big* b)
{
    for (int i = BIG_LIMBS - 1; i >= 0; --i)
        if (a->d[i] != b->d[i]) return a->d[i] > b->d[i] ? 1 : -1;
    return 0;
}

static void big_add(big* a, const big* b)           /* a += b */
{
    uint64_t carry = 0;
    for (int i = 0; i < BIG_LIMBS; ++i) {
        const uint64_t t = (uint64_t)a->d[i] + b->d[i] + carry;
        a->d[i] = (uint32_t)t;
        carry = t >> 32;
    }
}

static void big_sub(big* a, const big* b)           /* a -= b, for a >= b */
{
    int64_t borrow = 0;
    for (int i = 0; i < BIG_LIMBS; ++i) {
        int64_t t = (int64_t)a->d[i] - b->d[i] - borrow;
        borrow = t < 0;
        a->d[i] = (uint32_t)(t + (borrow ? ((int64_t)1 << 32) : 0));
    }
}

static void big_shl(big* out, const big* a, int s)  /* out = a * 2^s */
{
    big r;
    big_zero(&r);
    for (int i = BIG_LIMBS - 1; i >= 0; --i) {
        const int j = i - s / 32;
        if (j < 0) continue;
        uint64_t v = (uint64_t)a->d[j] << (s % 32);
        if (s % 32 && j > 0) v |= (uint64_t)a->d[j - 1] >> (32 - s % 32);
        r.d[i] = (uint32_t)v;
    }
    *out = r;
}

static void big_mul_small(big* out, const big* a, uint32_t m)   /* out = a * m */
{
    uint64_t carry = 0;
    for (int i = 0; i < BIG_LIMBS; ++i) {
        const uint64_t t = (uint64_t)a->d[i] * m + carry;
        out->d[i] = (uint32_t)t;
        carry = t >> 32;
    }
}

/* Inverse-CDF draw from the non-negative weights w[0..V): the smallest j with
 * w_0 + ... + w_j > u * (w_0 + ... + w_{V-1}), decided exactly.  With u = U *
 * 2^-149 (U an integer, from u's bits), the test is
 * (w_0 + ... + w_j) * 2^149 > U * total, in integers.  -1 if the total is 0. */
static int32_t draw(const big* w, int V, float u)
{
    big total, rhs, run, lhs;
    big_zero(&total);
    for (int j = 0; j < V; ++j) big_add(&total, &w[j]);
    if (big_is_zero(&total)) return -1;
    /* rhs = U * total: u's significand times total, shifted by u's exponent
     * (U < 2^149 because 0 <= u < 1) */
    uint32_t ubits;
    memcpy(&ubits, &u, sizeof ubits);
    const uint32_t e = (ubits >> 23) & 0xffu;
    const uint32_t m = (ubits & 0x7fffffu) | (e ? 0x800000u : 0u);
    big_mul_small(&rhs, &total, m);
    big_shl(&rhs, &rhs, e ? (int)e - 1 : 0);
    big_zero(&run);
    for (int j = 0; j < V; ++j) {
        big_add(&run, &w[j]);
        big_shl(&lhs, &run, 149);
        if (big_cmp(&lhs, &rhs) > 0) return j;
    }
    return -1;   /* unreachable: run ends at total and total * 2^149 > U * total */
}

int oracle_rejection_sample(const float* p, const float* q, const int32_t* draft,
                            const float* u_accept, const float* u_sample,
                            int batch, int K, int V, int32_t* tokens, int32_t* accepted)
{
    if (batch < 0 || K < 0 || V < 1) return ORACLE_BAD_ARG;
    for (size_t i = 0; i < (size_t)batch * K; ++i)
        if (draft[i] < 0 || draft[i] >= V) return ORACLE_BAD_ARG;
    for (size_t i = 0; i < (size_t)batch * (K + 1) * V; ++i)
        if (!(p[i] >= 0.0f) || isinf(p[i])) return ORACLE_BAD_ARG;
    for (size_t i = 0; i < (size_t)batch * K * V; ++i)
        if (!(q[i] >= 0.0f) || isinf(q[i])) return ORACLE_BAD_ARG;
    big* w = (big*)malloc(sizeof(big) * (size_t)V);
    if (!w) return ORACLE_NO_MEMORY;
    for (int b = 0; b < batch; ++b) {
        const float* pb = p + (size_t)b * (K + 1) * V;
        const float* qb = q + (size_t)b * K * V;
        int32_t* out = tokens + (size_t)b * (K + 1);
        /* acceptance tests, in order, up to the first rejection */
        int r = 0;
        while (r < K) {
            const int x = draft[(size_t)b * K + r];
            const double px = pb[(size_t)r * V + x], qx = qb[(size_t)r * V + x];
            if (!((double)u_accept[(size_t)b * K + r] * qx < px)) break;
            out[r] = x;
            ++r;
        }
        accepted[b] = r;
        /* the one sampled token: residual after a rejection, else the bonus */
        const float* pr = pb + (size_t)r * V;
        int32_t tok;
        if (r < K) {
            const float* qr = qb + (size_t)r * V;
            for (int j = 0; j < V; ++j) {      /* w = max(0, p - q), exactly */
                big qj;
                big_from_f32(&w[j], pr[j]);
                big_from_f32(&qj, qr[j]);
                if (big_cmp(&w[j], &qj) > 0) big_sub(&w[j], &qj);
                else big_zero(&w[j]);
            }
            tok = draw(w, V, u_sample[b]);
            if (tok < 0) {                      /* no residual mass: p itself */
                for (int j = 0; j < V; ++j) big_from_f32(&w[j], pr[j]);
                tok = draw(w, V, u_sample[b]);
            }
        } else {
            for (int j = 0; j < V; ++j) big_from_f32(&w[j], pr[j]);
            tok = draw(w, V, u_sample[b]);
        }
        out[r] = tok;
        for (int i = r + 1; i <= K; ++i) out[i] = -1;
    }
    free(w);
    return ORACLE_OK;
}
