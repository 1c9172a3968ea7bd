// spec_sample.hip -- speculative-sampling acceptance (rejection sampling) on
// MI355X (gfx950), the step after the verify pass.
//
// The operation is defined in include/paged_attn.h (paged_attn_rejection_sample).
// Sources: "Latency and cost in production" §10.6.2 (a draft token passes
// when p >= q and otherwise with probability p/q; after a rejection the
// replacement comes from norm(max(0, p - q)); when every draft passes, the
// target's extra position gives a bonus token) and "Speculative decoding
// principles" (7.2.1), acceptance rule and residual distribution (the test is
// one uniform u with u < p/q; the residual is a transient distribution
// computed at the rejected position only).
//
// Design: the work is one pass over one vocabulary row per sequence (the
// residual's p and q rows, or the bonus row), so it is HBM-bound; the rest is
// K scalar lookups.  The draw is decided exactly: every float32 is an integer
// multiple of 2^-149, and with entries below 2^22 a row of up to 2^20 weights
// sums to an integer below 2^192, held as six 32-bit columns.  Two kernels,
// each with four waves per workgroup and 16 consecutive entries per thread:
//  * pass 1, one workgroup per (4096-entry chunk of the row, sequence): finds
//    the first rejection (one lane per draft, a wave ballot); each thread
//    loads 16 entries straight into registers (coalesced 16-byte loads, all in
//    flight at once: a sum does not care which thread holds which entry) and
//    adds each entry, as an integer piece below 2^56 times 2^(32 k), into its
//    bucket k (int64 words in LDS, one set per thread): where p > q, p and q
//    into the two sets whose difference is the residual, elsewhere p into a
//    third set, which with the first gives the sum of p.  The buckets become
//    columns, the columns are summed over the workgroup, and the chunk's exact
//    sums of the sampling weights and of p are written;
//  * pass 2, one workgroup per sequence: scans the chunk sums exactly, takes
//    F = floor(u * total) (the running sum is an integer, so it exceeds u *
//    total iff it exceeds F), finds the first chunk whose running sum exceeds
//    F, re-reads that chunk, scans the threads' 16-entry sums to find the
//    thread, and scans that thread's 16 entries (one per lane, from LDS) to
//    find the token.
// A running sum rises only on positive weights, so a zero-weight token is
// never drawn.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "paged_attn.h"
#include "status.h"

#define PA_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kLanes = 64;                     // one wave
constexpr int kWaves = 4;                      // waves per workgroup
constexpr int kThreads = kLanes * kWaves;
constexpr int kPerThread = 16;                 // consecutive entries held by one thread
constexpr int kChunk = kThreads * kPerThread;  // vocabulary entries per chunk (one workgroup)
constexpr int kMaxDrafts = kLanes;
constexpr int kMaxChunks = 256;                // vocabulary up to 1,048,576
constexpr int kBlocks = kMaxChunks / kLanes;   // chunks per lane in the pass-2 scan
constexpr int kCols = 6;                       // 32-bit columns of an exact sum
constexpr int kBuckets = 5;                    // 32-bit exponent windows below 2^22
constexpr int kSlots = kBuckets + 1;           // and one slot that takes what is not added
constexpr int kRecord = 2 * kCols;             // uint32 per chunk: weight sum, p sum
constexpr int kEntryStride = kThreads + 1;     // LDS row of the entry transpose (bank skew)

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64;

struct SampleArgs {
    const float* p;          // [B][K+1][V]
    const float* q;          // [B][K][V]
    const int32_t* draft;    // [B][K]
    const float* u_accept;   // [B][K]
    const float* u_sample;   // [B]
    int32_t* tokens;         // [B][K+1]
    int32_t* accepted;       // [B]
    uint32_t* chunk_sums;    // [B][chunks][2][6]: exact sums of the weights and of p
    int32_t* first_rej;      // [B]: index of the first rejected draft (K if none)
    int32_t K, V, chunks;
    int32_t vec4;            // rows are 16-byte aligned (V % 4 == 0, aligned bases)
};

// an exact non-negative integer (units of 2^-149) as 32-bit columns in 64-bit
// words; normalised when every word is below 2^32
struct Cols {
    u64 c[kCols];
};

__device__ __forceinline__ Cols zero_cols()
{
    Cols r;
#pragma unroll
    for (int i = 0; i < kCols; ++i) r.c[i] = 0ull;
    return r;
}

// x in [0, 2^22) as x / 2^-149 = piece * 2^(32 k): piece = significand (with
// the hidden bit for normal numbers) shifted by the low five bits of
// max(exponent field - 1, 0).  The exponent field is clamped so that values
// outside the contract keep k in range (their token is then unspecified).
__device__ __forceinline__ void split(float x, uint32_t& k, u64& piece)
{
    const uint32_t b = __float_as_uint(x);
    const uint32_t e = min(b >> 23, 148u);
    const uint32_t h = min(e, 1u);
    const uint32_t m = (b & 0x7fffffu) | (h << 23);
    const uint32_t s = e - h;
    k = s >> 5;
    piece = (u64)m << (s & 31);
}

// the integer of x as columns (piece in columns k and k + 1)
__device__ __forceinline__ Cols cols_of(float x)
{
    uint32_t k;
    u64 piece;
    split(x, k, piece);
    Cols r;
#pragma unroll
    for (int i = 0; i < kCols; ++i)
        r.c[i] = i == (int)k ? (piece & 0xffffffffull) : i == (int)k + 1 ? (piece >> 32) : 0ull;
    return r;
}

// carry the columns so that each is below 2^32 (the value must be below 2^192)
__device__ __forceinline__ void normalise(Cols& a)
{
    u64 carry = 0;
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
        const u64 t = a.c[i] + carry;
        a.c[i] = t & 0xffffffffull;
        carry = t >> 32;
    }
}

// a - b for normalised a >= b
__device__ __forceinline__ Cols minus(const Cols& a, const Cols& b)
{
    Cols r;
    u64 borrow = 0;
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
        const u64 t = a.c[i] - b.c[i] - borrow;           // modulo 2^64
        borrow = (t >> 63) & 1ull;
        r.c[i] = t & 0xffffffffull;
    }
    return r;
}

__device__ __forceinline__ void plus_eq(Cols& a, const Cols& b)
{
#pragma unroll
    for (int i = 0; i < kCols; ++i) a.c[i] += b.c[i];
}

// a > b for normalised a, b
__device__ __forceinline__ bool greater(const Cols& a, const Cols& b)
{
    bool res = false, done = false;
#pragma unroll
    for (int i = kCols - 1; i >= 0; --i) {
        const bool diff = a.c[i] != b.c[i];
        res = (!done && diff) ? a.c[i] > b.c[i] : res;
        done = done || diff;
    }
    return res;
}

__device__ __forceinline__ bool is_zero(const Cols& a)
{
    bool z = true;
#pragma unroll
    for (int i = 0; i < kCols; ++i) z = z && a.c[i] == 0ull;
    return z;
}

__device__ __forceinline__ u64 readlane64(u64 x, int l)
{
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)x, l);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(x >> 32), l);
    return ((u64)hi << 32) | lo;
}

// Inclusive prefix sum over the wave's lanes with DPP moves (no LDS): within
// each row of 16 lanes by shifts of 1, 2, 4 and 8 (lanes shifted in from
// outside the row read 0), then row 0's total into row 1 and row 2's into
// row 3, then rows 0-1's total into rows 2 and 3.  The total must fit 32 bits.
__device__ __forceinline__ uint32_t dpp_scan(uint32_t x)
{
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// inclusive scan over the wave's lanes of normalised columns (each below
// 2^32): 16-bit halves scanned separately, so no partial sum leaves 32 bits
__device__ __forceinline__ void wave_scan(Cols& a)
{
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
        const uint32_t lo = dpp_scan((uint32_t)(a.c[i] & 0xffffu));
        const uint32_t hi = dpp_scan((uint32_t)(a.c[i] >> 16));
        a.c[i] = (u64)lo + ((u64)hi << 16);
    }
}

__device__ __forceinline__ Cols read_lane(const Cols& a, int l)
{
    Cols r;
#pragma unroll
    for (int i = 0; i < kCols; ++i) r.c[i] = readlane64(a.c[i], l);
    return r;
}

// floor(u * t) for normalised t and u in [0, 1): u = m * 2^(s - 149)
__device__ __forceinline__ Cols times_u(const Cols& t, float u)
{
    const uint32_t b = __float_as_uint(u);
    const uint32_t e = min(b >> 23, 148u);
    const uint32_t h = min(e, 1u);
    const u64 m = (b & 0x7fffffu) | (h << 23);
    const int sh = 149 - (int)(e - h);                    // >= 1
    u64 prod[kCols + 1];
    u64 carry = 0;
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
        const u64 x = t.c[i] * m + carry;                 // < 2^56 + 2^24
        prod[i] = x & 0xffffffffull;
        carry = x >> 32;
    }
    prod[kCols] = carry;
    const int qw = sh >> 5, rb = sh & 31;
    Cols f;
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
        u64 lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j <= kCols; ++j) {
            lo = j == i + qw ? prod[j] : lo;
            hi = j == i + qw + 1 ? prod[j] : hi;
        }
        f.c[i] = ((lo >> rb) | (hi << (32 - rb))) & 0xffffffffull;
    }
    return f;
}

// Index of the first rejected draft of sequence b (K if all pass), in every
// lane of the calling wave.  Draft i passes iff u * q(x) < p(x), exact in
// binary64 (both factors carry 24-bit significands).
__device__ __forceinline__ int first_rejection(const SampleArgs& a, int b, int lane)
{
    bool rejected = false;
    if (lane < a.K) {
        const int64_t di = (int64_t)b * a.K + lane;
        const int x = min(max(a.draft[di], 0), a.V - 1);
        const float px = a.p[((int64_t)b * (a.K + 1) + lane) * a.V + x];
        const float qx = a.q[di * a.V + x];
        rejected = !((double)a.u_accept[di] * (double)qx < (double)px);
    }
    const uint64_t m = __ballot(rejected);
    return m ? __ffsll((unsigned long long)m) - 1 : a.K;
}

// Entries [j0, j0 + 16) of a row into registers (0 past the end of the row);
// all loads are issued before any is used.
__device__ __forceinline__ void load_run(const float* row, int j0, int V, bool vec4,
                                         float (&x)[kPerThread])
{
    if (vec4 && j0 + kPerThread <= V) {
        const f32x4* s = reinterpret_cast<const f32x4*>(row + j0);
#pragma unroll
        for (int i = 0; i < kPerThread / 4; ++i) {
            const f32x4 v = s[i];
            x[4 * i] = v.x;
            x[4 * i + 1] = v.y;
            x[4 * i + 2] = v.z;
            x[4 * i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int j = j0 + i;
            const float v = row[min(j, V - 1)];
            x[i] = j < V ? v : 0.f;
        }
    }
}

// LDS buckets of one workgroup: [set][slot][thread]; set 0 sums p where p > q
// (all p for the bonus row), set 1 p where p <= q, set 2 q where p > q; slot
// kBuckets takes the entries a set does not count.  The residual is set 0 -
// set 2, the sum of p set 0 + set 1.
struct Buckets {
    u64 w[3][kSlots][kThreads];
};

typedef __attribute__((address_space(3))) u64 lds_u64;

// word `idx` of the buckets += v (an LDS atomic with no return: 32-bit address)
__device__ __forceinline__ void bucket_add(Buckets& bk, uint32_t idx, u64 v)
{
    lds_u64* base = (lds_u64*)(&bk.w[0][0][0]);
    __hip_atomic_fetch_add(base + idx, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ uint32_t slot(int set, uint32_t k, int tid)
{
    return ((uint32_t)set * kSlots + k) * kThreads + (uint32_t)tid;
}

// Exact sums of a thread's 16 entries: the sampling weights (max(0, p - q)
// when `residual`, else p) and, when `with_p`, p itself (else a copy of the
// weights).
template <bool WITH_P>
__device__ __forceinline__ void run_sums(const float (&xp)[kPerThread],
                                         const float (&xq)[kPerThread], bool residual,
                                         Buckets& bk, int tid, Cols& w, Cols& ps)
{
#pragma unroll
    for (int st = 0; st < 3; ++st)
#pragma unroll
        for (int k = 0; k < kBuckets; ++k) bk.w[st][k][tid] = 0ull;
    if (residual) {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            uint32_t kp, kq;
            u64 pp, pq;
            split(xp[i], kp, pp);
            split(xq[i], kq, pq);
            const bool gt = xp[i] > xq[i];
            bucket_add(bk, slot(gt ? 0 : 1, (WITH_P || gt) ? kp : kBuckets, tid), pp);
            bucket_add(bk, slot(2, gt ? kq : kBuckets, tid), pq);
        }
    } else {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            uint32_t kp;
            u64 pp;
            split(xp[i], kp, pp);
            bucket_add(bk, slot(0, kp, tid), pp);
        }
    }
    // buckets to columns; the residual's buckets are differences (signed), its
    // total is not
    int64_t cw = 0, cp = 0;
#pragma unroll
    for (int k = 0; k < kBuckets; ++k) {
        const u64 add = bk.w[0][k][tid];
        const u64 sub = residual ? bk.w[2][k][tid] : 0ull;
        const int64_t t = (int64_t)(add - sub) + cw;
        w.c[k] = (u64)(uint32_t)t;
        cw = t >> 32;
        if (WITH_P) {
            const u64 pk = bk.w[0][k][tid] + (residual ? bk.w[1][k][tid] : 0ull);
            const int64_t tp = (int64_t)pk + cp;
            ps.c[k] = (u64)(uint32_t)tp;
            cp = tp >> 32;
        }
    }
    w.c[kBuckets] = (u64)cw;
    ps.c[kBuckets] = (u64)cp;
    if (!WITH_P || !residual) ps = w;
}

// Rows of sequence b at position r: p, and q when r is a rejected draft.
__device__ __forceinline__ const float* p_row(const SampleArgs& a, int b, int r)
{
    return a.p + ((int64_t)b * (a.K + 1) + r) * a.V;
}
__device__ __forceinline__ const float* q_row(const SampleArgs& a, int b, int r)
{
    return a.q + ((int64_t)b * a.K + r) * a.V;
}

__device__ __forceinline__ void load_rows(const SampleArgs& a, int b, int r, bool residual,
                                          int j0, float (&xp)[kPerThread],
                                          float (&xq)[kPerThread])
{
    load_run(p_row(a, b, r), j0, a.V, a.vec4, xp);
    if (residual) {
        load_run(q_row(a, b, r), j0, a.V, a.vec4, xq);
    } else {
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) xq[k] = 0.f;
    }
}

// Entries of a chunk for its sums, in coalesced order: load j of thread t
// holds entries 4 (j * 256 + t) .. + 3 of the chunk (0 past the end of the
// row); a sum does not depend on which thread holds which entry.
__device__ __forceinline__ void load_spread(const float* row, int c0, int V, bool vec4, int tid,
                                            float (&x)[kPerThread])
{
#pragma unroll
    for (int j = 0; j < kPerThread / 4; ++j) {
        const int j0 = c0 + 4 * (j * kThreads + tid);
        if (vec4 && j0 + 4 <= V) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(row + j0);
            x[4 * j] = v.x;
            x[4 * j + 1] = v.y;
            x[4 * j + 2] = v.z;
            x[4 * j + 3] = v.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = row[min(j0 + e, V - 1)];
                x[4 * j + e] = j0 + e < V ? v : 0.f;
            }
        }
    }
}

// Pass 1: one workgroup per (chunk, sequence); writes the chunk's exact sums.
__global__ __launch_bounds__(kThreads) void spec_sample_chunks(SampleArgs a)
{
    __shared__ Buckets bk;
    __shared__ u64 part[kWaves][2][kCols];
    const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & (kLanes - 1), wave = tid / kLanes;
    const int r = first_rejection(a, b, lane);
    const bool residual = r < a.K;
    float xp[kPerThread], xq[kPerThread];
    load_spread(p_row(a, b, r), c * kChunk, a.V, a.vec4, tid, xp);
    if (residual) {
        load_spread(q_row(a, b, r), c * kChunk, a.V, a.vec4, tid, xq);
    } else {
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) xq[k] = 0.f;
    }
    Cols w, ps;
    run_sums<true>(xp, xq, residual, bk, tid, w, ps);
    // column totals of each wave (lane 63 of the scans), then of the workgroup
    wave_scan(w);
    wave_scan(ps);
    if (lane == kLanes - 1) {
#pragma unroll
        for (int i = 0; i < kCols; ++i) {
            part[wave][0][i] = w.c[i];
            part[wave][1][i] = ps.c[i];
        }
    }
    __syncthreads();
    // threads 0 and 1: the workgroup's sums of the weights and of p, carried
    // to 32-bit columns and stored
    if (tid < 2) {
        Cols t;
#pragma unroll
        for (int i = 0; i < kCols; ++i) {
            u64 sum = 0;
#pragma unroll
            for (int wv = 0; wv < kWaves; ++wv) sum += part[wv][tid][i];
            t.c[i] = sum;
        }
        normalise(t);
        uint32_t* out = a.chunk_sums + ((int64_t)b * a.chunks + c) * kRecord + tid * kCols;
#pragma unroll
        for (int i = 0; i < kCols; ++i) out[i] = (uint32_t)t.c[i];
    }
    if (c == 0 && tid == 0) a.first_rej[b] = r;
}

// Pass 2: one workgroup per sequence; picks the chunk, the thread's run and
// the token.  Every wave scans the chunk sums itself (the same values, so the
// same decisions); the chunk is then re-read by all four waves.
__global__ __launch_bounds__(kThreads) void spec_sample_pick(SampleArgs a)
{
    __shared__ Buckets bk;
    __shared__ float sp[kPerThread * kEntryStride];    // the chunk's entries, [entry][thread]
    __shared__ float sq[kPerThread * kEntryStride];
    __shared__ u64 wave_tot[kWaves][kCols];
    __shared__ int wave_hit[kWaves];
    __shared__ u64 f_run[kCols];                        // target inside the chosen run
    const int b = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & (kLanes - 1), wave = tid / kLanes;
    // everything the scan needs from pass 1 and the inputs, in one round trip
    const int r = a.first_rej[b];
    const float u = a.u_sample[b];
    const int32_t my_draft = lane < a.K ? a.draft[(int64_t)b * a.K + lane] : -1;
    uint32_t rec[kBlocks][kRecord];
#pragma unroll
    for (int blk = 0; blk < kBlocks; ++blk) {
        const int c = min(blk * kLanes + lane, a.chunks - 1);
        const uint32_t* in = a.chunk_sums + ((int64_t)b * a.chunks + c) * kRecord;
#pragma unroll
        for (int i = 0; i < kRecord; ++i) rec[blk][i] = blk * kLanes < a.chunks ? in[i] : 0u;
    }
    const int nblk = (a.chunks + kLanes - 1) / kLanes;

    // exact running sums over the chunks of one set (0 weights, 1 p); the total
    Cols pre[kBlocks];
    auto scan_chunks = [&](int set, Cols& total) {
        Cols carry_in = zero_cols();
#pragma unroll
        for (int blk = 0; blk < kBlocks; ++blk) {
            if (blk < nblk) {
                const bool valid = blk * kLanes + lane < a.chunks;
                Cols x;
#pragma unroll
                for (int i = 0; i < kCols; ++i) x.c[i] = valid ? rec[blk][set * kCols + i] : 0ull;
                wave_scan(x);
                plus_eq(x, carry_in);
                carry_in = read_lane(x, kLanes - 1);
                normalise(x);
                pre[blk] = x;
            }
        }
        total = carry_in;
        normalise(total);
    };
    Cols total;
    scan_chunks(0, total);
    int kind = 0;                                   // 0: the weights, 1: p (empty residual)
    if (is_zero(total) && r < a.K) {
        scan_chunks(1, total);
        kind = 1;
    }
    int32_t token = -1;
    if (!is_zero(total)) {
        const Cols f = times_u(total, u);           // the running sum must exceed this
        // the first chunk whose running sum exceeds f, and the sum before it
        int chunk = -1;
        Cols before = zero_cols();
#pragma unroll
        for (int blk = 0; blk < kBlocks; ++blk) {
            if (chunk < 0 && blk < nblk) {
                const bool valid = blk * kLanes + lane < a.chunks;
                const uint64_t m = __ballot(valid && greater(pre[blk], f));
                if (m) {
                    const int l = __ffsll((unsigned long long)m) - 1;
                    chunk = blk * kLanes + l;
                    if (l > 0) before = read_lane(pre[blk], l - 1);
                    else if (blk > 0) before = read_lane(pre[blk - 1], kLanes - 1);
                }
            }
        }
        if (chunk >= 0) {                            // the same in every wave
            const Cols f1 = minus(f, before);         // target inside the chunk
            const bool residual = r < a.K && kind == 0;
            float xp[kPerThread], xq[kPerThread];
            load_rows(a, b, r, residual, chunk * kChunk + tid * kPerThread, xp, xq);
#pragma unroll
            for (int k = 0; k < kPerThread; ++k) {
                sp[k * kEntryStride + tid] = xp[k];
                sq[k * kEntryStride + tid] = xq[k];
            }
            Cols w, ps;
            run_sums<false>(xp, xq, residual, bk, tid, w, ps);
            const Cols own = w;
            wave_scan(w);
            if (lane == kLanes - 1) {
#pragma unroll
                for (int i = 0; i < kCols; ++i) wave_tot[wave][i] = w.c[i];
            }
            __syncthreads();
            for (int wv = 0; wv < wave; ++wv)
#pragma unroll
                for (int i = 0; i < kCols; ++i) w.c[i] += wave_tot[wv][i];
            normalise(w);                             // running sum through this thread
            const uint64_t hit = __ballot(greater(w, f1));
            if (lane == 0) wave_hit[wave] = hit ? __ffsll((unsigned long long)hit) - 1 : kLanes;
            __syncthreads();
            int run = -1;
            for (int wv = 0; wv < kWaves && run < 0; ++wv)
                if (wave_hit[wv] < kLanes) run = wv * kLanes + wave_hit[wv];
            if (tid == run) {
                const Cols f2 = minus(f1, minus(w, own));   // target inside this run
#pragma unroll
                for (int i = 0; i < kCols; ++i) f_run[i] = f2.c[i];
            }
            __syncthreads();
            if (wave == 0 && run >= 0) {
                // entry `lane` of that run, its exact weight, and the running sums
                const int e = min(lane, kPerThread - 1);
                const float ep = lane < kPerThread ? sp[e * kEntryStride + run] : 0.f;
                const float eq = lane < kPerThread ? sq[e * kEntryStride + run] : 0.f;
                Cols x = cols_of(ep);
                if (residual) x = ep > eq ? minus(x, cols_of(eq)) : zero_cols();
                wave_scan(x);
                normalise(x);
                Cols f2;
#pragma unroll
                for (int i = 0; i < kCols; ++i) f2.c[i] = f_run[i];
                const uint64_t me = __ballot(greater(x, f2));
                if (me)
                    token = chunk * kChunk + run * kPerThread +
                            (__ffsll((unsigned long long)me) - 1);
            }
        }
    }
    if (wave == 0) {
        if (lane == 0) a.accepted[b] = r;
        for (int i = lane; i <= a.K; i += kLanes)   // i < r only for i == lane (r <= 64)
            a.tokens[(int64_t)b * (a.K + 1) + i] = i < r ? my_draft : i == r ? token : -1;
    }
}

int chunks_for(int32_t vocab) { return (vocab + kChunk - 1) / kChunk; }

}  // namespace

PA_API size_t paged_attn_rejection_sample_workspace_bytes(int32_t batch, int32_t vocab)
{
    if (batch < 1 || vocab < 1) return 0;
    return (size_t)batch * chunks_for(vocab) * kRecord * sizeof(uint32_t) +
           (size_t)batch * sizeof(int32_t);
}

PA_API pa_status paged_attn_rejection_sample(const float* p, const float* q, const int32_t* draft,
                                             const float* u_accept, const float* u_sample,
                                             int32_t batch, int32_t num_drafts, int32_t vocab,
                                             int32_t* tokens, int32_t* num_accepted,
                                             void* workspace, size_t workspace_bytes, void* stream)
{
    if (!p || !u_sample || !tokens || !num_accepted)
        return pa_record_error(PA_ERR_INVALID_ARG, "null p, u_sample, tokens or num_accepted");
    if (num_drafts > 0 && (!q || !draft || !u_accept))
        return pa_record_error(PA_ERR_INVALID_ARG, "null q, draft or u_accept with num_drafts > 0");
    if (batch < 1 || vocab < 1 || num_drafts < 0)
        return pa_record_error(PA_ERR_INVALID_ARG, "batch and vocab must be >= 1, num_drafts >= 0");
    if (num_drafts > kMaxDrafts)
        return pa_record_error(PA_ERR_UNSUPPORTED, "at most 64 drafts per sequence");
    if (chunks_for(vocab) > kMaxChunks)
        return pa_record_error(PA_ERR_UNSUPPORTED, "vocabulary above 1,048,576 entries");
    if (batch > 65535) return pa_record_error(PA_ERR_UNSUPPORTED, "batch above 65535");
    const size_t need = paged_attn_rejection_sample_workspace_bytes(batch, vocab);
    if (!workspace || workspace_bytes < need)
        return pa_record_error(PA_ERR_WORKSPACE, "workspace missing or too small");
    if (reinterpret_cast<uintptr_t>(workspace) % alignof(uint32_t))
        return pa_record_error(PA_ERR_INVALID_ARG, "workspace must be 4-byte aligned");
    SampleArgs a;
    a.p = p;
    a.q = q;
    a.draft = draft;
    a.u_accept = u_accept;
    a.u_sample = u_sample;
    a.tokens = tokens;
    a.accepted = num_accepted;
    a.chunk_sums = static_cast<uint32_t*>(workspace);
    a.first_rej = reinterpret_cast<int32_t*>(a.chunk_sums +
                                             (size_t)batch * chunks_for(vocab) * kRecord);
    a.K = num_drafts;
    a.V = vocab;
    a.chunks = chunks_for(vocab);
    a.vec4 = vocab % 4 == 0 && reinterpret_cast<uintptr_t>(p) % 16 == 0 &&
             reinterpret_cast<uintptr_t>(q) % 16 == 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(spec_sample_chunks, dim3((unsigned)a.chunks, (unsigned)batch),
                       dim3(kThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return pa_record_hip_error(e, "rejection sample pass 1 launch");
    hipLaunchKernelGGL(spec_sample_pick, dim3((unsigned)batch), dim3(kThreads), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return pa_record_hip_error(e, "rejection sample pass 2 launch");
    return PA_OK;
}
