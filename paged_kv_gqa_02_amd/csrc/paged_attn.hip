// paged_attn.hip -- paged GQA decode / verify attention for MI355X (gfx950).
//
// The operation is defined in include/paged_attn.h.  Sources: "Latency and
// cost in production" ch. 10 (§10.3.1 attention over every earlier key,
// §10.1.2 softmax / online softmax / GQA groups, §10.4.2 block table,
// §10.8.2-§10.8.3 symmetric scale); "Batching, speculative decoding, paged
// attention" §5.3.1 (decode is HBM-bound) and §5.3.7 (the kernel follows the
// block table to gather scattered 16-token blocks); "Speculative decoding
// principles" 7.2.1 (one forward scores K + 1 positions under a causal mask).
//
// Design (gfx950, wave64):
//  * One workgroup = one (sequence, kv head, row chunk, context partition).
//    Its waves walk the partition's pages round-robin; every K/V byte is read
//    from HBM once per (sequence, kv head) and used by all G * n query rows
//    of the group at once.
//  * QK^T and PV run on MFMA with the tokens of one page as the 16-wide M /
//    K dimension and the group's query rows as N (padded to 16 per tile), so
//    the GQA group and the verify rows share each K/V fragment in registers.
//    Pages are loaded straight from HBM into VGPRs in the MFMA operand
//    layout with non-temporal loads: K pages are stored in 16-byte head-dim
//    chunks so one K fragment is 1 KiB contiguous, a V fragment is 4 whole
//    256-byte token rows; V is transposed in registers with v_perm.  The QK output layout is exactly the PV B-operand layout, so the
//    probabilities never leave their lanes.
//  * Online softmax in the log2 domain (scale * log2 e folded into the
//    scores, v_exp_f32), running max reduced across the 4 lane groups with
//    two shuffles per page; the running sum stays lane-local until the end.
//  * Waves of a workgroup are merged in LDS in a fixed order; context
//    partitions (split-K, at most 64 per sequence) are merged by a second
//    small kernel, one workgroup per output row.  Both merges weight a part
//    by 2^(m_part - m_max).
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

#include "cdna4.h"
#include "paged_attn.h"
#include "staged.h"
#include "status.h"

#define PA_API extern "C" __attribute__((visibility("default")))

namespace {

using namespace cdna4;

constexpr int kPage = 16;
constexpr int kHeadDim = 128;
constexpr int kSlab = kPage * kHeadDim;     // elements of one (page, kv head) slab
constexpr int kWave = 64;
constexpr int kMaxRowTiles = 4;             // 16-row MFMA tiles per workgroup
constexpr int kMaxSplits = 64;              // context partitions per sequence
constexpr float kLog2e = 1.4426950408889634f;
// Running max before any key is seen.  Finite, so exp2(m_old - m_new) is
// never inf - inf; masked scores are -inf and give exp2(-inf) = 0.
constexpr float kNoMax = -1.0e30f;
constexpr int kAccStride = kHeadDim + 4;    // LDS row stride of the wave merge (bank skew)
// The running max of a row moves only when a page's max exceeds it by more
// than this many log2 units, so weights stay <= 2^8 (safe in fp32 and bf16)
// and the accumulator is rescaled on few pages.
constexpr float kRescaleSlack = 8.0f;

enum KvKind { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

struct Args {
    const void* k;
    const void* v;
    const float* k_scale;
    const float* v_scale;
    const void* q;
    void* out;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const uint64_t* tree_mask; // [B][n] ancestor masks of a draft tree, or null (causal)
    float* part_acc;       // [B][n][Hq][num_splits][128]
    float* part_ml;        // [B][n][Hq][num_splits][2]  (max in log2 units, sum)
    int64_t page_stride;   // elements from one page to the next (Hkv * 16 * 128)
    int32_t num_pages;
    int32_t max_pages;
    int32_t n;
    int32_t hq;
    int32_t hkv;
    int32_t group;         // G = Hq / Hkv
    int32_t rows;          // G * n query rows per (sequence, kv head)
    int32_t row_chunks;
    int32_t num_splits;
    int32_t part_pages;
    float scale_log2;      // scale * log2(e)
};

// ---------------------------------------------------------------------------
// one page of K and V for one kv head, in MFMA operand layout
//   l16 = lane % 16, g = lane / 16
//   K slab: 16-byte chunks of the head dimension, the 16 tokens of a chunk
//   stored one after another; byte offset of (chunk q, token t) = (16 q + t) * 16.
//   The lanes of one load instruction c read chunks 4c .. 4c+3 of every token:
//   1 KiB contiguous, lane (l16, g) gets chunk 4c + g of token l16.
//   V slab: token-major rows; lane (l16, g) reads 16 bytes of token 4g + s per
//   instruction s, so one instruction covers four whole rows.
//   Loads are non-temporal: every K/V byte is used once per call.
// ---------------------------------------------------------------------------
template <int KV> struct Page;

template <> struct Page<KV_BF16> {
    u32x4 k[4];   // k[c]: K[l16][32c + 8g .. +8]
    u32x4 v[4];   // v[s]: V[4g + s][8 l16 .. +8]
};

template <> struct Page<KV_FP8> {
    u32x4 k[2];   // k[h]: K[l16][64h + 16g .. +16] bytes
    u32x2 v[4];   // v[s]: V[4g + s][8 l16 .. +8] bytes
    float ks, vs;
};

template <> struct Page<KV_F32> {
    f32x4 k[8];   // k[c]: K[l16][16c + 4g .. +4]
    f32x4 v[8];   // v[2s + h]: V[4g + s][8 l16 + 4h .. +4]
};

template <typename T>
__device__ __forceinline__ T stream_load(const T* p)
{
    return __builtin_nontemporal_load(p);
}

// chunk (4c + g) of token l16: byte offset ((4c + g) * 16 + l16) * 16 = 1024 c + lane * 16
__device__ __forceinline__ const u32x4* k_fragment(const void* slab, int lane)
{
    return reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(slab) + 16 * lane);
}

__device__ __forceinline__ void load_page(Page<KV_BF16>& p, const Args& a, int phys, int kh,
                                          int l16, int g)
{
    const int64_t off = (int64_t)phys * a.page_stride + (int64_t)kh * kSlab;
    const uint16_t* kb = static_cast<const uint16_t*>(a.k) + off;
    const uint16_t* vb = static_cast<const uint16_t*>(a.v) + off;
    const u32x4* kp = k_fragment(kb, 16 * g + l16);
    const u32x4* vp = reinterpret_cast<const u32x4*>(vb + 4 * g * kHeadDim + 8 * l16);
#pragma unroll
    for (int c = 0; c < 4; ++c) p.k[c] = stream_load(kp + 64 * c);
#pragma unroll
    for (int s = 0; s < 4; ++s) p.v[s] = stream_load(vp + 16 * s);
}

__device__ __forceinline__ void load_page(Page<KV_FP8>& p, const Args& a, int phys, int kh,
                                          int l16, int g)
{
    const int64_t off = (int64_t)phys * a.page_stride + (int64_t)kh * kSlab;
    const uint8_t* kb = static_cast<const uint8_t*>(a.k) + off;
    const uint8_t* vb = static_cast<const uint8_t*>(a.v) + off;
    const u32x4* kp = k_fragment(kb, 16 * g + l16);
    const u32x2* vp = reinterpret_cast<const u32x2*>(vb + 4 * g * kHeadDim + 8 * l16);
#pragma unroll
    for (int h = 0; h < 2; ++h) p.k[h] = stream_load(kp + 64 * h);
#pragma unroll
    for (int s = 0; s < 4; ++s) p.v[s] = stream_load(vp + 16 * s);
    const int64_t si = (int64_t)phys * a.hkv + kh;
    p.ks = a.k_scale[si];
    p.vs = a.v_scale[si];
}

__device__ __forceinline__ void load_page(Page<KV_F32>& p, const Args& a, int phys, int kh,
                                          int l16, int g)
{
    const int64_t off = (int64_t)phys * a.page_stride + (int64_t)kh * kSlab;
    const float* kb = static_cast<const float*>(a.k) + off;
    const float* vb = static_cast<const float*>(a.v) + off;
    const f32x4* kp = reinterpret_cast<const f32x4*>(k_fragment(kb, 16 * g + l16));
    const f32x4* vp = reinterpret_cast<const f32x4*>(vb + 4 * g * kHeadDim + 8 * l16);
#pragma unroll
    for (int c = 0; c < 8; ++c) p.k[c] = stream_load(kp + 64 * c);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        p.v[2 * s] = stream_load(vp + 32 * s);
        p.v[2 * s + 1] = stream_load(vp + 32 * s + 1);
    }
}

// V rows of tokens at or past the sequence end (their slots may hold NaN) are
// replaced by zeros once loaded; s counts this lane's tokens 4g + s
__device__ __forceinline__ void clear_dead_v(Page<KV_BF16>& p, int first_dead_s)
{
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) p.v[s][e] = (s < first_dead_s) ? p.v[s][e] : 0u;
}
__device__ __forceinline__ void clear_dead_v(Page<KV_FP8>& p, int first_dead_s)
{
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 2; ++e) p.v[s][e] = (s < first_dead_s) ? p.v[s][e] : 0u;
}
__device__ __forceinline__ void clear_dead_v(Page<KV_F32>& p, int first_dead_s)
{
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p.v[2 * s][e] = (s < first_dead_s) ? p.v[2 * s][e] : 0.f;
            p.v[2 * s + 1][e] = (s < first_dead_s) ? p.v[2 * s + 1][e] : 0.f;
        }
}

// ---------------------------------------------------------------------------
// query rows in MFMA B-operand layout (lane holds row l16 of its tile)
// ---------------------------------------------------------------------------
template <int KV> struct QFrag;
template <> struct QFrag<KV_BF16> { bf16x8 b[4]; };   // dims 32c + 8g .. +8
template <> struct QFrag<KV_FP8>  { bf16x8 b[4]; };   // dims 64(c/2) + 16g + 8(c%2) .. +8
template <> struct QFrag<KV_F32>  { f32x4 b[8]; };    // dims 16c + 4g .. +4

// Loads are unconditional (the row pointer of a padding row is a valid row)
// and padding rows are zeroed afterwards, so the loads can stay in flight.
__device__ __forceinline__ void load_q(QFrag<KV_BF16>& f, const uint16_t* row, bool valid, int g)
{
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(row + 32 * c + 8 * g);
        f.b[c] = __builtin_bit_cast(bf16x8, valid ? x : u32x4{0u, 0u, 0u, 0u});
    }
}
__device__ __forceinline__ void load_q(QFrag<KV_FP8>& f, const uint16_t* row, bool valid, int g)
{
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int d0 = 64 * (c >> 1) + 16 * g + 8 * (c & 1);
        const u32x4 x = *reinterpret_cast<const u32x4*>(row + d0);
        f.b[c] = __builtin_bit_cast(bf16x8, valid ? x : u32x4{0u, 0u, 0u, 0u});
    }
}
__device__ __forceinline__ void load_q(QFrag<KV_F32>& f, const float* row, bool valid, int g)
{
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(row + 16 * c + 4 * g);
        f.b[c] = valid ? x : f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// S^T[token][row] for one 16-row tile: lane holds tokens 4g + v of row l16
__device__ __forceinline__ f32x4 scores(const Page<KV_BF16>& p, const QFrag<KV_BF16>& q)
{
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, p.k[c]), q.b[c],
                                                    s, 0, 0, 0);
    return s;
}
__device__ __forceinline__ f32x4 scores(const Page<KV_FP8>& p, const QFrag<KV_FP8>& q)
{
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const u32x4& w = p.k[c >> 1];
        const int h = c & 1;
        u32x4 kb = fp8x8_to_bf16x8(w[2 * h], w[2 * h + 1]);
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb), q.b[c], s,
                                                    0, 0, 0);
    }
    return s * p.ks;
}
__device__ __forceinline__ f32x4 scores(const Page<KV_F32>& p, const QFrag<KV_F32>& q)
{
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(p.k[c][e], q.b[c][e], s, 0, 0, 0);
    return s;
}

// o[db] holds O[row l16][32g + 8v + db], v = 0..3 (the PV output layout)
template <int KV> struct Acc { f32x4 o[8]; };

// V of one page as PV A operands: a[db] = {V[4g + s][8 l16 + db], s = 0..3},
// built once per page and shared by every row tile.
struct VOps {
    i16x4 a[8];
    float vs;       // V scale folded into the probabilities (1 for bf16)
};

__device__ __forceinline__ void transpose_v(VOps& o, const u32x4 (&v)[4]) { v_operands(o.a, v); }

__device__ __forceinline__ void prepare_v(VOps& o, const Page<KV_BF16>& pg)
{
    transpose_v(o, pg.v);
    o.vs = 1.0f;
}

__device__ __forceinline__ void prepare_v(VOps& o, const Page<KV_FP8>& pg)
{
    u32x4 vb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) vb[s] = fp8x8_to_bf16x8(pg.v[s][0], pg.v[s][1]);
    transpose_v(o, vb);
    o.vs = pg.vs;
}

// acc += P * V for one tile; p[s] is the weight of token 4g + s for row l16.
// Returns the sum of the weights as they entered the product (bf16-rounded
// for bf16 K/V, so the running sum matches the products).
template <int KV>
__device__ __forceinline__ float pv(Acc<KV>& acc, const VOps& vo, const float (&p)[4])
{
    uint32_t b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) b[s] = bf16_bits(KV == KV_FP8 ? p[s] * vo.vs : p[s]);
    const i16x4 pb = __builtin_bit_cast(i16x4, u32x2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)});
#pragma unroll
    for (int db = 0; db < 8; ++db)
        acc.o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vo.a[db], pb, acc.o[db], 0, 0, 0);
    if constexpr (KV == KV_FP8)
        return p[0] + p[1] + p[2] + p[3];
    else
        return bf16_float(b[0]) + bf16_float(b[1]) + bf16_float(b[2]) + bf16_float(b[3]);
}

__device__ __forceinline__ float pv_f32(Acc<KV_F32>& acc, const Page<KV_F32>& pg,
                                       const float (&p)[4])
{
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int db = 0; db < 8; ++db)
            acc.o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(pg.v[2 * s + (db >> 2)][db & 3], p[s],
                                                              acc.o[db], 0, 0, 0);
    return p[0] + p[1] + p[2] + p[3];
}

template <int KV> struct QPtr { typedef uint16_t type; };
template <> struct QPtr<KV_F32> { typedef float type; };

template <int KV> struct OutT { typedef uint16_t type; };
template <> struct OutT<KV_F32> { typedef float type; };

__device__ __forceinline__ void store_out(uint16_t* o, float x) { *o = (uint16_t)bf16_bits(x); }
__device__ __forceinline__ void store_out(float* o, float x) { *o = x; }

// ---------------------------------------------------------------------------
// partition kernel
// ---------------------------------------------------------------------------
// Occupancy hints measured on MI355X.  Two row tiles (the verify shape) ask
// for two waves per SIMD: without the hint the compiler spends 272 VGPRs and
// only one wave per SIMD keeps pages in flight (verify 40 -> 33 us).  The
// fp8 one-tile kernel with a two-page pipeline fits four waves per SIMD in
// 116 VGPRs (2% faster).  Deeper pipelines keep the compiler's choice, which
// does not spill; they are meant for plans with one workgroup per CU.
template <int KV, int NT, int PF>
constexpr int min_waves_per_simd()
{
    return (NT == 2 && KV != KV_F32 && PF <= 3) ? 2 : (NT == 1 && KV == KV_FP8 && PF == 2) ? 4 : 1;
}

template <int KV, int NT, int W, int PF>
__global__ __launch_bounds__(W * kWave, (min_waves_per_simd<KV, NT, PF>())) void paged_attn_partition(Args a)
{
    constexpr int RT = 16 * NT;   // rows per workgroup
    __shared__ float sm_ml[W][RT][2];
    __shared__ float sm_acc[RT * kAccStride];
    __shared__ float sm_fin[RT][2];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int l16 = lane & 15;
    const int g = lane >> 4;

    int unit = blockIdx.x;
    const int split = unit % a.num_splits;
    unit /= a.num_splits;
    const int rc = unit % a.row_chunks;
    unit /= a.row_chunks;
    const int kh = unit % a.hkv;
    const int b = unit / a.hkv;

    // Block-table ids and query rows do not depend on the sequence length,
    // so they are requested together with it: the first page loads then wait
    // for one memory round trip instead of two.
    const int pg0 = split * a.part_pages;
    const int row0 = rc * RT;
    const int32_t* bt_row = a.block_table + (int64_t)b * a.max_pages;
    // (unconditional loads from clamped, in-bounds addresses: a lane-masked
    // load would make the compiler wait for it on the spot)
    const int raw_id = bt_row[min(pg0 + wave + lane * W, min(pg0 + a.part_pages, a.max_pages) - 1)];
    QFrag<KV> qf[NT];
    int qi[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = row0 + nt * 16 + l16;
        const bool valid = r < a.rows;
        const int i = valid ? r / a.group : 0;
        const int h = kh * a.group + (valid ? r - i * a.group : 0);
        const typename QPtr<KV>::type* qrow =
            static_cast<const typename QPtr<KV>::type*>(a.q) +
            (((int64_t)b * a.n + i) * a.hq + h) * kHeadDim;
        load_q(qf[nt], qrow, valid, g);
        qi[nt] = valid ? i : -1;
    }
    // draft-tree verification: row i sees tree token j iff bit j of its mask
    uint64_t tmask[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) tmask[nt] = ~uint64_t(0);
    if (a.tree_mask) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const uint64_t mk = a.tree_mask[(int64_t)b * a.n + max(qi[nt], 0)];
            tmask[nt] = qi[nt] >= 0 ? mk : ~uint64_t(0);
        }
    }

    // lengths are clamped to what the block table can describe, and page ids
    // to the pool, so that arrays breaking the contract give wrong numbers
    // but never an access outside the caller's buffers
    const int L = min(a.seq_lens[b], a.max_pages * kPage);
    const int npages = (L + kPage - 1) / kPage;
    const int nsplit_b = min((npages + a.part_pages - 1) / a.part_pages, a.num_splits);
    if (split >= nsplit_b) return;
    const int pg1 = min(pg0 + a.part_pages, npages);
    const int rows_here = min(RT, a.rows - row0);
    const int first_limit = L - a.n;          // row 0 sees tokens 0 .. L - n
    // first token that some row may not see: L - n + 1 for the causal chain,
    // L - n (the root) under a tree mask
    const int mask_from = a.tree_mask ? first_limit : first_limit + 1;

    // per-row visibility limits (padding rows see every live token)
    int lim[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) lim[nt] = qi[nt] >= 0 ? first_limit + qi[nt] : L - 1;

    Acc<KV> acc[NT];
    float m[NT], l[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[nt].o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[nt] = kNoMax;
        l[nt] = 0.f;
    }

    // this wave's pages: pg0 + wave + j * W, j < nj (nj <= 64 by construction)
    const int nj = (pg1 - pg0 - wave + W - 1) / W;
    const int my_id = (lane < nj) ? min(max(raw_id, 0), a.num_pages - 1) : 0;

    auto consume = [&](Page<KV>& pg, int j) {
        const int base = (pg0 + wave + j * W) * kPage;
        const bool need_mask = base + kPage - 1 >= mask_from;
        VOps vo;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 sv = scores(pg, qf[nt]);
            float s[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) s[v] = sv[v] * a.scale_log2;
            if (need_mask) {
                if (a.tree_mask) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int tok = base + 4 * g + v;
                        const bool vis = tok < L && (tok < first_limit ||
                                         ((tmask[nt] >> (tok - first_limit)) & 1u));
                        s[v] = vis ? s[v] : -INFINITY;
                    }
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        s[v] = (base + 4 * g + v <= lim[nt]) ? s[v] : -INFINITY;
                }
            }
            const float mx = group_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
            const bool grow = mx > m[nt] + kRescaleSlack;
            if (__any(grow)) {
                const float mnew = grow ? mx : m[nt];
                const float alpha = fast_exp2(m[nt] - mnew);
                m[nt] = mnew;
                l[nt] *= alpha;
#pragma unroll
                for (int db = 0; db < 8; ++db) acc[nt].o[db] *= alpha;
            }
            float p[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) p[v] = fast_exp2(s[v] - m[nt]);
            if (nt == 0 && base + kPage > L) clear_dead_v(pg, L - base - 4 * g);
            if constexpr (KV == KV_F32) {
                l[nt] += pv_f32(acc[nt], pg, p);
            } else {
                if (nt == 0) prepare_v(vo, pg);
                l[nt] += pv<KV>(acc[nt], vo, p);
            }
        }
    };

    // Software pipeline: page j + PF - 1 is requested before page j is used.
    // Loads are unconditional (indices past the last page repeat the last
    // page) so that the wait before each use covers only that page's loads.
    if (nj > 0) {
        auto phys_of = [&](int j) { return __builtin_amdgcn_readlane(my_id, min(j, nj - 1)); };
        Page<KV> buf[PF];
#pragma unroll
        for (int st = 0; st < PF - 1; ++st) load_page(buf[st], a, phys_of(st), kh, l16, g);
        int j0 = 0;
        for (; j0 + PF <= nj; j0 += PF) {
#pragma unroll
            for (int st = 0; st < PF; ++st) {
                load_page(buf[(st + PF - 1) % PF], a, phys_of(j0 + st + PF - 1), kh, l16, g);
                consume(buf[st], j0 + st);
            }
        }
#pragma unroll
        for (int st = 0; st < PF - 1; ++st)
            if (j0 + st < nj) consume(buf[st], j0 + st);
    }

    // ---- merge the waves of this workgroup (fixed order) ----
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        l[nt] = group_sum(l[nt]);
        if (g == 0) {
            sm_ml[wave][nt * 16 + l16][0] = m[nt];
            sm_ml[wave][nt * 16 + l16][1] = l[nt];
        }
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int row = nt * 16 + l16;
        float mm = kNoMax;
#pragma unroll
        for (int w = 0; w < W; ++w) mm = fmaxf(mm, sm_ml[w][row][0]);
        const float fac = fast_exp2(m[nt] - mm);
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[nt].o[db] *= fac;
        if (wave == 0 && g == 0) {
            float ls = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) ls += sm_ml[w][row][1] * fast_exp2(sm_ml[w][row][0] - mm);
            sm_fin[row][0] = mm;
            sm_fin[row][1] = ls;
        }
    }
#pragma unroll
    for (int w = 0; w < W; ++w) {
        if (wave == w) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int row = nt * 16 + l16;
                if (row < rows_here) {
                    float* dst = sm_acc + row * kAccStride + 32 * g;
#pragma unroll
                    for (int v = 0; v < 4; ++v)
#pragma unroll
                        for (int db = 0; db < 8; ++db) {
                            if (w == 0) dst[8 * v + db] = acc[nt].o[db][v];
                            else dst[8 * v + db] += acc[nt].o[db][v];
                        }
                }
            }
        }
        __syncthreads();
    }

    // ---- epilogue: final output (one partition) or a split-K partial ----
    const bool single = nsplit_b == 1;
    for (int e = threadIdx.x; e < rows_here * kHeadDim; e += W * kWave) {
        const int row = e / kHeadDim;
        const int d = e - row * kHeadDim;
        const int r = row0 + row;
        const int i = r / a.group;
        const int h = kh * a.group + (r - i * a.group);
        const int64_t orow = ((int64_t)b * a.n + i) * a.hq + h;
        const float x = sm_acc[row * kAccStride + d];
        if (single) {
            typename OutT<KV>::type* o = static_cast<typename OutT<KV>::type*>(a.out);
            store_out(o + orow * kHeadDim + d, x / sm_fin[row][1]);
        } else {
            const int64_t pidx = orow * a.num_splits + split;
            a.part_acc[pidx * kHeadDim + d] = x;
            if (d == 0) {
                a.part_ml[pidx * 2] = sm_fin[row][0];
                a.part_ml[pidx * 2 + 1] = sm_fin[row][1];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// split-K reduce: one 128-thread workgroup per output row (sequence, query
// row, head), one head-dim element per thread.  The first 16 partials of the
// element are fetched in the same round as the row's (max, sum) pairs, so a
// merge of up to 16 partitions costs one memory round trip.
// ---------------------------------------------------------------------------
constexpr int kReduceThreads = kHeadDim;
constexpr int kReduceInFlight = 16;

template <typename OT>
__global__ __launch_bounds__(kReduceThreads) void paged_attn_reduce(Args a)
{
    __shared__ float sm_m[kMaxSplits];
    __shared__ float sm_l[kMaxSplits];
    const int64_t orow = blockIdx.x;                 // (b * n + i) * hq + h
    const int b = (int)(orow / ((int64_t)a.n * a.hq));
    const int t = threadIdx.x;
    // The partials and (max, sum) pairs of the plan's splits are requested
    // together with the sequence length, before the number this sequence
    // actually wrote is known (entries past it are read but never used), so
    // the merge waits for one memory round trip instead of two.
    const float* src = a.part_acc + orow * a.num_splits * kHeadDim + t;
    float x[kReduceInFlight];
#pragma unroll
    for (int sp = 0; sp < kReduceInFlight; ++sp)
        x[sp] = src[min(sp, a.num_splits - 1) * kHeadDim];
    float mt = 0.f, lt = 0.f;
    if (t < a.num_splits) {
        const float* ml = a.part_ml + (orow * a.num_splits + t) * 2;
        mt = ml[0];
        lt = ml[1];
    }
    const int L = min(a.seq_lens[b], a.max_pages * kPage);
    const int npages = (L + kPage - 1) / kPage;
    const int ns = min((npages + a.part_pages - 1) / a.part_pages, a.num_splits);
    if (ns <= 1) return;                             // written by the partition kernel
    if (t < ns) {
        sm_m[t] = mt;
        sm_l[t] = lt;
    }
    __syncthreads();
    float mm = kNoMax;
    for (int sp = 0; sp < ns; ++sp) mm = fmaxf(mm, sm_m[sp]);
    float ls = 0.f, acc = 0.f;
#pragma unroll
    for (int sp = 0; sp < kReduceInFlight; ++sp)
        if (sp < ns) {
            const float w = fast_exp2(sm_m[sp] - mm);
            ls += sm_l[sp] * w;
            acc += w * x[sp];
        }
    for (int sp = kReduceInFlight; sp < ns; ++sp) {
        const float w = fast_exp2(sm_m[sp] - mm);
        ls += sm_l[sp] * w;
        acc += w * src[sp * kHeadDim];
    }
    store_out(static_cast<OT*>(a.out) + orow * kHeadDim + t, acc / ls);
}

// ---------------------------------------------------------------------------
// KV append (quantize-on-write): the n_new newest tokens of every sequence are
// written into their pages ("Latency and cost in production" §10.12.2: a
// request's blocks fill one token at a time; §10.8.2-§10.8.3: q =
// round(x / scale) with zero-point 0).  Pages are independent (each has its
// own scale), so one workgroup of one wave takes one (sequence, kv head, K or
// V, page touched by the new tokens); its work unit is one 16-byte chunk of
// one token row (K chunked, V token-major), read from the source with 16-byte
// loads.  fp8 pages: scale = absmax / 448 over the new values of a page none
// of whose earlier slots are live (1 if 0); otherwise max(old, absmax / 448),
// and the earlier live bytes are re-encoded when it grows.  All in binary32.
// ---------------------------------------------------------------------------
struct AppendArgs {
    void* k;
    void* v;
    float* k_scale;
    float* v_scale;
    const void* k_new;     // [B][n_new][Hkv][128]
    const void* v_new;
    const int32_t* block_table;
    const int32_t* seq_lens;
    int64_t page_stride;   // elements from one page to the next (Hkv * 16 * 128)
    int32_t num_pages;
    int32_t max_pages;
    int32_t hkv;
    int32_t n_new;
};

// E4M3 value of a byte, exactly (sign, 4-bit exponent with bias 7, 3-bit mantissa)
__device__ __forceinline__ float e4m3_to_float(uint32_t byte)
{
    const uint32_t e = (byte >> 3) & 0xF, m = byte & 0x7;
    const float mag = e == 0 ? (float)m * 0.001953125f                       // m * 2^-9
                             : __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (byte & 0x80) ? -mag : mag;
}

// Nearest E4M3 byte to x, ties to even, saturating at +-448
__device__ __forceinline__ uint32_t float_to_e4m3(float x)
{
    const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80;
    const float a = fabsf(x);
    uint32_t code;
    if (!(a < 448.0f)) {
        code = 0x7E;
    } else if (a < 0.015625f) {                                  // below 2^-6: steps of 2^-9
        code = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        const int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;   // a in [2^e, 2^(e+1))
        const uint32_t steps = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - e));  // 8..16
        code = min((uint32_t)((e + 7) << 3) + steps - 8u, 0x7Eu);
    }
    return sign | code;
}

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

template <int KV, bool SRC_BF16>
__global__ __launch_bounds__(kWave) void paged_attn_append(AppendArgs a)
{
    constexpr int esz = KV == KV_F32 ? 4 : KV == KV_BF16 ? 2 : 1;
    constexpr int X = 16 / esz;                     // elements per 16-byte chunk of the pool
    constexpr int C = kHeadDim / X;                 // chunks per token row
    constexpr int SW = SRC_BF16 ? 2 : 4;            // source bytes per element
    constexpr int SV = X * SW / 16;                 // 16-byte source loads per chunk
    constexpr int kPerLane = kPage * C / kWave;     // most chunks one lane holds (fp8: 2)
    const int lane = threadIdx.x;
    const int which = blockIdx.x & 1;               // 0: K, 1: V
    const int kh = (blockIdx.x >> 1) % a.hkv;
    const int b = (blockIdx.x >> 1) / a.hkv;
    const int L = min(a.seq_lens[b], a.max_pages * kPage);
    const int first = L - a.n_new;
    if (first < 0) return;
    const int p = first / kPage + (int)blockIdx.y;  // logical page of this workgroup
    if (p > (L - 1) / kPage) return;
    const int phys = min(max(a.block_table[(int64_t)b * a.max_pages + p], 0), a.num_pages - 1);
    const int s0 = p * kPage;
    const int lo = max(first - s0, 0);              // first new slot of this page
    const int hi = min(L - s0, kPage);              // one past the last
    const int nchunks = (hi - lo) * C;
    uint8_t* pool = static_cast<uint8_t*>(which ? a.v : a.k) +
                    ((int64_t)phys * a.page_stride + (int64_t)kh * kSlab) * esz;
    const uint8_t* src = static_cast<const uint8_t*>(which ? a.v_new : a.k_new);

    // byte offset of chunk c of slot `slot` in this slab
    auto at = [&](int slot, int c) -> int64_t {
        return which ? (int64_t)(slot * kHeadDim + c * X) * esz : (int64_t)(c * kPage + slot) * 16;
    };
    auto src_at = [&](int slot, int c) -> const u32x4* {
        const int64_t e = (((int64_t)b * a.n_new + (s0 + slot - first)) * a.hkv + kh) * kHeadDim +
                          c * X;
        return reinterpret_cast<const u32x4*>(src + e * SW);
    };
    auto load_chunk = [&](int slot, int c, float (&x)[X]) {
        const u32x4* s = src_at(slot, c);
#pragma unroll
        for (int j = 0; j < SV; ++j) {
            const u32x4 w = s[j];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (SRC_BF16) {
                    x[8 * j + 2 * i] = bf16_float(w[i] & 0xFFFF);
                    x[8 * j + 2 * i + 1] = bf16_float(w[i] >> 16);
                } else {
                    x[4 * j + i] = __uint_as_float(w[i]);
                }
            }
        }
    };

    if constexpr (KV != KV_FP8) {
        for (int e = lane; e < nchunks; e += kWave) {
            const int slot = lo + e / C, c = e % C;
            u32x4 w;
            if constexpr (KV == KV_F32 || SRC_BF16) {
                w = *src_at(slot, c);                   // already in the pool format
            } else {
                float x[X];
                load_chunk(slot, c, x);
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = bf16_bits(x[2 * i]) | (bf16_bits(x[2 * i + 1]) << 16);
            }
            *reinterpret_cast<u32x4*>(pool + at(slot, c)) = w;
        }
    } else {
        float x[kPerLane][X];
        float amax = 0.f;
#pragma unroll
        for (int r = 0; r < kPerLane; ++r) {
            const int e = lane + r * kWave;
            if (e < nchunks) {
                load_chunk(lo + e / C, e % C, x[r]);
#pragma unroll
                for (int i = 0; i < X; ++i) amax = fmaxf(amax, fabsf(x[r][i]));
            }
        }
        amax = wave_max(amax);
        const float cand = amax / 448.0f;
        float* scales = which ? a.v_scale : a.k_scale;
        const int64_t si = (int64_t)phys * a.hkv + kh;
        float scale;
        if (lo == 0) {
            scale = amax > 0.f ? cand : 1.0f;
        } else {
            const float old = scales[si];
            scale = cand > old ? cand : old;
            if (scale != old) {
                // the page's earlier live bytes move to the larger scale
                for (int e = lane; e < lo * C; e += kWave) {
                    u32x4* ptr = reinterpret_cast<u32x4*>(pool + at(e / C, e % C));
                    u32x4 w = *ptr;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        uint32_t out = 0;
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const float val = e4m3_to_float((w[i] >> (8 * k)) & 0xFF) * old;
                            out |= float_to_e4m3(val / scale) << (8 * k);
                        }
                        w[i] = out;
                    }
                    *ptr = w;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < kPerLane; ++r) {
            const int e = lane + r * kWave;
            if (e < nchunks) {
                u32x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint32_t out = 0;
#pragma unroll
                    for (int k = 0; k < 4; ++k) out |= float_to_e4m3(x[r][4 * i + k] / scale) << (8 * k);
                    w[i] = out;
                }
                *reinterpret_cast<u32x4*>(pool + at(lo + e / C, e % C)) = w;
            }
        }
        if (lane == 0) scales[si] = scale;
    }
}

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
// per workgroup and a three-page register pipeline for one row tile; two
// pages when the query tile (two row tiles, or fp8 conversion) needs the
// registers.
constexpr int kWaves = 4;
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
        const int64_t grid = (int64_t)batch * d.num_kv_heads * row_blocks;
        if (grid > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "grid too large");
        pl->partition_pages = (max_len + kPage - 1) / kPage;
        pl->num_splits = 1;
        pl->row_tiles = kStagedPrefillRows / 16;
        pl->row_chunks = (int32_t)row_blocks;
        pl->waves = 4;
        pl->grid = (int32_t)grid;
        pl->reduce = 0;
        pl->kernel = 1;
        return PA_OK;
    }
    const int nt = (int)std::min<int64_t>(kMaxRowTiles, (rows + 15) / 16);
    const int64_t row_chunks = (rows + 16 * nt - 1) / (16 * nt);
    const int max_pages = (max_len + kPage - 1) / kPage;
    const int64_t units = (int64_t)batch * d.num_kv_heads * row_chunks;
    int part;
    if (d.partition_pages > 0) {
        part = std::min(d.partition_pages, max_pages);
    } else {
        // two workgroups per CU for one row tile; one for wider query tiles,
        // whose workgroups already fill the register file (MI355X sweep)
        const int64_t target = (nt == 1 ? 2LL : 1LL) * cu_count();
        int64_t ns = (target + units - 1) / units;
        const int64_t ns_cap =
            std::max<int64_t>(1, max_pages / (2 * (d.waves > 0 ? d.waves : kWaves)));
        ns = std::max<int64_t>(1, std::min(ns, ns_cap));
        part = (int)((max_pages + ns - 1) / ns);
    }
    const int waves = d.waves > 0 ? d.waves : kWaves;
    part = std::min(part, 64 * waves);         // each wave holds at most 64 page ids
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

template <int KV, int NT, int W, int PF>
void launch_partition(const Args& a, int grid, hipStream_t st)
{
    hipLaunchKernelGGL((paged_attn_partition<KV, NT, W, PF>), dim3(grid), dim3(W * kWave), 0, st,
                       a);
}

// (waves, prefetch) variants are instantiated for the bf16 and fp8 paths with
// one or two row tiles; every other shape runs the default variant
template <int KV, int NT>
void launch_tuned(int waves, int prefetch, const Args& a, int grid, hipStream_t st)
{
    if constexpr (KV == KV_F32 || NT > 2) {
        launch_partition<KV, NT, kWaves, 2>(a, grid, st);
        return;
    } else {
    const int key = waves * 10 + prefetch;
    switch (key) {
    case 42: launch_partition<KV, NT, 4, 2>(a, grid, st); break;
    case 43: launch_partition<KV, NT, 4, 3>(a, grid, st); break;
    case 44: launch_partition<KV, NT, 4, 4>(a, grid, st); break;
    case 45: launch_partition<KV, NT, 4, 5>(a, grid, st); break;
    case 46: launch_partition<KV, NT, 4, 6>(a, grid, st); break;
    case 83: launch_partition<KV, NT, 8, 3>(a, grid, st); break;
    case 84: launch_partition<KV, NT, 8, 4>(a, grid, st); break;
    case 82: launch_partition<KV, NT, 8, 2>(a, grid, st); break;
    default: launch_partition<KV, NT, 4, 2>(a, grid, st); break;
    }
    }
}

template <int KV>
void launch_partition_nt(int nt, int waves, int prefetch, const Args& a, int grid,
                         hipStream_t st)
{
    switch (nt) {
    case 1: launch_tuned<KV, 1>(waves, prefetch, a, grid, st); break;
    case 2: launch_tuned<KV, 2>(waves, prefetch, a, grid, st); break;
    case 3: launch_tuned<KV, 3>(waves, prefetch, a, grid, st); break;
    default: launch_tuned<KV, 4>(waves, prefetch, a, grid, st); break;
    }
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
    // the LDS-staged kernel writes O in 8- and 16-byte pieces
    const bool out16 = reinterpret_cast<uintptr_t>(out) % 16 == 0;
    pa_status stt = make_plan(pool, batch, n, hq, max_seq_len, &pl, out16);
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

    Args a;
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
    if (pl.kernel == 1 && tree_mask)
        return fail(PA_ERR_UNSUPPORTED, "draft trees have at most 64 nodes");
    // draft trees on bf16 / fp8 pools: the LDS-staged kernel, 64 rows per
    // workgroup, under the same split plan (and workspace) as the partition kernel
    const bool staged_tree = tree_mask && d.kv_dtype != PA_F32 && d.staged_from != -1 && out16 &&
                             pl.partition_pages <= kStagedTreeMaxPages;
    if (ev_begin && (e = hipEventRecord(static_cast<hipEvent_t>(ev_begin), st)) != hipSuccess)
        return hip_fail(e, "hipEventRecord(begin)");
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
        if ((e = launch_staged(sa, d.kv_dtype == PA_FP8_E4M3, staged_tree, st)) != hipSuccess)
            return hip_fail(e, "staged kernel launch");
    } else {
        const int pf = d.prefetch > 0 ? d.prefetch : default_prefetch(d.kv_dtype, pl.row_tiles);
        switch (d.kv_dtype) {
        case PA_F32: launch_partition_nt<KV_F32>(pl.row_tiles, pl.waves, pf, a, pl.grid, st); break;
        case PA_BF16: launch_partition_nt<KV_BF16>(pl.row_tiles, pl.waves, pf, a, pl.grid, st); break;
        default: launch_partition_nt<KV_FP8>(pl.row_tiles, pl.waves, pf, a, pl.grid, st); break;
        }
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "partition kernel launch");
    }
    if (ev_end && (e = hipEventRecord(static_cast<hipEvent_t>(ev_end), st)) != hipSuccess)
        return hip_fail(e, "hipEventRecord(end)");
    if (pl.reduce) {
        const unsigned rows_out = (unsigned)((int64_t)batch * n * hq);
        if (q_dtype == PA_F32)
            hipLaunchKernelGGL(paged_attn_reduce<float>, dim3(rows_out), dim3(kReduceThreads), 0,
                               st, a);
        else
            hipLaunchKernelGGL(paged_attn_reduce<uint16_t>, dim3(rows_out), dim3(kReduceThreads),
                               0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "reduce kernel launch");
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
    pa_plan pl;
    pa_status st = make_plan(pool, batch, q_per_seq, num_q_heads, max_seq_len, &pl);
    if (st != PA_OK) return st;
    *bytes = workspace_for(pl, batch, q_per_seq, num_q_heads);
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
    const bool bf = src_dtype == PA_BF16;
    switch (d.kv_dtype) {
    case PA_F32: hipLaunchKernelGGL((paged_attn_append<KV_F32, false>), grid, dim3(kWave), 0, st, a); break;
    case PA_BF16:
        if (bf) hipLaunchKernelGGL((paged_attn_append<KV_BF16, true>), grid, dim3(kWave), 0, st, a);
        else hipLaunchKernelGGL((paged_attn_append<KV_BF16, false>), grid, dim3(kWave), 0, st, a);
        break;
    default:
        if (bf) hipLaunchKernelGGL((paged_attn_append<KV_FP8, true>), grid, dim3(kWave), 0, st, a);
        else hipLaunchKernelGGL((paged_attn_append<KV_FP8, false>), grid, dim3(kWave), 0, st, a);
        break;
    }
    hipError_t e = hipGetLastError();
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
