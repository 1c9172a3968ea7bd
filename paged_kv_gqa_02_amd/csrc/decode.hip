// decode.hip -- paged GQA decode / verify attention kernels for MI355X
// (gfx950): the partition kernel and the split-K reduce.
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
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "cdna4.h"
#include "decode.h"

namespace {

using namespace cdna4;
using Args = DecodeArgs;

// Running max before any key is seen.  Finite, so exp2(m_old - m_new) is
// never inf - inf; masked scores are -inf and give exp2(-inf) = 0.
constexpr float kNoMax = -1.0e30f;
constexpr int kAccStride = kHeadDim + 4;    // LDS row stride of the wave merge (bank skew)
// The running max of a row moves only when a page's max exceeds it by more
// than this many log2 units, so weights stay <= 2^8 (safe in fp32 and bf16)
// and the accumulator is rescaled on few pages.
constexpr float kRescaleSlack = 8.0f;

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
// only one wave per SIMD keeps pages in flight (verify 40 -> 33 us).  The bf16
// one-tile kernel with up to three pages in flight (decode) asks for two as
// well: it then fits 179 VGPRs and keeps its accumulators out of AGPRs, whose
// per-page copies out and back it otherwise pays (same speed, HBM-bound).  The
// fp8 one-tile kernel with a two-page pipeline fits four waves per SIMD in
// 116 VGPRs (2% faster).  Deeper pipelines keep the compiler's choice, which
// does not spill; they are meant for plans with one workgroup per CU.
template <int KV, int NT, int PF>
constexpr int min_waves_per_simd()
{
    if (KV != KV_F32 && PF <= 3 && (NT == 2 || (NT == 1 && KV == KV_BF16))) return 2;
    return (NT == 1 && KV == KV_FP8 && PF == 2) ? 4 : 1;
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
    // (the first round of this wave's page ids: see the pipeline below)
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

    // this wave's pages: pg0 + wave + j * W, j < nj.  A lane holds one page id,
    // so the wave takes its ids in rounds of 64 pages; the next round's ids are
    // requested when a round starts.  Automatic plans keep nj <= 64 (one round)
    // up to 64 * W * kMaxSplits pages per sequence.
    const int nj = (pg1 - pg0 - wave + W - 1) / W;
    const int id_last = min(pg0 + a.part_pages, a.max_pages) - 1;

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
    // Loads are unconditional (indices past the round's last page repeat that
    // page) so that the wait before each use covers only that page's loads.
    int ids = raw_id;                               // round 0: requested with the length
    for (int r0 = 0; r0 < nj; r0 += kWave) {
        const int nr = min(nj - r0, kWave);
        const int my_id = (lane < nr) ? min(max(ids, 0), a.num_pages - 1) : 0;
        if (r0 + kWave < nj)
            ids = bt_row[min(pg0 + wave + (r0 + kWave + lane) * W, id_last)];
        auto phys_of = [&](int j) { return __builtin_amdgcn_readlane(my_id, min(j, nr - 1)); };
        Page<KV> buf[PF];
#pragma unroll
        for (int st = 0; st < PF - 1; ++st) load_page(buf[st], a, phys_of(st), kh, l16, g);
        int j0 = 0;
        for (; j0 + PF <= nr; j0 += PF) {
#pragma unroll
            for (int st = 0; st < PF; ++st) {
                load_page(buf[(st + PF - 1) % PF], a, phys_of(j0 + st + PF - 1), kh, l16, g);
                consume(buf[st], r0 + j0 + st);
            }
        }
#pragma unroll
        for (int st = 0; st < PF - 1; ++st)
            if (j0 + st < nr) consume(buf[st], r0 + j0 + st);
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
// launches
// ---------------------------------------------------------------------------
template <int KV, int NT, int W, int PF>
void launch_variant(const Args& a, int grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    // the events are attached to the dispatch itself: no marker between them
    hipExtLaunchKernelGGL((paged_attn_partition<KV, NT, W, PF>), dim3(grid), dim3(W * kWave), 0,
                          st, e0, e1, 0, a);
}

// (waves, prefetch) variants are instantiated for the bf16 and fp8 paths with
// one or two row tiles; every other shape runs the default variant
template <int KV, int NT>
void launch_tuned(int waves, int prefetch, const Args& a, int grid, hipStream_t st,
                  hipEvent_t e0, hipEvent_t e1)
{
    if constexpr (KV == KV_F32 || NT > 2) {
        launch_variant<KV, NT, kDefaultWaves, 2>(a, grid, st, e0, e1);
    } else {
        switch (waves * 10 + prefetch) {
        case 42: launch_variant<KV, NT, 4, 2>(a, grid, st, e0, e1); break;
        case 43: launch_variant<KV, NT, 4, 3>(a, grid, st, e0, e1); break;
        case 44: launch_variant<KV, NT, 4, 4>(a, grid, st, e0, e1); break;
        case 45: launch_variant<KV, NT, 4, 5>(a, grid, st, e0, e1); break;
        case 46: launch_variant<KV, NT, 4, 6>(a, grid, st, e0, e1); break;
        case 82: launch_variant<KV, NT, 8, 2>(a, grid, st, e0, e1); break;
        case 83: launch_variant<KV, NT, 8, 3>(a, grid, st, e0, e1); break;
        case 84: launch_variant<KV, NT, 8, 4>(a, grid, st, e0, e1); break;
        default: launch_variant<KV, NT, 4, 2>(a, grid, st, e0, e1); break;
        }
    }
}

template <int KV>
void launch_rows(int nt, int waves, int prefetch, const Args& a, int grid, hipStream_t st,
                 hipEvent_t e0, hipEvent_t e1)
{
    switch (nt) {
    case 1: launch_tuned<KV, 1>(waves, prefetch, a, grid, st, e0, e1); break;
    case 2: launch_tuned<KV, 2>(waves, prefetch, a, grid, st, e0, e1); break;
    case 3: launch_tuned<KV, 3>(waves, prefetch, a, grid, st, e0, e1); break;
    default: launch_tuned<KV, 4>(waves, prefetch, a, grid, st, e0, e1); break;
    }
}

}  // namespace

hipError_t launch_partition(const DecodeArgs& a, int kv, int row_tiles, int waves, int prefetch,
                            int grid, hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end)
{
    switch (kv) {
    case KV_F32: launch_rows<KV_F32>(row_tiles, waves, prefetch, a, grid, st, ev_begin, ev_end); break;
    case KV_BF16: launch_rows<KV_BF16>(row_tiles, waves, prefetch, a, grid, st, ev_begin, ev_end); break;
    default: launch_rows<KV_FP8>(row_tiles, waves, prefetch, a, grid, st, ev_begin, ev_end); break;
    }
    return hipGetLastError();
}

hipError_t launch_reduce(const DecodeArgs& a, bool f32_out, unsigned rows_out, hipStream_t st)
{
    if (f32_out)
        hipLaunchKernelGGL(paged_attn_reduce<float>, dim3(rows_out), dim3(kReduceThreads), 0, st, a);
    else
        hipLaunchKernelGGL(paged_attn_reduce<uint16_t>, dim3(rows_out), dim3(kReduceThreads), 0, st,
                           a);
    return hipGetLastError();
}
