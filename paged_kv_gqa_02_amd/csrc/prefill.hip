// prefill.hip -- chunked-prefill attention over the paged KV cache on MI355X
// (gfx950): many query rows per sequence, each attending to every key of the
// earlier chunks and causally within its own chunk.
//
// Sources: "Latency and cost in production" §10.2.6 (chunked prefill splits a
// long prompt's prefill into chunks interleaved with decode steps) and
// "Batching, speculative decoding, paged attention" §5.3.15 (a later chunk
// attends again to the earlier chunks' KV), over the block-table gather of
// §5.3.7 and the online softmax of "Latency and cost in production" §10.1.2.
// The result is the causal verify of include/paged_attn.h with large n: row i
// of a sequence with L keys sees keys 0 .. L - n + i.
//
// Design (gfx950, wave64).  The work is a dense contraction (about 630 FLOP
// per HBM byte at a 512-token chunk), so it is laid out for the MFMA pipes:
//  * one workgroup = 8 waves = 256 query rows of one (sequence, kv head);
//    each wave owns 32 rows as two 16-row MFMA tiles.  Two waves per SIMD let
//    one wave's softmax arithmetic overlap the other's MFMAs;
//  * the keys are walked in steps of two pages (32 tokens).  The workgroup
//    copies each pair once into a ring of four LDS stages with direct
//    global-to-LDS loads, three pairs ahead of the one being consumed, so no
//    register holds data in flight.  Pages keep the pool's layouts: a wave's
//    K operand is one contiguous KiB per LDS read, a V operand four 256-byte
//    rows.  E4M3 pages are converted to bf16 (exactly) as operands are read,
//    their scales applied to the scores and probabilities.  bf16 V operands
//    come straight from LDS with gfx950's transposing read (ds_read_b64_tr_b16),
//    V rows being stored with a 16-byte-chunk XOR swizzle (chosen per lane in
//    the direct copy) so that those reads are free of bank conflicts;
//  * QK^T is v_mfma_f32_16x16x32_bf16 per page (tokens as M, rows as N); PV is
//    the same instruction over the 32 tokens of the pair: the K index of the
//    MFMA is free to enumerate tokens in any order, so the two pages' QK
//    outputs, held lane by lane, are already the PV B operand, and the two
//    pages' transposed V fragments concatenate into the A operand;
//  * online softmax in the log2 domain with the lazy rescale of the decode
//    kernel, the scale folded into the exponent's FMA; bf16 row sums come from
//    one more MFMA with an all-ones operand (the sum of exactly the bf16
//    weights that enter PV).  Only pairs that cross a row's causal limit are
//    masked, and pairs beyond every row's limit are never visited.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "cdna4.h"
#include "prefill.h"

namespace {

using namespace cdna4;

constexpr int kPage = 16;
constexpr int kHeadDim = 128;
constexpr int kSlab = kPage * kHeadDim;
constexpr int kWave = 64;
constexpr int kWaves = 8;                              // two per SIMD
constexpr int kTiles = 2;                              // 16-row tiles per wave
constexpr int kThreads = kWaves * kWave;
constexpr int kRowsPerWave = 16 * kTiles;
static_assert(kWaves * kRowsPerWave == kPrefillRows, "rows per workgroup");
constexpr int kStages = 4;                             // LDS ring of page pairs
constexpr float kNoMax = -1.0e30f;
constexpr float kRescaleSlack = 8.0f;

// One pair of pages in LDS, exactly as in the pool: [K page 0][K page 1]
// [V page 0][V page 1], each one (page, kv head) slab of 16 * 128 elements.
template <bool FP8> struct Layout {
    static constexpr int kElem = FP8 ? 1 : 2;
    static constexpr int kPageBytes = kSlab * kElem;            // 4 KiB bf16, 2 KiB fp8
    static constexpr int kStage = 4 * kPageBytes;
    static constexpr int kLoadsPerWave = kStage / 1024 / kWaves;   // 1 KiB per wave instruction
};

// Asynchronous copy of 16 bytes per lane from global memory straight into LDS:
// lane l's bytes (base + voff) land at lds + 16 l, so one wave instruction
// fills 1 KiB.  base and lds are wave-uniform (scalar registers).  Issued as
// inline assembly so that the compiler does not wait for it before every LDS
// read; the kernel counts these loads itself (s_waitcnt vmcnt) and there are
// no other global loads in its main loop.
__device__ __forceinline__ void dma16(const void* src, uint32_t voff, uint32_t lds)
{
    const uint64_t addr = reinterpret_cast<uint64_t>(src);
    // (the builtin returns a signed int: widen through uint32_t, never sign-extend)
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    const uint64_t base = (uint64_t)lo | ((uint64_t)hi << 32);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 1\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(lds)
                 : "memory");
}

template <int N>
__device__ __forceinline__ void wait_dma()
{
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// bf16 V rows in LDS: 16-byte chunk c of row r is stored at chunk c ^ vswz(r),
// so that the eight rows one transposing read touches fall in distinct banks.
__device__ __forceinline__ int vswz(int row) { return 2 * (row & 7); }

// Pair j into its stage, 1 KiB per wave instruction: piece p of the stage is
// slab p / (pieces per slab) (K page 0, K page 1, V page 0, V page 1) at
// offset 1 KiB * (p % pieces per slab); wave w copies pieces w * n .. w * n + n - 1.
// A bf16 V piece holds rows 4i .. 4i + 3; lane l lands at row 4i + l / 16,
// chunk l % 16, and fetches the chunk that the swizzle puts there.
template <bool FP8>
__device__ __forceinline__ void issue_pair(const PrefillArgs& a, const int32_t* ids, int npairs,
                                           int j, int kh, int wave, int lane, uint32_t stage_lds)
{
    using Ly = Layout<FP8>;
    constexpr int kPieces = Ly::kPageBytes / 1024;       // per slab
    const int jj = min(j, npairs - 1);                   // past the end: a harmless repeat
#pragma unroll
    for (int i = 0; i < Ly::kLoadsPerWave; ++i) {
        const int piece = wave * Ly::kLoadsPerWave + i;
        const int slab = piece / kPieces;
        // page ids are wave-uniform: the slab address is formed on the scalar unit
        const int page = __builtin_amdgcn_readfirstlane(ids[2 * jj + (slab & 1)]);
        const uint8_t* src = static_cast<const uint8_t*>(slab < 2 ? a.k : a.v) +
                             ((int64_t)page * a.page_stride + (int64_t)kh * kSlab) * Ly::kElem +
                             1024 * (piece % kPieces);
        uint32_t voff = 16 * lane;
        if (!FP8 && slab >= 2) {
            const int row = 4 * (piece % kPieces) + (lane >> 4);
            voff = 256 * (lane >> 4) + 16 * ((lane & 15) ^ vswz(row));
        }
        dma16(src, voff, __builtin_amdgcn_readfirstlane(stage_lds + 1024 * piece));
    }
}

// E4M3 K operand c (dims 32c + 8g .. +8 of token l16, the bf16 layout's chunk
// 4c + g): bytes 8 (g % 2) .. +8 of fp8 chunk 2c + g / 2 of that token
__device__ __forceinline__ u32x4 k_operand_fp8(const uint8_t* kp, int c, int l16, int g)
{
    const u32x2 w = *reinterpret_cast<const u32x2*>(kp + ((2 * c + (g >> 1)) * 16 + l16) * 16 +
                                                    8 * (g & 1));
    return fp8x8_to_bf16x8(w[0], w[1]);
}

template <bool FP8>
__global__ __launch_bounds__(kThreads) void paged_attn_prefill(PrefillArgs a)
{
    using Ly = Layout<FP8>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * Ly::kStage];
    __shared__ int32_t ids[kPrefillMaxPages];
    __shared__ float scales[FP8 ? 2 * kPrefillMaxPages : 1];   // k then v, per page of the block

    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wave = t / kWave;
    const int l16 = lane & 15;
    const int g = lane >> 4;

    // heavy row blocks first; all row blocks of one (sequence, kv head) share
    // blockIdx mod (B * Hkv), hence one XCD and its L2 when that is a multiple of 8
    const int bh_count = a.batch * a.hkv;
    const int bh = blockIdx.x % bh_count;
    const int rb = a.row_blocks - 1 - (int)(blockIdx.x / bh_count);
    const int kh = bh % a.hkv;
    const int b = bh / a.hkv;

    // lengths clamped to what the block table and the page-id table describe:
    // arrays that break the contract give wrong numbers, never a stray access
    const int L = max(min(min(a.seq_lens[b], a.max_pages * kPage), kPrefillMaxPages * kPage), 1);
    const int row0 = rb * kPrefillRows;
    const int last_row = min(row0 + kPrefillRows, a.rows) - 1;
    // keys the block needs: up to the causal limit of its last row
    const int key_end = max(min(L, L - a.n + last_row / a.group + 1), 1);
    const int npages = (key_end + kPage - 1) / kPage;
    const int npairs = (npages + 1) / 2;
    const int seq_pages = (L + kPage - 1) / kPage;

    // query rows of this wave (MFMA B-operand layout: lane holds row l16 of a tile)
    bf16x8 qf[kTiles][4];
    int lim[kTiles];
    const int wrow0 = row0 + wave * kRowsPerWave;
#pragma unroll
    for (int tt = 0; tt < kTiles; ++tt) {
        const int r = wrow0 + tt * 16 + l16;
        const bool valid = r < a.rows;
        const int i = valid ? r / a.group : 0;
        const int h = kh * a.group + (valid ? r - i * a.group : 0);
        const uint16_t* qrow = a.q + (((int64_t)b * a.n + i) * a.hq + h) * kHeadDim;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * g);
            qf[tt][c] = __builtin_bit_cast(bf16x8, valid ? x : u32x4{0u, 0u, 0u, 0u});
        }
        lim[tt] = valid ? L - a.n + i : L - 1;     // padding rows see every live key
    }
    // the smallest limit among this wave's rows decides which pairs need masks
    const int wave_lim = L - a.n + min(wrow0, a.rows - 1) / a.group;

    // page ids (and E4M3 scales) of the block, clamped to the sequence and the pool
    const int32_t* bt_row = a.block_table + (int64_t)b * a.max_pages;
    for (int p = t; p < 2 * npairs; p += kThreads) {
        const int id = min(max(bt_row[min(p, seq_pages - 1)], 0), a.num_pages - 1);
        ids[p] = id;
        if constexpr (FP8) {
            scales[p] = a.k_scale[(int64_t)id * a.hkv + kh];
            scales[kPrefillMaxPages + p] = a.v_scale[(int64_t)id * a.hkv + kh];
        }
    }
    __syncthreads();

    f32x4 acc[kTiles][8];
    f32x4 lsum[kTiles];      // bf16 pools: row sums of the weights, from an all-ones MFMA
    float m[kTiles], l[kTiles];
#pragma unroll
    for (int tt = 0; tt < kTiles; ++tt) {
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[tt][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        lsum[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[tt] = kNoMax;
        l[tt] = 0.f;
    }
    // A operand of all ones (bf16 1.0 = 0x3F80): C[m][row] = sum over the 32
    // tokens of the row's weights, exactly the bf16 values that enter PV
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u,
                                                         0x3F803F80u});

    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
    // prologue: pairs 0 .. kStages - 2 in flight
#pragma unroll
    for (int j = 0; j < kStages - 1; ++j)
        issue_pair<FP8>(a, ids, npairs, j, kh, wave, lane, lds0 + j * Ly::kStage);

    for (int j = 0; j < npairs; ++j) {
        // this wave's part of pair j has landed once at most the later pairs'
        // loads are outstanding; the barrier then covers every wave's part, and
        // every wave is done with pair j - 1, whose stage is refilled next
        wait_dma<(kStages - 2) * Ly::kLoadsPerWave>();
        __syncthreads();
        issue_pair<FP8>(a, ids, npairs, j + kStages - 1, kh, wave, lane,
                        lds0 + ((j + kStages - 1) % kStages) * Ly::kStage);

        uint8_t* st = lds + (j % kStages) * Ly::kStage;
        const int base = 32 * j;
        const bool need_mask = base + 31 > wave_lim;
        if (base + 31 >= L) {
            // the pair holding the sequence end: V rows past it may hold NaN,
            // which a zero weight would still carry through the MFMA, so they
            // are zeroed in LDS (once per workgroup, on this pair only)
            constexpr int kRowBytes = kHeadDim * Ly::kElem;
            for (int e = t; e < 32 * kRowBytes / 16; e += kThreads) {
                const int tok = e / (kRowBytes / 16);
                if (base + tok >= L)
                    *reinterpret_cast<u32x4*>(st + (2 + tok / 16) * Ly::kPageBytes +
                                              (tok % 16) * kRowBytes + 16 * (e % (kRowBytes / 16))) =
                        u32x4{0u, 0u, 0u, 0u};
            }
            __syncthreads();
        }
        float ks[2] = {1.f, 1.f}, vs[2] = {1.f, 1.f};
        if constexpr (FP8) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                ks[h] = scales[2 * j + h];
                vs[h] = scales[kPrefillMaxPages + 2 * j + h];
            }
        }
        // K operands of both pages
        u32x4 kf[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint8_t* kp = st + h * Ly::kPageBytes;
                if constexpr (FP8)
                    kf[h][c] = k_operand_fp8(kp, c, l16, g);
                else
                    kf[h][c] = *reinterpret_cast<const u32x4*>(kp + 1024 * c + 16 * lane);
            }
        // V operands over the 32 tokens: {page 0 rows 4g..4g+3, page 1 rows 4g..4g+3}
        bf16x8 va[8];
        {
            i16x4 av[2][8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint8_t* vp = st + (2 + h) * Ly::kPageBytes;
                if constexpr (FP8) {
                    // a[db] = {V[4g + s][8 l16 + db], s = 0..3}: rows read, then permuted
                    u32x4 vr[4];
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) {
                        const u32x2 w = *reinterpret_cast<const u32x2*>(vp + (4 * g + s4) * kHeadDim + 8 * l16);
                        vr[s4] = fp8x8_to_bf16x8(w[0], w[1]);
                    }
                    v_operands(av[h], vr);
                } else {
                    // a[db] = {V[4g + k][16 db + l16], k = 0..3} from one transposing
                    // read: in each 16-lane group, lane j names 4 elements of row
                    // 4g + j / 4 at dims 16 db + 4 (j % 4), and lane i receives the
                    // i % 4-th element of lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4
                    const int row = 4 * g + (l16 >> 2);
                    const uint8_t* rp = vp + 2 * kHeadDim * row + 8 * (l16 & 1);
#pragma unroll
                    for (int db = 0; db < 8; ++db) {
                        const int chunk = 2 * db + ((l16 & 3) >> 1);
                        av[h][db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4*)(rp + 16 * (chunk ^ vswz(row))));
                    }
                }
            }
#pragma unroll
            for (int db = 0; db < 8; ++db)
                va[db] = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(av[0][db], av[1][db], 0, 1, 2, 3, 4, 5, 6, 7));
        }
        // Phase 1, every tile: raw scores.  The scale (and an E4M3 page's K
        // scale) is folded into the exponent: p = exp2(s * f - m) with f > 0,
        // so max(s * f) = f * max(s).
        float f[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) f[h] = FP8 ? a.scale_log2 * ks[h] : a.scale_log2;
        float sc[kTiles][8];
#pragma unroll
        for (int tt = 0; tt < kTiles; ++tt)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[h][c]),
                                                                 qf[tt][c], s4, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) sc[tt][4 * h + v] = s4[v];
            }
        if (need_mask) {
#pragma unroll
            for (int tt = 0; tt < kTiles; ++tt)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int tok = base + 16 * (e >> 2) + 4 * g + (e & 3);
                    sc[tt][e] = tok <= lim[tt] ? sc[tt][e] : -INFINITY;
                }
        }
        // Phase 2: row maxima, and one rescale branch for all tiles (a tile
        // whose maximum did not move is multiplied by exp2(0) = 1, exactly)
        float mx[kTiles];
        bool grow_any = false;
#pragma unroll
        for (int tt = 0; tt < kTiles; ++tt) {
            float x = -INFINITY;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float ph = fmaxf(fmaxf(sc[tt][4 * h], sc[tt][4 * h + 1]),
                                       fmaxf(sc[tt][4 * h + 2], sc[tt][4 * h + 3]));
                x = fmaxf(x, ph * f[h]);
            }
            mx[tt] = group_max(x);
            grow_any |= mx[tt] > m[tt] + kRescaleSlack;
        }
        if (__any(grow_any)) {
#pragma unroll
            for (int tt = 0; tt < kTiles; ++tt) {
                const float mnew = mx[tt] > m[tt] + kRescaleSlack ? mx[tt] : m[tt];
                const float alpha = fast_exp2(m[tt] - mnew);
                m[tt] = mnew;
                l[tt] *= alpha;
                lsum[tt] *= alpha;
#pragma unroll
                for (int db = 0; db < 8; ++db) acc[tt][db] *= alpha;
            }
        }
        // Phase 3, one basic block: weights and PV of every tile, so that one
        // tile's exponentials can issue while the other's MFMAs run
#pragma unroll
        for (int tt = 0; tt < kTiles; ++tt) {
            uint32_t pb[8];
            float psum = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = fast_exp2(__builtin_fmaf(sc[tt][e], f[e >> 2], -m[tt]));
                pb[e] = bf16_bits(FP8 ? p * vs[e >> 2] : p);
                if constexpr (FP8) psum += p;
            }
            const bf16x8 pf = __builtin_bit_cast(
                bf16x8, u32x4{pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16), pb[4] | (pb[5] << 16),
                              pb[6] | (pb[7] << 16)});
            if constexpr (FP8)
                l[tt] += psum;      // the V scale rides on the weights, not on their sum
            else
                lsum[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf, lsum[tt], 0, 0, 0);
#pragma unroll
            for (int db = 0; db < 8; ++db)
                acc[tt][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], pf, acc[tt][db], 0, 0, 0);
        }
    }
    // no copy may still be writing this workgroup's LDS when it exits
    wait_dma<0>();

    // epilogue: lane holds O[row l16][32 g + 8 v + db] (E4M3 pools) or
    // O[row l16][16 db + 4 g + v] (bf16 pools) of each tile
#pragma unroll
    for (int tt = 0; tt < kTiles; ++tt) {
        const int r = wrow0 + tt * 16 + l16;
        const float inv = 1.0f / (FP8 ? group_sum(l[tt]) : lsum[tt][0]);
        if (r < a.rows) {
            const int i = r / a.group;
            const int h = kh * a.group + (r - i * a.group);
            uint16_t* orow = a.out + (((int64_t)b * a.n + i) * a.hq + h) * kHeadDim;
            if constexpr (FP8) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w[e] = bf16_bits(acc[tt][2 * e][v] * inv) |
                               (bf16_bits(acc[tt][2 * e + 1][v] * inv) << 16);
                    *reinterpret_cast<u32x4*>(orow + 32 * g + 8 * v) = u32x4{w[0], w[1], w[2], w[3]};
                }
            } else {
#pragma unroll
                for (int db = 0; db < 8; ++db) {
                    const f32x4 x = acc[tt][db] * inv;
                    *reinterpret_cast<u32x2*>(orow + 16 * db + 4 * g) =
                        u32x2{bf16_bits(x[0]) | (bf16_bits(x[1]) << 16),
                              bf16_bits(x[2]) | (bf16_bits(x[3]) << 16)};
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, bool fp8, hipStream_t st)
{
    const dim3 grid((unsigned)((int64_t)a.batch * a.hkv * a.row_blocks));
    if (fp8)
        hipLaunchKernelGGL(paged_attn_prefill<true>, grid, dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(paged_attn_prefill<false>, grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}
