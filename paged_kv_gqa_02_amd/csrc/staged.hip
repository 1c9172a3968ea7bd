// staged.hip -- attention with the KV pages staged once in LDS and shared by
// every wave of a workgroup, for calls with many query rows per (sequence, kv
// head): chunked prefill and draft-tree verification, on MI355X (gfx950).
//
// Sources: "Latency and cost in production" §10.2.6 (chunked prefill splits a
// long prompt's prefill into chunks interleaved with decode steps) and
// "Batching, speculative decoding, paged attention" §5.3.15 (a later chunk
// attends again to the earlier chunks' KV) and §5.3.13 (a tree of candidate
// branches verified in one forward with tree attention), over the block-table
// gather of §5.3.7 and the online softmax of "Latency and cost in production"
// §10.1.2.  The results are those of include/paged_attn.h: row i of a sequence
// with L keys sees keys 0 .. L - n + i (causal), or every context key and its
// draft-tree ancestors (tree).
//
// Design (gfx950, wave64):
//  * a workgroup takes WAVES * TILES * 16 query rows of one (sequence, kv head)
//    and one context partition; each wave owns TILES 16-row MFMA tiles.
//    Chunked prefill uses 4 waves x 2 tiles (128 rows), draft trees 4 waves
//    x 1 tile (64 rows, few registers per wave), both with two key groups
//    (below): a row block's chain of pairs, which sets its workgroup's time,
//    is cut in two.  Chunked-prefill row blocks are dispatched heaviest first;
//  * the keys are walked in pairs of pages (32 tokens), one pair per key group
//    and step.  The workgroup copies each pair once into a ring of four LDS
//    stages with direct global-to-LDS loads, three steps ahead of the one
//    being consumed, so no register holds data in flight.  Pages keep the pool's layouts: a wave's
//    K operand is one contiguous KiB per LDS read.  E4M3 pages are converted
//    to bf16 (exactly) as operands are read, their scales applied to the
//    scores and probabilities.  bf16 V operands come straight from LDS with
//    gfx950's transposing read (ds_read_b64_tr_b16), V rows being stored with
//    a 16-byte-chunk XOR swizzle (chosen per lane in the direct copy) so that
//    those reads are free of bank conflicts;
//  * QK^T is v_mfma_f32_16x16x32_bf16 per page (tokens as M, rows as N); PV is
//    the same instruction over the 32 tokens of the pair: the K index of the
//    MFMA is free to enumerate tokens in any order, so the two pages' QK
//    outputs, held lane by lane, are already the PV B operand, and the two
//    pages' transposed V fragments concatenate into the A operand;
//  * online softmax in the log2 domain with the lazy rescale of the decode
//    kernel, the scale folded into the exponent's FMA; bf16 row sums come from
//    one more MFMA with an all-ones operand (the sum of exactly the bf16
//    weights that enter PV).  Per pair, both tiles' scores come first, then one
//    rescale branch, then the weights and PV of every tile in one basic block.
//    Only pairs that reach a row's masked keys are masked, and pairs beyond
//    every causal row's limit are never visited;
//  * a partition of a split sequence ends with its (max, sum, accumulator)
//    partial in the split-K reduce kernel's layout.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "cdna4.h"
#include "staged.h"

namespace {

using namespace cdna4;

constexpr int kPage = 16;
constexpr int kHeadDim = 128;
constexpr int kSlab = kPage * kHeadDim;
constexpr int kWave = 64;
constexpr float kNoMax = -1.0e30f;
// LDS ring depth in page pairs.  Four stages (three pairs in flight) keep two
// draft-tree workgroups on a CU and the accumulators in VGPRs; deeper rings
// measured no faster on MI355X.
constexpr int kRing = 4;
// key groups: the draft-tree kernel (8 waves, each pair of waves on one row
// tile) and the chunked-prefill kernel (8 waves, each pair on two row tiles)
constexpr int kTreeKeyGroups = 2;
constexpr int kPrefillKeyGroups = 2;
constexpr float kRescaleSlack = 8.0f;

// One pair of pages in LDS, in the pool's layouts: [K page 0][K page 1]
// [V page 0][V page 1], each one (page, kv head) slab of 16 * 128 elements.
template <bool FP8, int WAVES> struct Layout {
    static constexpr int kElem = FP8 ? 1 : 2;
    static constexpr int kPageBytes = kSlab * kElem;            // 4 KiB bf16, 2 KiB fp8
    static constexpr int kStage = 4 * kPageBytes;
    static constexpr int kLoadsPerWave = kStage / 1024 / WAVES;  // 1 KiB per wave instruction
    static_assert(kLoadsPerWave * 1024 * WAVES == kStage, "stage split over the waves");
};

// Asynchronous copy of 16 bytes per lane from global memory straight into LDS:
// lane l's bytes (base + voff) land at lds + 16 l, so one wave instruction
// fills 1 KiB.  base and lds are wave-uniform (scalar registers).  Issued as
// inline assembly so that the compiler does not wait for it before every LDS
// read; the kernel counts these loads itself (s_waitcnt vmcnt) and there are
// no other global loads in its main loop.  NT: a non-temporal load, for pages
// that no other workgroup reads again (draft trees: 5 % faster); chunked
// prefill keeps the default policy, as its row blocks re-read pages through L2.
template <bool NT>
__device__ __forceinline__ void dma16(const void* src, uint32_t voff, uint32_t lds)
{
    const uint64_t addr = reinterpret_cast<uint64_t>(src);
    // (the builtin returns a signed int: widen through uint32_t, never sign-extend)
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    const uint64_t base = (uint64_t)lo | ((uint64_t)hi << 32);
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 1\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                     :
                     : "v"(voff), "s"(base), "s"(lds)
                     : "memory");
    else
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

// Waits until at most `ahead` (<= N, wave-uniform) later steps of L loads each
// are outstanding.
template <int N, int L>
__device__ __forceinline__ void wait_steps(int ahead)
{
    if constexpr (N == 0) {
        wait_dma<0>();
    } else {
        if (ahead >= N)
            wait_dma<N * L>();
        else
            wait_steps<N - 1, L>(ahead);
    }
}

// bf16 V rows in LDS: 16-byte chunk c of row r is stored at chunk c ^ vswz(r),
// so that the eight rows one transposing read touches fall in distinct banks.
__device__ __forceinline__ int vswz(int row) { return 2 * (row & 7); }

// Pair j into its stage, 1 KiB per wave instruction: piece p of the stage is
// slab p / (pieces per slab) (K page 0, K page 1, V page 0, V page 1) at
// offset 1 KiB * (p % pieces per slab); wave w copies pieces w * n .. w * n + n - 1.
// A bf16 V piece holds rows 4i .. 4i + 3; lane l lands at row 4i + l / 16,
// chunk l % 16, and fetches the chunk that the swizzle puts there.
// ids[last] is the sequence's last page: a pair reaching past it repeats that
// page (its tokens are masked and its V rows zeroed).
template <bool FP8, int WAVES, bool NT>
__device__ __forceinline__ void issue_pair(const StagedArgs& a, const int32_t* ids, int npairs,
                                           int last, int j, int kh, int wave, int lane,
                                           uint32_t stage_lds)
{
    using Ly = Layout<FP8, WAVES>;
    constexpr int kPieces = Ly::kPageBytes / 1024;       // per slab
    const int jj = uni(min(j, npairs - 1));              // past the end: a harmless repeat
    // both page ids of the pair in one LDS read, before any copy is issued (each
    // copy is a compiler barrier for memory, which would re-read them); page ids
    // are wave-uniform, so slab addresses are formed on the scalar unit
    const uint64_t pp = *reinterpret_cast<const uint64_t*>(ids + 2 * jj);
    const int p0 = uni((int)(uint32_t)pp);
    const int p1 = uni((int)(uint32_t)(pp >> 32));
    const int page[2] = {p0, 2 * jj + 1 <= last ? p1 : p0};
    const uint8_t* src[Ly::kLoadsPerWave];
    uint32_t voff[Ly::kLoadsPerWave];
#pragma unroll
    for (int i = 0; i < Ly::kLoadsPerWave; ++i) {
        const int piece = wave * Ly::kLoadsPerWave + i;
        const int slab = piece / kPieces;
        src[i] = static_cast<const uint8_t*>(slab < 2 ? a.k : a.v) +
                 ((int64_t)page[slab & 1] * a.page_stride + (int64_t)kh * kSlab) * Ly::kElem +
                 1024 * (piece % kPieces);
        voff[i] = 16 * lane;
        if (!FP8 && slab >= 2) {
            const int row = 4 * (piece % kPieces) + (lane >> 4);
            voff[i] = 256 * (lane >> 4) + 16 * ((lane & 15) ^ vswz(row));
        }
    }
#pragma unroll
    for (int i = 0; i < Ly::kLoadsPerWave; ++i)
        dma16<NT>(src[i], voff[i],
              __builtin_amdgcn_readfirstlane(stage_lds + 1024 * (wave * Ly::kLoadsPerWave + i)));
}

// E4M3 K operand c (dims 32c + 8g .. +8 of token l16, the bf16 layout's chunk
// 4c + g): bytes 8 (g % 2) .. +8 of fp8 chunk 2c + g / 2 of that token
__device__ __forceinline__ u32x4 k_operand_fp8(const uint8_t* kp, int c, int l16, int g)
{
    const u32x2 w = *reinterpret_cast<const u32x2*>(kp + ((2 * c + (g >> 1)) * 16 + l16) * 16 +
                                                    8 * (g & 1));
    return fp8x8_to_bf16x8(w[0], w[1]);
}

// STAGES: LDS ring of page pairs (STAGES - 1 pairs in flight); MAXP: most
// pages of one partition, whose page ids (and E4M3 scales) are held in LDS,
// with the odd page its last pair may reach into the next partition.  Asking
// for at least two waves per SIMD caps a lane at 256 registers, so the MFMA
// accumulators stay in VGPRs, where the rescale can reach them (in AGPRs they
// would be copied out and back on every pair).
//
// KG key groups: the workgroup has WAVES * KG waves; waves w and w + WAVES
// hold the same query rows (WAVES row waves) and walk alternate pairs of the
// partition (key group k takes pairs KG j + k), each group copying its own
// pairs; their online-softmax states merge in LDS at the end.  This puts two
// waves on every SIMD, and twice the copies in flight, without a second
// workgroup's entry cost; for chunked prefill it halves the chain of pairs of
// the heaviest row blocks, which set the kernel's time.
template <bool FP8, int WAVES, int TILES, bool TREE, int STAGES, int MAXP, int KG>
__global__ __launch_bounds__(WAVES * KG * kWave, 2) void paged_attn_staged(StagedArgs a)
{
    using Ly = Layout<FP8, WAVES>;
    constexpr int kStages = STAGES;
    constexpr int kThreads = WAVES * KG * kWave;
    constexpr int kRowsPerWave = 16 * TILES;
    constexpr int kRows = WAVES * kRowsPerWave;
    constexpr int kStep = KG * Ly::kStage;         // LDS bytes of one step (KG pairs)
    static_assert((kStages - 2) * Ly::kLoadsPerWave <= 63, "vmcnt counts at most 63 loads");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * kStep];
    constexpr int kIds = MAXP + 2;
    __shared__ __attribute__((aligned(8))) int32_t ids[kIds];
    __shared__ float scales[FP8 ? 2 * kIds : 1];   // k then v, per page of the block

    // (the index builtins: this file is built without IEEE mode, and the
    // device library's threadIdx / blockIdx helpers, built with it, would be
    // called rather than inlined)
    const int t = (int)__builtin_amdgcn_workitem_id_x();
    const int lane = t & (kWave - 1);
    // (read through readfirstlane, so that the compiler knows them to be
    // wave-uniform and keeps what derives from them in scalar registers)
    const int wave_id = __builtin_amdgcn_readfirstlane(t / kWave);
    const int wave = KG == 1 ? wave_id : wave_id % WAVES;       // row wave
    const int kg = KG == 1 ? 0 : wave_id / WAVES;               // key group
    const int l16 = lane & 15;
    const int g = lane >> 4;

    // Work items are (row block, partition) units, taken in rounds of W =
    // a.workgroups: in round r, workgroup w takes item r * W + w, or
    // r * W + W - 1 - w in odd rounds, so that the items (heaviest first)
    // pair up heavy with light on each workgroup.  Draft trees launch one
    // workgroup per item; chunked prefill one per CU, which then runs its
    // items back to back with no dispatch in between.
    const int items = a.batch * a.hkv * a.row_blocks * a.num_splits;
    // chunked prefill with up to 64 sequences: lane u holds the length of
    // sequence u and its rank by length (longest first, ties by index)
    int my_rank = 0;
    int mine = INT_MIN;
    if constexpr (!TREE) {
        if (a.batch <= kWave) {
            mine = lane < a.batch ? a.seq_lens[lane] : INT_MIN;
            for (int u = 0; u < a.batch; ++u) {
                const int lu = __builtin_amdgcn_readlane(mine, u);
                my_rank += (lu > mine || (lu == mine && u < lane)) ? 1 : 0;
            }
        }
    }
    auto item = [&](const int x) {
        int sp, b, kh, rb, seq_len;
        {
            sp = x % a.num_splits;
            const int rest = x / a.num_splits;
            if constexpr (TREE) {
                // (sequence, kv head) pairs in item order, one row block each
                const int bh_count = a.batch * a.hkv;
                const int bh = rest % bh_count;
                rb = a.row_blocks - 1 - rest / bh_count;
                kh = bh % a.hkv;
                b = bh / a.hkv;
                seq_len = a.seq_lens[b];
            } else {
                // Causal row blocks differ in work: a block of a sequence with c
                // earlier tokens walks c / 32 + (its index + 1) * (tokens per block) / 32
                // pairs, and an item's time follows its pair count.  Items take
                // the slots (sequence rank, row block) heaviest first, sequences
                // ranked by length (longest first).  The kv head is the items'
                // fastest index: the row blocks of one (sequence, kv head) share
                // item mod Hkv, so with workgroups placed round-robin on the 8
                // XCDs (and a multiple of 8 of them) they run on two XCDs at most,
                // one per round direction, whose L2s serve their re-reads.
                kh = rest % a.hkv;
                const int q = rest / a.hkv;
                const int rank = q / a.row_blocks;
                rb = a.row_blocks - 1 - (q - rank * a.row_blocks);
                if (a.batch <= kWave) {
                    const uint64_t hit = __ballot(lane < a.batch && my_rank == rank);
                    b = hit ? (int)__builtin_ctzll(hit) : rank;   // (ranks are a permutation)
                    seq_len = __builtin_amdgcn_readlane(mine, b);
                } else {
                    b = rank;                          // many sequences: index order
                    seq_len = a.seq_lens[b];
                }
            }
            sp = uni(sp);
            b = uni(b);
            kh = uni(kh);
            rb = uni(rb);
        }

        // Every load of the prologue is issued before the first one is waited for:
        // this partition's block-table entries, the query rows and their tree masks
        // (only the sequence length decides what is used of them).
        const int pg0 = sp * a.part_pages;
        const int part = min(a.part_pages, MAXP);     // a larger partition is cut short
        const int32_t* bt_row = a.block_table + (int64_t)b * a.max_pages;
        // Page ids are fetched and staged by the loader threads: in chunked
        // prefill the waves of key groups 1 .., which are idle while group 0
        // writes the previous item's output and so fetch the next item's ids
        // meanwhile; every thread otherwise.  (Unconditional loads from
        // clamped, in-bounds addresses: under a lane mask the compiler would
        // wait for each load before issuing the next.)
        constexpr bool kGroupLoaders = KG > 1 && !TREE;
        constexpr int kLoaders = kGroupLoaders ? (KG - 1) * WAVES * kWave : kThreads;
        const int lt = kGroupLoaders ? t - WAVES * kWave : t;      // < 0: not a loader
        constexpr int kIdLoads = (kIds + kLoaders - 1) / kLoaders;
        int idv[kIdLoads];
        if (lt >= 0) {
#pragma unroll
            for (int k = 0; k < kIdLoads; ++k)
                idv[k] = bt_row[min(pg0 + min(lt + k * kLoaders, part), a.max_pages - 1)];
        }
        const int row0 = rb * kRows;
        const int wrow0 = row0 + wave * kRowsPerWave;
        // query rows of this wave (MFMA B-operand layout: lane holds row l16 of a tile)
        bf16x8 qf[TILES][4];
        int qi[TILES];
        uint64_t tmask[TILES];
#pragma unroll
        for (int tt = 0; tt < TILES; ++tt) {
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
            qi[tt] = valid ? i : -1;
            if constexpr (TREE) {
                const uint64_t mk = a.tree_mask[(int64_t)b * a.n + i];
                tmask[tt] = valid ? mk : ~uint64_t(0);
            }
        }

        // lengths clamped to what the block table describes: arrays that break the
        // contract give wrong numbers, never a stray access
        // (the values below are wave-uniform; readfirstlane keeps them, and the
        // loop control and page addresses derived from them, in scalar registers
        // where a division or a loaded value would otherwise leave them in VGPRs)
        const int L = uni(max(min(seq_len, a.max_pages * kPage), 1));
        const int seq_pages = (L + kPage - 1) / kPage;
        const int nsplit_b = uni(min((seq_pages + a.part_pages - 1) / a.part_pages, a.num_splits));
        if (sp >= nsplit_b) return;                   // this sequence has fewer partitions
        const int last_row = min(row0 + kRows, a.rows) - 1;
        const int first_limit = L - a.n;              // row 0 sees tokens 0 .. L - n (causal)
        // keys the block needs: up to the causal limit of its last row, or all (tree)
        const int key_end = TREE ? L : uni(max(min(L, first_limit + last_row / a.group + 1), 1));
        const int pg_end = uni(min(pg0 + part, (key_end + kPage - 1) / kPage));
        const int npairs = uni(max(pg_end - pg0 + 1, 0) / 2);
        const int last = uni(seq_pages - 1 - pg0);    // the sequence's last page, partition-relative
        // the last pair of a partition with an odd page count reaches one page
        // into the next partition: keys from here on are masked like dead ones
        const int tok_end = min(L, kPage * pg_end);
        int lim[TILES];
#pragma unroll
        for (int tt = 0; tt < TILES; ++tt)
            lim[tt] = qi[tt] >= 0 ? first_limit + qi[tt] : L - 1;   // padding rows see every live key
        // the pairs that need masks: those past the smallest causal limit among
        // this wave's rows, or reaching the tree tokens
        const int wave_lim = TREE ? first_limit - 1 : uni(first_limit + min(wrow0, a.rows - 1) / a.group);

        // page ids (and E4M3 scales) of the partition, clamped to the pool
#pragma unroll
        for (int k = 0; k < kIdLoads; ++k) {
            const int p = lt + k * kLoaders;
            if (lt >= 0 && p < 2 * npairs) {
                const int id = min(max(idv[k], 0), a.num_pages - 1);
                ids[p] = id;
                if constexpr (FP8) {
                    scales[p] = a.k_scale[(int64_t)id * a.hkv + kh];
                    scales[kIds + p] = a.v_scale[(int64_t)id * a.hkv + kh];
                }
            }
        }
        __syncthreads();

        f32x4 acc[TILES][8];
        f32x4 lsum[TILES];      // bf16 pools: row sums of the weights, from an all-ones MFMA
        float m[TILES], l[TILES];
#pragma unroll
        for (int tt = 0; tt < TILES; ++tt) {
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

        // Scores of pair jp for every tile, raw: K operands of both pages from LDS,
        // QK^T on the MFMAs.  The scale (and an E4M3 page's K scale) is folded into
        // the exponent later: p = exp2(s * f - m) with f > 0, so max(s * f) = f * max(s).
        auto scores = [&](const uint8_t* st, float (&sc)[TILES][8]) {
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
            // MFMA runs at raised wave priority, here and for PV: a wave about to
            // issue MFMAs goes first, and the other waves of the SIMD fill its
            // MFMA time with their softmax arithmetic (about 2 % on prefill)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int tt = 0; tt < TILES; ++tt)
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
            __builtin_amdgcn_s_setprio(0);
        };

        // step j holds pairs KG j .. KG j + KG - 1, pair KG j + k in sub-stage k;
        // key group k copies and computes pair KG j + k
        const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
        const int nsteps = KG == 1 ? npairs : (npairs + KG - 1) / KG;
        // prologue: steps 0 .. kStages - 2 in flight.  No step past the last is
        // copied, so the loads outstanding after step j are those of the
        // min(kStages - 2, nsteps - 1 - j) steps that follow it.
#pragma unroll
        for (int j = 0; j < kStages - 1; ++j)
            if (j < nsteps)
                issue_pair<FP8, WAVES, TREE>(a, ids, npairs, last, KG * j + kg, kh, wave, lane,
                                             lds0 + j * kStep + kg * Ly::kStage);

        for (int j = 0; j < nsteps; ++j) {
            // this wave's part of step j has landed once at most the later steps'
            // loads are outstanding; the barrier then covers every wave's part, and
            // every wave is done with step j - 1, whose stage is refilled next
            wait_steps<kStages - 2, Ly::kLoadsPerWave>(min(kStages - 2, nsteps - 1 - j));
            __syncthreads();
            if (j + kStages - 1 < nsteps)
                issue_pair<FP8, WAVES, TREE>(a, ids, npairs, last, KG * (j + kStages - 1) + kg, kh,
                                             wave, lane, lds0 + ((j + kStages - 1) % kStages) * kStep +
                                                             kg * Ly::kStage);

            const int step_base = 16 * pg0 + 32 * KG * j;     // first token of the step
            if (step_base + 32 * KG - 1 >= L) {
                // the step holding the sequence end: V rows past it may hold NaN,
                // which a zero weight would still carry through the MFMA, so they
                // are zeroed in LDS (once per workgroup, on this step only)
                constexpr int kRowBytes = kHeadDim * Ly::kElem;
                constexpr int kChunks = 32 * kRowBytes / 16;   // 16-byte pieces of a pair's V rows
                for (int e = t; e < KG * kChunks; e += kThreads) {
                    const int sub = KG == 1 ? 0 : e / kChunks;
                    const int ep = KG == 1 ? e : e % kChunks;
                    const int tok = ep / (kRowBytes / 16);
                    if (step_base + 32 * sub + tok >= L)
                        *reinterpret_cast<u32x4*>(lds + (j % kStages) * kStep + sub * Ly::kStage +
                                                  (2 + tok / 16) * Ly::kPageBytes + (tok % 16) * kRowBytes +
                                                  16 * (ep % (kRowBytes / 16))) = u32x4{0u, 0u, 0u, 0u};
                }
                __syncthreads();
            }
            const int jp = KG * j + kg;               // this wave's pair
            if constexpr (KG > 1)
                if (jp >= npairs) continue;           // (a key group past the end idles)
            uint8_t* st = lds + (j % kStages) * kStep + kg * Ly::kStage;
            const int base = 16 * pg0 + 32 * jp;      // first token of the pair
            const bool need_mask = base + 31 > wave_lim || base + 31 >= tok_end;
            float sc[TILES][8];
            scores(st, sc);
            float ks[2] = {1.f, 1.f}, vs[2] = {1.f, 1.f};
            if constexpr (FP8) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int pg = min(2 * jp + h, last);
                    ks[h] = scales[pg];
                    vs[h] = scales[kIds + pg];
                }
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
            float f[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) f[h] = FP8 ? a.scale_log2 * ks[h] : a.scale_log2;
            if (need_mask) {
#pragma unroll
                for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int tok = base + 16 * (e >> 2) + 4 * g + (e & 3);
                        bool vis;
                        if constexpr (TREE)
                            vis = tok < first_limit ||
                                  ((tmask[tt] >> min(max(tok - first_limit, 0), 63)) & 1u);
                        else
                            vis = tok <= lim[tt];
                        vis = vis && tok < tok_end;
                        sc[tt][e] = vis ? sc[tt][e] : -INFINITY;
                    }
            }
            // Phase 2: row maxima, and one rescale branch for all tiles (a tile
            // whose maximum did not move is multiplied by exp2(0) = 1, exactly)
            float mx[TILES];
            bool grow_any = false;
#pragma unroll
            for (int tt = 0; tt < TILES; ++tt) {
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
                for (int tt = 0; tt < TILES; ++tt) {
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
            for (int tt = 0; tt < TILES; ++tt) {
                float pw[8];
                float psum = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float p = fast_exp2(__builtin_fmaf(sc[tt][e], f[e >> 2], -m[tt]));
                    pw[e] = FP8 ? p * vs[e >> 2] : p;
                    if constexpr (FP8) psum += p;
                }
                const bf16x8 pf = __builtin_bit_cast(
                    bf16x8, u32x4{bf16x2_bits(pw[0], pw[1]), bf16x2_bits(pw[2], pw[3]),
                                  bf16x2_bits(pw[4], pw[5]), bf16x2_bits(pw[6], pw[7])});
                if constexpr (FP8)
                    l[tt] += psum;      // the V scale rides on the weights, not on their sum
                else
                    lsum[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf, lsum[tt], 0, 0, 0);
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int db = 0; db < 8; ++db)
                    acc[tt][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], pf, acc[tt][db], 0, 0, 0);
                __builtin_amdgcn_s_setprio(0);
            }
        }
        // no copy may still be writing this item's ring when it is reused
        wait_dma<0>();
        if constexpr (KG > 1) {
            // key groups 1 .. KG - 1 hand their (max, sum, accumulator) to group 0
            // through the ring, one tile at a time, value x of a lane at
            // xs[x * kLanes + lane id] (consecutive lanes, consecutive words);
            // group 0 merges them with weights 2^(m_k - max) and writes the result
            constexpr int kLanes = (KG - 1) * WAVES * kWave;
            constexpr int kVals = 34;                  // acc (32), m, l of one tile
            float* xs = reinterpret_cast<float*>(lds);
            static_assert(kLanes * kVals * 4 <= kStages * kStep, "merge fits the ring");
            __syncthreads();                           // every wave is done with the ring
#pragma unroll
            for (int tt = 0; tt < TILES; ++tt) {
                if (kg > 0) {
                    float* my = xs + ((kg - 1) * WAVES + wave) * kWave + lane;
#pragma unroll
                    for (int db = 0; db < 8; ++db)
#pragma unroll
                        for (int v = 0; v < 4; ++v) my[(4 * db + v) * kLanes] = acc[tt][db][v];
                    my[32 * kLanes] = m[tt];
                    my[33 * kLanes] = FP8 ? l[tt] : lsum[tt][0];
                }
                __syncthreads();
                if (kg == 0) {
                    float mm = m[tt];
#pragma unroll
                    for (int k = 1; k < KG; ++k)
                        mm = fmaxf(mm, xs[32 * kLanes + ((k - 1) * WAVES + wave) * kWave + lane]);
                    const float s0 = fast_exp2(m[tt] - mm);
                    float lt = (FP8 ? l[tt] : lsum[tt][0]) * s0;
#pragma unroll
                    for (int db = 0; db < 8; ++db) acc[tt][db] *= s0;
#pragma unroll
                    for (int k = 1; k < KG; ++k) {
                        const float* o = xs + ((k - 1) * WAVES + wave) * kWave + lane;
                        const float sk = fast_exp2(o[32 * kLanes] - mm);
                        lt += o[33 * kLanes] * sk;
#pragma unroll
                        for (int db = 0; db < 8; ++db)
#pragma unroll
                            for (int v = 0; v < 4; ++v) acc[tt][db][v] += o[(4 * db + v) * kLanes] * sk;
                    }
                    m[tt] = mm;
                    if constexpr (FP8)
                        l[tt] = lt;
                    else
                        lsum[tt][0] = lt;
                }
                if (tt + 1 < TILES) __syncthreads();   // group 0 is done reading the slots
            }
        }

        // epilogue: lane holds O[row l16][32 g + 8 v + db] (E4M3 pools) or
        // O[row l16][16 db + 4 g + v] (bf16 pools) of each tile; the final output
        // when the sequence has one partition, else this partition's partial
        const bool single = nsplit_b == 1;
        if (kg == 0) {    // (the other key groups handed their states to group 0)
#pragma unroll
            for (int tt = 0; tt < TILES; ++tt) {
                const int r = wrow0 + tt * 16 + l16;
                const float lt = FP8 ? group_sum(l[tt]) : lsum[tt][0];
                if (r < a.rows) {
                    const int i = r / a.group;
                    const int h = kh * a.group + (r - i * a.group);
                    const int64_t orow = ((int64_t)b * a.n + i) * a.hq + h;
                    if (single) {
                        const float inv = 1.0f / lt;
                        uint16_t* o = a.out + orow * kHeadDim;
                        if constexpr (FP8) {
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                uint32_t w[4];
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    w[e] = bf16x2_bits(acc[tt][2 * e][v] * inv, acc[tt][2 * e + 1][v] * inv);
                                *reinterpret_cast<u32x4*>(o + 32 * g + 8 * v) = u32x4{w[0], w[1], w[2], w[3]};
                            }
                        } else {
#pragma unroll
                            for (int db = 0; db < 8; ++db) {
                                const f32x4 x = acc[tt][db] * inv;
                                *reinterpret_cast<u32x2*>(o + 16 * db + 4 * g) =
                                    u32x2{bf16x2_bits(x[0], x[1]), bf16x2_bits(x[2], x[3])};
                            }
                        }
                    } else {
                        const int64_t pidx = orow * a.num_splits + sp;
                        float* pa = a.part_acc + pidx * kHeadDim;
                        if constexpr (FP8) {
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                f32x4 lo, hi;
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    lo[e] = acc[tt][e][v];
                                    hi[e] = acc[tt][4 + e][v];
                                }
                                *reinterpret_cast<f32x4*>(pa + 32 * g + 8 * v) = lo;
                                *reinterpret_cast<f32x4*>(pa + 32 * g + 8 * v + 4) = hi;
                            }
                        } else {
#pragma unroll
                            for (int db = 0; db < 8; ++db)
                                *reinterpret_cast<f32x4*>(pa + 16 * db + 4 * g) = acc[tt][db];
                        }
                        if (g == 0) {
                            a.part_ml[pidx * 2] = m[tt];
                            a.part_ml[pidx * 2 + 1] = lt;
                        }
                    }
                }
            }
        }
        // (one key group: no merge barrier separates this item's last reads of
        // the page ids from the next item's writes)
        if constexpr (KG == 1) __syncthreads();
    };
    if constexpr (TREE) {
        item((int)__builtin_amdgcn_workgroup_id_x());
    } else {
        const int wgs = a.workgroups;
        const int w = (int)__builtin_amdgcn_workgroup_id_x();
        for (int x0 = 0; x0 < items; x0 += wgs) {
            const int x = x0 + (((x0 / wgs) & 1) ? wgs - 1 - w : w);
            if (x < items) item(x);
        }
    }
}

}  // namespace

namespace {

template <bool FP8, int WAVES, int TILES, bool TREE, int STAGES, int MAXP, int KG>
hipError_t launch(const StagedArgs& a, dim3 grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    hipExtLaunchKernelGGL((paged_attn_staged<FP8, WAVES, TILES, TREE, STAGES, MAXP, KG>), grid,
                          dim3(WAVES * KG * kWave), 0, st, e0, e1, 0, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_staged(const StagedArgs& a, bool fp8, bool tree, hipStream_t st,
                         hipEvent_t e0, hipEvent_t e1)
{
    const dim3 grid((unsigned)a.workgroups);
    if (tree)
        return fp8 ? launch<true, 4, 1, true, kRing, kStagedTreeMaxPages, kTreeKeyGroups>(a, grid, st,
                                                                                        e0, e1)
                   : launch<false, 4, 1, true, kRing, kStagedTreeMaxPages, kTreeKeyGroups>(a, grid, st,
                                                                                         e0, e1);
    return fp8 ? launch<true, 4, 2, false, kRing, kStagedMaxPages, kPrefillKeyGroups>(a, grid, st,
                                                                                    e0, e1)
               : launch<false, 4, 2, false, kRing, kStagedMaxPages, kPrefillKeyGroups>(a, grid, st,
                                                                                     e0, e1);
}
