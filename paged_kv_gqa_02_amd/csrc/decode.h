// decode.h -- launch interface of the paged decode / verify kernels (the
// partition kernel and the split-K reduce, decode.hip) and of the KV append
// kernel (append.hip), for the host side of the library (paged_attn.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

// geometry of the page pool (include/paged_attn.h)
constexpr int kPage = 16;
constexpr int kHeadDim = 128;
constexpr int kSlab = kPage * kHeadDim;     // elements of one (page, kv head) slab
constexpr int kWave = 64;
constexpr int kMaxRowTiles = 4;             // 16-row MFMA tiles per workgroup
constexpr int kMaxSplits = 64;              // context partitions per sequence
constexpr int kDefaultWaves = 4;            // waves per partition workgroup
constexpr float kLog2e = 1.4426950408889634f;

// KV element kinds (the values of pa_dtype)
enum KvKind { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

struct DecodeArgs {
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

// The partition kernel for KV kind `kv` with `row_tiles` 16-row MFMA tiles per
// workgroup, `waves` waves and `prefetch` pages in flight per wave (shapes
// outside the tuned set run 4 waves x 2 pages), on `grid` workgroups.  ev_begin
// and ev_end (either may be null) are attached to the kernel's dispatch and
// take its start and end times.
hipError_t launch_partition(const DecodeArgs& a, int kv, int row_tiles, int waves, int prefetch,
                            int grid, hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end);

// The split-K reduce, one workgroup per output row; float or bf16 output.
hipError_t launch_reduce(const DecodeArgs& a, bool f32_out, unsigned rows_out, hipStream_t st);

// The KV append kernel for pool kind `kv` and a bf16 (else f32) source.
hipError_t launch_append(const AppendArgs& a, int kv, bool src_bf16, dim3 grid, hipStream_t st);
