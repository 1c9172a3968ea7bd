// staged.h -- launch interface of the LDS-staged attention kernel (chunked
// prefill and draft-tree verification), used by the verify entry points.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

struct StagedArgs {
    const void* k;              // pool K, chunked layout, bf16 or E4M3
    const void* v;              // pool V, token-major
    const float* k_scale;       // [num_pages][Hkv] (E4M3 pools)
    const float* v_scale;
    const uint16_t* q;          // [B][n][Hq][128] bf16
    uint16_t* out;              // [B][n][Hq][128] bf16
    const int32_t* block_table; // [B][max_pages]
    const int32_t* seq_lens;    // [B]
    const uint64_t* tree_mask;  // [B][n] ancestor masks (tree calls)
    float* part_acc;            // [B][n][Hq][num_splits][128] split-K partials
    float* part_ml;             // [B][n][Hq][num_splits][2]   (max in log2 units, sum)
    int64_t page_stride;        // elements from one page to the next (Hkv * 16 * 128)
    int32_t num_pages;
    int32_t max_pages;
    int32_t batch;
    int32_t n;
    int32_t hq;
    int32_t hkv;
    int32_t group;              // Hq / Hkv
    int32_t rows;               // group * n rows per (sequence, kv head)
    int32_t row_blocks;         // workgroups per (sequence, kv head, partition)
    int32_t num_splits;         // context partitions of the longest sequence
    int32_t part_pages;         // pages per partition
    float scale_log2;           // scale * log2(e)
    int32_t workgroups;         // launched: one per work item (draft trees), or up to one
                                // per CU taking the items in turn (chunked prefill)
};

// rows of one (sequence, kv head) per workgroup: chunked prefill, draft trees
constexpr int kStagedPrefillRows = 128;
constexpr int kStagedTreeRows = 64;
// pages one workgroup can address (their page ids are staged in LDS): chunked
// prefill (one partition per sequence), draft-tree partitions
constexpr int kStagedMaxPages = 2048;
constexpr int kStagedTreeMaxPages = 512;
// Launches the kernel on `st` with a.workgroups workgroups over the
// batch * hkv * row_blocks * num_splits work items (one each for draft trees).
// ev_begin / ev_end (either may be null) take the kernel's start and end times.
hipError_t launch_staged(const StagedArgs& a, bool fp8, bool tree, hipStream_t st,
                         hipEvent_t ev_begin, hipEvent_t ev_end);
