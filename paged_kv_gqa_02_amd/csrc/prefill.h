// prefill.h -- the chunked-prefill attention kernel's launch interface (used
// by the verify entry points when a call has many query rows per sequence).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

struct PrefillArgs {
    const void* k;              // pool K, chunked layout, bf16 or E4M3
    const void* v;              // pool V, token-major
    const float* k_scale;       // [num_pages][Hkv] (E4M3 pools)
    const float* v_scale;
    const uint16_t* q;          // [B][n][Hq][128] bf16
    uint16_t* out;              // [B][n][Hq][128] bf16
    const int32_t* block_table; // [B][max_pages]
    const int32_t* seq_lens;    // [B]
    int64_t page_stride;        // elements from one page to the next (Hkv * 16 * 128)
    int32_t num_pages;
    int32_t max_pages;
    int32_t batch;
    int32_t n;
    int32_t hq;
    int32_t hkv;
    int32_t group;              // Hq / Hkv
    int32_t rows;               // group * n rows per (sequence, kv head)
    int32_t row_blocks;         // ceil(rows / kPrefillRows)
    float scale_log2;           // scale * log2(e)
};

// rows of one (sequence, kv head) per workgroup
constexpr int kPrefillRows = 256;
// pages of one sequence the kernel can address (its page ids are staged in LDS)
constexpr int kPrefillMaxPages = 2048;

// Launches the kernel on `st`; grid = batch * hkv * row_blocks workgroups.
hipError_t launch_prefill(const PrefillArgs& a, bool fp8, hipStream_t st);
