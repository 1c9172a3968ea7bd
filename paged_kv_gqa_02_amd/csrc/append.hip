// append.hip -- KV append with fp8 quantise-on-write for MI355X (gfx950).
//
// The n_new newest tokens of every sequence are written into their pages ("Latency and cost in production" §10.12.2: a
// request's blocks fill one token at a time; §10.8.2-§10.8.3: q =
// round(x / scale) with zero-point 0).  Pages are independent (each has its
// own scale), so one workgroup of one wave takes one (sequence, kv head, K or
// V, page touched by the new tokens); its work unit is one 16-byte chunk of
// one token row (K chunked, V token-major), read from the source with 16-byte
// loads.  fp8 pages: scale = absmax / 448 over the new values of a page none
// of whose earlier slots are live (1 if 0); otherwise max(old, absmax / 448),
// and the earlier live bytes are re-encoded when it grows.  All in binary32.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "cdna4.h"
#include "decode.h"

namespace {

using namespace cdna4;

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

}  // namespace

hipError_t launch_append(const AppendArgs& a, int kv, bool src_bf16, dim3 grid, hipStream_t st)
{
    switch (kv) {
    case KV_F32: hipLaunchKernelGGL((paged_attn_append<KV_F32, false>), grid, dim3(kWave), 0, st, a); break;
    case KV_BF16:
        if (src_bf16) hipLaunchKernelGGL((paged_attn_append<KV_BF16, true>), grid, dim3(kWave), 0, st, a);
        else hipLaunchKernelGGL((paged_attn_append<KV_BF16, false>), grid, dim3(kWave), 0, st, a);
        break;
    default:
        if (src_bf16) hipLaunchKernelGGL((paged_attn_append<KV_FP8, true>), grid, dim3(kWave), 0, st, a);
        else hipLaunchKernelGGL((paged_attn_append<KV_FP8, false>), grid, dim3(kWave), 0, st, a);
        break;
    }
    return hipGetLastError();
}
