// cdna4.h -- gfx950 device helpers shared by the library's kernels: operand
// vector types, bf16 rounding, exp2, reductions across the four 16-lane groups
// of a wave, exact E4M3 -> bf16 conversion and the V-page transpose into the
// MFMA A-operand layout.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace cdna4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16_bits(float x)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// two floats to bf16 (round to nearest even, as bf16_bits) in one packed
// conversion: lo in bits 0..15, hi in bits 16..31
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi)
{
    typedef __bf16 bf16v2 __attribute__((ext_vector_type(2)));
    typedef float f32v2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32v2){lo, hi}, bf16v2));
}

__device__ __forceinline__ float bf16_float(uint32_t bits16)
{
    return __uint_as_float(bits16 << 16);
}

// a wave-uniform value, marked as such for the compiler (readfirstlane), so
// that what derives from it is computed on the scalar unit
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float fast_exp2(float x)
{
    return __builtin_amdgcn_exp2f(x);
}

// Reductions across the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48) with the gfx950 lane-swap instructions: swapping a register with
// itself leaves one copy of each partner value in the returned pair.
__device__ __forceinline__ float group_max(float x)
{
    const uint32_t u = __float_as_uint(x);
    auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t w = __float_as_uint(y);
    auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float group_sum(float x)
{
    const uint32_t u = __float_as_uint(x);
    auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t w = __float_as_uint(y);
    auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Two E4M3 bytes (low or high half of w) -> two bf16 in one dword.  E4M3 is
// a subset of bf16, so the conversion is exact.
template <bool kHigh>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w)
{
    bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHigh);
    return __builtin_bit_cast(uint32_t, r);
}

// 8 E4M3 bytes -> 8 bf16
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1)
{
    u32x4 r;
    r[0] = fp8x2_to_bf16x2<false>(w0);
    r[1] = fp8x2_to_bf16x2<true>(w0);
    r[2] = fp8x2_to_bf16x2<false>(w1);
    r[3] = fp8x2_to_bf16x2<true>(w1);
    return r;
}

// Four 16-byte rows r = 0..3 of 8 bf16 each (v[r] = row r, elements e = 0..7)
// -> a[e] = {v[0][e], v[1][e], v[2][e], v[3][e]}: the MFMA A operand whose K
// index runs over the rows.
__device__ __forceinline__ void v_operands(i16x4 (&a)[8], const u32x4 (&v)[4])
{
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t lo = __builtin_amdgcn_perm(v[1][w], v[0][w], sel);
        const uint32_t hi = __builtin_amdgcn_perm(v[3][w], v[2][w], sel);
        a[e] = __builtin_bit_cast(i16x4, u32x2{lo, hi});
    }
}

}  // namespace cdna4
