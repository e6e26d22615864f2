// Device helpers shared by the kernels: cross-lane moves, and the K/V row stores of
// k_rope.hip and k_qkv.hip, so that every path rounds, rotates and quantizes with the same
// instructions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kvc_internal.hpp"

namespace kvc {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Combine a value with the lane 16 (32) positions away without an LDS round trip: the
// gfx950 lane-swap instructions exchange rows of 16 lanes (halves of 32) between two
// registers, so swapping a register with itself leaves each lane's value and its
// partner's in the two results.  Both lanes of a pair get the same bits (IEEE max and
// addition are commutative).
__device__ __forceinline__ float max_xor16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Store 4 f32 values at dst: as they are for an f32 region, rounded to binary16 (nearest,
// ties to even: v_cvt_f16_f32 in the default rounding mode) for a half region.
__device__ __forceinline__ void store4(float *dst, float4 v)
{
    *reinterpret_cast<float4 *>(dst) = v;
}
__device__ __forceinline__ void store4(_Float16 *dst, float4 v)
{
    half4_t h;
    h[0] = (_Float16)v.x;
    h[1] = (_Float16)v.y;
    h[2] = (_Float16)v.z;
    h[3] = (_Float16)v.w;
    *reinterpret_cast<half4_t *>(dst) = h;
}

// Rotate one pair.  Contraction is off for this function: four rounded products, one
// rounded difference and one rounded sum.
__device__ __forceinline__ void rotate_pair(float x0, float x1, float2 cs_sn, float &y0,
                                            float &y1)
{
#pragma clang fp contract(off)
    const float a = x0 * cs_sn.x;
    const float b = x1 * cs_sn.y;
    const float c = x0 * cs_sn.y;
    const float d = x1 * cs_sn.x;
    y0 = a - b;
    y1 = c + d;
}

// Q8_0 store of 4 consecutive values of a row, held by lane group member (idx % 8) of the
// 8 aligned lanes that together hold one 32-value block: the block's max |x| is reduced
// across the 8 lanes (DPP within each half-row), every lane derives the same scale and
// reciprocal (IEEE f32 division), writes its 4 codes as one dword at `codes`, and the
// group's first lane writes the binary16 scale at `scale`.
__device__ __forceinline__ void q8_store4(float4 y, int8_t *codes, _Float16 *scale, int32_t idx)
{
#pragma clang fp contract(off)
    float a = fmaxf(fmaxf(fabsf(y.x), fabsf(y.y)), fmaxf(fabsf(y.z), fabsf(y.w)));
    a = fmaxf(a, dpp<0xB1>(a));   // lane ^ 1
    a = fmaxf(a, dpp<0x4E>(a));   // lane ^ 2
    a = fmaxf(a, dpp<0x141>(a));  // i <-> 7 - i within 8 lanes: the other quad
    const float d = a / 127.0f;
    const float r = d != 0.0f ? 1.0f / d : 0.0f;
    const int32_t c0 = (int32_t)roundf(y.x * r), c1 = (int32_t)roundf(y.y * r);
    const int32_t c2 = (int32_t)roundf(y.z * r), c3 = (int32_t)roundf(y.w * r);
    const uint32_t packed = (uint32_t)(c0 & 0xff) | ((uint32_t)(c1 & 0xff) << 8) |
                            ((uint32_t)(c2 & 0xff) << 16) | ((uint32_t)(c3 & 0xff) << 24);
    *reinterpret_cast<uint32_t *>(codes) = packed;
    if ((idx & 7) == 0) *scale = (_Float16)d;
}

}  // namespace kvc
