// Device-side helpers shared by the gfx950 kernels of the BlockFFN layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace blockffn {

// Operand and accumulator vectors of the bf16 matrix-core (MFMA) instructions.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;     // CDNA wavefront width
constexpr int kTileM = 32;    // token rows per tile: one n = 32 chunk

// 16-byte load of eight bf16 values.
__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t *p)
{
    u32x4 v = *reinterpret_cast<const u32x4 *>(p);
    return __builtin_bit_cast(bf16x8, v);
}

// Same, but bypassing reuse in the caches: for weights that are streamed once.
__device__ __forceinline__ bf16x8 load_bf16x8_stream(const uint16_t *p)
{
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 zero_bf16x8()
{
    return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b)
{
    return __uint_as_float((uint32_t)b << 16);
}

// Swish / SiLU with beta = 1: a * sigmoid(a) = a / (1 + e^-a).
__device__ __forceinline__ float swish_fast(float a)
{
    return a / (1.0f + __expf(-a));
}

__device__ __forceinline__ float swish_precise(float a)
{
    return a / (1.0f + expf(-a));
}

// Sum over the 64 lanes of a wavefront, returned to every lane; every lane must be
// active. DPP butterflies inside each row of 16 lanes (each lane adds its partner's
// value, and a + b == b + a exactly, so all lanes of a row agree bit for bit), then
// the four row sums are read out in a fixed order.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                              0xf, 0xf, false));
}
// Sum over each 16-lane row of the wave, returned in every lane of the row (the same
// bits in all of them: every step adds two values in either order).
__device__ __forceinline__ float row16_sum_f32(float v)
{
    v += dpp_f32<0xb1>(v);    // quad_perm [1,0,3,2]
    v += dpp_f32<0x4e>(v);    // quad_perm [2,3,0,1]
    v += dpp_f32<0x141>(v);   // row_half_mirror
    v += dpp_f32<0x140>(v);   // row_mirror
    return v;
}
__device__ __forceinline__ float wave_sum_f32(float v)
{
    v += dpp_f32<0xb1>(v);    // quad_perm [1,0,3,2]
    v += dpp_f32<0x4e>(v);    // quad_perm [2,3,0,1]
    v += dpp_f32<0x141>(v);   // row_half_mirror
    v += dpp_f32<0x140>(v);   // row_mirror
    const int b = __builtin_bit_cast(int, v);
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xf, 0xf, false);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double readlane_f64(double v, int lane)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double wave_sum_f64(double v)
{
    v += dpp_f64<0xb1>(v);
    v += dpp_f64<0x4e>(v);
    v += dpp_f64<0x141>(v);
    v += dpp_f64<0x140>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

}  // namespace blockffn
