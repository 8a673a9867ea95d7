// wkv7_device.h -- device helpers shared by the libwkv7 kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv7 {

constexpr int kN = 64;  // head size; the only one the library is built for

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Element loads: bf16 widens to fp32 exactly (its bits are the top half of an fp32).
__device__ __forceinline__ float load_elem(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t *p, size_t i)
{
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x)
{
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ void store_elem(float *p, size_t i, float x) { p[i] = x; }
__device__ __forceinline__ void store_elem(uint16_t *p, size_t i, float x) { p[i] = f32_to_bf16_bits(x); }

// Broadcast lane `src` (a compile-time constant after unrolling) of a wave-wide value.
__device__ __forceinline__ float lane_bcast(float x, int src)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), src));
}

}  // namespace wkv7
