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

// Sum of x over the 64 lanes of a wave (every lane active), returned to every lane.
__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        x += __shfl_xor(x, off);
    return x;
}

// The time-mix tail after WKV for one (b, t, h) row held one channel per lane
// (the SwiftRWKV Inference guide fuses its three named parts: group norm,
// bonus, gate): the row of o is normalised over its 64 channels (mean,
// biased variance, eps), scaled and shifted per channel, the bonus
// (sum over keys of r k r_k) times v is added, and the gate multiplies.
// Lane j passes o[j], v[j], g[j], ln_w[j], ln_b[j] and also r[j], k[j], r_k[j]
// for the bonus sum over the key index.
// tail_norm takes the bonus sum already formed (it does not depend on o).
__device__ __forceinline__ float tail_norm(float oj, float bonus, float vj, float gj, float wj, float bj, float eps)
{
    const float mu = wave_sum(oj) * (1.0f / kN);
    const float d = oj - mu;
    const float var = wave_sum(d * d) * (1.0f / kN);
    return (d / sqrtf(var + eps) * wj + bj + bonus * vj) * gj;
}
__device__ __forceinline__ float tail_lane(float oj, float rj, float kj, float rkj, float vj, float gj, float wj,
                                           float bj, float eps)
{
    return tail_norm(oj, wave_sum(rj * kj * rkj), vj, gj, wj, bj, eps);
}

}  // namespace wkv7
