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

// x from another lane of the same 16-lane row, by a DPP control (no LDS round trip).
// Every control used here reads inside the row, so bound_ctrl never applies; setting
// it lets the compiler fold the move into the add that consumes it.
template <int CTRL>
__device__ __forceinline__ float row_dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over the 16 lanes of a row group (lanes 16 g .. 16 g + 15), returned to all of
// them: the other lane of each pair (quad_perm 1,0,3,2), of each quad (2,3,0,1), then
// the mirrored quad of the half row and the mirrored half of the row.  Each step adds
// two partial sums that the lanes hold in swapped roles, so every lane gets the same
// bits.
__device__ __forceinline__ float group16_sum(float x)
{
    x += row_dpp<0xb1>(x);   // quad_perm [1, 0, 3, 2]
    x += row_dpp<0x4e>(x);   // quad_perm [2, 3, 0, 1]
    x += row_dpp<0x141>(x);  // row_half_mirror
    x += row_dpp<0x140>(x);  // row_mirror
    return x;
}

// The same tail for one (b, t, h) row held by the 16 lanes of a row group, four
// channels per lane: o4, r4, k4, v4, g4 are the lane's channels of the row, rk4,
// w4, b4 its channels of r_k, ln_w, ln_b.  Every lane of the group must take part.
__device__ __forceinline__ f32x4 tail_row4(const f32x4 o4, const f32x4 r4, const f32x4 k4, const f32x4 v4,
                                           const f32x4 g4, const f32x4 rk4, const f32x4 w4, const f32x4 b4,
                                           float eps)
{
    const float mu = group16_sum((o4[0] + o4[1]) + (o4[2] + o4[3])) * (1.0f / kN);
    f32x4 d;
    float ss = 0.f, bon = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        d[c] = o4[c] - mu;
        ss += d[c] * d[c];
        bon += r4[c] * k4[c] * rk4[c];
    }
    const float inv = rsqrtf(group16_sum(ss) * (1.0f / kN) + eps);
    const float bonus = group16_sum(bon);
    f32x4 xo;
#pragma unroll
    for (int c = 0; c < 4; ++c)
        xo[c] = (d[c] * inv * w4[c] + b4[c] + bonus * v4[c]) * g4[c];
    return xo;
}

}  // namespace wkv7
