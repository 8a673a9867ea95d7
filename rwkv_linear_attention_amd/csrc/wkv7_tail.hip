// wkv7_tail.hip -- the time-mix tail after WKV as a pass of its own: group
// norm, bonus and gate per (batch, token, head) row (tail_lane in
// wkv7_device.h).  The SwiftRWKV Inference guide fuses these three steps into
// the kernel the recurrent step uses; wkv7_step_tail does that.  After the
// chunked prefill, whose outputs of one token are spread over several waves,
// this pass applies the same arithmetic: one row per 16 lanes, four channels
// per lane, every input read once and x written once.
#include "wkv7_device.h"
#include "wkv7_launch.h"

namespace wkv7 {
namespace {

// Four consecutive elements as fp32 (bf16 widens exactly) and back.
__device__ __forceinline__ f32x4 load4(const float *p, size_t i) { return *reinterpret_cast<const f32x4 *>(p + i); }
__device__ __forceinline__ f32x4 load4(const uint16_t *p, size_t i)
{
    const uint2 u = *reinterpret_cast<const uint2 *>(p + i);
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
}
__device__ __forceinline__ void store4(float *p, size_t i, const f32x4 &x) { *reinterpret_cast<f32x4 *>(p + i) = x; }
__device__ __forceinline__ void store4(uint16_t *p, size_t i, const f32x4 &x)
{
    const uint32_t lo = f32_to_bf16_bits(x[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(x[1])) << 16);
    const uint32_t hi = f32_to_bf16_bits(x[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(x[3])) << 16);
    *reinterpret_cast<uint2 *>(p + i) = uint2{lo, hi};
}

// One (b, t, h) row per 16 lanes, four channels per lane (wide loads): tail_row4.
template <typename Tin, typename To, typename Tx>
__global__ __launch_bounds__(256) void tmix_tail_kernel(const To *o, const Tin *r, const Tin *k, const Tin *v,
                                                        const Tin *gate, const float *r_k, const float *ln_w,
                                                        const float *ln_b, float eps, Tx *x, long long rows, int H)
{
    const long long row = (blockIdx.x * 256ll + threadIdx.x) >> 4;  // sixteen rows per workgroup
    if (row >= rows)
        return;  // whole 16-lane groups: the sums below stay inside a group
    const int c0 = 4 * (threadIdx.x & 15);
    const int hh = static_cast<int>(row % H);
    const size_t e = static_cast<size_t>(row) * kN + c0;
    const int pj = hh * kN + c0;
    const f32x4 o4 = load4(o, e);
    const f32x4 r4 = load4(r, e), k4 = load4(k, e), v4 = load4(v, e), g4 = load4(gate, e);
    const f32x4 rk4 = load4(r_k, pj), w4 = load4(ln_w, pj), b4 = load4(ln_b, pj);
    store4(x, e, tail_row4(o4, r4, k4, v4, g4, rk4, w4, b4, eps));
}

template <typename Tin, typename To, typename Tx>
hipError_t launch_t(const TailArgs &p, hipStream_t stream)
{
    const long long blocks = (p.rows + 15) / 16;
    hipLaunchKernelGGL((tmix_tail_kernel<Tin, To, Tx>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       static_cast<const To *>(p.o), static_cast<const Tin *>(p.r), static_cast<const Tin *>(p.k),
                       static_cast<const Tin *>(p.v), static_cast<const Tin *>(p.gate), p.r_k, p.ln_w, p.ln_b,
                       p.eps, static_cast<Tx *>(p.x), p.rows, p.H);
    return hipGetLastError();
}

template <typename Tin, typename To>
hipError_t launch_x(const TailArgs &p, hipStream_t stream)
{
    return p.x_bf16 ? launch_t<Tin, To, uint16_t>(p, stream) : launch_t<Tin, To, float>(p, stream);
}

template <typename Tin>
hipError_t launch_o(const TailArgs &p, hipStream_t stream)
{
    return p.o_bf16 ? launch_x<Tin, uint16_t>(p, stream) : launch_x<Tin, float>(p, stream);
}

}  // namespace

hipError_t launch_tail(const TailArgs &p, hipStream_t stream)
{
    return p.in_bf16 ? launch_o<uint16_t>(p, stream) : launch_o<float>(p, stream);
}

}  // namespace wkv7
