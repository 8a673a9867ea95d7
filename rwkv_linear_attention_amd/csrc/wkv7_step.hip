// wkv7_step.hip -- the recurrent WKV-7 pass (decode and short speculative-verify steps).
//
// One step per token, per (batch, head), exactly as defined for the recurrent
// pass: the RWKV-X Architecture page, section "WKV-7 Kernel (Generalized Delta
// Rule)" (decay, rank-1 delta term, key-value write, readout, per head and
// timestep) with the Core AI RWKV-7 note, section 1 (S = [K,V]; both the decay
// and the rank-1 term act on the state the step starts from; o = r^T S after
// the write).  Optional per-position states serve the verify step of the
// RWKV7-MTP-Exp model card, section "Inference" (state rolled back to the
// accepted prefix).
//
// Mapping to gfx950: one 64-lane wavefront per head; lane j owns VALUE column
// j of the 64x64 fp32 state, i.e. 64 VGPRs holding S[0..63][j].  Because every
// value column evolves independently given the shared key-side vectors, both
// reductions over the key index (a^T S and r^T S) are in-lane dot products and
// need no cross-lane traffic; the key-side scalars a[i], w[i], b[i], k[i], r[i]
// are broadcast from the lane that loaded them.  A state row S[i][0..63] is
// 256 contiguous bytes, so each of the 64 state loads and stores of a wave is
// one fully coalesced 256-byte access.
#include "wkv7_device.h"
#include "wkv7_launch.h"

namespace wkv7 {
namespace {

template <typename Tin, typename Tout, bool HAS_STATE_IN, bool WRITE_POS>
__global__ __launch_bounds__(64) void wkv7_step_kernel(SeqArgs p)
{
    const int j = threadIdx.x;                 // value column owned by this lane
    const int bh = blockIdx.x;                 // (batch, head) pair
    const int H = p.H, T = p.T;
    const int bb = bh / H, hh = bh - bb * H;
    const Tin *__restrict__ r = static_cast<const Tin *>(p.r);
    const Tin *__restrict__ w = static_cast<const Tin *>(p.w);
    const Tin *__restrict__ k = static_cast<const Tin *>(p.k);
    const Tin *__restrict__ v = static_cast<const Tin *>(p.v);
    const Tin *__restrict__ a = static_cast<const Tin *>(p.a);
    const Tin *__restrict__ b = static_cast<const Tin *>(p.b);
    Tout *__restrict__ o = static_cast<Tout *>(p.o);

    const size_t sbase = static_cast<size_t>(bh) * (kN * kN) + j;
    float S[kN];
#pragma unroll
    for (int i = 0; i < kN; ++i)
        S[i] = HAS_STATE_IN ? p.state_in[sbase + i * kN] : 0.0f;

    for (int t = 0; t < T; ++t) {
        const size_t base = ((static_cast<size_t>(bb) * T + t) * H + hh) * kN + j;
        // lane j holds element j of every key-side vector and of v
        const float a_j = load_elem(a, base), w_j = load_elem(w, base);
        const float b_j = load_elem(b, base), k_j = load_elem(k, base);
        const float r_j = load_elem(r, base), v_j = load_elem(v, base);

        // sa = a^T S (state before the step), in-lane over the key index
        float sa = 0.0f;
#pragma unroll
        for (int i = 0; i < kN; ++i)
            sa = fmaf(lane_bcast(a_j, i), S[i], sa);
        // S[i][j] = w[i] S[i][j] + b[i] sa[j] + k[i] v[j]
#pragma unroll
        for (int i = 0; i < kN; ++i)
            S[i] = fmaf(lane_bcast(w_j, i), S[i], fmaf(lane_bcast(b_j, i), sa, lane_bcast(k_j, i) * v_j));
        // o[j] = r^T S (after the write)
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < kN; ++i)
            acc = fmaf(lane_bcast(r_j, i), S[i], acc);
        store_elem(o, base, acc);

        if (WRITE_POS) {
            float *dst = p.state_pos + ((static_cast<size_t>(bb) * T + t) * H + hh) * (kN * kN) + j;
#pragma unroll
            for (int i = 0; i < kN; ++i)
                dst[i * kN] = S[i];
        }
    }
#pragma unroll
    for (int i = 0; i < kN; ++i)
        p.state_out[sbase + i * kN] = S[i];
}

template <typename Tin, typename Tout>
hipError_t launch_typed(const SeqArgs &p, hipStream_t stream)
{
    const dim3 grid(static_cast<unsigned>(p.B) * static_cast<unsigned>(p.H)), block(64);
    const bool sin = p.state_in != nullptr, pos = p.state_pos != nullptr;
    if (sin && pos)
        hipLaunchKernelGGL((wkv7_step_kernel<Tin, Tout, true, true>), grid, block, 0, stream, p);
    else if (sin)
        hipLaunchKernelGGL((wkv7_step_kernel<Tin, Tout, true, false>), grid, block, 0, stream, p);
    else if (pos)
        hipLaunchKernelGGL((wkv7_step_kernel<Tin, Tout, false, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((wkv7_step_kernel<Tin, Tout, false, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

// Copy (or zero, when src is null) n_floats of state; n_floats is a multiple of 4.
__global__ __launch_bounds__(256) void state_copy_kernel(const float4 *src, float4 *dst, long long n4)
{
    for (long long i = blockIdx.x * 256ll + threadIdx.x; i < n4; i += static_cast<long long>(gridDim.x) * 256)
        dst[i] = src ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

// Zero the [H,64,64] block of every batch row b with mask[b] != 0 (all rows when mask is null).
__global__ __launch_bounds__(256) void state_reset_kernel(float4 *state, const unsigned char *mask,
                                                          long long per_row4, long long n4)
{
    for (long long i = blockIdx.x * 256ll + threadIdx.x; i < n4; i += static_cast<long long>(gridDim.x) * 256) {
        if (mask && !mask[i / per_row4])
            continue;
        state[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

unsigned grid_for(long long n4)
{
    long long blocks = (n4 + 255) / 256;
    return static_cast<unsigned>(blocks < 4096 ? (blocks > 0 ? blocks : 1) : 4096);
}

}  // namespace

hipError_t launch_step(const SeqArgs &p, hipStream_t stream)
{
    if (p.in_bf16)
        return p.o_bf16 ? launch_typed<uint16_t, uint16_t>(p, stream) : launch_typed<uint16_t, float>(p, stream);
    return p.o_bf16 ? launch_typed<float, uint16_t>(p, stream) : launch_typed<float, float>(p, stream);
}

hipError_t launch_state_copy(const float *src, float *dst, long long n_floats, hipStream_t stream)
{
    const long long n4 = n_floats / 4;
    hipLaunchKernelGGL(state_copy_kernel, dim3(grid_for(n4)), dim3(256), 0, stream,
                       reinterpret_cast<const float4 *>(src), reinterpret_cast<float4 *>(dst), n4);
    return hipGetLastError();
}

hipError_t launch_state_reset(float *state, int B, int H, const unsigned char *row_mask, hipStream_t stream)
{
    const long long per_row4 = static_cast<long long>(H) * kN * kN / 4;
    const long long n4 = per_row4 * B;
    hipLaunchKernelGGL(state_reset_kernel, dim3(grid_for(n4)), dim3(256), 0, stream,
                       reinterpret_cast<float4 *>(state), row_mask, per_row4, n4);
    return hipGetLastError();
}

}  // namespace wkv7
