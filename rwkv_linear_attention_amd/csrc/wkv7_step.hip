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
// Mapping to gfx950: one workgroup of NW wavefronts per head (four for one
// token, eight for longer runs, whose per-position state stores are then
// spread over more waves).  Lane j owns
// VALUE column j of the 64x64 fp32 state; wave g holds the 64/NW key rows
// i = g*RW .. g*RW + RW-1 of that column in registers.  Every value column
// evolves independently given the shared key-side vectors, so the update is
// lane-local; the reductions over the key index (a^T S and r^T S) are
// in-lane partial sums over a wave's rows, combined across the NW waves
// through LDS in a fixed order.  The key-side scalars a, w, b, k, r of a
// wave's rows are uniform across its lanes.
// A state row S[i][0..63] is 256 contiguous bytes, so every state load and
// store of a wave is one fully coalesced 256-byte access; the state streams
// through once per call, so its loads and stores are marked nontemporal.  Splitting a head's
// rows over several short waves lets the loads, arithmetic and stores of
// different waves overlap, which is what a bandwidth-bound step needs.
#include "wkv7_device.h"
#include "wkv7_launch.h"

namespace wkv7 {
namespace {

constexpr int TB = 8;          // tokens per staged block

// RW consecutive elements of a key-side vector, widened to fp32, from a
// wave-uniform address (scalar loads).
template <int RW>
__device__ __forceinline__ void load_rows(const uint16_t *__restrict__ p, float (&x)[RW])
{
    const uint32_t *p32 = reinterpret_cast<const uint32_t *>(p);
#pragma unroll
    for (int u = 0; u < RW / 2; ++u) {
        const uint32_t bits = p32[u];
        x[2 * u] = __uint_as_float(bits << 16);
        x[2 * u + 1] = __uint_as_float(bits & 0xffff0000u);
    }
}
template <int RW>
__device__ __forceinline__ void load_rows(const float *__restrict__ p, float (&x)[RW])
{
#pragma unroll
    for (int u = 0; u < RW; ++u)
        x[u] = p[u];
}

// The key-side inputs of a step reach the waves in one of two ways, chosen by
// the launcher: a single token (decode) is read with scalar loads issued
// together with the state loads; longer runs (speculative verify, replays)
// stage blocks of TB tokens, widened to fp32, in LDS with one cooperative
// load, so no global latency sits inside the token loop.  The arithmetic is
// the same code either way.
// With VARLEN, row b runs its first lengths[b] tokens only (clamped to [0, T]);
// T stays the row stride of the [B, T, H, N] tensors.  With TAIL, the time-mix
// tail (group norm, bonus, gate; see tail_lane) is applied to each token's o
// in the wave that reduces it, and o receives x.
struct TailIn {
    const void *gate;
    const float *r_k, *ln_w, *ln_b;
    float eps;
};
template <typename Tin, typename Tout, bool HAS_STATE_IN, bool WRITE_POS, bool STAGED, int NW, bool VARLEN,
          bool TAIL>
__global__ __launch_bounds__(NW * 64) void wkv7_step_kernel(
    const Tin *__restrict__ r, const Tin *__restrict__ w, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const Tin *__restrict__ a, const Tin *__restrict__ b, const float *state_in, Tout *__restrict__ o,
    float *state_out, float *__restrict__ state_pos, int T, int H, const int *__restrict__ lengths, TailIn tail)
{
    constexpr int RW = kN / NW;                                       // key rows per wave
    const int j = threadIdx.x & 63;                                   // value column of this lane
    const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // row block of this wave
    const int i0 = g * RW;
    const int bh = blockIdx.x;                                        // (batch, head) pair
    const int bb = bh / H, hh = bh - bb * H;
    const int L = VARLEN ? min(max(lengths[bb], 0), T) : T;  // tokens of this row
    __shared__ float part_a[2][NW][kN];  // a^T S partial sums, alternating between tokens
    __shared__ float part_r[NW][kN];     // r^T S partial sums
    __shared__ alignas(16) float xin[STAGED ? TB : 1][6][kN];  // staged a, w, b, k, r, v

    const Tin *const vecs[6] = {a, w, b, k, r, v};
    constexpr int PER = STAGED ? (TB * 6 * kN) / (NW * 64) : 1;  // staged elements per thread
    float stage[PER];
    auto stage_load = [&](int t0, int nt) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = u * NW * 64 + threadIdx.x;
            // rows past the end re-read the last token (unconditional loads keep the
            // waits for them out of the issue sequence); they are never stored
            const int tt = min(e / (6 * kN), nt - 1), rem = e % (6 * kN), vec = rem / kN, n = rem % kN;
            stage[u] = load_elem(vecs[vec], ((static_cast<size_t>(bb) * T + t0 + tt) * H + hh) * kN + n);
        }
    };
    if constexpr (STAGED)
        stage_load(0, max(min(TB, L), 1));  // issued before the state loads: waiting for it skips them

    // the tail's per-head parameters of this lane's channel
    float t_w = 0.f, t_b = 0.f, t_rk = 0.f;
    if constexpr (TAIL) {
        t_w = tail.ln_w[hh * kN + j];
        t_b = tail.ln_b[hh * kN + j];
        t_rk = tail.r_k[hh * kN + j];
    }
    const size_t sbase = static_cast<size_t>(bh) * (kN * kN) + static_cast<size_t>(i0) * kN + j;
    float S[RW];
#pragma unroll
    for (int u = 0; u < RW; ++u)
        S[u] = HAS_STATE_IN ? __builtin_nontemporal_load(state_in + sbase + u * kN) : 0.0f;

    constexpr int BLK = STAGED ? TB : 1;
    for (int t0 = 0; t0 < L; t0 += BLK) {
        const int nt = min(BLK, L - t0);
        if constexpr (STAGED) {
            if (t0 > 0) {
                __syncthreads();  // the previous block's inputs are no longer read
                stage_load(t0, nt);
            }
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int e = u * NW * 64 + threadIdx.x;
                if (e < nt * 6 * kN)
                    (&xin[0][0][0])[e] = stage[u];
            }
            __syncthreads();
        }
        for (int tt = 0; tt < nt; ++tt) {
            const int t = t0 + tt;
            const size_t base = ((static_cast<size_t>(bb) * T + t) * H + hh) * kN;  // uniform
            // this wave's rows of a, w, b, k, r (uniform across lanes) and v[j]
            float ar[RW], wr[RW], br[RW], kr[RW], rr[RW], vj;
            if constexpr (STAGED) {
                vj = xin[tt][5][j];
            } else {
                load_rows(a + base + i0, ar);
                load_rows(w + base + i0, wr);
                load_rows(b + base + i0, br);
                load_rows(k + base + i0, kr);
                load_rows(r + base + i0, rr);
                vj = load_elem(v, base + j);
            }
            // the tail's bonus sum and gate do not depend on the state: wave 0 forms them
            // here, beside the other waves' partial sums
            float t_bonus = 0.f, t_g = 0.f;
            if constexpr (TAIL) {
                if (g == 0) {
                    float rj, kj;
                    if constexpr (STAGED) {
                        rj = xin[tt][4][j];
                        kj = xin[tt][3][j];
                    } else {
                        rj = load_elem(r, base + j);
                        kj = load_elem(k, base + j);
                    }
                    t_g = load_elem(static_cast<const Tin *>(tail.gate), base + j);
                    t_bonus = wave_sum(rj * kj * t_rk);
                }
            }
            auto rows4 = [&](int vec, const float (&reg)[RW], int u) -> f32x4 {
                if constexpr (STAGED)
                    return *reinterpret_cast<const f32x4 *>(&xin[tt][vec][i0 + u]);
                else
                    return f32x4{reg[u], reg[u + 1], reg[u + 2], reg[u + 3]};
            };

            // sa[j] = a^T S over the state before this token: partial over this wave's rows
            float sa = 0.0f;
#pragma unroll
            for (int u = 0; u < RW; u += 4) {
                const f32x4 a4 = rows4(0, ar, u);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sa = fmaf(a4[e], S[u + e], sa);
            }
            part_a[t & 1][g][j] = sa;
            __syncthreads();
            sa = part_a[t & 1][0][j];
#pragma unroll
            for (int gg = 1; gg < NW; ++gg)
                sa += part_a[t & 1][gg][j];
            // S[i][j] = w[i] S[i][j] + b[i] sa[j] + k[i] v[j], then o[j] = r^T S
            float op = 0.0f;
#pragma unroll
            for (int u = 0; u < RW; u += 4) {
                const f32x4 w4 = rows4(1, wr, u), b4 = rows4(2, br, u), k4 = rows4(3, kr, u), r4 = rows4(4, rr, u);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    S[u + e] = fmaf(w4[e], S[u + e], fmaf(b4[e], sa, k4[e] * vj));
                    op = fmaf(r4[e], S[u + e], op);
                }
            }
            if (WRITE_POS) {
                float *dst = state_pos + ((static_cast<size_t>(bb) * T + t) * H + hh) * (kN * kN) + i0 * kN + j;
#pragma unroll
                for (int u = 0; u < RW; ++u)
                    __builtin_nontemporal_store(S[u], dst + u * kN);
            }
            if (STAGED && state_out && t == L - 1)  // the final state leaves before the o reduction
#pragma unroll
                for (int u = 0; u < RW; ++u)
                    __builtin_nontemporal_store(S[u], state_out + sbase + u * kN);
            part_r[g][j] = op;
            __syncthreads();
            if (g == 0) {
                float acc = part_r[0][j];
#pragma unroll
                for (int gg = 1; gg < NW; ++gg)
                    acc += part_r[gg][j];
                if constexpr (TAIL)
                    acc = tail_norm(acc, t_bonus, vj, t_g, t_w, t_b, tail.eps);
                store_elem(o, base + j, acc);
            }
        }
    }
    if (state_out && (!STAGED || L == 0))  // (staged runs store it with their last token)
#pragma unroll
        for (int u = 0; u < RW; ++u)
            __builtin_nontemporal_store(S[u], state_out + sbase + u * kN);
}

template <typename Tin, typename Tout, bool STAGED, int NW>
hipError_t launch_mode(const SeqArgs &p, hipStream_t stream)
{
    const dim3 grid(static_cast<unsigned>(p.B) * static_cast<unsigned>(p.H)), block(NW * 64);
    const Tin *r = static_cast<const Tin *>(p.r), *w = static_cast<const Tin *>(p.w);
    const Tin *k = static_cast<const Tin *>(p.k), *v = static_cast<const Tin *>(p.v);
    const Tin *a = static_cast<const Tin *>(p.a), *b = static_cast<const Tin *>(p.b);
    Tout *o = static_cast<Tout *>(p.o);
    const bool sin = p.state_in != nullptr, pos = p.state_pos != nullptr;
    const TailIn tail{p.gate, p.r_k, p.ln_w, p.ln_b, p.eps};
#define WKV7_STEP_LAUNCH_T(SIN, POS, VL, TL)                                                                   \
    hipLaunchKernelGGL((wkv7_step_kernel<Tin, Tout, SIN, POS, STAGED, NW, VL, TL>), grid, block, 0, stream, r, w, \
                       k, v, a, b, p.state_in, o, p.state_out, p.state_pos, p.T, p.H, p.lengths, tail)
#define WKV7_STEP_LAUNCH(SIN, POS, VL) WKV7_STEP_LAUNCH_T(SIN, POS, VL, false)
    if (p.gate) {  // the fused tail (whole rows, per-position states optional)
        if (sin && pos)
            WKV7_STEP_LAUNCH_T(true, true, false, true);
        else if (sin)
            WKV7_STEP_LAUNCH_T(true, false, false, true);
        else if (pos)
            WKV7_STEP_LAUNCH_T(false, true, false, true);
        else
            WKV7_STEP_LAUNCH_T(false, false, false, true);
    } else if (p.lengths && sin)  // rows of their own lengths (the forward pass, no per-position states)
        WKV7_STEP_LAUNCH(true, false, true);
    else if (p.lengths)
        WKV7_STEP_LAUNCH(false, false, true);
    else if (sin && pos)
        WKV7_STEP_LAUNCH(true, true, false);
    else if (sin)
        WKV7_STEP_LAUNCH(true, false, false);
    else if (pos)
        WKV7_STEP_LAUNCH(false, true, false);
    else
        WKV7_STEP_LAUNCH(false, false, false);
#undef WKV7_STEP_LAUNCH
#undef WKV7_STEP_LAUNCH_T
    return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_typed(const SeqArgs &p, hipStream_t stream)
{
    // waves per head: four for a single token, eight for longer runs (measured best)
    return p.T > 1 ? launch_mode<Tin, Tout, true, 8>(p, stream) : launch_mode<Tin, Tout, false, 4>(p, stream);
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

// Commit of a speculative step: per (batch row b, head), with n = accepted[b],
// the state after the first n tokens (state_pos[b, n-1]; state_in[b] for n = 0,
// zeros when state_in is null); rows with n outside [0, T] keep state_out.
__global__ __launch_bounds__(256) void state_commit_kernel(const float4 *state_pos, const int *accepted,
                                                           const float4 *state_in, float4 *state_out, int T,
                                                           int H)
{
    constexpr int PER = kN * kN / 4;  // float4 per head
    const int bh = blockIdx.x, bb = bh / H, hh = bh - bb * H;
    const int n = accepted[bb];
    if (n < 0 || n > T)
        return;
    float4 *dst = state_out + static_cast<size_t>(bh) * PER;
    const float4 *src = nullptr;
    if (n > 0)
        src = state_pos + ((static_cast<size_t>(bb) * T + (n - 1)) * H + hh) * PER;
    else if (state_in)
        src = state_in + static_cast<size_t>(bh) * PER;
    if (src == dst)
        return;
    // all of a lane's loads first, then its stores: four loads in flight per lane
    // (a load-store loop waits for each load before the next)
    constexpr int PL = PER / 256;
    float4 x[PL];
#pragma unroll
    for (int q = 0; q < PL; ++q)
        x[q] = src ? src[threadIdx.x + 256 * q] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int q = 0; q < PL; ++q)
        dst[threadIdx.x + 256 * q] = x[q];
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

hipError_t launch_state_commit(const float *state_pos, const int *accepted, const float *state_in,
                               float *state_out, int B, int T, int H, hipStream_t stream)
{
    hipLaunchKernelGGL(state_commit_kernel, dim3(static_cast<unsigned>(B) * static_cast<unsigned>(H)), dim3(256), 0,
                       stream, reinterpret_cast<const float4 *>(state_pos), accepted,
                       reinterpret_cast<const float4 *>(state_in), reinterpret_cast<float4 *>(state_out), T, H);
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
