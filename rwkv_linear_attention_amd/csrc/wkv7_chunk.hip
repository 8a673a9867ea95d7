// wkv7_chunk.hip -- the parallel (prefill) WKV-7 pass: chunked, on the matrix cores.
//
// The SwiftRWKV Inference guide describes a parallel pass over a whole prompt
// that computes the same function as the token-by-token recurrent pass, run as
// one launch whose sequence length is a kernel input.  This file is such a
// pass for gfx950.  The recurrence itself (RWKV-X Architecture page, section
// "WKV-7 Kernel (Generalized Delta Rule)"; Core AI RWKV-7 note, section 1) is
//     S_t = diag(w_t) S_{t-1} + b_t (a_t^T S_{t-1}) + k_t v_t^T,   o_t = S_t^T r_t,
// with S = [K,V] (row = key channel i, column = value channel j).
//
// CHUNK FORM.  Unrolling the recurrence over a chunk of C = 16 tokens that
// starts from state S0 (tau, sigma = 0..15 are positions in the chunk, P_tau
// the product of w over positions 0..tau, per key channel) gives
//     z_tau = S_{tau-1}^T a_tau   (rows of Z)
//     Z = (I - M_ab)^{-1} (A~ S0 + M_ak V)
//     O = R~ S0 + M_rb Z + M_rk V
//     S_C = P_15 S0 + B^T Z + K^T V        (B, K scaled by P_15 / P_sigma)
// where M_xy[tau][sigma] = sum_i x_tau[i] y_sigma[i] P_{tau-1 or tau}[i] / P_sigma[i]
// (strictly lower triangular for the a rows, lower with the diagonal for the
// r rows).  The decays are factored around a reference position inside the
// chunk (after token 7) so that no factor leaves the fp32 exponent range:
//     d_tau = P_tau / P_7,   A'[tau] = a_tau d_{tau-1},   R'[tau] = r_tau d_tau,
//     B'[s] = b_s / d_s,     K'[s] = k_s / d_s,          S^ = diag(P_7) S0,
// so that M_xy = tril(X' Y'^T), and with T = (I - M_ab)^{-1} (a forward
// substitution), E = T M_ak, F = M_rb T, G = F M_ak + M_rk:
//     Z = (T A') S^ + E V
//     O = (R' + F A') S^ + G V
//     S_C = diag(d_15) (S^ + B'^T Z + K'^T V).
// Decay multipliers are raised to at least 2^-15 so that every factor stays
// within 2^(+-120); RWKV-7's decays (>= 0.545) never reach that bound.
//
// MAPPING.  One workgroup of 4 waves per (batch, head, block of NC value
// columns); it walks the chunks of its head in order and keeps its state
// columns in registers, in the accumulator layout of the 16x16 matrix-core
// tiles, for the whole sequence.  Value columns are independent, so a head
// can be split into J = 64/NC column blocks with no communication.  All
// products run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation; fp32
// operands are split into bf16 pieces (x = x0 + x1 [+ x2]) and the piece
// products summed, which keeps fp32-level accuracy on the matrix cores.
#include <type_traits>

#include "wkv7_device.h"
#include "wkv7_launch.h"

namespace wkv7 {
namespace {

constexpr int CH = 16;            // chunk length
constexpr int REF = 7;            // decays are measured relative to the state after this position
constexpr float W_MIN = 0x1p-15f; // lower bound applied to decay multipliers in this kernel
constexpr int NTHREADS = 256;     // 4 waves
constexpr int LDP = kN + 4;       // padded row pitch (floats) of [16][64] tiles
constexpr int LDM = CH + 1;       // padded row pitch of [16][16] tiles

// Split x into NP bf16 pieces whose sum reproduces x to ~2^(-8 NP).
template <int NP>
__device__ __forceinline__ void split_bf16(float x, __bf16 (&out)[3])
{
    __bf16 h0 = static_cast<__bf16>(x);
    out[0] = h0;
    if constexpr (NP > 1) {
        float r1 = x - static_cast<float>(h0);
        __bf16 h1 = static_cast<__bf16>(r1);
        out[1] = h1;
        if constexpr (NP > 2)
            out[2] = static_cast<__bf16>(r1 - static_cast<float>(h1));
    }
}

// acc += A(16 x 32) * B(32 x 16).  av[e] is A[m][slot(q,e)] and bv[e] is
// B[slot(q,e)][n] for this lane (q = lane/16, m = n = lane%16); the slot ->
// k assignment is the caller's (any bijection shared by A and B gives the
// product).  NPA / NPB bf16 pieces per operand; piece products (p, r) with
// p + r < max(NPA, NPB) are kept.
template <int NPA, int NPB>
__device__ __forceinline__ void mma_split(f32x4 &acc, const float (&av)[8], const float (&bv)[8])
{
    bf16x8 A[3], Bm[3];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        __bf16 pa[3], pb[3];
        split_bf16<NPA>(av[e], pa);
        split_bf16<NPB>(bv[e], pb);
#pragma unroll
        for (int p = 0; p < NPA; ++p)
            A[p][e] = pa[p];
#pragma unroll
        for (int p = 0; p < NPB; ++p)
            Bm[p][e] = pb[p];
    }
    constexpr int NPM = NPA > NPB ? NPA : NPB;
    // smallest pieces first
#pragma unroll
    for (int s = NPM - 1; s >= 0; --s)
#pragma unroll
        for (int p = 0; p < NPA; ++p) {
            const int r = s - p;
            if (r >= 0 && r < NPB)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[p], Bm[r], acc, 0, 0, 0);
        }
}

template <int NC>
struct ChunkSmem {
    float Ap[CH][LDP];   // A'[tau][i]
    float Rp[CH][LDP];   // R'[tau][i]
    float Bp[CH][LDP];   // B'[s][i]
    float Kp[CH][LDP];   // K'[s][i]
    float Wm[CH][LDP];   // T A'
    float Pm[CH][LDP];   // R' + F A'
    float V[CH][NC + 4]; // value columns of this workgroup
    float Mab[CH][LDM], Mak[CH][LDM], Mrb[CH][LDM], Mrk[CH][LDM];
    float Tm[CH][LDM], Em[CH][LDM], Fm[CH][LDM], Gm[CH][LDM];
    float d15[kN];       // P_15 / P_7 per key channel
    float p7[kN];        // P_7 per key channel
};

template <typename Tin, typename Tout, int J, bool HAS_STATE_IN>
__global__ __launch_bounds__(NTHREADS) void wkv7_chunk_kernel(SeqArgs p, int per_xcd, int nblocks)
{
    constexpr int NC = kN / J;            // value columns of this workgroup
    constexpr int NSW = NC / 16;          // waves that own state columns
    constexpr bool F32IN = std::is_same<Tin, float>::value;
    constexpr int NP = F32IN ? 3 : 2;     // bf16 pieces of derived fp32 operands
    constexpr int NPV = F32IN ? 3 : 1;    // pieces of v (exact in one piece when it is bf16)
    __shared__ ChunkSmem<NC> sm;

    // Workgroup -> (batch*head, column block).  Workgroups are dealt to the
    // XCDs round-robin; keep the J column blocks of one head on one XCD so the
    // key-side inputs they share are fetched into one L2.
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int lid = xcd * per_xcd + slot;
    if (lid >= nblocks)
        return;
    const int bh = lid / J, jb = lid - bh * J;
    const int H = p.H, T = p.T;
    const int bb = bh / H, hh = bh - bb * H;

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, q = lane >> 4, m = lane & 15;
    const Tin *__restrict__ gw = static_cast<const Tin *>(p.w);
    const Tin *__restrict__ gv = static_cast<const Tin *>(p.v);
    // the key-side input this wave turns into a decay-scaled operand
    const Tin *__restrict__ gx = static_cast<const Tin *>(wv == 0 ? p.a : wv == 1 ? p.r : wv == 2 ? p.b : p.k);
    Tout *__restrict__ go = static_cast<Tout *>(p.o);

    const int j0 = jb * NC;          // first value column of the workgroup
    const int jw = j0 + 16 * wv;     // first value column of this wave's state tile (wv < NSW)
    const size_t rowstride = static_cast<size_t>(H) * kN;            // elements between tokens
    const size_t head0 = (static_cast<size_t>(bb) * T * H + hh) * kN;  // (b, t=0, h, 0)

    // State tile in accumulator layout: Sx[pt][e] = S[16 pt + 4 q + e][jw + m].
    float Sx[4][4];
    const size_t sbase = static_cast<size_t>(bh) * (kN * kN);
    if (wv < NSW) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Sx[pt][e] = HAS_STATE_IN ? p.state_in[sbase + (16 * pt + 4 * q + e) * kN + jw + m] : 0.0f;
    }

    // Register prefetch of one chunk's inputs: lane = key channel for w and x;
    // v is spread over the workgroup.
    constexpr int VPT = CH * NC / NTHREADS;  // v elements per thread
    float wn[CH], xn[CH], vn[VPT];
    auto fetch = [&](int c) {
        const int t0 = c * CH;
#pragma unroll
        for (int tau = 0; tau < CH; ++tau) {
            const bool ok = t0 + tau < T;
            const size_t idx = head0 + static_cast<size_t>(t0 + tau) * rowstride + lane;
            wn[tau] = ok ? load_elem(gw, idx) : 1.0f;
            xn[tau] = ok ? load_elem(gx, idx) : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int flat = u * NTHREADS + tid, tau = flat / NC, jj = flat - tau * NC;
            const bool ok = t0 + tau < T;
            vn[u] = ok ? load_elem(gv, head0 + static_cast<size_t>(t0 + tau) * rowstride + j0 + jj) : 0.0f;
        }
    };

    const int nchunks = (T + CH - 1) / CH;
    fetch(0);
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * CH;
        float wc[CH], xc[CH], vc[VPT];
#pragma unroll
        for (int tau = 0; tau < CH; ++tau) {
            wc[tau] = fmaxf(wn[tau], W_MIN);
            xc[tau] = xn[tau];
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u)
            vc[u] = vn[u];
        if (c + 1 < nchunks)
            fetch(c + 1);

        // ---- A: decay factors and decay-scaled operands (lane = key channel i)
        {
            // d[tau + 1] = d_tau = P_tau / P_7 for tau = -1..15; id[] = 1 / d.
            float d[CH + 1], id[CH + 1];
            d[REF + 1] = 1.0f;
            id[REF + 1] = 1.0f;
            float fwd = 1.0f;
#pragma unroll
            for (int tau = REF + 1; tau < CH; ++tau) {
                fwd *= wc[tau];
                d[tau + 1] = fwd;
                id[tau + 1] = 1.0f / fwd;
            }
            float bwd = 1.0f;  // prod of w over positions tau+1 .. REF
#pragma unroll
            for (int tau = REF - 1; tau >= -1; --tau) {
                bwd *= wc[tau + 1];
                id[tau + 1] = bwd;
                d[tau + 1] = 1.0f / bwd;
            }
            const int i = lane;
#pragma unroll
            for (int tau = 0; tau < CH; ++tau) {
                if (wv == 0)
                    sm.Ap[tau][i] = xc[tau] * d[tau];        // a_tau * d_{tau-1}
                else if (wv == 1)
                    sm.Rp[tau][i] = xc[tau] * d[tau + 1];    // r_tau * d_tau
                else if (wv == 2)
                    sm.Bp[tau][i] = xc[tau] * id[tau + 1];   // b_tau / d_tau
                else
                    sm.Kp[tau][i] = xc[tau] * id[tau + 1];   // k_tau / d_tau
            }
            if (wv == 0) {
                sm.p7[i] = id[0];      // P_7 = 1 / d_{-1}
                sm.d15[i] = d[CH];     // d_15
            }
#pragma unroll
            for (int u = 0; u < VPT; ++u) {
                const int flat = u * NTHREADS + tid, tau = flat / NC, jj = flat - tau * NC;
                sm.V[tau][jj] = vc[u];
            }
        }
        __syncthreads();

        // ---- B: M_ab, M_ak, M_rb, M_rk (one 16x16 tile per wave, K = 64 key channels)
        {
            const float(*X1)[LDP] = wv < 2 ? sm.Ap : sm.Rp;
            const float(*X2)[LDP] = (wv & 1) ? sm.Kp : sm.Bp;
            float(*Md)[LDM] = wv == 0 ? sm.Mab : wv == 1 ? sm.Mak : wv == 2 ? sm.Mrb : sm.Mrk;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                float av[8], bv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    av[e] = X1[m][32 * s + 8 * q + e];
                    bv[e] = X2[m][32 * s + 8 * q + e];
                }
                mma_split<NP, NP>(acc, av, bv);
            }
            const bool strict = wv < 2;  // a rows exclude the diagonal, r rows include it
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tau = 4 * q + e, sg = m;
                Md[tau][sg] = (sg < tau || (!strict && sg == tau)) ? acc[e] : 0.0f;
            }
        }
        __syncthreads();

        // ---- C: T = (I - M_ab)^{-1} by forward substitution, one column per lane
        if (wv == 0 && lane < CH) {
            float x[CH];
#pragma unroll
            for (int tau = 0; tau < CH; ++tau)
                x[tau] = tau == lane ? 1.0f : 0.0f;
#pragma unroll
            for (int sg = 0; sg < CH; ++sg)
#pragma unroll
                for (int tau = sg + 1; tau < CH; ++tau)
                    x[tau] = fmaf(sm.Mab[tau][sg], x[sg], x[tau]);
#pragma unroll
            for (int tau = 0; tau < CH; ++tau)
                sm.Tm[tau][lane] = x[tau];
        }
        __syncthreads();

        // ---- D1: E = T M_ak (wave 0), F = M_rb T (wave 1), W = T A' (tile wv of 4)
        {
            float av[8], bv[8];
            if (wv < 2) {
                const float(*LA)[LDM] = wv == 0 ? sm.Tm : sm.Mrb;
                const float(*LB)[LDM] = wv == 0 ? sm.Mak : sm.Tm;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int kk = 8 * q + e;
                    av[e] = kk < CH ? LA[m][kk] : 0.0f;
                    bv[e] = kk < CH ? LB[kk][m] : 0.0f;
                }
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                mma_split<NP, NP>(acc, av, bv);
                float(*Dd)[LDM] = wv == 0 ? sm.Em : sm.Fm;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Dd[4 * q + e][m] = acc[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kk = 8 * q + e;
                av[e] = kk < CH ? sm.Tm[m][kk] : 0.0f;
                bv[e] = kk < CH ? sm.Ap[kk][16 * wv + m] : 0.0f;
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_split<NP, NP>(acc, av, bv);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sm.Wm[4 * q + e][16 * wv + m] = acc[e];
        }
        __syncthreads();

        // ---- D2: G = F M_ak + M_rk (wave 0), P = R' + F A' (tile wv of 4)
        {
            float av[8], bv[8];
            if (wv == 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int kk = 8 * q + e;
                    av[e] = kk < CH ? sm.Fm[m][kk] : 0.0f;
                    bv[e] = kk < CH ? sm.Mak[kk][m] : 0.0f;
                }
                f32x4 acc;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[e] = sm.Mrk[4 * q + e][m];
                mma_split<NP, NP>(acc, av, bv);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sm.Gm[4 * q + e][m] = acc[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kk = 8 * q + e;
                av[e] = kk < CH ? sm.Fm[m][kk] : 0.0f;
                bv[e] = kk < CH ? sm.Ap[kk][16 * wv + m] : 0.0f;
            }
            f32x4 acc;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[e] = sm.Rp[4 * q + e][16 * wv + m];
            mma_split<NP, NP>(acc, av, bv);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sm.Pm[4 * q + e][16 * wv + m] = acc[e];
        }
        __syncthreads();

        // ---- E: the state-dependent part, per wave on its 16 value columns
        if (wv < NSW) {
            const int jl = 16 * wv + m;  // this lane's column inside the workgroup block
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Sx[pt][e] *= sm.p7[16 * pt + 4 * q + e];  // S^ = diag(P_7) S0
            // Key slot (q, e) of k-step s stands for key row 16 (2 s + e/4) + 4 q + e%4,
            // which is exactly what this lane holds of S^ in Sx[2 s + e/4][e % 4].
            f32x4 z = {0.f, 0.f, 0.f, 0.f}, ov = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                float aw[8], ap[8], bs[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int krow = 16 * (2 * s + e / 4) + 4 * q + (e & 3);
                    aw[e] = sm.Wm[m][krow];
                    ap[e] = sm.Pm[m][krow];
                    bs[e] = Sx[2 * s + e / 4][e & 3];
                }
                mma_split<NP, NP>(z, aw, bs);
                mma_split<NP, NP>(ov, ap, bs);
            }
            {
                float ae[8], ag[8], bvv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int kk = 8 * q + e;
                    ae[e] = kk < CH ? sm.Em[m][kk] : 0.0f;
                    ag[e] = kk < CH ? sm.Gm[m][kk] : 0.0f;
                    bvv[e] = kk < CH ? sm.V[kk][jl] : 0.0f;
                }
                mma_split<NP, NPV>(z, ae, bvv);
                mma_split<NP, NPV>(ov, ag, bvv);
            }
            // outputs: lane (q, m) holds O[4q + e][jw + m]
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tau = 4 * q + e;
                if (t0 + tau < T)
                    store_elem(go, head0 + static_cast<size_t>(t0 + tau) * rowstride + jw + m, ov[e]);
            }
            // S^ += B'^T Z + K'^T V, then S = diag(d_15) S^.  Slot (q, e): e < 4 is
            // Z row 4q + e (held by this lane in z[e]); e >= 4 is V row 4q + e - 4.
            float bz[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bz[e] = z[e];
                bz[e + 4] = sm.V[4 * q + e][jl];
            }
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                float ak[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ak[e] = sm.Bp[4 * q + e][16 * pt + m];
                    ak[e + 4] = sm.Kp[4 * q + e][16 * pt + m];
                }
                f32x4 acc = {Sx[pt][0], Sx[pt][1], Sx[pt][2], Sx[pt][3]};
                mma_split<NP, NP>(acc, ak, bz);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Sx[pt][e] = acc[e] * sm.d15[16 * pt + 4 * q + e];
            }
        }
        __syncthreads();
    }

    if (wv < NSW) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.state_out[sbase + (16 * pt + 4 * q + e) * kN + jw + m] = Sx[pt][e];
    }
}

template <typename Tin, typename Tout, int J>
hipError_t launch_j(const SeqArgs &p, hipStream_t stream)
{
    const int nblocks = p.B * p.H * J;
    int per_xcd = (nblocks + 7) / 8;
    per_xcd = (per_xcd + J - 1) / J * J;  // a head's column blocks never straddle two XCDs
    const dim3 grid(8 * per_xcd), block(NTHREADS);
    if (p.state_in)
        hipLaunchKernelGGL((wkv7_chunk_kernel<Tin, Tout, J, true>), grid, block, 0, stream, p, per_xcd, nblocks);
    else
        hipLaunchKernelGGL((wkv7_chunk_kernel<Tin, Tout, J, false>), grid, block, 0, stream, p, per_xcd, nblocks);
    return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_typed(const SeqArgs &p, hipStream_t stream)
{
    // Split heads into column blocks until the grid covers the 256 compute units.
    const long long heads = static_cast<long long>(p.B) * p.H;
    if (heads >= 256)
        return launch_j<Tin, Tout, 1>(p, stream);
    if (heads >= 128)
        return launch_j<Tin, Tout, 2>(p, stream);
    return launch_j<Tin, Tout, 4>(p, stream);
}

}  // namespace

hipError_t launch_chunk(const SeqArgs &p, hipStream_t stream)
{
    if (p.in_bf16)
        return p.o_bf16 ? launch_typed<uint16_t, uint16_t>(p, stream) : launch_typed<uint16_t, float>(p, stream);
    return p.o_bf16 ? launch_typed<float, uint16_t>(p, stream) : launch_typed<float, float>(p, stream);
}

}  // namespace wkv7
