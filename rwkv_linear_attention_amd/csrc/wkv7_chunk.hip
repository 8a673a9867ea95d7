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
// the product of w over positions 0..tau, per key channel) gives, for the
// rows z_tau = S_{tau-1}^T a_tau of Z,
//     Z   = (I - M_ab)^{-1} (A~ S0 + M_ak V)
//     O   = R~ S0 + M_rb Z + M_rk V
//     S_C = diag(P_15) S0 + B^^T Z + K^^T V
// where A~[tau] = a_tau P_{tau-1}, R~[tau] = r_tau P_tau, B^[s] = b_s P_15/P_s,
// K^[s] = k_s P_15/P_s, and M_xy[tau][s] = sum_i x_tau[i] y_s[i] P_{tau-1 or
// tau}[i] / P_s[i] (strictly lower triangular for the a rows, lower with the
// diagonal for the r rows).  The decays are factored around a reference
// position inside the chunk (after position 7) so that no factor leaves the
// fp32 exponent range:
//     d_tau = P_tau / P_7,   A'[tau] = a_tau d_{tau-1},   R'[tau] = r_tau d_tau,
//     B'[s] = b_s / d_s,     K'[s] = k_s / d_s,          S^ = diag(P_7) S0,
// so that M_xy = tril(X' Y'^T) and, with T = (I - M_ab)^{-1},
//     Z   = T (A' S^ + M_ak V)
//     O   = R' S^ + [M_rb | M_rk] [Z ; V]
//     S_C = diag(d_15) (S^ + [B'^T | K'^T] [Z ; V]).
// Decay multipliers are raised to at least 2^-15 so that every factor stays
// within 2^(+-120); RWKV-7's decays (>= 0.545) never come near that bound.
//
// MAPPING (gfx950).  One workgroup per (batch, head, block of NC value
// columns); value columns evolve independently, so a head splits into
// J = 64/NC blocks with no communication.  The workgroup is a software
// pipeline with one barrier per chunk and two kinds of waves:
//  * consumer waves (NC/16 of them) each keep a 64x16 slice of the fp32 state
//    in registers, in the accumulator layout of a 16x16 matrix-core tile, for
//    the whole sequence, and run only the state-dependent products of chunk c;
//  * four producer waves compute, one iteration ahead, the intra-chunk
//    matrices M and the triangular inverse T of chunk c+1, and, two
//    iterations ahead, the decay-scaled operands of chunk c+2, from inputs they
//    prefetched two iterations before that.
// Chunk data lives in a ring of three LDS slots.  All products run on
// v_mfma_f32_16x16x{32,16}_bf16 with fp32 accumulation; fp32 operands are
// split into bf16 pieces (x = x0 + x1 [+ x2], stored pre-split in LDS) and
// the piece products summed, which keeps fp32-level accuracy on the matrix
// cores.  bf16 inputs (v here) are exact in one piece.
#include <type_traits>

#include "wkv7_device.h"
#include "wkv7_launch.h"

namespace wkv7 {
namespace {

constexpr int CH = 16;             // chunk length
constexpr int REF = 7;             // decays are measured relative to the state after this position
constexpr float W_MIN = 0x1p-15f;  // lower bound applied to decay multipliers in this kernel
constexpr int NPROD = 4;           // producer waves
constexpr int LDA = kN + 8;        // row pitch (bf16) of [16][64] operand planes
constexpr int LDT = CH + 8;        // row pitch (bf16) of [64][16] transposed planes
constexpr int LDM = CH + 1;        // row pitch (fp32) of [16][16] matrices

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint16_t bf16_bits(float x)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));  // round to nearest even
}
__device__ __forceinline__ float bf16_val(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

// x = sum of NP bf16 pieces (to ~2^(-8 NP) relative).
template <int NP>
__device__ __forceinline__ void split(float x, uint16_t (&o)[NP])
{
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        o[p] = bf16_bits(x);
        x -= bf16_val(o[p]);
    }
}

// Piece products acc += sum_{p + r < max(NPA,NPB)} A_p B_r, smallest first.
template <int NPA, int NPB>
__device__ __forceinline__ void mma32(f32x4 &acc, const s16x8 (&A)[NPA], const s16x8 (&B)[NPB])
{
    constexpr int NPM = NPA > NPB ? NPA : NPB;
#pragma unroll
    for (int s = NPM - 1; s >= 0; --s)
#pragma unroll
        for (int p = 0; p < NPA; ++p) {
            const int r = s - p;
            if (r >= 0 && r < NPB)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[p]),
                                                              __builtin_bit_cast(bf16x8, B[r]), acc, 0, 0, 0);
        }
}
template <int NPA, int NPB>
__device__ __forceinline__ void mma16(f32x4 &acc, const s16x4 (&A)[NPA], const s16x4 (&B)[NPB])
{
    constexpr int NPM = NPA > NPB ? NPA : NPB;
#pragma unroll
    for (int s = NPM - 1; s >= 0; --s)
#pragma unroll
        for (int p = 0; p < NPA; ++p) {
            const int r = s - p;
            if (r >= 0 && r < NPB)
                acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A[p], B[r], acc, 0, 0, 0);
        }
}

// Split 8 (or 4) fp32 values into NP fragment planes.
template <int NP>
__device__ __forceinline__ void split8(const float (&v)[8], s16x8 (&out)[NP])
{
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint16_t pc[NP];
        split<NP>(v[e], pc);
#pragma unroll
        for (int p = 0; p < NP; ++p)
            out[p][e] = static_cast<short>(pc[p]);
    }
}
template <int NP>
__device__ __forceinline__ void split4(const float (&v)[4], s16x4 (&out)[NP])
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint16_t pc[NP];
        split<NP>(v[e], pc);
#pragma unroll
        for (int p = 0; p < NP; ++p)
            out[p][e] = static_cast<short>(pc[p]);
    }
}

__device__ __forceinline__ s16x4 lds4(const uint16_t *p) { return *reinterpret_cast<const s16x4 *>(p); }

// One chunk's data in LDS.  Operand planes hold bf16 bit patterns.
template <int NP, int NPV, int NC>
struct Slot {
    uint16_t Ap[NP][CH][LDA];    // A'[tau][i]
    uint16_t Rp[NP][CH][LDA];    // R'[tau][i]
    uint16_t BpT[NP][kN][LDT];   // B'[s][i] stored as [i][s]
    uint16_t KpT[NP][kN][LDT];   // K'[s][i] stored as [i][s]
    uint16_t Vt[NPV][NC][LDT];   // v[s][j] stored as [j][s]
    float M[3][CH][LDM];         // M_ak, M_rb, M_rk (masked)
    float Tm[CH][LDM];           // (I - M_ab)^{-1}
    float p7[kN];                // P_7 per key channel
    float d15[kN];               // P_15 / P_7 per key channel
};

template <int NP, int NPV, int NC>
struct Smem {
    Slot<NP, NPV, NC> slot[3];
    float Mab[CH][LDM];          // scratch of the wave that solves for T
};

// Decay factors of one key channel over a chunk: d[tau+1] = P_tau / P_7 and
// id[tau+1] = P_7 / P_tau for tau = -1..15 (P_-1 = 1), with two reciprocals.
__device__ __forceinline__ void decay_factors(const float (&w)[CH], float (&d)[CH + 1], float (&id)[CH + 1])
{
    // id for tau <= REF: product of w over tau+1 .. REF
    id[REF + 1] = 1.0f;
#pragma unroll
    for (int tau = REF - 1; tau >= -1; --tau)
        id[tau + 1] = id[tau + 2] * w[tau + 1];
    // d for tau >= REF: product of w over REF+1 .. tau
    d[REF + 1] = 1.0f;
#pragma unroll
    for (int tau = REF + 1; tau < CH; ++tau)
        d[tau + 1] = d[tau] * w[tau];
    // d for tau < REF: P_tau / P_7 = (1 / P_7) * prod_{0..tau} w
    const float inv_p7 = __builtin_amdgcn_rcpf(id[0]);
    float pre = inv_p7;
    d[0] = inv_p7;
#pragma unroll
    for (int tau = 0; tau < REF; ++tau) {
        pre *= w[tau];
        d[tau + 1] = pre;
    }
    // id for tau > REF: P_7 / P_tau = (1 / d_15) * prod_{tau+1..15} w
    const float inv_d15 = __builtin_amdgcn_rcpf(d[CH]);
    float post = inv_d15;
    id[CH] = inv_d15;
#pragma unroll
    for (int tau = CH - 2; tau >= REF + 1; --tau) {
        post *= w[tau + 1];
        id[tau + 1] = post;
    }
}

template <typename Tin, typename Tout, int J, bool HAS_STATE_IN>
__global__ __launch_bounds__((kN / J / 16 + NPROD) * 64) void wkv7_chunk_kernel(SeqArgs p, int per_xcd,
                                                                                   int nblocks)
{
    constexpr int NC = kN / J;            // value columns of this workgroup
    constexpr int NSW = NC / 16;          // consumer waves (16 state columns each)
    constexpr bool F32IN = std::is_same<Tin, float>::value;
    constexpr int NP = F32IN ? 3 : 2;     // bf16 pieces of derived fp32 operands
    constexpr int NPV = F32IN ? 3 : 1;    // pieces of v (one is exact for bf16 inputs)
    using SlotT = Slot<NP, NPV, NC>;
    __shared__ Smem<NP, NPV, NC> sm;

    // Workgroup -> (batch*head, column block).  Workgroups are dealt to the
    // XCDs round-robin; the J column blocks of one head stay on one XCD so the
    // key-side inputs they share are fetched into one L2.
    const int xcd = blockIdx.x & 7, slot_id = blockIdx.x >> 3;
    const int lid = xcd * per_xcd + slot_id;
    if (lid >= nblocks)
        return;
    const int bh = lid / J, jb = lid - bh * J;
    const int H = p.H, T = p.T;
    const int bb = bh / H, hh = bh - bb * H;
    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, m = lane & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j0 = jb * NC;
    const size_t rowstride = static_cast<size_t>(H) * kN;              // elements between tokens
    const size_t head0 = (static_cast<size_t>(bb) * T * H + hh) * kN;   // (b, t=0, h, 0)
    const size_t sbase = static_cast<size_t>(bh) * (kN * kN);
    const int nchunks = (T + CH - 1) / CH;

    if (wv < NSW) {
        // ------------------------------------------------------------ consumer
        const int jw = j0 + 16 * wv;      // this wave's first state column
        const int jl = 16 * wv + m;       // this lane's column inside the workgroup block
        Tout *__restrict__ go = static_cast<Tout *>(p.o);
        // Sx[pt][e] = S[16 pt + 4 q + e][jw + m] (the true state between chunks)
        float Sx[4][4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Sx[pt][e] = HAS_STATE_IN ? p.state_in[sbase + (16 * pt + 4 * q + e) * kN + jw + m] : 0.0f;

        for (int i = -2; i < nchunks; ++i) {
            if (i >= 0) {
                const SlotT &sl = sm.slot[i % 3];
                const int t0 = i * CH;
                // S^ = diag(P_7) S, as matrix-core B operands over the key index:
                // key slot (q, e) of k-step s is key row 16 (2 s + e/4) + 4 q + e%4,
                // which this lane holds in Sx[2 s + e/4][e % 4].
                s16x8 Bs[2][NP];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    float v8[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int pt = 2 * s + e / 4;
                        v8[e] = Sx[pt][e & 3] * sl.p7[16 * pt + 4 * q + (e & 3)];
                    }
                    split8<NP>(v8, Bs[s]);
                }
                // A'-rows and R'-rows as A operands with the same key slots
                f32x4 y = {0.f, 0.f, 0.f, 0.f}, o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    s16x8 Af[NP], Rf[NP];
#pragma unroll
                    for (int pl = 0; pl < NP; ++pl) {
                        const s16x4 a0 = lds4(&sl.Ap[pl][m][32 * s + 4 * q]);
                        const s16x4 a1 = lds4(&sl.Ap[pl][m][32 * s + 16 + 4 * q]);
                        const s16x4 r0 = lds4(&sl.Rp[pl][m][32 * s + 4 * q]);
                        const s16x4 r1 = lds4(&sl.Rp[pl][m][32 * s + 16 + 4 * q]);
                        Af[pl] = s16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                        Rf[pl] = s16x8{r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
                    }
                    mma32<NP, NP>(y, Af, Bs[s]);
                    mma32<NP, NP>(o, Rf, Bs[s]);
                }
                // V rows as a B operand over the token index (slot (q, e) = token 4 q + e)
                s16x4 Vf[NPV];
#pragma unroll
                for (int pl = 0; pl < NPV; ++pl)
                    Vf[pl] = lds4(&sl.Vt[pl][jl][4 * q]);
                // y += M_ak V
                {
                    float a4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        a4[e] = sl.M[0][m][4 * q + e];
                    s16x4 Mf[NP];
                    split4<NP>(a4, Mf);
                    mma16<NP, NPV>(y, Mf, Vf);
                }
                // Z = T Y  (Y held in accumulator layout: Y[4 q + e][col m] = y[e])
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
                {
                    float t4[4], y4[4] = {y[0], y[1], y[2], y[3]};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        t4[e] = sl.Tm[m][4 * q + e];
                    s16x4 Tf[NP], Yf[NP];
                    split4<NP>(t4, Tf);
                    split4<NP>(y4, Yf);
                    mma16<NP, NP>(z, Tf, Yf);
                }
                // [Z ; V] as one B operand over 32 token slots: (q, e<4) is Z row 4q+e
                // (this lane's z[e]), (q, e>=4) is V row 4q+e-4.
                s16x8 ZV[NP];
                {
                    float z4[4] = {z[0], z[1], z[2], z[3]};
                    s16x4 Zf[NP];
                    split4<NP>(z4, Zf);
#pragma unroll
                    for (int pl = 0; pl < NP; ++pl) {
                        const s16x4 vv = pl < NPV ? Vf[pl < NPV ? pl : 0] : s16x4{0, 0, 0, 0};
                        ZV[pl] = s16x8{Zf[pl][0], Zf[pl][1], Zf[pl][2], Zf[pl][3], vv[0], vv[1], vv[2], vv[3]};
                    }
                }
                // o += [M_rb | M_rk] [Z ; V]
                {
                    float a8[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a8[e] = sl.M[1][m][4 * q + e];
                        a8[e + 4] = sl.M[2][m][4 * q + e];
                    }
                    s16x8 Mf[NP];
                    split8<NP>(a8, Mf);
                    mma32<NP, NP>(o, Mf, ZV);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tau = 4 * q + e;
                    if (t0 + tau < T)
                        store_elem(go, head0 + static_cast<size_t>(t0 + tau) * rowstride + jw + m, o[e]);
                }
                // S = diag(d_15) (S^ + [B'^T | K'^T] [Z ; V]), one 16-row tile at a time
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    s16x8 Uf[NP];
#pragma unroll
                    for (int pl = 0; pl < NP; ++pl) {
                        const s16x4 b4 = lds4(&sl.BpT[pl][16 * pt + m][4 * q]);
                        const s16x4 k4 = lds4(&sl.KpT[pl][16 * pt + m][4 * q]);
                        Uf[pl] = s16x8{b4[0], b4[1], b4[2], b4[3], k4[0], k4[1], k4[2], k4[3]};
                    }
                    f32x4 acc;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[e] = Sx[pt][e] * sl.p7[16 * pt + 4 * q + e];
                    mma32<NP, NP>(acc, Uf, ZV);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        Sx[pt][e] = acc[e] * sl.d15[16 * pt + 4 * q + e];
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.state_out[sbase + (16 * pt + 4 * q + e) * kN + jw + m] = Sx[pt][e];
        return;
    }

    // ---------------------------------------------------------------- producers
    const int pw = wv - NSW;  // 0: M_ab and T; 1: A' K' and M_ak; 2: R' and M_rb; 3: B' v and M_rk
    const Tin *__restrict__ gw = static_cast<const Tin *>(p.w);
    const Tin *__restrict__ gx0 = static_cast<const Tin *>(pw == 1 ? p.a : pw == 2 ? p.r : p.b);
    const Tin *__restrict__ gx1 = static_cast<const Tin *>(pw == 1 ? p.k : p.v);
    const bool has_x1 = pw == 1 || pw == 3;   // second stream: k for wave 1, v for wave 3
    // Prefetched raw inputs of one chunk (lane = key channel, or value column for v).
    struct Raw {
        Tin w[CH], x0[CH], x1[CH];
    };
    Raw ra, rb;
    auto fetch = [&](Raw &R, int c) {
        if (pw == 0 || c >= nchunks)
            return;
        const int t0 = c * CH;
#pragma unroll
        for (int tau = 0; tau < CH; ++tau) {
            const int t = min(t0 + tau, T - 1);
            const size_t row = head0 + static_cast<size_t>(t) * rowstride;
            R.w[tau] = gw[row + lane];
            R.x0[tau] = gx0[row + lane];
            if (has_x1)
                R.x1[tau] = gx1[row + (pw == 3 ? (j0 + (lane < NC ? lane : 0)) : lane)];
        }
    };
    // Operand stage: decay-scaled operands of chunk c into its slot.
    auto operands = [&](const Raw &R, int c) {
        if (pw == 0 || c >= nchunks)
            return;
        SlotT &sl = sm.slot[c % 3];
        const int t0 = c * CH, i = lane;
        float w[CH], x0[CH], x1[CH];
#pragma unroll
        for (int tau = 0; tau < CH; ++tau) {
            const bool ok = t0 + tau < T;
            w[tau] = ok ? fmaxf(load_elem(R.w, tau), W_MIN) : 1.0f;
            x0[tau] = ok ? load_elem(R.x0, tau) : 0.0f;
            x1[tau] = (ok && has_x1) ? load_elem(R.x1, tau) : 0.0f;
        }
        float d[CH + 1], id[CH + 1];
        decay_factors(w, d, id);
        if (pw == 1 || pw == 2) {
            // A' (wave 1) or R' (wave 2), rows over tau, one bf16 write per plane and row
            uint16_t(*dst)[CH][LDA] = pw == 1 ? sl.Ap : sl.Rp;
#pragma unroll
            for (int tau = 0; tau < CH; ++tau) {
                uint16_t pc[NP];
                split<NP>(x0[tau] * (pw == 1 ? d[tau] : d[tau + 1]), pc);
#pragma unroll
                for (int pl = 0; pl < NP; ++pl)
                    dst[pl][tau][i] = pc[pl];
            }
        }
        // K' (wave 1, from x1) or B' (wave 3, from x0): transposed rows, 16 bf16 per plane
        if (pw == 1 || pw == 3) {
            uint16_t(*dst)[kN][LDT] = pw == 1 ? sl.KpT : sl.BpT;
            const float *src = pw == 1 ? x1 : x0;
            s16x8 lo[NP], hi[NP];
#pragma unroll
            for (int s = 0; s < CH; ++s) {
                uint16_t pc[NP];
                split<NP>(src[s] * id[s + 1], pc);
#pragma unroll
                for (int pl = 0; pl < NP; ++pl) {
                    if (s < 8)
                        lo[pl][s] = static_cast<short>(pc[pl]);
                    else
                        hi[pl][s - 8] = static_cast<short>(pc[pl]);
                }
            }
#pragma unroll
            for (int pl = 0; pl < NP; ++pl) {
                *reinterpret_cast<s16x8 *>(&dst[pl][i][0]) = lo[pl];
                *reinterpret_cast<s16x8 *>(&dst[pl][i][8]) = hi[pl];
            }
        }
        if (pw == 3) {
            sl.p7[i] = id[0];      // P_7
            sl.d15[i] = d[CH];     // P_15 / P_7
            if (lane < NC) {
                // v column j0 + lane over the chunk, transposed
#pragma unroll
                for (int pl = 0; pl < NPV; ++pl) {
                    s16x8 lo, hi;
#pragma unroll
                    for (int s = 0; s < CH; ++s) {
                        uint16_t pc[NPV];
                        split<NPV>(x1[s], pc);
                        if (s < 8)
                            lo[s] = static_cast<short>(pc[pl]);
                        else
                            hi[s - 8] = static_cast<short>(pc[pl]);
                    }
                    *reinterpret_cast<s16x8 *>(&sl.Vt[pl][lane][0]) = lo;
                    *reinterpret_cast<s16x8 *>(&sl.Vt[pl][lane][8]) = hi;
                }
            }
        }
    };
    // Matrix stage: one 16x16 tile M = tril(X' Y'^T) of chunk c per wave over
    // the 64 key channels; wave 0 also inverts I - M_ab by forward substitution.
    auto matrices = [&](int c) {
        if (c < 0 || c >= nchunks)
            return;
        SlotT &sl = sm.slot[c % 3];
        const uint16_t(*X)[CH][LDA] = (pw == 0 || pw == 1) ? sl.Ap : sl.Rp;
        const uint16_t(*Y)[kN][LDT] = (pw == 0 || pw == 2) ? sl.BpT : sl.KpT;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            s16x8 Af[NP], Bf[NP];
#pragma unroll
            for (int pl = 0; pl < NP; ++pl) {
                Af[pl] = *reinterpret_cast<const s16x8 *>(&X[pl][m][32 * s + 8 * q]);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    Bf[pl][e] = static_cast<short>(Y[pl][32 * s + 8 * q + e][m]);
            }
            mma32<NP, NP>(acc, Af, Bf);
        }
        const bool strict = pw < 2;  // a rows exclude the diagonal, r rows include it
        float(*dst)[LDM] = pw == 0 ? sm.Mab : sl.M[pw - 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tau = 4 * q + e;
            dst[tau][m] = (m < tau || (!strict && m == tau)) ? acc[e] : 0.0f;
        }
        if (pw == 0) {
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's M_ab writes are done
            __builtin_amdgcn_wave_barrier();
            if (lane < CH) {
                // column `lane` of (I - M_ab)^{-1}
                float x[CH];
#pragma unroll
                for (int tau = 0; tau < CH; ++tau)
                    x[tau] = tau == lane ? 1.0f : 0.0f;
#pragma unroll
                for (int s = 0; s < CH; ++s)
#pragma unroll
                    for (int tau = s + 1; tau < CH; ++tau)
                        x[tau] = fmaf(sm.Mab[tau][s], x[s], x[tau]);
#pragma unroll
                for (int tau = 0; tau < CH; ++tau)
                    sl.Tm[tau][lane] = x[tau];
            }
        }
    };

    // Pipeline: iteration i consumes chunk i (consumer waves), builds the
    // matrices of chunk i+1 and the operands of chunk i+2, and prefetches the
    // inputs of chunk i+4.  Two register sets alternate between even and odd i.
    fetch(ra, 0);
    fetch(rb, 1);
    for (int i = -2; i < nchunks; i += 2) {
        matrices(i + 1);
        operands(ra, i + 2);
        fetch(ra, i + 4);
        __syncthreads();
        if (i + 1 < nchunks) {
            matrices(i + 2);
            operands(rb, i + 3);
            fetch(rb, i + 5);
            __syncthreads();
        }
    }
}

template <typename Tin, typename Tout, int J>
hipError_t launch_j(const SeqArgs &p, hipStream_t stream)
{
    const int nblocks = p.B * p.H * J;
    int per_xcd = (nblocks + 7) / 8;
    per_xcd = (per_xcd + J - 1) / J * J;  // a head's column blocks never straddle two XCDs
    const dim3 grid(8 * per_xcd), block((kN / J / 16 + NPROD) * 64);
    if (p.state_in)
        hipLaunchKernelGGL((wkv7_chunk_kernel<Tin, Tout, J, true>), grid, block, 0, stream, p, per_xcd, nblocks);
    else
        hipLaunchKernelGGL((wkv7_chunk_kernel<Tin, Tout, J, false>), grid, block, 0, stream, p, per_xcd, nblocks);
    return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_typed(const SeqArgs &p, hipStream_t stream)
{
    // One workgroup fills a compute unit's LDS; split heads into column blocks
    // only while the grid still fits in one pass over the 256 compute units.
    const long long heads = static_cast<long long>(p.B) * p.H;
    if (heads * 4 <= 256)
        return launch_j<Tin, Tout, 4>(p, stream);
    if (heads * 2 <= 256)
        return launch_j<Tin, Tout, 2>(p, stream);
    return launch_j<Tin, Tout, 1>(p, stream);
}

}  // namespace

hipError_t launch_chunk(const SeqArgs &p, hipStream_t stream)
{
    if (p.in_bf16)
        return p.o_bf16 ? launch_typed<uint16_t, uint16_t>(p, stream) : launch_typed<uint16_t, float>(p, stream);
    return p.o_bf16 ? launch_typed<float, uint16_t>(p, stream) : launch_typed<float, float>(p, stream);
}

}  // namespace wkv7
