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
constexpr int LDM = CH + 4;        // row pitch (fp32) of [16][16] matrices (16-byte rows)

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

template <int NP, bool ON>
struct RowMajorBK {
    uint16_t Bp[NP][CH][LDA];
    uint16_t Kp[NP][CH][LDA];
};
template <int NP>
struct RowMajorBK<NP, false> {};

// One chunk's data in LDS.  Operand planes hold bf16 bit patterns.  With
// bf16 inputs (NP == 2) B' and K' are also kept row-major, so the matrix
// stage reads its operands with 16-byte loads; the fp32-input build (NP == 3)
// has no room for them and gathers from the transposed copies instead.
template <int NP, int NPV, int NC>
struct alignas(16) Slot {
    uint16_t Ap[NP][CH][LDA];    // A'[tau][i]
    uint16_t Rp[NP][CH][LDA];    // R'[tau][i]
    RowMajorBK<NP, NP == 2> bk;  // B'[s][i], K'[s][i]  (NP == 2 only)
    uint16_t BpT[NP][kN][LDT];   // B'[s][i] stored as [i][s]
    uint16_t KpT[NP][kN][LDT];   // K'[s][i] stored as [i][s]
    uint16_t Vt[NPV][NC][LDT];   // v[s][j] stored as [j][s]
    float M[3][CH][LDM];         // M_ak, M_rb, M_rk (masked)
    float Tm[CH][LDM];           // (I - M_ab)^{-1}
    alignas(16) float p7[kN];    // P_7 per key channel
    alignas(16) float d15[kN];   // P_15 / P_7 per key channel
};

// Raw bf16 input rows of one chunk, staged by the producers: [stream][tau][i]
// with streams w, a, r, k, b, v (v holds all 64 columns of the head).
struct alignas(16) RawSlot {
    uint16_t x[6][CH][kN];
};

template <bool ON>
struct RawRing {
    RawSlot raw[2];
};
template <>
struct RawRing<false> {};

template <int NP, int NPV, int NC>
struct Smem {
    Slot<NP, NPV, NC> slot[3];
    RawRing<NP == 2> rr;         // staged raw rows (bf16 inputs only)
    float Mab[CH][LDM];          // scratch of the wave that solves for T
    float Xs[8][9];              // scratch of the blocked triangular inverse
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
    constexpr bool STAGED = !F32IN;  // bf16 rows go through the LDS staging ring

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

        if constexpr (STAGED)
            __syncthreads();  // matches the producers' prologue
        for (int i = -2; i < nchunks; ++i) {
            if (i >= 0) {
                const SlotT &sl = sm.slot[i % 3];
                const int t0 = i * CH;
                // P_7 and d_15 of this lane's 16 key rows 16 pt + 4 q + e
                f32x4 p7v[4], d15v[4];
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    p7v[pt] = *reinterpret_cast<const f32x4 *>(&sl.p7[16 * pt + 4 * q]);
                    d15v[pt] = *reinterpret_cast<const f32x4 *>(&sl.d15[16 * pt + 4 * q]);
                }
                // S^ = diag(P_7) S, as matrix-core B operands over the key index:
                // key slot (q, e) of k-step s is key row 16 (2 s + e/4) + 4 q + e%4,
                // which this lane holds in Sx[2 s + e/4][e % 4].
                float Sh[4][4];
#pragma unroll
                for (int pt = 0; pt < 4; ++pt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        Sh[pt][e] = Sx[pt][e] * p7v[pt][e];
                s16x8 Bs[2][NP];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    float v8[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v8[e] = Sh[2 * s + e / 4][e & 3];
                    split8<NP>(v8, Bs[s]);
                }
                // A'-rows and R'-rows as A operands with the same key slots;
                // independent accumulators per k-step keep the chains short.
                f32x4 y2[2], o2[2];
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
                    y2[s] = f32x4{0.f, 0.f, 0.f, 0.f};
                    o2[s] = f32x4{0.f, 0.f, 0.f, 0.f};
                    mma32<NP, NP>(y2[s], Af, Bs[s]);
                    mma32<NP, NP>(o2[s], Rf, Bs[s]);
                }
                // V rows as a B operand over the token index (slot (q, e) = token 4 q + e)
                s16x4 Vf[NPV];
#pragma unroll
                for (int pl = 0; pl < NPV; ++pl)
                    Vf[pl] = lds4(&sl.Vt[pl][jl][4 * q]);
                // M_ak V
                f32x4 ym = {0.f, 0.f, 0.f, 0.f};
                {
                    const f32x4 mv = *reinterpret_cast<const f32x4 *>(&sl.M[0][m][4 * q]);
                    const float a4[4] = {mv[0], mv[1], mv[2], mv[3]};
                    s16x4 Mf[NP];
                    split4<NP>(a4, Mf);
                    mma16<NP, NPV>(ym, Mf, Vf);
                }
                // Z = T Y  (Y = A' S^ + M_ak V in accumulator layout: Y[4 q + e][col m])
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
                {
                    const f32x4 tv = *reinterpret_cast<const f32x4 *>(&sl.Tm[m][4 * q]);
                    const float t4[4] = {tv[0], tv[1], tv[2], tv[3]};
                    float y4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        y4[e] = (y2[0][e] + y2[1][e]) + ym[e];
                    s16x4 Tf[NP], Yf[NP];
                    split4<NP>(t4, Tf);
                    split4<NP>(y4, Yf);
                    mma16<NP, NP>(z, Tf, Yf);
                }
                // [Z ; V] as one B operand over 32 token slots: (q, e<4) is Z row 4q+e
                // (this lane's z[e]), (q, e>=4) is V row 4q+e-4.
                s16x8 ZV[NP];
                {
                    const float z4[4] = {z[0], z[1], z[2], z[3]};
                    s16x4 Zf[NP];
                    split4<NP>(z4, Zf);
#pragma unroll
                    for (int pl = 0; pl < NP; ++pl) {
                        const s16x4 vv = pl < NPV ? Vf[pl < NPV ? pl : 0] : s16x4{0, 0, 0, 0};
                        ZV[pl] = s16x8{Zf[pl][0], Zf[pl][1], Zf[pl][2], Zf[pl][3], vv[0], vv[1], vv[2], vv[3]};
                    }
                }
                // o = R' S^ + [M_rb | M_rk] [Z ; V]
                f32x4 o3 = {0.f, 0.f, 0.f, 0.f};
                {
                    const f32x4 mrb = *reinterpret_cast<const f32x4 *>(&sl.M[1][m][4 * q]);
                    const f32x4 mrk = *reinterpret_cast<const f32x4 *>(&sl.M[2][m][4 * q]);
                    const float a8[8] = {mrb[0], mrb[1], mrb[2], mrb[3], mrk[0], mrk[1], mrk[2], mrk[3]};
                    s16x8 Mf[NP];
                    split8<NP>(a8, Mf);
                    mma32<NP, NP>(o3, Mf, ZV);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tau = 4 * q + e;
                    if (t0 + tau < T)
                        store_elem(go, head0 + static_cast<size_t>(t0 + tau) * rowstride + jw + m,
                                   (o2[0][e] + o2[1][e]) + o3[e]);
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
                    f32x4 acc = {Sh[pt][0], Sh[pt][1], Sh[pt][2], Sh[pt][3]};
                    mma32<NP, NP>(acc, Uf, ZV);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        Sx[pt][e] = acc[e] * d15v[pt][e];
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
    // Wave 0 builds M_ab and inverts I - M_ab; waves 1..3 build the operands
    // (wave 1: A' and K'; wave 2: R'; wave 3: B', v and the decay factors) and
    // the matrices M_ak (1), M_rb (2), M_rk (3).
    const int pw = wv - NSW;
    // ---- input path
    // STAGED: producer pw in 1..3 owns two of the six input streams (w a | r k | b v)
    // and moves them, as 16-byte pieces of whole 128-byte rows, from HBM to the
    // staging ring: the loads of chunk c are issued in iteration c-5, written
    // to ring slot c%2 in iteration c-3 and read in iteration c-2.
    // Otherwise (fp32 inputs): per-lane loads straight into registers.
    const uint16_t *gs0 = nullptr, *gs1 = nullptr;
    int sidx0 = 0, sidx1 = 0;
    if (pw == 1) { gs0 = static_cast<const uint16_t *>(p.w); sidx0 = 0; gs1 = static_cast<const uint16_t *>(p.a); sidx1 = 1; }
    if (pw == 2) { gs0 = static_cast<const uint16_t *>(p.r); sidx0 = 2; gs1 = static_cast<const uint16_t *>(p.k); sidx1 = 3; }
    if (pw == 3) { gs0 = static_cast<const uint16_t *>(p.b); sidx0 = 4; gs1 = static_cast<const uint16_t *>(p.v); sidx1 = 5; }
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    struct Stage {
        u32x4 v[2][2];  // [stream][half]: rows 8*half + lane/8, bytes 16*(lane%8) .. +16
    };
    Stage sa, sb;
    auto stage_load = [&](Stage &S, int c) {
        if constexpr (STAGED) {
            if (pw == 0 || c >= nchunks)
                return;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int t = min(c * CH + 8 * h + (lane >> 3), T - 1);
                const size_t off = head0 + static_cast<size_t>(t) * rowstride + 8 * (lane & 7);
                S.v[0][h] = *reinterpret_cast<const u32x4 *>(gs0 + off);
                S.v[1][h] = *reinterpret_cast<const u32x4 *>(gs1 + off);
            }
        }
    };
    auto stage_store = [&](const Stage &S, int c) {
        if constexpr (STAGED) {
            if (pw == 0 || c >= nchunks)
                return;
            RawSlot &rs = sm.rr.raw[c & 1];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int tau = 8 * h + (lane >> 3);
                *reinterpret_cast<u32x4 *>(&rs.x[sidx0][tau][8 * (lane & 7)]) = S.v[0][h];
                *reinterpret_cast<u32x4 *>(&rs.x[sidx1][tau][8 * (lane & 7)]) = S.v[1][h];
            }
        }
    };
    // fp32 inputs: registers of one chunk (lane = key channel, or value column for v)
    const Tin *__restrict__ gw = static_cast<const Tin *>(p.w);
    const Tin *__restrict__ gx0 = static_cast<const Tin *>(pw == 1 ? p.a : pw == 2 ? p.r : p.b);
    const Tin *__restrict__ gx1 = static_cast<const Tin *>(pw == 1 ? p.k : p.v);
    struct Raw {
        Tin w[CH], x0[CH], x1[CH];
    };
    Raw ra, rb;
    auto reg_load = [&](Raw &R, int c) {
        if constexpr (!STAGED) {
            if (pw == 0 || c >= nchunks)
                return;
#pragma unroll
            for (int tau = 0; tau < CH; ++tau) {
                const int t = min(c * CH + tau, T - 1);
                const size_t row = head0 + static_cast<size_t>(t) * rowstride;
                R.w[tau] = gw[row + lane];
                R.x0[tau] = gx0[row + lane];
                R.x1[tau] = gx1[row + (pw == 3 ? j0 + (lane < NC ? lane : 0) : lane)];
            }
        }
    };

    // ---- operand stage: decay-scaled operands of chunk c into its slot
    auto operands = [&](const Raw &R, int c) {
        if (pw == 0 || c >= nchunks)
            return;
        SlotT &sl = sm.slot[c % 3];
        const int t0 = c * CH, i = lane;
        float w[CH], x0[CH], x1[CH];
        if constexpr (STAGED) {
            const RawSlot &rs = sm.rr.raw[c & 1];
            // this wave's streams: wave 1 (a, k), wave 2 (r, -), wave 3 (b, v)
            const int s0 = pw == 1 ? 1 : pw == 2 ? 2 : 4;
            const int s1 = pw == 1 ? 3 : 5;
            const int col1 = pw == 3 ? j0 + (lane < NC ? lane : 0) : lane;
            // Read every row (rows past the end hold valid, clamped data), then
            // mask with uniform bit masks, so the reads are not split by branches.
            uint32_t rw[CH], r0[CH], r1[CH];
#pragma unroll
            for (int tau = 0; tau < CH; ++tau) {
                rw[tau] = rs.x[0][tau][i];
                r0[tau] = rs.x[s0][tau][i];
                r1[tau] = rs.x[s1][tau][col1];
            }
#pragma unroll
            for (int tau = 0; tau < CH; ++tau) {
                const uint32_t keep = t0 + tau < T ? 0xffffu : 0u;          // uniform
                const uint32_t keep1 = pw != 2 ? keep : 0u;
                w[tau] = fmaxf(bf16_val(static_cast<uint16_t>((rw[tau] & keep) | (0x3f80u & ~keep))), W_MIN);
                x0[tau] = bf16_val(static_cast<uint16_t>(r0[tau] & keep));
                x1[tau] = bf16_val(static_cast<uint16_t>(r1[tau] & keep1));
            }
        } else {
#pragma unroll
            for (int tau = 0; tau < CH; ++tau) {
                const bool ok = t0 + tau < T;
                w[tau] = ok ? fmaxf(load_elem(R.w, tau), W_MIN) : 1.0f;
                x0[tau] = ok ? load_elem(R.x0, tau) : 0.0f;
                x1[tau] = (ok && pw != 2) ? load_elem(R.x1, tau) : 0.0f;
            }
        }
        float d[CH + 1], id[CH + 1];
        decay_factors(w, d, id);
        if (pw == 1 || pw == 2) {
            // A' (wave 1) or R' (wave 2): row-major, one bf16 per plane and row
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
        if (pw == 1 || pw == 3) {
            // K' (wave 1, from x1) or B' (wave 3, from x0): transposed rows of 16
            // bf16 per plane, and (bf16 inputs) the row-major copy as well
            uint16_t(*dstT)[kN][LDT] = pw == 1 ? sl.KpT : sl.BpT;
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
                    if constexpr (NP == 2)
                        (pw == 1 ? sl.bk.Kp : sl.bk.Bp)[pl][s][i] = pc[pl];
                }
            }
#pragma unroll
            for (int pl = 0; pl < NP; ++pl) {
                *reinterpret_cast<s16x8 *>(&dstT[pl][i][0]) = lo[pl];
                *reinterpret_cast<s16x8 *>(&dstT[pl][i][8]) = hi[pl];
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

    // ---- matrix stage: one 16x16 tile M = tril(X' Y'^T) of chunk c per wave
    // over the 64 key channels; wave 0 then inverts I - M_ab.
    auto matrices = [&](int c) {
        if (c < 0 || c >= nchunks)
            return;
        SlotT &sl = sm.slot[c % 3];
        const uint16_t(*X)[CH][LDA] = (pw == 0 || pw == 1) ? sl.Ap : sl.Rp;
        const bool yb = pw == 0 || pw == 2;  // Y' = B' (else K')
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            s16x8 Af[NP], Bf[NP];
#pragma unroll
            for (int pl = 0; pl < NP; ++pl) {
                Af[pl] = *reinterpret_cast<const s16x8 *>(&X[pl][m][32 * s + 8 * q]);
                if constexpr (NP == 2) {
                    Bf[pl] = *reinterpret_cast<const s16x8 *>(&(yb ? sl.bk.Bp : sl.bk.Kp)[pl][m][32 * s + 8 * q]);
                } else {
                    const uint16_t(*Y)[kN][LDT] = yb ? sl.BpT : sl.KpT;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        Bf[pl][e] = static_cast<short>(Y[pl][32 * s + 8 * q + e][m]);
                }
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
            // (I - M_ab)^{-1} in 8x8 blocks: T11 = (I - M11)^{-1}, T22 = (I - M22)^{-1}
            // by forward substitution (lanes 0..7 and 8..15, one column each), then
            // T21 = T22 (M21 T11) with one entry per lane.  This wave's own LDS
            // writes are complete before it reads them back.
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
            __builtin_amdgcn_wave_barrier();
            if (lane < CH) {
                const int off = lane < 8 ? 0 : 8, col = lane - off;
                float x[8];
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    x[t] = t == col ? 1.0f : 0.0f;
#pragma unroll
                for (int s2 = 0; s2 < 8; ++s2)
#pragma unroll
                    for (int t = s2 + 1; t < 8; ++t)
                        x[t] = fmaf(sm.Mab[off + t][off + s2], x[s2], x[t]);
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    sl.Tm[off + t][off + col] = x[t];
                    if (off == 0)
                        sl.Tm[t][8 + col] = 0.0f;  // upper-right block
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
            const int r8 = lane >> 3, c8 = lane & 7;
            float xv = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k)
                xv = fmaf(sm.Mab[8 + r8][k], sl.Tm[k][c8], xv);
            sm.Xs[r8][c8] = xv;
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
            float tv = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k)
                tv = fmaf(sl.Tm[8 + r8][8 + k], sm.Xs[k][c8], tv);
            sl.Tm[8 + r8][c8] = tv;
        }
    };

    // Pipeline: iteration i consumes chunk i (consumer waves), builds the
    // matrices of chunk i+1 and the operands of chunk i+2 (reading ring slot
    // (i+2)%2), writes the staged rows of chunk i+3 into the other ring slot
    // and issues the loads of chunk i+5 (fp32 inputs: loads of chunk i+4).
    // Register sets alternate between even and odd iterations.
    if constexpr (STAGED) {
        stage_load(sa, 0);
        stage_load(sb, 1);
        stage_store(sa, 0);
        stage_load(sa, 2);
        __syncthreads();  // ring slot 0 holds chunk 0 (matched by the consumers)
    } else {
        reg_load(ra, 0);
        reg_load(rb, 1);
    }
    for (int i = -2; i < nchunks; i += 2) {
        matrices(i + 1);
        operands(ra, i + 2);
        if constexpr (STAGED) {
            stage_store(sb, i + 3);
            stage_load(sb, i + 5);
        } else {
            reg_load(ra, i + 4);
        }
        __syncthreads();
        if (i + 1 < nchunks) {
            matrices(i + 2);
            operands(rb, i + 3);
            if constexpr (STAGED) {
                stage_store(sa, i + 4);
                stage_load(sa, i + 6);
            } else {
                reg_load(rb, i + 5);
            }
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
