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
// pipeline with one barrier per chunk:
//  * consumer waves (NC/16 of them) each keep a 64x16 slice of the fp32 state
//    in registers, in the accumulator layout of a 16x16 matrix-core tile, for
//    the whole sequence, and run only the state-dependent products of chunk c;
//  * eight producer waves work ahead: four build the intra-chunk matrices of
//    chunk c+1 (M_ab with the triangular inverse T, M_ak, M_rb, M_rk), four
//    build the decay-scaled operands of chunk c+2 (A', R', B', K' and v), and
//    three of them also move the raw input rows of chunk c+3 into a staging
//    ring in LDS, from 16-byte loads issued two iterations earlier.
// Chunk data lives in a ring of three LDS slots.  All products run on
// v_mfma_f32_16x16x{32,16}_bf16 with fp32 accumulation; fp32 operands are
// split into bf16 pieces (x = x0 + x1 [+ x2], stored pre-split in LDS by the
// wave that makes them) and the piece products summed, which keeps
// fp32-level accuracy on the matrix cores.  bf16 inputs are exact in one piece.
#include <type_traits>

#include "wkv7_device.h"
#include "wkv7_launch.h"

namespace wkv7 {
namespace {

constexpr int CH = 16;             // chunk length
constexpr int REF = 7;             // decays are measured relative to the state after this position
constexpr float W_MIN = 0x1p-15f;  // lower bound applied to decay multipliers in this kernel
constexpr int NPROD = 8;           // producer waves
constexpr int LDA = kN + 8;        // row pitch (bf16) of [16][64] operand planes
constexpr int LDT = CH + 8;        // row pitch (bf16) of [64][16] transposed planes and [16][16] planes
constexpr int LDU = 32 + 8;        // row pitch (bf16) of interleaved [rows][32] planes
constexpr int LDM = CH + 4;        // row pitch (fp32) of [16][16] scratch matrices (16-byte rows)
constexpr uint32_t W_MIN_BITS = 0x38000000u;  // 2^-15 as fp32 bits

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint16_t bf16_bits(float x)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));  // round to nearest even
}
__device__ __forceinline__ float bf16_val(uint32_t h) { return __uint_as_float(h << 16); }

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
__device__ __forceinline__ s16x8 lds8(const uint16_t *p) { return *reinterpret_cast<const s16x8 *>(p); }

// Column of key channel i in the row-major operand planes.  A matrix-core
// lane (q, .) of k-step s consumes key rows 16 (2 s + e/4) + 4 q + e%4,
// e = 0..7 (the rows it holds of the state tile); storing those eight keys
// next to each other makes its fragment one 16-byte read.  Products over
// the key index are unaffected as long as both operands use the same order.
__device__ __forceinline__ int key_slot(int i)
{
    return 32 * (i >> 5) + 8 * ((i >> 2) & 3) + 4 * ((i >> 4) & 1) + (i & 3);
}
__device__ __forceinline__ s16x8 cat(const s16x4 a, const s16x4 b)
{
    return s16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <int NP, bool ON>
struct RowMajorBK {
    uint16_t Bp[NP][CH][LDA];
    uint16_t Kp[NP][CH][LDA];
};
template <int NP>
struct RowMajorBK<NP, false> {};

// One chunk's data in LDS.  Planes hold bf16 bit patterns.  With bf16
// inputs (NP == 2) B' and K' are also kept row-major, so the matrix stage
// reads its operands with 16-byte loads; the fp32-input build (NP == 3) has
// no room for them and gathers from the transposed copies instead.
template <int NP, int NPV, int NC>
struct alignas(16) Slot {
    uint16_t Ap[NP][CH][LDA];    // A'[tau][key_slot(i)]
    uint16_t Rp[NP][CH][LDA];    // R'[tau][key_slot(i)]
    RowMajorBK<NP, NP == 2> bk;  // B'[s][key_slot(i)], K'[s][key_slot(i)]  (NP == 2 only)
    uint16_t Ut[NP][kN][LDU];    // [i][8 g + e]: B'[4 g + e][i] for e < 4, K'[4 g + e - 4][i] for e >= 4
    uint16_t Vt[NPV][NC][LDT];   // v[s][j] stored as [j][s]
    uint16_t Mak[NP][CH][LDT];   // M_ak (masked)
    uint16_t Mrr[NP][CH][LDU];   // [tau][8 g + e]: M_rb[tau][4 g + e] for e < 4, M_rk[tau][4 g + e - 4] for e >= 4
    uint16_t Tp[NP][CH][LDT];    // T = (I - M_ab)^{-1}
    alignas(16) float p7[kN];    // P_7 per key channel
    alignas(16) float f[kN];     // d_15 of this chunk times P_7 of the next one (d_15 alone for the last)
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
    float Mab[CH][LDM];          // scratch of the wave that builds T
    float Tf[CH][LDM];           // T in fp32 while it is built
    float Xs[8][LDM];
};

// Decay factors of one key channel over a chunk: d[tau+1] = P_tau / P_7 and
// id[tau+1] = P_7 / P_tau for tau = -1..15 (P_-1 = 1), with two reciprocals.
__device__ __forceinline__ void decay_factors(const float (&w)[CH], float (&d)[CH + 1], float (&id)[CH + 1])
{
    id[REF + 1] = 1.0f;  // id for tau <= REF: product of w over tau+1 .. REF
#pragma unroll
    for (int tau = REF - 1; tau >= -1; --tau)
        id[tau + 1] = id[tau + 2] * w[tau + 1];
    d[REF + 1] = 1.0f;   // d for tau >= REF: product of w over REF+1 .. tau
#pragma unroll
    for (int tau = REF + 1; tau < CH; ++tau)
        d[tau + 1] = d[tau] * w[tau];
    const float inv_p7 = __builtin_amdgcn_rcpf(id[0]);  // d for tau < REF: (1/P_7) prod_{0..tau} w
    float pre = inv_p7;
    d[0] = inv_p7;
#pragma unroll
    for (int tau = 0; tau < REF; ++tau) {
        pre *= w[tau];
        d[tau + 1] = pre;
    }
    const float inv_d15 = __builtin_amdgcn_rcpf(d[CH]);  // id for tau > REF: (1/d_15) prod_{tau+1..15} w
    float post = inv_d15;
    id[CH] = inv_d15;
#pragma unroll
    for (int tau = CH - 2; tau >= REF + 1; --tau) {
        post *= w[tau + 1];
        id[tau + 1] = post;
    }
}

// Wait for this wave's outstanding LDS accesses (its writes become visible to
// its own later reads from other lanes).
__device__ __forceinline__ void lds_fence_wave()
{
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
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
    constexpr bool STAGED = !F32IN;       // bf16 rows go through the LDS staging ring
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
        // Sx[pt][e] holds row 16 pt + 4 q + e, column jw + m of the state: the input
        // state before the first chunk, S^ of the coming chunk between chunks, and
        // the output state after the last one.
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
                if (i == 0) {
                    // S^ = diag(P_7) S_in for the first chunk; afterwards every chunk
                    // leaves S^ of the next one (its row factor folds both scalings).
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt) {
                        const f32x4 p7v = *reinterpret_cast<const f32x4 *>(&sl.p7[16 * pt + 4 * q]);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            Sx[pt][e] *= p7v[e];
                    }
                }
                // S^ as matrix-core B operands over the key index: key slot (q, e) of
                // k-step s is key row 16 (2 s + e/4) + 4 q + e%4, which this lane holds
                // in Sx[2 s + e/4][e % 4].
                s16x8 Bs[2][NP];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    float v8[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v8[e] = Sx[2 * s + e / 4][e & 3];
                    split8<NP>(v8, Bs[s]);
                }
                // A'-rows and R'-rows as A operands with the same key slots (stored
                // contiguously, see key_slot); one accumulator per k-step.
                f32x4 y2[2], o2[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    s16x8 Af[NP], Rf[NP];
#pragma unroll
                    for (int pl = 0; pl < NP; ++pl) {
                        Af[pl] = lds8(&sl.Ap[pl][m][32 * s + 8 * q]);
                        Rf[pl] = lds8(&sl.Rp[pl][m][32 * s + 8 * q]);
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
                    s16x4 Mf[NP];
#pragma unroll
                    for (int pl = 0; pl < NP; ++pl)
                        Mf[pl] = lds4(&sl.Mak[pl][m][4 * q]);
                    mma16<NP, NPV>(ym, Mf, Vf);
                }
                // Z = T Y  (Y = A' S^ + M_ak V in accumulator layout: Y[4 q + e][col m])
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
                {
                    float y4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        y4[e] = (y2[0][e] + y2[1][e]) + ym[e];
                    s16x4 Tf[NP], Yf[NP];
#pragma unroll
                    for (int pl = 0; pl < NP; ++pl)
                        Tf[pl] = lds4(&sl.Tp[pl][m][4 * q]);
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
                    for (int pl = 0; pl < NP; ++pl)
                        ZV[pl] = cat(Zf[pl], pl < NPV ? Vf[pl < NPV ? pl : 0] : s16x4{0, 0, 0, 0});
                }
                // o = R' S^ + [M_rb | M_rk] [Z ; V]
                f32x4 o3 = {0.f, 0.f, 0.f, 0.f};
                {
                    s16x8 Mf[NP];
#pragma unroll
                    for (int pl = 0; pl < NP; ++pl)
                        Mf[pl] = lds8(&sl.Mrr[pl][m][8 * q]);
                    mma32<NP, NP>(o3, Mf, ZV);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tau = 4 * q + e;
                    if (t0 + tau < T)
                        store_elem(go, head0 + static_cast<size_t>(t0 + tau) * rowstride + jw + m,
                                   (o2[0][e] + o2[1][e]) + o3[e]);
                }
                // S^ <- diag(f) (S^ + [B'^T | K'^T] [Z ; V]), one 16-row tile at a time
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    s16x8 Uf[NP];
#pragma unroll
                    for (int pl = 0; pl < NP; ++pl)
                        Uf[pl] = lds8(&sl.Ut[pl][16 * pt + m][8 * q]);
                    f32x4 acc = {Sx[pt][0], Sx[pt][1], Sx[pt][2], Sx[pt][3]};
                    mma32<NP, NP>(acc, Uf, ZV);
                    const f32x4 fv = *reinterpret_cast<const f32x4 *>(&sl.f[16 * pt + 4 * q]);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        Sx[pt][e] = acc[e] * fv[e];
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
    //   pw 0: M_ab and T                pw 4: A'  (from w, a)
    //   pw 1: M_ak, stages w a          pw 5: R'  (from w, r)
    //   pw 2: M_rb, stages r k          pw 6: B'  (from w, b), P_7 and d_15
    //   pw 3: M_rk, stages b v          pw 7: K'  (from w, k) and v
    const int pw = wv - NSW;
    const bool stager = pw >= 1 && pw <= 3;
    const bool maker = pw >= 4;

    // ---- input path
    // STAGED: waves 1..3 each own two of the six input streams and move them,
    // as 16-byte pieces of whole 128-byte rows, from HBM to the staging ring:
    // the loads of chunk c are issued in iteration c-5, written to ring slot
    // c%2 in iteration c-3 and read by the operand makers in iteration c-2.
    // Otherwise (fp32 inputs) the operand makers load straight into registers.
    const uint16_t *gs0 = static_cast<const uint16_t *>(pw == 1 ? p.w : pw == 2 ? p.r : p.b);
    const uint16_t *gs1 = static_cast<const uint16_t *>(pw == 1 ? p.a : pw == 2 ? p.k : p.v);
    const int sidx0 = pw == 1 ? 0 : pw == 2 ? 2 : 4;
    const int sidx1 = sidx0 + 1;
    struct Stage {
        u32x4 v[2][2];  // [stream][half]: row 8*half + lane/8, elements 8*(lane%8) .. +8
    };
    Stage sa, sb;
    auto stage_load = [&](Stage &S, int c) {
        if constexpr (STAGED) {
            if (!stager || c >= nchunks)
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
            if (!stager || c >= nchunks)
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
    // operand makers: the stream each one scales, and (wave 7) v
    const int xs = pw == 4 ? 1 : pw == 5 ? 2 : pw == 6 ? 4 : 3;   // a, r, b, k
    const int vcol = j0 + (lane < NC ? lane : 0);
    const Tin *__restrict__ gw = static_cast<const Tin *>(p.w);
    const Tin *__restrict__ gx =
        static_cast<const Tin *>(pw == 4 ? p.a : pw == 5 ? p.r : pw == 6 ? p.b : p.k);
    const Tin *__restrict__ gv = static_cast<const Tin *>(p.v);
    struct Raw {
        Tin w[CH], x[CH], v[CH];
    };
    Raw ra, rb;
    auto reg_load = [&](Raw &R, int c) {
        if constexpr (!STAGED) {
            if (!maker || c >= nchunks)
                return;
#pragma unroll
            for (int tau = 0; tau < CH; ++tau) {
                const int t = min(c * CH + tau, T - 1);
                const size_t row = head0 + static_cast<size_t>(t) * rowstride;
                R.w[tau] = gw[row + lane];
                R.x[tau] = gx[row + lane];
                if (pw == 7)
                    R.v[tau] = gv[row + vcol];
            }
        }
    };

    // ---- operand stage (waves 4..7): decay-scaled operands of chunk c into its slot
    const int ks = key_slot(lane);
    float prev_d15 = 0.0f;  // wave 6: d_15 of the chunk before (its row factor is finished here)
    auto operands = [&](const Raw &R, int c) {
        if (!maker || c >= nchunks)
            return;
        SlotT &sl = sm.slot[c % 3];
        const int t0 = c * CH, i = lane;
        float w[CH], x[CH], v[CH];
        if constexpr (STAGED) {
            const RawSlot &rs = sm.rr.raw[c & 1];
            // Read every row (rows past the end hold valid, clamped data) before
            // any use, so the reads are not split by branches.
            uint32_t rw[CH], rx[CH], rv[CH];
#pragma unroll
            for (int tau = 0; tau < CH; ++tau) {
                rw[tau] = rs.x[0][tau][i];
                rx[tau] = rs.x[xs][tau][i];
                rv[tau] = rs.x[5][tau][vcol];
            }
            if (t0 + CH <= T) {
#pragma unroll
                for (int tau = 0; tau < CH; ++tau) {
                    w[tau] = __uint_as_float(max(rw[tau] << 16, W_MIN_BITS));
                    x[tau] = bf16_val(rx[tau]);
                    v[tau] = bf16_val(rv[tau]);
                }
            } else {
                // last, partial chunk: positions past the end act as w = 1 and zero vectors
#pragma unroll
                for (int tau = 0; tau < CH; ++tau) {
                    const uint32_t keep = t0 + tau < T ? 0xffffu : 0u;  // uniform
                    w[tau] = __uint_as_float(max(((rw[tau] & keep) | (0x3f80u & ~keep)) << 16, W_MIN_BITS));
                    x[tau] = bf16_val(rx[tau] & keep);
                    v[tau] = bf16_val(rv[tau] & keep);
                }
            }
        } else {
#pragma unroll
            for (int tau = 0; tau < CH; ++tau) {
                const bool ok = t0 + tau < T;
                w[tau] = ok ? fmaxf(load_elem(R.w, tau), W_MIN) : 1.0f;
                x[tau] = ok ? load_elem(R.x, tau) : 0.0f;
                v[tau] = (ok && pw == 7) ? load_elem(R.v, tau) : 0.0f;
            }
        }
        float d[CH + 1], id[CH + 1];
        decay_factors(w, d, id);
        if (pw == 4 || pw == 5) {
            // A' (wave 4) or R' (wave 5): row-major, key columns in key_slot order
            uint16_t(*dst)[CH][LDA] = pw == 4 ? sl.Ap : sl.Rp;
#pragma unroll
            for (int tau = 0; tau < CH; ++tau) {
                uint16_t pc[NP];
                split<NP>(x[tau] * (pw == 4 ? d[tau] : d[tau + 1]), pc);
#pragma unroll
                for (int pl = 0; pl < NP; ++pl)
                    dst[pl][tau][ks] = pc[pl];
            }
            return;
        }
        // B' (wave 6) or K' (wave 7): the interleaved transposed planes (four runs
        // of four tokens per key row) and, with bf16 inputs, the row-major copy
        const int half = pw == 6 ? 0 : 4;
        s16x4 g4[NP][4];
#pragma unroll
        for (int s2 = 0; s2 < CH; ++s2) {
            uint16_t pc[NP];
            split<NP>(x[s2] * id[s2 + 1], pc);
#pragma unroll
            for (int pl = 0; pl < NP; ++pl) {
                g4[pl][s2 >> 2][s2 & 3] = static_cast<short>(pc[pl]);
                if constexpr (NP == 2)
                    (pw == 6 ? sl.bk.Bp : sl.bk.Kp)[pl][s2][ks] = pc[pl];
            }
        }
#pragma unroll
        for (int pl = 0; pl < NP; ++pl)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<s16x4 *>(&sl.Ut[pl][i][8 * g + half]) = g4[pl][g];
        if (pw == 6) {
            // P_7 of this chunk; row factor d_15 * P_7(next) of the previous chunk,
            // and of this one when it is the last
            sl.p7[i] = id[0];
            if (c > 0)
                sm.slot[(c + 2) % 3].f[i] = prev_d15 * id[0];
            prev_d15 = d[CH];
            if (c == nchunks - 1)
                sl.f[i] = d[CH];
        } else if (lane < NC) {
            // v column j0 + lane over the chunk, transposed
#pragma unroll
            for (int pl = 0; pl < NPV; ++pl) {
                s16x8 vlo, vhi;
#pragma unroll
                for (int s2 = 0; s2 < CH; ++s2) {
                    uint16_t pc[NPV];
                    split<NPV>(v[s2], pc);
                    if (s2 < 8)
                        vlo[s2] = static_cast<short>(pc[pl]);
                    else
                        vhi[s2 - 8] = static_cast<short>(pc[pl]);
                }
                *reinterpret_cast<s16x8 *>(&sl.Vt[pl][lane][0]) = vlo;
                *reinterpret_cast<s16x8 *>(&sl.Vt[pl][lane][8]) = vhi;
            }
        }
    };

    // ---- matrix stage (waves 0..3): one 16x16 tile M = tril(X' Y'^T) of chunk c
    // per wave over the 64 key channels; wave 0 then inverts I - M_ab.
    auto matrices = [&](int c) {
        if (maker || c < 0 || c >= nchunks)
            return;
        SlotT &sl = sm.slot[c % 3];
        const uint16_t(*X)[CH][LDA] = pw <= 1 ? sl.Ap : sl.Rp;
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
                    // key slot (q, e) of k-step s is key 16 (2 s + e/4) + 4 q + e%4
                    const int col = 8 * (m >> 2) + (yb ? 0 : 4) + (m & 3);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        Bf[pl][e] = static_cast<short>(sl.Ut[pl][16 * (2 * s + e / 4) + 4 * q + (e & 3)][col]);
                }
            }
            mma32<NP, NP>(acc, Af, Bf);
        }
        const bool strict = pw < 2;  // a rows exclude the diagonal, r rows include it
        if (pw > 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tau = 4 * q + e;
                uint16_t pc[NP];
                split<NP>((m < tau || (!strict && m == tau)) ? acc[e] : 0.0f, pc);
#pragma unroll
                for (int pl = 0; pl < NP; ++pl) {
                    if (pw == 1)
                        sl.Mak[pl][tau][m] = pc[pl];
                    else
                        sl.Mrr[pl][tau][8 * (m >> 2) + (pw == 2 ? 0 : 4) + (m & 3)] = pc[pl];
                }
            }
            return;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tau = 4 * q + e;
            sm.Mab[tau][m] = m < tau ? acc[e] : 0.0f;
        }
        // (I - M_ab)^{-1} in 8x8 blocks: T11 = (I - M11)^{-1} and T22 = (I - M22)^{-1}
        // by forward substitution (lanes 0..7 and 8..15, one column each), then
        // T21 = T22 (M21 T11) with one entry per lane; finally split into planes.
        lds_fence_wave();
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
                sm.Tf[off + t][off + col] = x[t];
                if (off == 0)
                    sm.Tf[t][8 + col] = 0.0f;  // upper-right block
            }
        }
        lds_fence_wave();
        const int r8 = lane >> 3, c8 = lane & 7;
        float xv = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            xv = fmaf(sm.Mab[8 + r8][k], sm.Tf[k][c8], xv);
        sm.Xs[r8][c8] = xv;
        lds_fence_wave();
        float tv = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            tv = fmaf(sm.Tf[8 + r8][8 + k], sm.Xs[k][c8], tv);
        sm.Tf[8 + r8][c8] = tv;
        lds_fence_wave();
        // planes: lane -> row lane/4, columns 4 (lane%4) .. +4
        const int tr = lane >> 2, tc = 4 * (lane & 3);
        const f32x4 tq = *reinterpret_cast<const f32x4 *>(&sm.Tf[tr][tc]);
        const float t4[4] = {tq[0], tq[1], tq[2], tq[3]};
        s16x4 tp[NP];
        split4<NP>(t4, tp);
#pragma unroll
        for (int pl = 0; pl < NP; ++pl)
            *reinterpret_cast<s16x4 *>(&sl.Tp[pl][tr][tc]) = tp[pl];
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
