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
// With every decay multiplier of a chunk at least 2^-15, every factor stays
// within 2^(+-120).  A chunk with a smaller decay anywhere (RWKV-7's decays,
// >= 0.545, never come near) is evaluated exactly instead: its decay table is
// all ones (so S^ enters it unscaled and leaves it scaled for the next chunk)
// and its consumers run the recurrence itself over its 16 tokens, reading the
// inputs from global memory.
//
// MAPPING (gfx950).  One workgroup per (batch, head, block of NC value
// columns); value columns evolve independently, so a head splits into
// J = 64/NC blocks with no communication.  The workgroup is a software
// pipeline with one barrier per chunk; in iteration i (fp32 inputs; the bf16
// build runs one stage deeper, see the pipeline below)
//  * consumer waves (NC/16 of them) each keep a 64x16 slice of the fp32 state
//    in registers, in the accumulator layout of a 16x16 matrix-core tile, for
//    the whole sequence, and run only the state-dependent products of chunk i;
//  * the matrix waves build M_ab, M_ak, M_rb and M_rk of chunk i+1; the
//    inverse wave inverts I - M_ab by repeated squaring on the matrix cores,
//    T = (I + M)(I + M^2)(I + M^4)(I + M^8) (M is strictly lower triangular,
//    so M^16 = 0), carrying each matrix and its transpose in registers (the
//    first transpose goes through LDS);
//  * four scale waves form the decay-scaled operands A', R', B', K' (and the
//    v rows) of chunk i+2, elementwise, from a table of decay factors;
//  * a decay wave turns the w rows of chunk i+3 into that table.
// With bf16 inputs two inverse waves and two decay waves take the even and the
// odd chunks, each spreading one chunk's work over two iterations.
// The decay and scale waves load their own input rows from HBM, in their own
// lane layouts, two or more iterations ahead; rows past the end of the sequence
// count as w = 1 and zero vectors.
// Every operand that a product needs transposed is read with the gfx950 LDS
// transpose load (ds_read_b64_tr_b16) from row-major storage, so no stage
// writes a second, transposed copy.  All products run on
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
// a decay of magnitude below this sends its chunk to the exact recurrent path
constexpr float W_EXACT = 0x1p-15f;
// producer waves: ten with bf16 inputs (two inverse and two decay waves), eight with fp32 inputs
template <typename Tin>
constexpr int nprod() { return std::is_same<Tin, float>::value ? 8 : 10; }
// LDS layouts are chosen so that every access pattern below runs free of
// bank conflicts on gfx950 (64 banks of 4 bytes): 160-byte rows for the
// [16][64] planes, and XOR-swizzled, unpadded [16][16] tiles and decay rows.
constexpr int LDA = kN + 16;       // row pitch (bf16) of [16][64] planes
constexpr int NDROW = 2 * CH + 1;  // decay table rows: d_0 .. d_16, then id_1 .. id_16

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values to a packed pair of bf16 (round to nearest even), element 0 low.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Split 2 NW fp32 values into NP planes of packed bf16 pairs: x = x0 + x1 [+ x2]
// (to ~2^(-8 NP) relative); each piece is the rounded remainder of the ones before.
template <int NP, int NW>
__device__ __forceinline__ void split_pk(const float (&v)[2 * NW], uint32_t (&o)[NP][NW])
{
    float r[2 * NW];
#pragma unroll
    for (int e = 0; e < 2 * NW; ++e)
        r[e] = v[e];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
#pragma unroll
        for (int w = 0; w < NW; ++w)
            o[p][w] = pk_bf16(r[2 * w], r[2 * w + 1]);
        if (p + 1 < NP) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                r[2 * w] -= bf16_lo(o[p][w]);
                r[2 * w + 1] -= bf16_hi(o[p][w]);
            }
        }
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
    uint32_t o[NP][4];
    split_pk<NP, 4>(v, o);
#pragma unroll
    for (int p = 0; p < NP; ++p)
        out[p] = __builtin_bit_cast(s16x8, u32x4{o[p][0], o[p][1], o[p][2], o[p][3]});
}
template <int NP>
__device__ __forceinline__ void split4(const f32x4 v, s16x4 (&out)[NP])
{
    const float a[4] = {v[0], v[1], v[2], v[3]};
    uint32_t o[NP][2];
    split_pk<NP, 2>(a, o);
#pragma unroll
    for (int p = 0; p < NP; ++p)
        out[p] = __builtin_bit_cast(s16x4, u32x2{o[p][0], o[p][1]});
}

__device__ __forceinline__ s16x8 lds8(const uint16_t *p) { return *reinterpret_cast<const s16x8 *>(p); }

// Four consecutive outputs to global memory (fp32, or bf16 rounded to nearest even).
__device__ __forceinline__ void store4(float *p, const f32x4 x) { *reinterpret_cast<f32x4 *>(p) = x; }
__device__ __forceinline__ void store4(uint16_t *p, const f32x4 x)
{
    const uint32_t lo = f32_to_bf16_bits(x[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(x[1])) << 16);
    const uint32_t hi = f32_to_bf16_bits(x[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(x[3])) << 16);
    *reinterpret_cast<u32x2 *>(p) = u32x2{lo, hi};
}

// Four consecutive input elements from global memory, widened to fp32.
__device__ __forceinline__ f32x4 load4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ f32x4 load4(const uint16_t *p)
{
    const u32x2 u = *reinterpret_cast<const u32x2 *>(p);
    return f32x4{bf16_lo(u[0]), bf16_hi(u[0]), bf16_lo(u[1]), bf16_hi(u[1])};
}

// LDS transpose load of a 16x16 bf16 tile stored row-major as X[k][n]: lane
// 16 q + i passes the address of X[4 q + i/4][4 (i%4)] (four consecutive n),
// and lane (n = l%16, q = l/16) receives X[4 q + e][n], e = 0..3 -- the
// fragment a 16x16x16 matrix-core operand takes over k.  The four n-groups of
// a row may sit anywhere: each lane names its own.
__device__ __forceinline__ s16x4 tr4(const uint16_t *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(p));
}
__device__ __forceinline__ s16x8 cat(const s16x4 a, const s16x4 b)
{
    return s16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Column of key channel i in the row-major operand planes.  A matrix-core
// lane (q, .) of k-step s consumes key rows 16 (2 s + e/4) + 4 q + e%4,
// e = 0..7 (the rows it holds of the state tile); storing those eight keys
// next to each other makes its fragment one 16-byte read.  Products over
// the key index are unaffected as long as both operands use the same order.
__device__ __forceinline__ int key_slot(int i)
{
    return 32 * (i >> 5) + 8 * ((i >> 2) & 3) + 4 * ((i >> 4) & 1) + (i & 3);
}
// Column of key channel i in row r of the decay table: key order, with the
// two 16-key halves of each 32-key group exchanged on odd rows.
__device__ __forceinline__ int dcol(int r, int i) { return i ^ (16 * (r & 1)); }
// Place of the four elements [row][4 c .. 4 c + 3] of a 16x16 matrix tile:
// the 8-byte unit c moves to c ^ (row / 4 % 4).
__device__ __forceinline__ int mcol(int row, int c) { return 4 * (c ^ ((row >> 2) & 3)); }

// One chunk's operands and matrices in LDS (bf16 bit patterns; NP planes).
// The 16x16 matrices are stored transposed, [s][tau], as their producers hold
// them, at mcol(); consumers read them back with transpose loads.
// Planes are selected by index (never by choosing between pointers), the
// operands as X[OP_A], X[OP_R], X[OP_B], X[OP_K] and the matrices as
// Mt[MT_T], Mt[MT_AK], Mt[MT_RB], Mt[MT_RK].
enum { OP_A = 0, OP_R = 1, OP_B = 2, OP_K = 3 };
enum { MT_T = 0, MT_AK = 1, MT_RB = 2, MT_RK = 3 };
template <int NP, int NPV>
struct alignas(16) Slot {
    uint16_t X[4][NP][CH][LDA];   // A'[tau], R'[tau], B'[s], K'[s] over key_slot(i)
    uint16_t Vr[NPV][CH][LDA];    // v[s][j], all 64 value columns
    uint16_t Mt[4][NP][CH][CH];   // T, M_ak, M_rb, M_rk: element [tau][s] stored at [s][tau]
    alignas(16) float f[kN];      // d_15 of this chunk times P_7 of the next one (d_15 alone for the last)
};

// Decay factors of one chunk per key channel, rows d_0 .. d_16 and id_1 .. id_16
// (d_{tau+1} = P_tau / P_7, id_{tau+1} = P_7 / P_tau), key i of row r at dcol(r, i).
struct alignas(16) DSlot {
    float v[NDROW][kN];
};

constexpr int MTP = 20;  // row pitch (floats) of the fp32 transpose tiles of M_ab
// The tail variant's o of the last two chunks, fp32, [token][column] with a row pitch
// of OTP floats (the consumers' writes of four token rows then hit different banks).
constexpr int OTP = kN + 4;
template <int NOT>
struct OTiles {
    alignas(16) float t[NOT][CH][OTP];
};
template <>
struct OTiles<0> {};
// The checkpoint variant's d_15 of each chunk in the operand ring (slot c % NS).
template <int NG>
struct GRing {
    alignas(16) float g[NG][kN];
};
template <>
struct GRing<0> {};

template <typename Tin, int NP, int NPV, int NS, int NT, int NOT, int NG>
struct Smem {
    Slot<NP, NPV> slot[NS];
    alignas(16) Tin wbuf[CH][kN];  // w rows of one chunk, transposed through here by the decay wave
    DSlot dt[2];
    alignas(16) float p7[kN];  // P_7 of the first chunk
    alignas(16) float d15[2][kN];  // d_15 of the last two chunks whose table was written
    alignas(16) float mt[NT][CH][MTP];  // M_ab of one chunk per inverse wave, row-major
    int exact[8];  // chunk c % 8 takes the exact path (its decay table is all ones)
    OTiles<NOT> ot;
    GRing<NG> gr;
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

// MODE_TAIL (bf16 inputs, J = 1): the time-mix tail is fused.  The consumers leave o in
// LDS, and NTAIL more waves turn each chunk's rows into x (written through p.o, of
// type Tout) one iteration later.
// MODE_CKPT: the consumers also write the state entering every chunk to p.state_pos
// as [B, ceil(T / 16), H, N, N] (chunk 0: the input state), the checkpoints from
// which a backward pass rebuilds each chunk's states.
enum { MODE_PLAIN = 0, MODE_TAIL = 1, MODE_CKPT = 2 };
constexpr int NTAIL = 2;
template <int MODE>
constexpr int nextra() { return MODE == MODE_TAIL ? NTAIL : 0; }
template <typename Tin, typename Tout, int J, bool HAS_STATE_IN, int MODE>
__global__ __launch_bounds__((kN / J / 16 + nprod<Tin>() + nextra<MODE>()) * 64) void wkv7_chunk_kernel(
    SeqArgs p, int per_xcd, int nblocks)
{
    constexpr bool TAIL = MODE == MODE_TAIL, CKPT = MODE == MODE_CKPT;
    constexpr int NC = kN / J;            // value columns of this workgroup
    constexpr int NSW = NC / 16;          // consumer waves (16 state columns each)
    constexpr bool F32IN = std::is_same<Tin, float>::value;
    constexpr int NP = F32IN ? 3 : 2;     // bf16 pieces of derived fp32 operands
    constexpr int NPV = F32IN ? 3 : 1;    // pieces of v (one is exact for bf16 inputs)
    // bf16 inputs: a four-slot ring, with the decay-table and inverse waves
    // each working on two chunks at once (see the pipeline below); fp32 inputs
    // (three bf16 pieces, larger slots) keep a three-slot ring.
    constexpr bool DEEP = !F32IN;
    constexpr int NS = DEEP ? 4 : 3;
    using SlotT = Slot<NP, NPV>;
    static_assert(!TAIL || (J == 1 && !F32IN), "the fused tail runs with bf16 inputs and whole heads");
    __shared__ Smem<Tin, NP, NPV, NS, DEEP ? 2 : 1, TAIL ? 2 : 0, CKPT ? NS : 0> sm;

    // Workgroup -> (batch*head, column block).  Workgroups are dealt to the
    // XCDs round-robin; the J column blocks of one head stay on one XCD so the
    // key-side inputs they share are fetched into one L2.
    const int xcd = blockIdx.x & 7, slot_id = blockIdx.x >> 3;
    const int lid = xcd * per_xcd + slot_id;
    if (lid >= nblocks)
        return;
    const int bh = lid / J, jb = lid - bh * J;
    const int H = p.H, T = p.T;  // T: the row stride of the [B, T, H, N] tensors
    const int bb = bh / H, hh = bh - bb * H;
    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, m = lane & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j0 = jb * NC;
    const size_t head0 = (static_cast<size_t>(bb) * T * H + hh) * kN;   // (b, t=0, h, 0)
    const size_t sbase = static_cast<size_t>(bh) * (kN * kN);
    // tokens of this row: all T, or its own length (clamped to [0, T])
    const int L = p.lengths ? min(max(p.lengths[bb], 0), T) : T;
    if (L == 0) {
        // an empty row: the state passes through (zeros without state_in)
        for (int e = 4 * tid; e < kN * (kN / J); e += 4 * static_cast<int>(blockDim.x)) {
            const int i = e / (kN / J), jj = j0 + e % (kN / J);  // this workgroup's columns of row i
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (HAS_STATE_IN)
                x = *reinterpret_cast<const f32x4 *>(&p.state_in[sbase + i * kN + jj]);
            *reinterpret_cast<f32x4 *>(&p.state_out[sbase + i * kN + jj]) = x;
        }
        return;
    }
    const int nchunks = (L + CH - 1) / CH;
    // element offset of token t in this (batch, head)'s rows: one 32x32->64 multiply-add
    const uint32_t rs32 = static_cast<uint32_t>(H) * kN;
    auto row_of = [&](int t) { return head0 + static_cast<uint64_t>(static_cast<uint32_t>(t)) * rs32; };
    // Pipeline depth: iteration i consumes chunk i and builds the matrices of
    // chunk i+1; the operands of chunk i+OFF_S and the decay table of chunk
    // i+OFF_D (DEEP: also M_ab of chunk i+2 and the decay factors of chunk i+5).
    constexpr int OFF_S = DEEP ? 3 : 2;
    constexpr int OFF_D = DEEP ? 4 : 3;
    constexpr int OFF_D1 = DEEP ? OFF_D + 1 : OFF_D;  // where the decay factors are computed
    constexpr int I0 = -OFF_D1;                        // first iteration: decay factors of chunk 0


    if (wv < NSW) {
        // ------------------------------------------------------------ consumer
        // The consumers' chain of dependent products is the longest per chunk;
        // the producer waves sharing their SIMDs have slack, so the consumers'
        // instructions go first.
        __builtin_amdgcn_s_setprio(2);
        const int jw = j0 + 16 * wv;      // this wave's first state column
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
        // The state is in registers before the chunk loop starts.  Without this wait the
        // compiler waits for these loads inside the loop, where the counter also holds the
        // previous chunk's output stores: every chunk would wait for those to drain.
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        // CKPT: [B, NCK, H, N*N] checkpoints in tile order (element (i, j) of a head's
        // state at ckpt_offset(i, j) from its base): this lane's four values of row tile pt
        // (rows 16 pt + 4 q + e, column jw + m) are one 16-byte unit, and the wave's store
        // of a row tile is one contiguous kilobyte
        const int nck = (T + CH - 1) / CH;
        auto ckpt_store = [&](int c, const f32x4 (&x)[4]) {
            float *const cb = p.ckpt + ((static_cast<size_t>(bb) * nck + c) * H + hh) * (kN * kN) +
                              ckpt_offset(4 * q, jw + m);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
                *reinterpret_cast<f32x4 *>(cb + ckpt_offset(16 * pt, 0)) = x[pt];
        };
        if constexpr (CKPT) {  // chunk 0 starts from the input state
            f32x4 x0[4];
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
                x0[pt] = f32x4{Sx[pt][0], Sx[pt][1], Sx[pt][2], Sx[pt][3]};
            ckpt_store(0, x0);
        }
        // transpose-load address pieces of this lane: row 4 q + m/4, column group m%4
        const int trow = 4 * q + (m >> 2), tcol = 4 * (m & 3);
        const int mcol_t = mcol(trow, m & 3);  // the same unit in a swizzled matrix tile
        // byte offsets of this lane's outputs (rows 4 q + e, column m) from a chunk's
        // base: 32-bit offsets from a uniform base keep the stores' addresses in one register
        uint32_t ooff[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            ooff[e] = (static_cast<uint32_t>(4 * q + e) * rs32 + m) * static_cast<uint32_t>(sizeof(Tout));
        auto store_o = [](Tout *base, uint32_t off, float x) {
            asm volatile("" : "+v"(off));  // keeps the offset 32-bit (not widened ahead of the loop)
            store_elem(reinterpret_cast<Tout *>(reinterpret_cast<char *>(base) + off), 0, x);
        };

        // The exact path of a chunk with a decay below 2^-15: the recurrence itself,
        // token by token, on this wave's 64x16 slice of the state (which enters such a
        // chunk unscaled).  Lane (q, m) holds rows 16 pt + 4 q + e of column jw + m; a
        // sum over the key rows adds the four lanes of a column (m, m+16, m+32, m+48)
        // by two exchanges, which give all four the same value.
        auto exact_chunk = [&](int t0, int c) {
            const int nt = min(CH, L - t0);
#pragma unroll 1
            for (int tau = 0; tau < nt; ++tau) {
                // uniform row bases; the lanes' keys are small offsets from them, made opaque
                // here so that no per-lane address is hoisted out of the chunk loop (it would
                // stay live through the other path and push that one into spills)
                int kq = 4 * q, jc = jw + m;
                asm volatile("" : "+v"(kq), "+v"(jc));
                const uint64_t row = row_of(t0 + tau);
                const Tin *__restrict__ ra = static_cast<const Tin *>(p.a) + row;
                const Tin *__restrict__ rw = static_cast<const Tin *>(p.w) + row;
                const Tin *__restrict__ rb = static_cast<const Tin *>(p.b) + row;
                const Tin *__restrict__ rk = static_cast<const Tin *>(p.k) + row;
                const Tin *__restrict__ rr = static_cast<const Tin *>(p.r) + row;
                const float vj = load_elem(static_cast<const Tin *>(p.v) + row, jc);
                float sa = 0.0f;
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const f32x4 a4 = load4(ra + 16 * pt + kq);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sa = fmaf(a4[e], Sx[pt][e], sa);
                }
                sa += __shfl_xor(sa, 16);
                sa += __shfl_xor(sa, 32);
                float op = 0.0f;
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    // one group of four keys at a time: this path is rare, and its registers
                    // count against the whole wave's budget
                    __builtin_amdgcn_sched_barrier(0);
                    const int key = 16 * pt + kq;
                    const f32x4 w4 = load4(rw + key), b4 = load4(rb + key);
                    const f32x4 k4 = load4(rk + key), r4 = load4(rr + key);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        Sx[pt][e] = fmaf(w4[e], Sx[pt][e], fmaf(b4[e], sa, k4[e] * vj));
                        op = fmaf(r4[e], Sx[pt][e], op);
                    }
                }
                op += __shfl_xor(op, 16);
                op += __shfl_xor(op, 32);
                if (q == 0) {
                    if constexpr (TAIL)
                        sm.ot.t[c & 1][tau][jc] = op;
                    else
                        store_elem(go + row, jc, op);
                }
            }
        };

        // A' and v of the next chunk are read at the end of each iteration
        // (they were final one or more iterations before) and stay in flight
        // across the barrier: this wave writes no LDS, so its barrier needs no
        // wait for its own LDS accesses.
        s16x8 pA[2][NP];
        s16x4 pV[NPV];
        auto prefetch = [&](int c) {
            const SlotT &sl = sm.slot[max(c, 0) % NS];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int pl = 0; pl < NP; ++pl)
                    pA[s][pl] = lds8(&sl.X[OP_A][pl][m][32 * s + 8 * q]);
#pragma unroll
            for (int pl = 0; pl < NPV; ++pl)
                pV[pl] = tr4(&sl.Vr[pl][trow][jw + tcol]);
        };
        // Whether chunk i takes the exact path, as a scalar.  Chunk i+1's flag (final since
        // its decay table was written) is read early in chunk i and becomes a scalar after
        // a wait that chunk i's own reads need anyway, so the branch waits for nothing.
        // The two paths meet on the state before its row factors (acc), so that the common
        // path keeps its registers (the copies fall on the rare path).
        int exact_next = 0;
        for (int i = I0; i < nchunks; ++i) {
            if (i == -1)
                exact_next = __builtin_amdgcn_readfirstlane(sm.exact[0]);
            if (i >= 0) {
                const SlotT &sl = sm.slot[i % NS];
                const int t0 = i * CH;
                const int flag_next = sm.exact[(i + 1) & 7];
                f32x4 acc[4], fv[4];  // the state before its row factors, and those factors
                if (exact_next) {
                    // S^ enters unscaled (this chunk's P_7 is 1) and leaves scaled by f = P_7
                    // of the next chunk (this chunk's d_15 is 1)
                    exact_chunk(t0, i);
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt)
                        acc[pt] = f32x4{Sx[pt][0], Sx[pt][1], Sx[pt][2], Sx[pt][3]};
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt)
                        fv[pt] = *reinterpret_cast<const f32x4 *>(&sl.f[16 * pt + 4 * q]);
                } else {
                    // this chunk's R' rows and the M_ak and T tiles, read first so that
                    // they arrive while S^ is split
                    s16x8 Rf[2][NP];
                    s16x4 Mak[NP], Tf[NP];
#pragma unroll
                    for (int s = 0; s < 2; ++s)
#pragma unroll
                        for (int pl = 0; pl < NP; ++pl)
                            Rf[s][pl] = lds8(&sl.X[OP_R][pl][m][32 * s + 8 * q]);
#pragma unroll
                    for (int pl = 0; pl < NP; ++pl) {
                        Mak[pl] = tr4(&sl.Mt[MT_AK][pl][trow][mcol_t]);
                        Tf[pl] = tr4(&sl.Mt[MT_T][pl][trow][mcol_t]);
                    }
                    if (i == 0) {
                        // S^ = diag(P_7) S_in for the first chunk; afterwards every chunk
                        // leaves S^ of the next one (its row factor folds both scalings).
#pragma unroll
                        for (int pt = 0; pt < 4; ++pt) {
                            const f32x4 p7v = *reinterpret_cast<const f32x4 *>(&sm.p7[16 * pt + 4 * q]);
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                Sx[pt][e] *= p7v[e];
                        }
                    }
                    // S^ as matrix-core B operands over the key index: key slot (q, e) of
                    // k-step s is key row 16 (2 s + e/4) + 4 q + e%4, which this lane holds
                    // in Sx[2 s + e/4][e % 4].
                    s16x8 Bs[2][NP];
                    auto split_state = [&](int s) {
                        float v8[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            v8[e] = Sx[2 * s + e / 4][e & 3];
                        split8<NP>(v8, Bs[s]);
                    };
                    // A'-rows and R'-rows as A operands with the same key slots (stored
                    // contiguously, see key_slot); one accumulator per k-step.
                    // Y = A' S^ + M_ak V in accumulator layout (Y[4 q + e][col m]): A' S^ in
                    // one accumulator over both k-steps and M_ak V in another (a 16x16x16
                    // product never accumulates onto a 16x16x32 one: the compiler inserts no
                    // wait states between the two shapes); R' S^ in one accumulator that the
                    // [M_rb | M_rk] product (the same shape) later continues
                    // V rows as a B operand over the token index (slot (q, e) = token 4 q + e)
                    s16x4 Vf[NPV];
#pragma unroll
                    for (int pl = 0; pl < NPV; ++pl)
                        Vf[pl] = pV[pl];
                    f32x4 ym = {0.f, 0.f, 0.f, 0.f}, ya = {0.f, 0.f, 0.f, 0.f}, oacc = {0.f, 0.f, 0.f, 0.f};
                    // The first k-step's products run while the second half of S^ is
                    // split: the scheduling groups interleave one product with a few
                    // elementwise instructions.
                    split_state(0);
                    __builtin_amdgcn_sched_barrier(0);
                    mma16<NP, NPV>(ym, Mak, Vf);
                    mma32<NP, NP>(ya, pA[0], Bs[0]);
                    split_state(1);
#pragma unroll
                    for (int g = 0; g < 5; ++g) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix-core product
                        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // then elementwise work
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    mma32<NP, NP>(ya, pA[1], Bs[1]);
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        mma32<NP, NP>(oacc, Rf[s], Bs[s]);
                    // The LDS reads for the rest of the chunk are issued here, once the
                    // products above have taken A', R' and S^ out of their registers,
                    // so that they arrive while Z is formed (the fences keep the
                    // compiler from sinking them to their first use).
                    __builtin_amdgcn_sched_barrier(0);
                    // the state update's [B'^T | K'^T] fragments (key rows 16 pt ..)
                    s16x8 Uf[4][NP];
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt) {
                        const int ukey = key_slot(16 * pt + tcol);
#pragma unroll
                        for (int pl = 0; pl < NP; ++pl)
                            Uf[pt][pl] = cat(tr4(&sl.X[OP_B][pl][trow][ukey]), tr4(&sl.X[OP_K][pl][trow][ukey]));
                    }
                    // [M_rb | M_rk] for the output
                    s16x8 Mf[NP];
#pragma unroll
                    for (int pl = 0; pl < NP; ++pl)
                        Mf[pl] = cat(tr4(&sl.Mt[MT_RB][pl][trow][mcol_t]), tr4(&sl.Mt[MT_RK][pl][trow][mcol_t]));
                    __builtin_amdgcn_sched_barrier(0);
                    // Z = T Y
                    f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    {
                        f32x4 y4;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            y4[e] = ya[e] + ym[e];
                        s16x4 Yf[NP];
                        split4<NP>(y4, Yf);
                        mma16<NP, NP>(z, Tf, Yf);
                    }
                    // [Z ; V] as one B operand over 32 token slots: (q, e<4) is Z row 4q+e
                    // (this lane's z[e]), (q, e>=4) is V row 4q+e-4.
                    s16x8 ZV[NP];
                    {
                        s16x4 Zf[NP];
                        split4<NP>(z, Zf);
#pragma unroll
                        for (int pl = 0; pl < NP; ++pl)
                            ZV[pl] = cat(Zf[pl], pl < NPV ? Vf[pl < NPV ? pl : 0] : s16x4{0, 0, 0, 0});
                    }
                    // o = R' S^ + [M_rb | M_rk] [Z ; V]
                    mma32<NP, NP>(oacc, Mf, ZV);
                    // S^ <- diag(f) (S^ + [B'^T | K'^T] [Z ; V]), one 16-row tile at a time;
                    // the [B'^T | K'^T] fragment of key rows 16 pt .. 16 pt + 15 comes from the
                    // row-major B' and K' planes by transpose loads.  The products go out
                    // before the output stores (a branch the compiler schedules nothing
                    // across), and the row factors are read behind them.
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt) {
                        acc[pt] = f32x4{Sx[pt][0], Sx[pt][1], Sx[pt][2], Sx[pt][3]};
                        mma32<NP, NP>(acc[pt], Uf[pt], ZV);
                    }
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt)
                        fv[pt] = *reinterpret_cast<const f32x4 *>(&sl.f[16 * pt + 4 * q]);
                    if constexpr (TAIL) {
                        // the chunk's o stays in LDS for the tail wave (rows past the end too:
                        // that wave writes x for the row's tokens only)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            sm.ot.t[i & 1][4 * q + e][jw + m] = oacc[e];
                    } else {
                        // one uniform base per chunk, per-lane 32-bit offsets
                        Tout *const ob = go + row_of(t0) + jw;
                        if (t0 + CH <= L) {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                store_o(ob, ooff[e], oacc[e]);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (t0 + 4 * q + e < L)
                                    store_o(ob, ooff[e], oacc[e]);
                        }
                    }
                }
#pragma unroll
                for (int pt = 0; pt < 4; ++pt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        Sx[pt][e] = acc[pt][e] * fv[pt][e];
                if constexpr (CKPT) {
                    // the state entering chunk i+1, unscaled: acc times this chunk's d_15
                    if (i + 1 < nchunks) {
                        f32x4 xs[4];
#pragma unroll
                        for (int pt = 0; pt < 4; ++pt)
                            xs[pt] = acc[pt] * *reinterpret_cast<const f32x4 *>(&sm.gr.g[i % NS][16 * pt + 4 * q]);
                        ckpt_store(i + 1, xs);
                    }
                }
                exact_next = __builtin_amdgcn_readfirstlane(flag_next);
            }
            if constexpr (TAIL)
                asm volatile("" ::: "memory");  // the o-tile writes are issued before the prefetch
            prefetch(i + 1);
            if constexpr (TAIL) {
                // this chunk's o-tile writes are complete before the barrier; the last
                // 2 NP + NPV LDS operations (the prefetch just issued) may stay in flight
                static_assert(2 * NP + NPV <= 15, "lgkmcnt field");
                __builtin_amdgcn_s_waitcnt(0xc07f | ((2 * NP + NPV) << 8));
            }
            __builtin_amdgcn_s_barrier();
            // The barrier alone is not a memory operation to the compiler: this
            // keeps it from moving or merging LDS reads across it (no instruction,
            // and no wait for the reads in flight).
            asm volatile("" ::: "memory");
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.state_out[sbase + (16 * pt + 4 * q + e) * kN + jw + m] = Sx[pt][e];
        return;
    }

    // ---------------------------------------------------------------- producers
    // Roles.  Waves go to the SIMDs round-robin (wave w on SIMD w % 4), so the
    // role table spreads the heavy producers (T, decay, K' with v) over
    // different SIMDs for every J.
    //   R_T : M_ab and T            R_D : decay table (from w)
    //   R_MA: M_ak                  R_SA, R_SR, R_SB, R_SK: A', R', B', K' (R_SK also v)
    //   R_MR: M_rb, M_rk
    enum { R_T = 0, R_MA = 1, R_MR = 2, R_D = 3, R_SA = 4, R_SR = 5, R_SB = 6, R_SK = 7, R_T1 = 8, R_D1 = 9,
           R_TAIL = 10 };
    // Producer k runs on SIMD (NSW + k) % 4, beside the consumer wave of that SIMD
    // if there is one.  The consumers set the pace, so the matrix-core work of the
    // producers (the inverse waves above all) is spread evenly over the consumers'
    // SIMDs, and the scale waves' elementwise work fills in around it.
    //   fp32 inputs (eight producers, J = 1): (T, MA) (SK, D) (SA, SR) (SB, MR)
    //   bf16 inputs, J = 1: (MR, SB, D) (SK, MA, D1) (T, SA) (T1, SR)
    //   bf16 inputs, J = 2 (consumers on SIMDs 0 and 1): (SK, SA) (SB, SR) on the
    //   consumers' SIMDs, (T, D1, MA) (T1, D, MR) on the other two
    // R_T / R_T1 and R_D / R_D1 take the even and the odd chunks.  The tail waves, when
    // there are any, are the last two (SIMDs 2 and 3, beside the inverse waves).
    constexpr unsigned long long ROLES = !DEEP ? 0x25316470ull : J == 1 ? 0xAA9354168072ull : 0x2154396780ull;
    const int role = static_cast<int>((ROLES >> (4 * (wv - NSW))) & 15);
    const int t_end = L;

    using F = std::integral_constant<bool, false>;
    using U = std::integral_constant<bool, true>;

    // ---- input path: the decay and scale waves load their own rows, in their
    // own lane layouts, two iterations ahead of use, into alternating register
    // sets (rows past the end are clamped here and masked where they are used).
    const int op = role - R_SA;                       // scale waves: OP_A, OP_R, OP_B, OP_K
    const Tin *__restrict__ gw = static_cast<const Tin *>(p.w);
    const Tin *__restrict__ gx = static_cast<const Tin *>((op & 2) ? ((op & 1) ? p.k : p.b) : ((op & 1) ? p.r : p.a));
    const Tin *__restrict__ gv = static_cast<const Tin *>(p.v);
    const int g8 = lane & 7;                          // scale waves: slot group of this lane
    const int k0 = 32 * (g8 >> 2) + 4 * (g8 & 3);     // its keys: k0 .. k0+3 and k0+16 .. k0+19
    // One register set holds, as 32-bit words, either the decay wave's w[tau]
    // (16 words) or a scale wave's rows: key runs x[pass][run] (words XW(pass,
    // run) ..) and, for R_SK, the v row of each pass (words VW(pass) ..).
    constexpr int EW = F32IN ? 1 : 2;                 // input elements per word
    constexpr int XRW = 4 / EW;                       // words of a four-key run
    constexpr int VRW = 8 / EW;                       // words of an eight-column v row piece
    constexpr int NU = 4 * XRW + 2 * VRW > CH ? 4 * XRW + 2 * VRW : CH;
    struct Raw {
        uint32_t u[NU];
    };
    auto XW = [](int pz, int h) { return (2 * pz + h) * XRW; };
    auto VW = [](int pz) { return 4 * XRW + pz * VRW; };
    // Loads are unconditional (a chunk past the end re-reads the last one, which
    // is never used): a load under a branch makes the compiler wait for it at
    // the join, right after issuing it.
    // decay wave: rows in the scale waves' layout (token 8 pass + lane/8, eight
    // keys from 8 g8), transposed to one key per lane through LDS when used
    auto load_w = [&](Raw &R, int c) {
        c = max(0, min(c, nchunks - 1));
#pragma unroll
        for (int pz = 0; pz < 2; ++pz) {
            const int t = min(c * CH + 8 * pz + (lane >> 3), t_end - 1);
            const uint32_t *src = reinterpret_cast<const uint32_t *>(gw + row_of(t) + 8 * g8);
#pragma unroll
            for (int h = 0; h < VRW / 4; ++h) {
                const u32x4 x4 = *reinterpret_cast<const u32x4 *>(src + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    R.u[pz * VRW + 4 * h + e] = x4[e];
            }
        }
    };
    auto load_x = [&](Raw &R, int c, auto with_v) {
        c = max(0, min(c, nchunks - 1));
#pragma unroll
        for (int pz = 0; pz < 2; ++pz) {
            const int t = min(c * CH + 8 * pz + (lane >> 3), t_end - 1);
            const uint64_t row = row_of(t);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t *src = reinterpret_cast<const uint32_t *>(gx + row + k0 + 16 * h);
                if constexpr (F32IN) {
                    const u32x4 x4 = *reinterpret_cast<const u32x4 *>(src);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        R.u[XW(pz, h) + e] = x4[e];
                } else {
                    const u32x2 x2 = *reinterpret_cast<const u32x2 *>(src);
                    R.u[XW(pz, h)] = x2[0];
                    R.u[XW(pz, h) + 1] = x2[1];
                }
            }
            if constexpr (decltype(with_v)::value) {
                const uint32_t *src = reinterpret_cast<const uint32_t *>(gv + row + 8 * g8);
#pragma unroll
                for (int h = 0; h < VRW / 4; ++h) {
                    const u32x4 v4 = *reinterpret_cast<const u32x4 *>(src + 4 * h);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        R.u[VW(pz) + 4 * h + e] = v4[e];
                }
            }
        }
    };

    // ---- decay waves.  Part 1 turns the w rows of chunk c into its decay
    // factors (kept in registers); part 2 writes them as the table of chunk c,
    // with P_7 of chunk 0 and the row factor f of chunk c-1 (d_15 of c-1, left
    // in LDS by the part 2 of chunk c-1, times P_7 of c; d_15 alone once c is
    // past the end).
    float dk[CH + 1], idk[CH + 1];  // factors of the chunk between the two parts
    int dexact = 0;                 // and whether it takes the exact path (uniform)
    auto decay1_body = [&](const Raw &R, int c) {
        const int i = lane;
        // transpose through LDS: rows in, one key channel per lane out (this
        // wave's own accesses, which LDS performs in order)
#pragma unroll
        for (int pz = 0; pz < 2; ++pz)
#pragma unroll
            for (int h = 0; h < VRW / 4; ++h)
                *reinterpret_cast<u32x4 *>(&sm.wbuf[8 * pz + (lane >> 3)][8 * g8 + 4 * EW * h]) =
                    u32x4{R.u[pz * VRW + 4 * h], R.u[pz * VRW + 4 * h + 1], R.u[pz * VRW + 4 * h + 2],
                          R.u[pz * VRW + 4 * h + 3]};
        float w[CH];
#pragma unroll
        for (int tau = 0; tau < CH; ++tau) {
            const uint32_t bits = F32IN ? __float_as_uint(load_elem(&sm.wbuf[0][0], tau * kN + i))
                                        : static_cast<uint32_t>(reinterpret_cast<const uint16_t *>(&sm.wbuf[0][0])[tau * kN + i]) << 16;
            w[tau] = __uint_as_float(bits);
        }
        if (c * CH + CH > t_end) {  // partial chunk (uniform): positions past the end decay by 1
#pragma unroll
            for (int tau = 0; tau < CH; ++tau)
                if (c * CH + tau >= t_end)
                    w[tau] = 1.0f;
        }
        // the smallest decay magnitude of this key channel; one channel below the bound
        // (-0.0 included) sends the whole chunk to the exact path, whose decay table is
        // all ones
        float wmin = fabsf(w[0]);
#pragma unroll
        for (int tau = 1; tau < CH; ++tau)
            wmin = fminf(wmin, fabsf(w[tau]));
        decay_factors(w, dk, idk);
        dexact = __builtin_amdgcn_readfirstlane(__ballot(wmin < W_EXACT) != 0ull);
        if (dexact) {
#pragma unroll
            for (int r = 0; r <= CH; ++r)
                dk[r] = idk[r] = 1.0f;
        }
    };
    auto decay1 = [&](const Raw &R, int c) {
        if (c >= 0 && c < nchunks)
            decay1_body(R, c);
    };
    auto decay2_body = [&](int c) {  // 0 <= c < nchunks
        const int i = lane;
        DSlot &D = sm.dt[c & 1];
#pragma unroll
        for (int r = 0; r <= CH; ++r)
            D.v[r][dcol(r, i)] = dk[r];
#pragma unroll
        for (int r = 1; r <= CH; ++r)
            D.v[CH + r][dcol(CH + r, i)] = idk[r];
        if (c == 0)
            sm.p7[i] = idk[0];
        else
            sm.slot[(c - 1) % NS].f[i] = sm.d15[(c - 1) & 1][i] * idk[0];
        if constexpr (CKPT)
            if (c > 0)
                sm.gr.g[(c - 1) % NS][i] = sm.d15[(c - 1) & 1][i];
        sm.d15[c & 1][i] = dk[CH];
        if (i == 0)
            sm.exact[c & 7] = dexact;
    };
    auto decay2 = [&](int c) {
        if (c == nchunks) {
            sm.slot[(c - 1) % NS].f[lane] = sm.d15[(c - 1) & 1][lane];
            if constexpr (CKPT)
                sm.gr.g[(c - 1) % NS][lane] = sm.d15[(c - 1) & 1][lane];
        } else if (c >= 0 && c < nchunks) {
            decay2_body(c);
        }
    };

    // ---- scale waves: X' = x * factor, elementwise, lane = (token, slot group):
    // token 8 pass + lane/8, key slots 8 g8 .. 8 g8 + 7.
    // The last, partial chunk has its own copy of the body (rows past the end
    // read as 0), so full chunks carry no per-row selects.
    auto scale_body = [&](const Raw &R, int c, auto with_v, auto partial_c) {
        constexpr bool partial = decltype(partial_c)::value;
        SlotT &sl = sm.slot[c % NS];
        const DSlot &D = sm.dt[c & 1];
        const int roff = op == 0 ? 0 : op == 1 ? 1 : CH + 1;  // table row of token tau
#pragma unroll
        for (int pz = 0; pz < 2; ++pz) {
            const int tau = 8 * pz + (lane >> 3);
            float x[8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if constexpr (F32IN) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        x[4 * h + e] = __uint_as_float(R.u[XW(pz, h) + e]);
                } else {
                    x[4 * h + 0] = bf16_lo(R.u[XW(pz, h)]);
                    x[4 * h + 1] = bf16_hi(R.u[XW(pz, h)]);
                    x[4 * h + 2] = bf16_lo(R.u[XW(pz, h) + 1]);
                    x[4 * h + 3] = bf16_hi(R.u[XW(pz, h) + 1]);
                }
            }
            if (partial && c * CH + tau >= t_end) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    x[e] = 0.0f;
            }
            const int drow = roff + tau;
            const f32x4 d0 = *reinterpret_cast<const f32x4 *>(&D.v[drow][dcol(drow, k0)]);
            const f32x4 d1 = *reinterpret_cast<const f32x4 *>(&D.v[drow][dcol(drow, k0 + 16)]);
            float y[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                y[e] = x[e] * d0[e];
                y[4 + e] = x[4 + e] * d1[e];
            }
            s16x8 pc[NP];
            split8<NP>(y, pc);
#pragma unroll
            for (int pl = 0; pl < NP; ++pl)
                *reinterpret_cast<s16x8 *>(&sl.X[op][pl][tau][8 * g8]) = pc[pl];
        }
        if constexpr (decltype(with_v)::value) {
            // v rows of the chunk (all 64 columns), row-major: lane -> row 8 pass + lane/8,
            // columns 8 g8 .. 8 g8 + 7
#pragma unroll
            for (int pz = 0; pz < 2; ++pz) {
                const int s = 8 * pz + (lane >> 3);
                const bool live = !partial || c * CH + s < t_end;
                if constexpr (F32IN) {
                    float v8[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v8[e] = live ? __uint_as_float(R.u[VW(pz) + e]) : 0.0f;
                    s16x8 pc[NPV];
                    split8<NPV>(v8, pc);
#pragma unroll
                    for (int pl = 0; pl < NPV; ++pl)
                        *reinterpret_cast<s16x8 *>(&sl.Vr[pl][s][8 * g8]) = pc[pl];
                } else {
                    const u32x4 v4 = {R.u[VW(pz)], R.u[VW(pz) + 1], R.u[VW(pz) + 2], R.u[VW(pz) + 3]};
                    *reinterpret_cast<u32x4 *>(&sl.Vr[0][s][8 * g8]) = live ? v4 : u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
    };
    auto scale = [&](const Raw &R, int c, auto with_v) {
        if (c < 0 || c >= nchunks)
            return;
        if (c * CH + CH > t_end)  // uniform
            scale_body(R, c, with_v, U{});
        else
            scale_body(R, c, with_v, F{});
    };

    // ---- matrix waves: 16x16 tiles M = tril(X' Y'^T) of chunk c over the 64 key
    // channels, stored transposed.  Each role has its own straight-line code
    // (mr is a compile-time flag): a branch between a matrix-core result and
    // the instruction reading it has been seen to lose the wait states that
    // read needs.
    auto matrices = [&](int c, auto mr_c) {
        constexpr bool MR = decltype(mr_c)::value;   // R_MR: (R',B') and (R',K'); else R_MA: (A',K')
        if (c < 0 || c >= nchunks)
            return;
        SlotT &sl = sm.slot[c % NS];
        constexpr int yo = MR ? OP_B : OP_K;
        constexpr int xo = MR ? OP_R : OP_A;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            s16x8 Af[NP], Bf[NP];
#pragma unroll
            for (int pl = 0; pl < NP; ++pl) {
                Af[pl] = lds8(&sl.X[xo][pl][m][32 * s + 8 * q]);
                Bf[pl] = lds8(&sl.X[yo][pl][m][32 * s + 8 * q]);
            }
            mma32<NP, NP>(acc, Af, Bf);           // lane (m, q): M[4 q + e][m]
            if constexpr (MR) {
                s16x8 Kf[NP];
#pragma unroll
                for (int pl = 0; pl < NP; ++pl)
                    Kf[pl] = lds8(&sl.X[OP_K][pl][m][32 * s + 8 * q]);
                mma32<NP, NP>(acc2, Af, Kf);      // M_rk
            }
        }
        // a rows exclude the diagonal, r rows include it
        f32x4 mv, mv2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tau = 4 * q + e;
            const bool keep = m < tau || (MR && m == tau);
            mv[e] = keep ? acc[e] : 0.0f;
            mv2[e] = keep ? acc2[e] : 0.0f;
        }
        s16x4 pc[NP];
        split4<NP>(mv, pc);
        constexpr int mt = MR ? MT_RB : MT_AK;
#pragma unroll
        for (int pl = 0; pl < NP; ++pl)
            *reinterpret_cast<s16x4 *>(&sl.Mt[mt][pl][m][mcol(m, q)]) = pc[pl];
        if constexpr (MR) {
            split4<NP>(mv2, pc);
#pragma unroll
            for (int pl = 0; pl < NP; ++pl)
                *reinterpret_cast<s16x4 *>(&sl.Mt[MT_RK][pl][m][mcol(m, q)]) = pc[pl];
        }
    };

    // ---- inverse wave.  Part A forms M = M_ab of chunk c (kept in registers)
    // and writes it to this wave's LDS tile; part B reads back M^T, inverts I - M,
    //   T = (I - M)^{-1} = (I + M)(I + M^2)(I + M^4)(I + M^8)   (M strictly lower),
    // and stores T.  A matrix X enters a product as the A operand through the
    // accumulator of X^T and as the B operand through its own accumulator, so
    // every product in part B is formed together with the transpose the next
    // one needs; the first transpose crosses the barrier between the parts in LDS.
    f32x4 tM;  // M of the chunk between the two parts
    float (*const mtile)[MTP] = sm.mt[role == R_T1 ? 1 : 0];
    auto inv_a_body = [&](int c) {
        const SlotT &sl = sm.slot[c % NS];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            s16x8 Af[NP], Bf[NP];
#pragma unroll
            for (int pl = 0; pl < NP; ++pl) {
                Af[pl] = lds8(&sl.X[OP_A][pl][m][32 * s + 8 * q]);
                Bf[pl] = lds8(&sl.X[OP_B][pl][m][32 * s + 8 * q]);
            }
            mma32<NP, NP>(acc, Af, Bf);           // lane (m, q): M[4 q + e][m]
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tau = 4 * q + e;
            tM[e] = m < tau ? acc[e] : 0.0f;      // M[tau][m]
            mtile[tau][m] = tM[e];
        }
    };
    auto inv_a = [&](int c) {
        if (c >= 0 && c < nchunks)
            inv_a_body(c);
    };
    auto inv_b_body = [&](int c) {
        SlotT &sl = sm.slot[c % NS];
        // M^T[4 q + e][m] = M[m][4 q + e]: row m of the tile
        const f32x4 tMt = *reinterpret_cast<const f32x4 *>(&mtile[m][4 * q]);
        f32x4 P = tM, Pt = tMt, Q, Qt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float one = m == 4 * q + e ? 1.0f : 0.0f;
            Q[e] = P[e] + one;
            Qt[e] = Pt[e] + one;
        }
#pragma unroll
        for (int lvl = 0; lvl < 3; ++lvl) {
            s16x4 Ps[NP], Pts[NP];
            split4<NP>(P, Ps);
            split4<NP>(Pt, Pts);
            f32x4 Pn = {0.f, 0.f, 0.f, 0.f}, Ptn = {0.f, 0.f, 0.f, 0.f};
            mma16<NP, NP>(Pn, Pts, Ps);          // P P
            if (lvl < 2)
                mma16<NP, NP>(Ptn, Ps, Pts);     // (P P)^T = P^T P^T
            s16x4 Qts[NP], Pns[NP];
            split4<NP>(Qt, Qts);
            split4<NP>(Pn, Pns);
            f32x4 Qn = Q, Qtn = Qt;
            mma16<NP, NP>(Qn, Qts, Pns);         // Q + Q Pn
            if (lvl < 2)
                mma16<NP, NP>(Qtn, Pns, Qts);    // Q^T + Pn^T Q^T
            P = Pn;
            Pt = Ptn;
            Q = Qn;
            Qt = Qtn;
        }
        s16x4 tp[NP];
        split4<NP>(Q, tp);
#pragma unroll
        for (int pl = 0; pl < NP; ++pl)
            *reinterpret_cast<s16x4 *>(&sl.Mt[MT_T][pl][m][mcol(m, q)]) = tp[pl];
    };
    auto inv_b = [&](int c) {
        if (c >= 0 && c < nchunks)
            inv_b_body(c);
    };

    // ---- tail waves (TAIL): in iteration i, the time-mix tail of chunk i-1, whose o the
    // consumers left in LDS in iteration i-1; the last chunk after the loop.  Tail wave
    // u takes tokens 8 u .. 8 u + 7 of each chunk in two passes; lane (r, c) of a pass
    // takes token 8 u + 4 pass + r, channels 4 c .. 4 c + 3 (tail_row4: one row per 16
    // lanes).  Its r, k, v and gate were loaded one iteration before.
    auto tail_role = [&]() {
        if constexpr (TAIL) {
            constexpr int NPASS = CH / 4 / NTAIL;
            const int tw = wv - (NSW + nprod<Tin>());  // which tail wave
            const int c0 = 4 * (lane & 15), rr = NPASS * 4 * tw + (lane >> 4);
            const int pj = hh * kN + c0;
            const f32x4 rk4 = *reinterpret_cast<const f32x4 *>(p.r_k + pj);
            const f32x4 w4 = *reinterpret_cast<const f32x4 *>(p.ln_w + pj);
            const f32x4 b4 = *reinterpret_cast<const f32x4 *>(p.ln_b + pj);
            const Tin *const ins[4] = {static_cast<const Tin *>(p.r), static_cast<const Tin *>(p.k),
                                       static_cast<const Tin *>(p.v), static_cast<const Tin *>(p.gate)};
            Tout *__restrict__ gxo = static_cast<Tout *>(p.o);
            // the rows of one chunk, [pass][r, k, v, gate], four bf16 channels each; three
            // sets in rotation, loaded three iterations before use (as the scale waves do)
            typedef u32x2 Rows[NPASS][4];
            Rows R0, R1, R2;
            // a chunk's rows as byte offsets (32-bit) from its first row: (15 H N + 60) * 2 < 2^32
            auto load_rows = [&](Rows &R, int c) {  // unconditional: chunks outside the row re-read one inside
                c = max(0, min(c, nchunks - 1));
                const uint64_t base = row_of(c * CH);
#pragma unroll
                for (int pz = 0; pz < NPASS; ++pz) {
                    const int tau = min(4 * pz + rr, t_end - 1 - c * CH);
                    const uint32_t off = (static_cast<uint32_t>(tau) * rs32 + c0) * 2u;
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        R[pz][x] = *reinterpret_cast<const u32x2 *>(
                            reinterpret_cast<const char *>(ins[x] + base) + off);
                }
            };
            auto unpack = [](const u32x2 u) {
                return f32x4{bf16_lo(u[0]), bf16_hi(u[0]), bf16_lo(u[1]), bf16_hi(u[1])};
            };
            auto tail_chunk = [&](int c, const Rows &R) {
                // the passes' rows straight-line (their chains interleave), then the stores
                f32x4 o4[NPASS], x4[NPASS];
#pragma unroll
                for (int pz = 0; pz < NPASS; ++pz)
                    o4[pz] = *reinterpret_cast<const f32x4 *>(&sm.ot.t[c & 1][4 * pz + rr][c0]);
#pragma unroll
                for (int pz = 0; pz < NPASS; ++pz)
                    x4[pz] = tail_row4(o4[pz], unpack(R[pz][0]), unpack(R[pz][1]), unpack(R[pz][2]),
                                       unpack(R[pz][3]), rk4, w4, b4, p.eps);
                Tout *const xb = gxo + row_of(c * CH);
#pragma unroll
                for (int pz = 0; pz < NPASS; ++pz) {
                    const int tau = 4 * pz + rr;
                    const uint32_t off = (static_cast<uint32_t>(tau) * rs32 + c0) * static_cast<uint32_t>(sizeof(Tout));
                    if (c * CH + tau < t_end)
                        store4(reinterpret_cast<Tout *>(reinterpret_cast<char *>(xb) + off), x4[pz]);
                }
            };
            // iteration i (set (i - I0) % 3) takes chunk i-1 and loads chunk i+2 into the same set
            auto work = [&](int i, Rows &R) {
                if (i >= 1)
                    tail_chunk(i - 1, R);
                load_rows(R, i + 2);
            };
            load_rows(R0, I0 - 1);
            load_rows(R1, I0);
            load_rows(R2, I0 + 1);
            int i = I0;
            for (; i + 2 < nchunks; i += 3) {
                work(i, R0);
                __syncthreads();
                work(i + 1, R1);
                __syncthreads();
                work(i + 2, R2);
                __syncthreads();
            }
            if (i < nchunks) {
                work(i, R0);
                __syncthreads();
                if (i + 1 < nchunks) {
                    work(i + 1, R1);
                    __syncthreads();
                }
            }
            // the last chunk, after the last barrier, from the set its iteration would use
            const int kf = (nchunks - I0) % 3;
            if (kf == 0)
                tail_chunk(nchunks - 1, R0);
            else if (kf == 1)
                tail_chunk(nchunks - 1, R1);
            else
                tail_chunk(nchunks - 1, R2);
        }
    };

    // Pipeline: each role runs its own copy of the loop, one barrier per
    // iteration.  The waves that load input rows unroll it by three and keep
    // three register sets: the rows a wave works on in iteration i were loaded
    // in iteration i-3 into set (i - I0) % 3.  Before the loop the three sets
    // are loaded in the same order as in every later round, so the compiler's
    // waits (which may also cover the set loaded one round before) only ever
    // wait for rows two or more iterations old.
    using K0 = std::integral_constant<int, 0>;
    using K1 = std::integral_constant<int, 1>;
    using K2 = std::integral_constant<int, 2>;
    auto run = [&](auto work) {
        for (int i = I0; i < nchunks; ++i) {
            work(i);
            __syncthreads();
        }
    };
    auto run2 = [&](auto work) {
        // whole pairs in the loop, the last iteration after it; K0 is i = I0 + 2j
        int i = I0;
        for (; i + 1 < nchunks; i += 2) {
            work(i, K0{});
            __syncthreads();
            work(i + 1, K1{});
            __syncthreads();
        }
        if (i < nchunks) {
            work(i, K0{});
            __syncthreads();
        }
    };
    auto run3 = [&](auto work) {
        // whole rounds in the loop (its back edge then has one predecessor, and
        // the wait analysis stays exact), the last one or two iterations after it
        int i = I0;
        for (; i + 2 < nchunks; i += 3) {
            work(i, K0{});
            __syncthreads();
            work(i + 1, K1{});
            __syncthreads();
            work(i + 2, K2{});
            __syncthreads();
        }
        if (i < nchunks) {
            work(i, K0{});
            __syncthreads();
            if (i + 1 < nchunks) {
                work(i + 1, K1{});
                __syncthreads();
            }
        }
    };
    auto scale_role = [&](auto with_v) {
        Raw f0, f1, f2;
        load_x(f0, I0 + OFF_S, with_v);  // chunks below 0 are nothing (rows of chunk 0 are read instead)
        load_x(f1, I0 + OFF_S + 1, with_v);
        load_x(f2, I0 + OFF_S + 2, with_v);
        run3([&](int i, auto k) {
            constexpr int K = decltype(k)::value;
            Raw &fr = K == 0 ? f0 : K == 1 ? f1 : f2;
            scale(fr, i + OFF_S, with_v);
            load_x(fr, i + OFF_S + 3, with_v);
        });
    };
    // one inverse wave per chunk parity: chunk c's M in iteration c-2, its T in c-1
    auto inv_role = [&](auto par_c) {
        constexpr int PAR = decltype(par_c)::value;
        run2([&](int i, auto k) {
            constexpr int PI = ((I0 & 1) + decltype(k)::value) & 1;  // parity of i
            if constexpr (((PI + 1) & 1) == PAR)
                inv_b(i + 1);
            else
                inv_a(i + 2);
        });
    };
    if (role == R_T || role == R_T1) {
        if constexpr (DEEP) {
            if (role == R_T)
                inv_role(std::integral_constant<int, 0>{});
            else
                inv_role(std::integral_constant<int, 1>{});
        } else {
            run([&](int i) {
                inv_a(i + 1);
                inv_b(i + 1);
            });
        }
    } else if (role == R_MA) {
        run([&](int i) { matrices(i + 1, F{}); });
    } else if (role == R_MR) {
        run([&](int i) { matrices(i + 1, U{}); });
    } else if (DEEP && (role == R_D || role == R_D1)) {
        // one decay wave per chunk parity: chunk c's factors in iteration c-5,
        // its table in c-4; its rows are loaded right after the factors of the
        // chunk two before (one register set, two iterations ahead)
        auto decay_role = [&](auto par_c) {
            constexpr int PAR = decltype(par_c)::value;
            Raw fr;
            load_w(fr, PAR);
            run2([&](int i, auto k) {
                constexpr int PI = ((I0 & 1) + decltype(k)::value) & 1;  // parity of i
                if constexpr (((PI + OFF_D) & 1) == PAR) {
                    decay2(i + OFF_D);
                } else {
                    decay1(fr, i + OFF_D1);
                    load_w(fr, i + OFF_D1 + 2);
                }
            });
        };
        if (role == R_D)
            decay_role(std::integral_constant<int, 0>{});
        else
            decay_role(std::integral_constant<int, 1>{});
    } else if (role == R_D) {
        Raw f0, f1, f2;
        load_w(f0, I0 + OFF_D1);
        load_w(f1, I0 + OFF_D1 + 1);
        load_w(f2, I0 + OFF_D1 + 2);
        run3([&](int i, auto k) {
            constexpr int K = decltype(k)::value;
            Raw &fr = K == 0 ? f0 : K == 1 ? f1 : f2;
            if constexpr (DEEP) {
                // table of chunk i+4 from factors computed last iteration, and the
                // factors of chunk i+5 (one block in the steady state)
                if (i + OFF_D >= 0 && i + OFF_D1 < nchunks) {
                    decay2_body(i + OFF_D);
                    decay1_body(fr, i + OFF_D1);
                } else {
                    decay2(i + OFF_D);
                    decay1(fr, i + OFF_D1);
                }
            } else {
                decay1(fr, i + OFF_D);
                decay2(i + OFF_D);
            }
            load_w(fr, i + OFF_D1 + 3);
        });
    } else if (TAIL && role == R_TAIL) {
        tail_role();
    } else if (role == R_SK) {
        scale_role(U{});
    } else {
        scale_role(F{});
    }
}

template <typename Tin, typename Tout, int J, int MODE = MODE_PLAIN>
hipError_t launch_j(const SeqArgs &p, hipStream_t stream)
{
    const int nblocks = p.B * p.H * J;
    int per_xcd = (nblocks + 7) / 8;
    per_xcd = (per_xcd + J - 1) / J * J;  // a head's column blocks never straddle two XCDs
    const dim3 grid(8 * per_xcd), block((kN / J / 16 + nprod<Tin>() + nextra<MODE>()) * 64);
    if (p.state_in)
        hipLaunchKernelGGL((wkv7_chunk_kernel<Tin, Tout, J, true, MODE>), grid, block, 0, stream, p, per_xcd,
                           nblocks);
    else
        hipLaunchKernelGGL((wkv7_chunk_kernel<Tin, Tout, J, false, MODE>), grid, block, 0, stream, p, per_xcd,
                           nblocks);
    return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_typed(const SeqArgs &p, hipStream_t stream)
{
    // The fused tail needs every column of a token in one workgroup: whole heads.
    if (p.gate) {
        if constexpr (std::is_same<Tin, uint16_t>::value)
            return launch_j<Tin, Tout, 1, MODE_TAIL>(p, stream);
        else
            return hipErrorInvalidValue;  // the C ABI routes fp32 inputs elsewhere
    }
    // One workgroup fills a compute unit's LDS; split heads into column blocks
    // only while the grid still fits in one pass over the 256 compute units.
    const long long heads = static_cast<long long>(p.B) * p.H;
    if (p.ckpt) {  // checkpoints (fp32 o only)
        if constexpr (std::is_same<Tout, float>::value) {
            if (heads * 4 <= 256)
                return launch_j<Tin, Tout, 4, MODE_CKPT>(p, stream);
            if (heads * 2 <= 256)
                return launch_j<Tin, Tout, 2, MODE_CKPT>(p, stream);
            return launch_j<Tin, Tout, 1, MODE_CKPT>(p, stream);
        } else {
            return hipErrorInvalidValue;  // the C ABI refuses a bf16 o with checkpoints
        }
    }
    if (heads * 4 <= 256)
        return launch_j<Tin, Tout, 4>(p, stream);
    if (heads * 2 <= 256)
        return launch_j<Tin, Tout, 2>(p, stream);
    return launch_j<Tin, Tout, 1>(p, stream);
}

// The checkpoint of a one-chunk pass: each head's input state (zeros when src is null)
// in tile order, one 16-byte unit (four rows of one column) per thread.
__global__ __launch_bounds__(256) void ckpt_from_state_kernel(const float *src, f32x4 *dst, long long n4)
{
    for (long long i = blockIdx.x * 256ll + threadIdx.x; i < n4; i += static_cast<long long>(gridDim.x) * 256) {
        const long long head = i >> 10;
        const int u = static_cast<int>(i & 1023);
        // unit u holds rows 16 (u/64 % 4) + 4 (u/16 % 4) + e, column 16 (u/256) + u % 16
        const int row0 = 16 * ((u >> 6) & 3) + 4 * ((u >> 4) & 3), col = 16 * (u >> 8) + (u & 15);
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (src)
            for (int e = 0; e < 4; ++e)
                x[e] = src[head * (kN * kN) + (row0 + e) * kN + col];
        dst[i] = x;
    }
}

}  // namespace

hipError_t launch_ckpt_from_state(const float *state, float *ckpt, int B, int H, hipStream_t stream)
{
    const long long n4 = static_cast<long long>(B) * H * (kN * kN / 4);
    const long long blocks = (n4 + 255) / 256;
    hipLaunchKernelGGL(ckpt_from_state_kernel, dim3(static_cast<unsigned>(blocks < 65536 ? blocks : 65536)), dim3(256),
                       0, stream, state, reinterpret_cast<f32x4 *>(ckpt), n4);
    return hipGetLastError();
}

hipError_t launch_chunk(const SeqArgs &p, hipStream_t stream)
{
    if (p.in_bf16)
        return p.o_bf16 ? launch_typed<uint16_t, uint16_t>(p, stream) : launch_typed<uint16_t, float>(p, stream);
    return p.o_bf16 ? launch_typed<float, uint16_t>(p, stream) : launch_typed<float, float>(p, stream);
}

}  // namespace wkv7
