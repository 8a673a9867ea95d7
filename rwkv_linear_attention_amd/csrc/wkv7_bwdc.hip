// wkv7_bwdc.hip -- the backward pass from chunk checkpoints, in chunk form.
//
// The pages name a trainable WKV kernel whose backward pass rebuilds the state
// chunk by chunk (the SwiftRWKV Inference guide, its `.rwkvq` backend section)
// and give no formulas.  The gradients are the reverse-mode adjoint of the
// recurrence of the RWKV-X Architecture page, section "WKV-7 Kernel
// (Generalized Delta Rule)":
//     S_t = diag(w_t) S_{t-1} + b_t (a_t^T S_{t-1}) + k_t v_t^T,    o_t = S_t^T r_t.
// With G = dL/dS_t, going back over the tokens,
//     G += r_t dO_t^T;   c_t = G^T b_t;   G <- diag(w_t) G + a_t c_t^T,
// which needs no states at all.  Everything else is local to a chunk of 16
// tokens once the state entering it (its checkpoint, S0) and the gradient for
// the state leaving it (G_end) are known.  So the pass runs as three launches:
//
//   1. the chunk kernel on every head's last chunk (its G_end is d_state_out);
//   2. the gradient chain, one workgroup per head, serial over the tokens: it
//      writes G_end of every other chunk, and the gradient of the input state;
//   3. the chunk kernel on every other chunk, all at once.
//
// G_end of chunk c is written into c's own rows of dr, dk, da and db (16 tokens
// x 64 channels each, four of them hold the 64 x 64 matrix), which the chunk
// kernel reads before it overwrites them with the gradients: no workspace.
//
// The chunk kernel.  With P_tau the running product of w over the chunk and the
// factors measured against position 7, d_tau = P_tau / P_7 (no absolute product
// is formed), A' = a d_{tau-1}, R' = r d_tau, B' = b / d_tau, K' = k / d_tau,
// S^ = diag(P_7) S0, G^ = diag(d_15) G_end, M_xy = tril(X'Y'^T) (strict for the
// a-rows) and T = (I - M_ab)^{-1}, the chunk's forward is
//     X = A' S^ + M_ak V,  Z = T X,  O = R' S^ + M_rb Z + M_rk V,
//     S_end = diag(d_15) (S^ + B'^T Z + K'^T V),
// and its reverse mode
//     dZ = B' G^ + M_rb^T dO,  dX = T^T dZ,  dV = K' G^ + M_rk^T dO + M_ak^T dX,
//     dM_ab = tril(dX Z^T, -1), dM_ak = tril(dX V^T, -1), dM_rb = tril(dO Z^T), dM_rk = tril(dO V^T),
//     dA' = dX S^T + dM_ab B' + dM_ak K',   dR' = dO S^T + dM_rb B' + dM_rk K',
//     dB' = Z G^T + dM_ab^T A' + dM_rb^T R', dK' = V G^T + dM_ak^T A' + dM_rk^T R',
//     da = dA' d_{tau-1},  dr = dR' d_tau,  db = dB' / d_tau,  dk = dK' / d_tau,  dv = dV.
// The decay gradient is taken in its direct form dw_t = rowsum(G_t * S_{t-1}),
// with both states written in the chunk's terms:
//     w_t dw_t = rowsum(G^ * S^) + sum_{u<t} (B'_u (G^ z_u) + K'_u (G^ v_u))
//              + sum_{s>=t} R'_s (S^ dO_s + sum_{u<t} (B'_u dO_s.z_u + K'_u dO_s.v_u))
//              + sum_{s>t}  A'_s (S^ dX_s + sum_{u<t} (B'_u dX_s.z_u + K'_u dX_s.v_u)),
// elementwise in the key index.  Every term carries w_t among its decay
// factors, so the division by w_t loses nothing.  (The log-decay form, a suffix
// sum of d log P divided by w, loses about eps / w to cancellation.)  The
// products run on the matrix cores in fp32 (16x16x4), so the chunk form is as
// exact as the recurrence; a chunk with a decay below 2^-15 (factors outside the
// fp32 range, w = 0 included) runs the recurrence itself instead.
#include "wkv7_device.h"
#include "wkv7_launch.h"

#include <algorithm>
#include <type_traits>

namespace wkv7 {
namespace {

constexpr int CC = 16;                          // chunk length: the checkpoint spacing
constexpr int kCUs = 256;                       // compute units of the chip
constexpr int REF = 7;                          // reference position of the decay factors
constexpr float kExactBelow = 1.0f / 32768.0f;  // 2^-15

// Four consecutive elements at p (16-byte aligned for fp32, 8-byte for bf16), widened.
__device__ __forceinline__ f32x4 load4w(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ f32x4 load4w(const uint16_t *p)
{
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
}

// ---------------------------------------------------------------------------------
// The gradient chain.  The value columns of G evolve independently: each head runs as
// two workgroups of 32 columns, four waves of 8 columns each.  Lane (rg, cg) of a wave,
// rg = lane % 16 and cg = lane / 16, holds key rows 4 rg .. 4 rg + 3 of the wave's
// columns 2 cg and 2 cg + 1.  Per token, c = G^T b is a sum over the key rows: in-lane
// over four rows, then over the 16 lanes of the lane's DPP row (the other rows of the
// same columns) -- inside the wave, so the token loop has no barrier and the waves run
// independently.  A chunk's r, w, a, b (per key) and dO (the workgroup's columns) are
// staged in LDS, loaded into registers one chunk ahead; each lane reads its four keys'
// values and its two columns' dO, one token ahead of their use.
constexpr int GNW = 4, GCOL = 32;

template <typename Tin>
struct ChainStage {
    // 16-byte pieces: 4 key-side tensors x 16 tokens x 64 channels (KPT per thread, tensor
    // after tensor, so a wave's pieces lie in one tensor), then dO 16 x 32 fp32 (one per
    // thread: 128 pieces, the second 128 threads load and store them again)
    static constexpr int EPP = 16 / sizeof(Tin);
    static constexpr int PPTEN = CC * kN / EPP;   // pieces per tensor
    static constexpr int KPT = 4 * PPTEN / (GNW * 64);
    static_assert(KPT * GNW * 64 == 4 * PPTEN && PPTEN % 64 == 0, "whole waves per tensor");
    static_assert(CC * GCOL / 4 == 128, "one dO piece per thread, twice");
};

#define GLOBAL_AS __attribute__((address_space(1)))
typedef unsigned long long u64;
typedef float f32x2 __attribute__((ext_vector_type(2)));

// x or y by a per-lane condition the compiler cannot see through (so it selects the
// values and does not build a table of them)
__device__ __forceinline__ u64 pick(bool f, u64 x, u64 y)
{
    unsigned m = f;
    asm volatile("" : "+v"(m));
    return m ? x : y;
}

struct ChainSmem {
    float in[2][4][CC][kN];   // r, w, a, b of a chunk (two chunks in turn)
    float dout[2][CC][GCOL];  // dO at the workgroup's columns
};

template <typename Tin, bool HAS_DOUT>
__global__ __launch_bounds__(GNW * 64) void wkv7_bwdc_chain_kernel(BwdArgs p)
{
    using SG = ChainStage<Tin>;
    __shared__ alignas(16) ChainSmem sm;
    const int lane = threadIdx.x & 63, rg = lane & 15, cg = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int bh = blockIdx.x >> 1, half = blockIdx.x & 1;
    const int H = p.H, T = p.T;
    const int bb = bh / H, hh = bh - bb * H;
    const int nck = (T + CC - 1) / CC;
    const int jw = wv * 8 + cg * 2;        // this lane's first column within the workgroup's
    const int j = half * GCOL + jw;        // ... and within the head's
    const int r0 = 4 * rg;                 // this lane's first key row
    const size_t tok_e = static_cast<size_t>(H) * kN;
    const size_t head_e = static_cast<size_t>(bb) * T * tok_e + static_cast<size_t>(hh) * kN;
    const size_t sbase = static_cast<size_t>(bh) * (kN * kN) + static_cast<size_t>(r0) * kN + j;
    float G[4][2];  // rows r0 + u, columns j, j + 1
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const float2 x = HAS_DOUT ? *reinterpret_cast<const float2 *>(&p.d_state_out[sbase + u * kN])
                                  : make_float2(0.f, 0.f);
        G[u][0] = x.x;
        G[u][1] = x.y;
    }
    auto put = [&](float *dst) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            *reinterpret_cast<float2 *>(dst + u * kN) = make_float2(G[u][0], G[u][1]);
    };
    if (T == 0) {  // no tokens: the gradient passes through
        put(p.d_state_in + sbase);
        return;
    }

    // staging of chunk c, without a branch: key-side piece n = tid + 256 q lies in tensor
    // n / PPTEN (uniform over the wave); tokens are clamped into the sequence (past T
    // they are never read)
    auto tensor = [&](int x) -> u64 {  // x is a constant after unrolling
        return reinterpret_cast<u64>(x == 0 ? p.r : x == 1 ? p.w : x == 2 ? p.a : p.b);
    };
    constexpr int WPT = SG::PPTEN / 64;  // waves per tensor in one slot
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    u32x4 stg[SG::KPT], sdo;  // raw bits: widened when stored to LDS, so no load is waited for early
    auto stage_load = [&](int c) {
#pragma unroll
        for (int q = 0; q < SG::KPT; ++q) {
            const int n = static_cast<int>(threadIdx.x) + q * GNW * 64, rem = n % SG::PPTEN;
            const int tau = rem / (kN / SG::EPP), col = (rem % (kN / SG::EPP)) * SG::EPP;
            const int t = min(c * CC + tau, T - 1);
            // slot q's first tensor is a constant; the wave's is that one or the next
            constexpr int per_slot = GNW / WPT;
            const int ten0 = q * per_slot;
            const u64 base = (per_slot > 1 && wv >= WPT) ? tensor(ten0 + 1) : tensor(ten0);
            const GLOBAL_AS Tin *src = reinterpret_cast<const GLOBAL_AS Tin *>(base) + head_e +
                                       static_cast<size_t>(t) * tok_e + col;
            stg[q] = *reinterpret_cast<const GLOBAL_AS u32x4 *>(src);
        }
        const int m = threadIdx.x & 127, tau = m / (GCOL / 4), col = (m % (GCOL / 4)) * 4;
        const int t = min(c * CC + tau, T - 1);
        sdo = *reinterpret_cast<const GLOBAL_AS u32x4 *>(reinterpret_cast<const GLOBAL_AS float *>(
                                                              reinterpret_cast<u64>(p.d_o)) +
                                                          head_e + static_cast<size_t>(t) * tok_e + half * GCOL + col);
    };
    auto stage_store = [&](int c) {
        const int bsel = c & 1;
#pragma unroll
        for (int q = 0; q < SG::KPT; ++q) {
            const int n = static_cast<int>(threadIdx.x) + q * GNW * 64;
            const int ten = n / SG::PPTEN, rem = n % SG::PPTEN;
            const int tau = rem / (kN / SG::EPP), col = (rem % (kN / SG::EPP)) * SG::EPP;
            float *const dst = &sm.in[bsel][ten][tau][col];
            if constexpr (sizeof(Tin) == 2) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    *reinterpret_cast<f32x4 *>(dst + 4 * h) =
                        f32x4{__uint_as_float(stg[q][2 * h] << 16), __uint_as_float(stg[q][2 * h] & 0xffff0000u),
                              __uint_as_float(stg[q][2 * h + 1] << 16),
                              __uint_as_float(stg[q][2 * h + 1] & 0xffff0000u)};
            } else {
                *reinterpret_cast<u32x4 *>(dst) = stg[q];
            }
        }
        const int m = threadIdx.x & 127, tau = m / (GCOL / 4), col = (m % (GCOL / 4)) * 4;
        *reinterpret_cast<u32x4 *>(&sm.dout[bsel][tau][col]) = sdo;
    };
    // G_end goes to tensor r0 / 16 of dr, dk, da, db: a per-lane choice, made once
    const int sidx = r0 / CC;
    const u64 gbase = pick(sidx == 0, reinterpret_cast<u64>(p.dr),
                           pick(sidx == 1, reinterpret_cast<u64>(p.dk),
                                pick(sidx == 2, reinterpret_cast<u64>(p.da), reinterpret_cast<u64>(p.db))));
    GLOBAL_AS float *const gdst = reinterpret_cast<GLOBAL_AS float *>(gbase) + head_e + (r0 % CC) * tok_e + j;
    // a token's r, w, a, b at this lane's four keys and dO at its two columns
    struct Tok {
        f32x4 r, w, a, b;
        float2 d;
    };
    auto read_tok = [&](int bsel, int tau) {
        Tok x;
        x.r = *reinterpret_cast<const f32x4 *>(&sm.in[bsel][0][tau][r0]);
        x.w = *reinterpret_cast<const f32x4 *>(&sm.in[bsel][1][tau][r0]);
        x.a = *reinterpret_cast<const f32x4 *>(&sm.in[bsel][2][tau][r0]);
        x.b = *reinterpret_cast<const f32x4 *>(&sm.in[bsel][3][tau][r0]);
        x.d = *reinterpret_cast<const float2 *>(&sm.dout[bsel][tau][jw]);
        return x;
    };

    stage_load(nck - 1);
    stage_store(nck - 1);
    __syncthreads();
    for (int c = nck - 1; c >= 0; --c) {
        const int bsel = c & 1;
        if (c > 0)
            stage_load(c - 1);  // in flight during this chunk
        if (c < nck - 1) {
            // G_end of chunk c: key row 16 s + tau goes to token 16 c + tau of tensor s
            GLOBAL_AS float *const dst = gdst + static_cast<size_t>(c * CC) * tok_e;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                *reinterpret_cast<GLOBAL_AS f32x2 *>(dst + u * tok_e) = f32x2{G[u][0], G[u][1]};
        }
        const int t_hi = min(T, (c + 1) * CC) - 1, t_lo = c * CC;
        Tok cur = read_tok(bsel, t_hi - t_lo);
        for (int t = t_hi; t >= t_lo; --t) {
            const Tok nxt = read_tok(bsel, max(t - 1 - t_lo, 0));
            float pc0 = 0.f, pc1 = 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                G[u][0] = fmaf(cur.r[u], cur.d.x, G[u][0]);
                G[u][1] = fmaf(cur.r[u], cur.d.y, G[u][1]);
                pc0 = fmaf(cur.b[u], G[u][0], pc0);
                pc1 = fmaf(cur.b[u], G[u][1], pc1);
            }
            const float c0 = group16_sum(pc0), c1 = group16_sum(pc1);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                G[u][0] = fmaf(cur.w[u], G[u][0], cur.a[u] * c0);
                G[u][1] = fmaf(cur.w[u], G[u][1], cur.a[u] * c1);
            }
            cur = nxt;
        }
        if (c > 0) {
            stage_store(c - 1);  // the other buffer: chunk c + 1 used it, long finished
            __syncthreads();
        }
    }
    put(p.d_state_in + sbase);
}

// ---------------------------------------------------------------------------------
// The chunk kernel: one workgroup of four waves per (chunk, batch, head).  S^ and G^
// never enter LDS: each lane loads the parts of S0 and G_end that its own matrix-core
// products take (a row segment and a column segment of each), so three workgroups
// share a compute unit.
constexpr int RS = kN + 1;  // row stride of the LDS matrices (column reads hit distinct banks)
// row stride of the 16 x 16 matrices: rows 16-byte aligned, and a column read by 16
// lanes (or a column per lane group) hits distinct banks
constexpr int SS = CC + 4;

// The 16 x 64 matrices.  dR0 = dO S^T, dA0 = dX S^T, dBz = Z G^T and dKv = V G^T (the
// first terms of dR', dA', dB', dK', kept for the decay gradient) take the places of dO,
// dX, Z and V once those are no longer read.
enum Row { X_R, X_W, X_K, X_V, X_A, X_B, X_DO, X_Z, X_DX, NROW };
constexpr int X_DR0 = X_DO, X_DA0 = X_DX, X_DBZ = X_Z, X_DKV = X_V;
// The 16 x 16 matrices: T is formed over M_ab; dM_rb = tril(dO Z^T), dM_ab = tril(dX Z^T, -1)
// and dM_ak = tril(dX V^T, -1) (also the token-pair products of the decay gradient) over
// M_ak, M_rb and M_rk; dM_rk = tril(dO V^T) has a slot of its own.
enum Small { M_AB, M_AK, M_RB, M_RK, W_OV, NSMALL };
constexpr int M_T = M_AB, W_OZ = M_AK, W_XZ = M_RB, W_XV = M_RK;

// 44.4 KB: three workgroups share a compute unit.
struct ChunkSmem {
    float rows[NROW][CC][RS];  // 16 x 64 matrices (tokens x channels)
    alignas(16) float sm[NSMALL][CC][SS];  // 16 x 16 matrices
    alignas(16) float p7[kN];  // P_7 per key
    alignas(16) float d15[kN]; // d_15 per key
    alignas(16) int flag[4];   // per wave: a decay below 2^-15 in its quarter of the chunk
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// x[4 q + e] for a per-lane q in 0 .. 3 (three selects; no table)
__device__ __forceinline__ float sel4(int q, float x0, float x1, float x2, float x3)
{
    return (q & 2) ? ((q & 1) ? x3 : x2) : ((q & 1) ? x1 : x0);
}

// T = (I - M)^{-1} for a strictly lower triangular 16 x 16 M (in LDS, rows of SS), by one
// wave.  M^16 = 0, so T = I + M + ... + M^15 = (I + M8)(I + M4)(I + M2)(I + M) (the
// factors commute): six products on the matrix cores instead of a row-by-row solve.  A
// product X Y takes X as the A operand (lane (q, n): X[n][4 q + i]) and Y in the
// accumulator layout (lane (q, n): Y[4 q + e][n]); a power needed as an A operand passes
// through m, which is overwritten.  T is written to t (m itself allowed).
__device__ __forceinline__ void unit_lower_inverse(float (*m)[SS], float (*t)[SS], int lane)
{
    const int q = lane >> 4, n = lane & 15;
    float am[4], cm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        am[i] = m[n][4 * q + i];
        cm[i] = m[4 * q + i][n];
    }
    auto prod = [&](const float (&a)[4], const f32x4 &c0, const float (&bm)[4]) {
        f32x4 acc = c0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = mfma4(a[i], bm[i], acc);
        return acc;
    };
    auto as_a = [&](const f32x4 &c, float (&a)[4]) {  // accumulator layout -> A operand
#pragma unroll
        for (int e = 0; e < 4; ++e)
            m[4 * q + e][n] = c[e];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = m[n][4 * q + i];
    };
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    float a2[4], a4[4], a8[4];
    const f32x4 c2 = prod(am, zero, cm);  // M^2
    as_a(c2, a2);
    const float c2v[4] = {c2[0], c2[1], c2[2], c2[3]};
    const f32x4 c4 = prod(a2, zero, c2v);  // M^4
    as_a(c4, a4);
    const float c4v[4] = {c4[0], c4[1], c4[2], c4[3]};
    const f32x4 c8 = prod(a4, zero, c4v);  // M^8
    as_a(c8, a8);
    // R = I + M, then R += M2 R, R += M4 R, R += M8 R
    float r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        r[e] = cm[e] + (4 * q + e == n ? 1.f : 0.f);
    f32x4 rc = {r[0], r[1], r[2], r[3]};
    rc = prod(a2, rc, r);
    const float r2[4] = {rc[0], rc[1], rc[2], rc[3]};
    rc = prod(a4, rc, r2);
    const float r4[4] = {rc[0], rc[1], rc[2], rc[3]};
    rc = prod(a8, rc, r4);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        t[4 * q + e][n] = rc[e];
}

// The exact path of a chunk with a decay below 2^-15 (w = 0 included): the recurrence
// itself.  Lane (q, m) of wave wv holds columns 16 q .. 16 q + 15 of key row 16 wv + m
// of S and of G (the raw S0 and G_end are passed in).  A forward sweep forms
// z_tau = S_{tau-1}^T a_tau (kept in LDS); then, going back over the tokens, S_{t-1} and
// S_t are replayed from the checkpoint with those z (no more column sums), and each
// token's gradients are those of the recurrent adjoint:
//     dr = S_t dO_t, dk = G v_t, dw = rowsum(G * S_{t-1}), db = G z_t,
//     c = G^T b_t, dv = G^T k_t, da = S_{t-1} c, then G <- diag(w_t) G + a_t c^T.
// The raw inputs are in LDS (no factors were applied).
__device__ void exact_chunk(const BwdArgs &p, ChunkSmem &sm, int t0, int L, size_t head_e, size_t tok_e,
                            const float (&S0r)[16], const float (&Gin)[16])
{
    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, m = lane & 15;
    const int wv = tid >> 6, i = 16 * wv + m, j0 = 16 * q;
    float *const part = &sm.sm[M_AB][0][0];  // [4 waves][64 columns] partial column sums
    float *const cvec = &sm.sm[W_OZ][0][0], *const dvvec = &sm.sm[W_OV][0][0];
    auto zrow = [&](int tau) { return &sm.rows[X_Z][tau][0]; };
    // the sum over the 64 key rows of f x (this lane's 16 columns): over the 16 rows of
    // the wave by shuffles, then over the four waves in LDS
    auto colsum = [&](float f, const float (&x)[16], float *dst) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            float v = f * x[jj];
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 4);
            v += __shfl_xor(v, 8);
            if (m == 0)
                part[wv * kN + j0 + jj] = v;
        }
        __syncthreads();
        if (tid < kN)
            dst[tid] = (part[tid] + part[kN + tid]) + (part[2 * kN + tid] + part[3 * kN + tid]);
        __syncthreads();
    };
    auto rsum = [](float x) {  // over the four column quarters of the row
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        return x;
    };
    float G[16];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
        G[jj] = Gin[jj];
    auto step = [&](int u, float (&S)[16]) {
        const float wu = sm.rows[X_W][u][i], bu = sm.rows[X_B][u][i], ku = sm.rows[X_K][u][i];
        const float *z = zrow(u);
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
            S[jj] = fmaf(wu, S[jj], fmaf(bu, z[j0 + jj], ku * sm.rows[X_V][u][j0 + jj]));
    };
    {
        float S[16];
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
            S[jj] = S0r[jj];
        for (int tau = 0; tau < L; ++tau) {
            colsum(sm.rows[X_A][tau][i], S, zrow(tau));
            step(tau, S);
        }
    }
    for (int t = L - 1; t >= 0; --t) {
        const float rt = sm.rows[X_R][t][i], wt = sm.rows[X_W][t][i], at = sm.rows[X_A][t][i];
        const float bt = sm.rows[X_B][t][i], kt = sm.rows[X_K][t][i];
        const float *z = zrow(t);
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
            G[jj] = fmaf(rt, sm.rows[X_DO][t][j0 + jj], G[jj]);
        float Sp[16], St[16];
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
            Sp[jj] = S0r[jj];
        for (int u = 0; u < t; ++u)
            step(u, Sp);
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
            St[jj] = Sp[jj];
        step(t, St);
        float s_dr = 0.f, s_dk = 0.f, s_dw = 0.f, s_db = 0.f;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            const int j = j0 + jj;
            s_dr = fmaf(St[jj], sm.rows[X_DO][t][j], s_dr);
            s_dk = fmaf(G[jj], sm.rows[X_V][t][j], s_dk);
            s_dw = fmaf(G[jj], Sp[jj], s_dw);
            s_db = fmaf(G[jj], z[j], s_db);
        }
        s_dr = rsum(s_dr);
        s_dk = rsum(s_dk);
        s_dw = rsum(s_dw);
        s_db = rsum(s_db);
        colsum(bt, G, cvec);
        colsum(kt, G, dvvec);
        float s_da = 0.f;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
            s_da = fmaf(Sp[jj], cvec[j0 + jj], s_da);
        s_da = rsum(s_da);
        const size_t row = head_e + static_cast<size_t>(t0 + t) * tok_e;
        if (q == 0) {
            p.dr[row + i] = s_dr;
            p.dk[row + i] = s_dk;
            p.dw[row + i] = s_dw;
            p.db[row + i] = s_db;
            p.da[row + i] = s_da;
        }
        if (tid < kN)
            p.dv[row + tid] = dvvec[tid];
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
            G[jj] = fmaf(wt, G[jj], at * cvec[j0 + jj]);
    }
}

template <typename Tin>
__global__ __launch_bounds__(256, 3) void wkv7_bwdc_chunk_kernel(BwdArgs p, int c_lo, int nbh)
{
    __shared__ ChunkSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, m = lane & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tc = 16 * wv + m;  // this lane's key: its column of every 16 x 64 tile
    const int c = c_lo + static_cast<int>(blockIdx.x) / nbh;
    const int bh = static_cast<int>(blockIdx.x) % nbh;
    const int H = p.H, T = p.T;
    const int bb = bh / H, hh = bh - bb * H;
    const int nck = (T + CC - 1) / CC;
    const int t0 = c * CC, L = min(CC, T - t0);
    const size_t tok_e = static_cast<size_t>(H) * kN;
    const size_t head_e = static_cast<size_t>(bb) * T * tok_e + static_cast<size_t>(hh) * kN;
    auto rowp = [&](int tau) { return head_e + static_cast<size_t>(t0 + min(tau, L - 1)) * tok_e; };

    // ---- load.  Of the checkpoint S0 and G_end this lane takes row tc, columns
    // 16 q .. 16 q + 15 (the B operand of the products against S^T and G^T), loaded first,
    // and column tc, rows 16 q .. 16 q + 15 (the B operand of the products against S^ and
    // G^), loaded once the chunk is known to take the factor path.  Row u of G_end's
    // block sb (rows 16 sb .. 16 sb + 15) is, for an inner chunk, token t0 + u of dr, dk,
    // da, db (sb = 0 .. 3); for the last chunk, row 16 sb + u of d_state_out (a missing
    // d_state_out reads the checkpoint and is zeroed).  The inputs go to LDS (tokens past
    // the end as identity steps: w = 1, the rest 0), with dO.
    float srow[16], scol[16], grow[16], gcol[16];
    const bool inner = c < nck - 1, has_g = inner || p.d_state_out != nullptr;
    u64 scol_a, gcol_a, gstride;
    {
        const u64 s0 = reinterpret_cast<u64>(p.ckpt) + 4ull * (((static_cast<size_t>(bb) * nck + c) * H + hh) * (kN * kN));
        gstride = inner ? 4ull * tok_e : 4ull * kN;
        const u64 ginner = 4ull * (head_e + static_cast<size_t>(t0) * tok_e);
        const u64 glast = p.d_state_out ? reinterpret_cast<u64>(p.d_state_out) + 4ull * static_cast<size_t>(bh) * (kN * kN)
                                        : s0;
        // block wv (uniform over the wave) for the row segment, block q for the column one
        u64 grb;
        if (inner) {
            const void *const t = wv == 0 ? p.dr : (wv == 1 ? p.dk : (wv == 2 ? p.da : p.db));
            grb = reinterpret_cast<u64>(t) + ginner;
        } else {
            grb = glast + 4ull * CC * kN * wv;
        }
        const u64 gcb = inner ? pick(q == 0, reinterpret_cast<u64>(p.dr),
                                     pick(q == 1, reinterpret_cast<u64>(p.dk),
                                          pick(q == 2, reinterpret_cast<u64>(p.da), reinterpret_cast<u64>(p.db)))) +
                                    ginner
                              : glast + 4ull * CC * kN * q;
        // the checkpoint in tile order: the row segment is 16 values 16 bytes apart, the
        // column segment four 16-byte units 256 bytes apart
        const u64 srow_a = s0 + 4ull * ckpt_offset(tc, 16 * q);
        const u64 grow_a = grb + m * gstride + 4ull * 16 * q;
        scol_a = s0 + 4ull * ckpt_offset(16 * q, tc);
        gcol_a = gcb + 4ull * tc;
#pragma unroll
        for (int h4 = 0; h4 < 4; ++h4) {
            const f32x4 gv = *reinterpret_cast<const GLOBAL_AS f32x4 *>(grow_a + 16u * h4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                srow[4 * h4 + e] = *reinterpret_cast<const GLOBAL_AS float *>(srow_a + 16u * (4 * h4 + e));
                grow[4 * h4 + e] = gv[e];
            }
        }

        const int tau = tid >> 4, col = (tid & 15) * 4;
        const bool live = tau < L;
        const Tin *const srcs[6] = {static_cast<const Tin *>(p.r), static_cast<const Tin *>(p.w),
                                    static_cast<const Tin *>(p.k), static_cast<const Tin *>(p.v),
                                    static_cast<const Tin *>(p.a), static_cast<const Tin *>(p.b)};
        f32x4 in4[6], o4;
#pragma unroll
        for (int x = 0; x < 6; ++x)
            in4[x] = load4w(srcs[x] + rowp(tau) + col);
        o4 = load4w(p.d_o + rowp(tau) + col);

        // the rows past the end by masks the compiler cannot turn into branches (a load
        // moved under one is waited for at once)
        unsigned keep = live ? ~0u : 0u;
        asm volatile("" : "+v"(keep));
        auto mask = [&](float v, float dflt) {
            return __uint_as_float((__float_as_uint(v) & keep) | (__float_as_uint(dflt) & ~keep));
        };
        bool tiny = false;
#pragma unroll
        for (int x = 0; x < 6; ++x) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = mask(in4[x][e], x == X_W ? 1.f : 0.f);
                sm.rows[x][tau][col + e] = v;
                if (x == X_W)
                    tiny = tiny || !(fabsf(v) >= kExactBelow);  // NaN included
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            sm.rows[X_DO][tau][col + e] = mask(o4[e], 0.f);
        const bool any_tiny = __ballot(tiny) != 0ull;
        if (lane == 0)
            sm.flag[wv] = any_tiny ? 1 : 0;
    }
    __syncthreads();
    if ((sm.flag[0] | sm.flag[1] | sm.flag[2] | sm.flag[3]) != 0) {
        if (!has_g)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj)
                grow[jj] = 0.f;
        exact_chunk(p, sm, t0, L, head_e, tok_e, srow, grow);
        return;
    }
#pragma unroll
    for (int h4 = 0; h4 < 4; ++h4) {
        const f32x4 sv = *reinterpret_cast<const GLOBAL_AS f32x4 *>(scol_a + 256u * h4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            scol[4 * h4 + e] = sv[e];
    }
#pragma unroll
    for (int ii = 0; ii < 16; ++ii)
        gcol[ii] = *reinterpret_cast<const GLOBAL_AS float *>(gcol_a + gstride * ii);

    // ---- decay factors of key tc (each lane of the key forms all 16), applied to this
    // lane's tokens 4 q .. 4 q + 3 of r, a, b, k
    float dq[4], dpq[4], iq[4];  // d, d_{tau-1} and 1/d at this lane's tokens
    float p7, d15;
    {
        float wcol[CC], xr[4], xa[4], xb[4], xk[4];
        // every read before the first write (see the chain's factors)
#pragma unroll
        for (int tau = 0; tau < CC; ++tau)
            wcol[tau] = sm.rows[X_W][tau][tc];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xr[e] = sm.rows[X_R][4 * q + e][tc];
            xa[e] = sm.rows[X_A][4 * q + e][tc];
            xb[e] = sm.rows[X_B][4 * q + e][tc];
            xk[e] = sm.rows[X_K][4 * q + e][tc];
        }
        float d[CC];
        d[REF] = 1.0f;
#pragma unroll
        for (int tau = REF + 1; tau < CC; ++tau)
            d[tau] = d[tau - 1] * wcol[tau];
#pragma unroll
        for (int tau = REF - 1; tau >= 0; --tau)
            d[tau] = d[tau + 1] * __builtin_amdgcn_rcpf(wcol[tau + 1]);
        float pr = wcol[0];
#pragma unroll
        for (int tau = 1; tau <= REF; ++tau)
            pr *= wcol[tau];
        p7 = pr;
        d15 = d[CC - 1];
        if (q == 0) {
            sm.p7[tc] = pr;
            sm.d15[tc] = d15;
        }
        const float dm1 = d[0] * __builtin_amdgcn_rcpf(wcol[0]);  // d_{-1}: the factor of a at the first token
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dq[e] = sel4(q, d[e], d[4 + e], d[8 + e], d[12 + e]);
            dpq[e] = sel4(q, e == 0 ? dm1 : d[e - 1], d[3 + e], d[7 + e], d[11 + e]);
            iq[e] = __builtin_amdgcn_rcpf(dq[e]);
            const int tau = 4 * q + e;
            sm.rows[X_R][tau][tc] = xr[e] * dq[e];
            sm.rows[X_A][tau][tc] = xa[e] * dpq[e];
            sm.rows[X_B][tau][tc] = xb[e] * iq[e];
            sm.rows[X_K][tau][tc] = xk[e] * iq[e];
        }
    }
    __syncthreads();

    // ---- S^ = diag(P_7) S0, G^ = diag(d_15) G_end on this lane's segments, and
    // rowsum(G^ * S^) of key tc (over the four lanes of the row)
    float gs_sum;
    {
        if (!has_g)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                grow[jj] = 0.f;
                gcol[jj] = 0.f;
            }
        float acc = 0.f;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            srow[jj] *= p7;
            grow[jj] *= d15;
            acc = fmaf(grow[jj], srow[jj], acc);
        }
        acc += __shfl_xor(acc, 16);
        gs_sum = acc + __shfl_xor(acc, 32);
#pragma unroll
        for (int h4 = 0; h4 < 4; ++h4) {
            const f32x4 pv = *reinterpret_cast<const f32x4 *>(&sm.p7[16 * q + 4 * h4]);
            const f32x4 dv = *reinterpret_cast<const f32x4 *>(&sm.d15[16 * q + 4 * h4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                scol[4 * h4 + e] *= pv[e];
                gcol[4 * h4 + e] *= dv[e];
            }
        }
    }

    // ---- matrix-core fragments (16x16x4 fp32: lane (q, m) supplies A[m][k] and B[k][m]
    // for k = 16 q + i over a 64-long sum, k = 4 q + i over a 16-long one; the result
    // holds rows 4 q + e of column m).  Wave wv owns column tile wv of every 16 x 64 result.
    auto frag_rows = [&](int x, float (&f)[16]) {  // X[m][16 q + i] (also X^T as a B operand)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            f[i] = sm.rows[x][m][16 * q + i];
    };
    auto frag_tile = [&](int x, float (&f)[4]) {  // X[4 q + i][16 wv + m]: B over tokens
#pragma unroll
        for (int i = 0; i < 4; ++i)
            f[i] = sm.rows[x][4 * q + i][tc];
    };
    // a 16 x 16 matrix as the A operand over tokens, optionally transposed (every one is
    // stored with its mask applied)
    auto frag_small = [&](int sx, bool trans, float (&f)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kk = 4 * q + i, row = trans ? kk : m, col = trans ? m : kk;
            f[i] = sm.sm[sx][row][col];
        }
    };
    auto mm64 = [](f32x4 &acc, const float (&a)[16], const float (&b)[16]) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            acc = mfma4(a[i], b[i], acc);
    };
    auto mm16 = [](f32x4 &acc, const float (&a)[4], const float (&b)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = mfma4(a[i], b[i], acc);
    };
    auto to_rows = [&](int x, const f32x4 &acc) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            sm.rows[x][4 * q + e][tc] = acc[e];
    };
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    float fa[16], fb[16], a4[4], b4[4];

    // ---- M_ab, M_ak (strict), M_rb, M_rk: one per wave
    {
        const int xa = wv < 2 ? X_A : X_R, xb = (wv & 1) ? X_K : X_B;
        frag_rows(xa, fa);
        frag_rows(xb, fb);
        f32x4 acc = zero4;
        mm64(acc, fa, fb);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tau = 4 * q + e;
            const bool keep = wv < 2 ? m < tau : m <= tau;  // entries above are dropped (they
            sm.sm[wv][tau][m] = keep ? acc[e] : 0.f;        // may have overflowed)
        }
    }
    // ---- this wave's tiles of X = A' S^, dZ = B' G^, dV = K' G^, dR0 = dO S^T, dKv = V G^T
    f32x4 xacc = zero4, dzacc = zero4, dvacc = zero4, dracc = zero4, dkacc = zero4;
    frag_rows(X_A, fa);
    mm64(xacc, fa, scol);
    frag_rows(X_B, fa);
    mm64(dzacc, fa, gcol);
    frag_rows(X_K, fa);
    mm64(dvacc, fa, gcol);
    frag_rows(X_DO, fa);
    mm64(dracc, fa, srow);
    frag_rows(X_V, fa);
    mm64(dkacc, fa, grow);
    __syncthreads();

    // ---- the 16-long products that need the M's; T = (I - M_ab)^{-1} (wave 0); dO V^T
    // (wave 1)
    frag_tile(X_V, b4);
    frag_small(M_AK, false, a4);
    mm16(xacc, a4, b4);      // X += M_ak V
    frag_tile(X_DO, b4);
    frag_small(M_RB, true, a4);
    mm16(dzacc, a4, b4);     // dZ += M_rb^T dO
    frag_small(M_RK, true, a4);
    mm16(dvacc, a4, b4);     // dV += M_rk^T dO
    if (wv == 0) {
        unit_lower_inverse(sm.sm[M_AB], sm.sm[M_T], lane);  // T over M_ab
    } else if (wv == 1) {
        frag_rows(X_DO, fa);
        frag_rows(X_V, fb);
        f32x4 acc = zero4;
        mm64(acc, fa, fb);
#pragma unroll
        for (int e = 0; e < 4; ++e)  // stored as dM_rk: lower triangle with the diagonal
            sm.sm[W_OV][4 * q + e][m] = m <= 4 * q + e ? acc[e] : 0.f;
    }
    __syncthreads();

    // ---- Z = T X, dX = T^T dZ (the B operands are this lane's own rows), dV += M_ak^T dX
    f32x4 zacc = zero4, dxacc = zero4;
    {
        float xb4[4] = {xacc[0], xacc[1], xacc[2], xacc[3]};
        float zb4[4] = {dzacc[0], dzacc[1], dzacc[2], dzacc[3]};
        frag_small(M_T, false, a4);
        mm16(zacc, a4, xb4);
        frag_small(M_T, true, a4);
        mm16(dxacc, a4, zb4);
        float db4[4] = {dxacc[0], dxacc[1], dxacc[2], dxacc[3]};
        frag_small(M_AK, true, a4);
        mm16(dvacc, a4, db4);
    }
    to_rows(X_Z, zacc);
    to_rows(X_DX, dxacc);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (4 * q + e < L)
            p.dv[rowp(4 * q + e) + tc] = dvacc[e];
    __syncthreads();

    // ---- dO Z^T (wave 0), dX Z^T (wave 2), dX V^T (wave 3); dA0 = dX S^T, dBz = Z G^T
    if (wv != 1) {
        frag_rows(wv == 0 ? X_DO : X_DX, fa);
        frag_rows(wv == 3 ? X_V : X_Z, fb);
        f32x4 acc = zero4;
        mm64(acc, fa, fb);
        const int dst = wv == 0 ? W_OZ : (wv == 2 ? W_XZ : W_XV);
        // stored as dM_rb (lower triangle with the diagonal), dM_ab and dM_ak (strict)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tau = 4 * q + e;
            sm.sm[dst][tau][m] = (wv == 0 ? m <= tau : m < tau) ? acc[e] : 0.f;
        }
    }
    f32x4 daacc = zero4, dbacc = zero4;
    frag_rows(X_DX, fa);
    mm64(daacc, fa, srow);
    frag_rows(X_Z, fa);
    mm64(dbacc, fa, grow);
    __syncthreads();
    // dO, dX, Z and V are read no more: their places take dR0, dA0, dBz, dKv
    to_rows(X_DR0, dracc);
    to_rows(X_DA0, daacc);
    to_rows(X_DBZ, dbacc);
    to_rows(X_DKV, dkacc);

    // ---- dR' = dR0 + dM_rb B' + dM_rk K',  dA' = dA0 + dM_ab B' + dM_ak K',
    //      dB' = dBz + dM_ab^T A' + dM_rb^T R',  dK' = dKv + dM_ak^T A' + dM_rk^T R'
    // (dM_rb, dM_rk: dO Z^T, dO V^T with the diagonal; dM_ab, dM_ak: dX Z^T, dX V^T strict;
    // stored masked)
    frag_tile(X_B, b4);
    frag_small(W_OZ, false, a4);
    mm16(dracc, a4, b4);
    frag_small(W_XZ, false, a4);
    mm16(daacc, a4, b4);
    frag_tile(X_K, b4);
    frag_small(W_OV, false, a4);
    mm16(dracc, a4, b4);
    frag_small(W_XV, false, a4);
    mm16(daacc, a4, b4);
    frag_tile(X_A, b4);
    frag_small(W_XZ, true, a4);
    mm16(dbacc, a4, b4);
    frag_small(W_XV, true, a4);
    mm16(dkacc, a4, b4);
    frag_tile(X_R, b4);
    frag_small(W_OZ, true, a4);
    mm16(dbacc, a4, b4);
    frag_small(W_OV, true, a4);
    mm16(dkacc, a4, b4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (4 * q + e < L) {
            const size_t at = rowp(4 * q + e) + tc;
            p.dr[at] = dracc[e] * dq[e];
            p.da[at] = daacc[e] * dpq[e];
            p.db[at] = dbacc[e] * iq[e];
            p.dk[at] = dkacc[e] * iq[e];
        }
    }

    // ---- dw, in its direct form.  With Q_s(t) = sum_{u<t} (B'_u dO_s.z_u + K'_u dO_s.v_u)
    // and P_s(t) the same with dX_s, per key:
    //   w_t dw_t = rowsum(G^ * S^) + sum_{u<t} (B'_u dBz_u + K'_u dKv_u)
    //            + sum_{s>=t} R'_s (dR0_s + Q_s(t)) + sum_{s>t} A'_s (dA0_s + P_s(t)).
    // Lane (q, m) forms the Q/P terms of key tc for the rows s = 4 j + q; the four
    // partials meet by shuffles.  Everything it reads is column tc, which this wave wrote
    // (or the 16 x 16 matrices, complete since the last barrier): no barrier here.
    {
        const int i = tc;
        float bu[CC], ku[CC], acc[CC];
#pragma unroll
        for (int u = 0; u < CC; ++u) {
            bu[u] = sm.rows[X_B][u][i];
            ku[u] = sm.rows[X_K][u][i];
            acc[u] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s = 4 * j + q;
            const float rs = sm.rows[X_R][s][i], as = sm.rows[X_A][s][i];
            // row s of the four token-pair matrices, entries 0 .. 4 j + 3, four at a time
            f32x4 oz[4], ov[4], xz[4], xv[4];
#pragma unroll
            for (int h = 0; h <= j; ++h) {
                oz[h] = *reinterpret_cast<const f32x4 *>(&sm.sm[W_OZ][s][4 * h]);
                ov[h] = *reinterpret_cast<const f32x4 *>(&sm.sm[W_OV][s][4 * h]);
                xz[h] = *reinterpret_cast<const f32x4 *>(&sm.sm[W_XZ][s][4 * h]);
                xv[h] = *reinterpret_cast<const f32x4 *>(&sm.sm[W_XV][s][4 * h]);
            }
            float qr = 0.f, qa = 0.f;
            // t runs to the largest s of the four lanes; past this lane's s the terms are
            // formed and dropped (selects, so a non-finite dropped term does no harm)
#pragma unroll
            for (int t = 1; t <= 4 * j + 3; ++t) {
                const int u = t - 1;
                qr = fmaf(bu[u], oz[u >> 2][u & 3], fmaf(ku[u], ov[u >> 2][u & 3], qr));
                qa = fmaf(bu[u], xz[u >> 2][u & 3], fmaf(ku[u], xv[u >> 2][u & 3], qa));
                const float cr = fmaf(rs, qr, acc[t]);
                const float ca = fmaf(as, qa, cr);
                acc[t] = t < s ? ca : (t == s ? cr : acc[t]);
            }
        }
        // The four lanes of key tc (lanes m + 16 q) hold partials of acc[t] over their rows
        // s.  A reduce-scatter leaves lane q the sums of its own tokens 4 q .. 4 q + 3: the
        // lane pairs q, q ^ 2 exchange token halves, then q, q ^ 1 token quarters.
        const bool hi2 = (q & 2) != 0, hi1 = (q & 1) != 0;
        float h8[8], mine[4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float keep = hi2 ? acc[8 + e] : acc[e], send = hi2 ? acc[e] : acc[8 + e];
            h8[e] = keep + __shfl_xor(send, 32);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float keep = hi1 ? h8[4 + e] : h8[e], send = hi1 ? h8[e] : h8[4 + e];
            mine[e] = keep + __shfl_xor(send, 16);
        }
        // This lane's tokens' R'_t dR0_t, A'_t dA0_t and B'_t dBz_t + K'_t dKv_t; the
        // suffix over s >= t (s > t for the A' terms) and the prefix over u < t run across
        // the four lanes' blocks by shuffles, then inside the block.
        float rd[4], ad[4], bk[4];
        float ra = 0.f, bks = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 4 * q + e;
            rd[e] = sm.rows[X_R][t][i] * sm.rows[X_DR0][t][i];
            ad[e] = sm.rows[X_A][t][i] * sm.rows[X_DA0][t][i];
            bk[e] = fmaf(sm.rows[X_B][t][i], sm.rows[X_DBZ][t][i], sm.rows[X_K][t][i] * sm.rows[X_DKV][t][i]);
            ra += rd[e] + ad[e];
            bks += bk[e];
        }
        float sr = 0.f, pr = gs_sum;
#pragma unroll
        for (int d = 1; d < 4; ++d) {
            const float up = __shfl(ra, (lane + 16 * d) & 63), down = __shfl(bks, (lane - 16 * d) & 63);
            sr += q + d < 4 ? up : 0.f;
            pr += q - d >= 0 ? down : 0.f;
        }
        float suf[4];
#pragma unroll
        for (int e = 3; e >= 0; --e) {
            sr += rd[e];
            suf[e] = sr;
            sr += ad[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 4 * q + e;
            const float tot = (pr + suf[e]) + mine[e];
            pr += bk[e];
            if (t < L)
                p.dw[rowp(t) + i] = tot * __builtin_amdgcn_rcpf(sm.rows[X_W][t][i]);
        }
    }
}
// ---------------------------------------------------------------------------------
// The gradient chain in chunk form, on the matrix cores.  One workgroup of eight waves
// per (batch, head).  Chain wave cw (waves 0 .. 3) holds value columns 16 cw .. 16 cw + 15
// of G in the accumulator layout: lane (q, n) holds G[16 pt + 4 q + e][16 cw + n] in
// g[pt][e].  Per chunk, last first:
//     G^ = diag(d_15) G_end,   dZ = B' G^ + M_rb^T dO,   dX = T^T dZ,
//     G_end of the chunk before = diag(P_7) (G^ + R'^T dO + A'^T dX).
// Only B' G^, T^T dZ and A'^T dX depend on G.  The rest is formed a phase or a chunk
// ahead, in two LDS buffers (chunk c in one, chunk c - 1 in the other).  A chunk step is
// two phases and two barriers:
//   phase 1: chain waves: dZ of chunk c, with the factors, A', R', B' of chunk c - 1
//            (from its staged raw rows) formed while the products run.  Prep waves
//            (4 .. 7, one beside each chain wave on its SIMD): T of chunk c (wave 7);
//            R'^T dO of chunk c at the chain waves' columns (waves 4 .. 6);
//   phase 2: chain waves: dX and G of chunk c, stored as G_end of chunk c - 1.  Prep
//            waves: M_ab (wave 4) and M_rb (wave 5) of chunk c - 1; the raw rows of chunk
//            c - 2 staged (their loads were issued a chunk before).
// In dZ = B' G^ a lane's own rows of G^ are its operand: the sum over the keys runs in
// the order (pt, q, e) of the accumulator layout, and B' is read in that order.  A chunk
// with a decay below 2^-15 runs the recurrence token by token instead (chain waves, in
// phase 1, on the raw rows, which the prep waves copied into its buffer).
struct GchainBuf {
    float der[4][CC][RS];   // A', R', B' (raw a, r, b on the exact path) and raw w
    float dout[CC][RS];     // dO (zero past the end)
    alignas(16) float sm[3][CC][SS];  // M_ab, M_rb, T
    alignas(16) float d15[kN];
    alignas(16) float p7[kN];
    int flag[4];            // per chain wave: a decay below 2^-15 among its keys
    float qd[4][16][64];    // R'^T dO of chain wave cw, value 4 pt + e of lane l
};
// 100.7 KB
struct GchainSmem {
    float raw[4][CC][RS];  // r, w, a, b of the chunk being prepared (identity steps past the end)
    GchainBuf buf[2];
};
enum { G_R, G_W, G_A, G_B };
enum { D_A, D_R, D_B, D_W };
enum { S_AB, S_RB, S_T };

template <typename Tin, bool HAS_DOUT>
__global__ __launch_bounds__(512) void wkv7_bwdc_gchain_kernel(BwdArgs p)
{
    __shared__ GchainSmem sm;
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
    using Raw = typename std::conditional<sizeof(Tin) == 2, u32x2, u32x4v>::type;
    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, n = lane & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool chain = wv < 4;
    const int w4 = wv & 3;    // chain wave cw, or the prep wave's place beside it
    const int ptid = tid & 255;
    const int bh = blockIdx.x;
    const int H = p.H, T = p.T;
    const int bb = bh / H, hh = bh - bb * H;
    const int nck = (T + CC - 1) / CC;
    const int col = 16 * w4 + n;  // a chain wave's column (and key, in the factors)
    const size_t tok_e = static_cast<size_t>(H) * kN;
    const size_t head_e = static_cast<size_t>(bb) * T * tok_e + static_cast<size_t>(hh) * kN;
    const size_t sbase = static_cast<size_t>(bh) * (kN * kN) + col;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    float g[4][4];
    auto put_state = [&](float *dst) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dst[sbase + (16 * pt + 4 * q + e) * kN] = g[pt][e];
    };
    if (chain) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                g[pt][e] = HAS_DOUT ? p.d_state_out[sbase + (16 * pt + 4 * q + e) * kN] : 0.0f;
        // the loads complete here: registers still awaiting a load at the loop's head
        // would make every chunk wait on the memory counter, which the G_end stores of
        // the chunk before also hold
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                asm volatile("" : "+v"(g[pt][e]));
        if (T == 0) {  // no tokens: the gradient passes through
            put_state(p.d_state_in);
            return;
        }
    } else if (T == 0) {
        return;
    }

    // staging (prep waves): thread (token ptid / 16, channels 4 (ptid % 16) ..) loads four
    // elements of r, w, a, b and of dO, kept as raw bits until they are stored to LDS
    const int s_tau = ptid >> 4, s_c4 = (ptid & 15) * 4;
    Raw rin[4];
    u32x4v rdo;
    auto stage_load = [&](int c) {
        const int t0 = c * CC, L = min(CC, T - t0);
        const size_t off = head_e + static_cast<size_t>(t0 + min(s_tau, L - 1)) * tok_e + s_c4;
        const Tin *const src[4] = {static_cast<const Tin *>(p.r), static_cast<const Tin *>(p.w),
                                   static_cast<const Tin *>(p.a), static_cast<const Tin *>(p.b)};
#pragma unroll
        for (int x = 0; x < 4; ++x)
            rin[x] = *reinterpret_cast<const GLOBAL_AS Raw *>(
                reinterpret_cast<const GLOBAL_AS Tin *>(reinterpret_cast<u64>(src[x])) + off);
        rdo = *reinterpret_cast<const GLOBAL_AS u32x4v *>(
            reinterpret_cast<const GLOBAL_AS float *>(reinterpret_cast<u64>(p.d_o)) + off);
    };
    auto stage_store = [&](int c, GchainBuf &b) {
        const bool live = s_tau < min(CC, T - c * CC);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            f32x4 v4;
            if constexpr (sizeof(Tin) == 2)
                v4 = f32x4{__uint_as_float(rin[x][0] << 16), __uint_as_float(rin[x][0] & 0xffff0000u),
                           __uint_as_float(rin[x][1] << 16), __uint_as_float(rin[x][1] & 0xffff0000u)};
            else
                v4 = f32x4{__uint_as_float(rin[x][0]), __uint_as_float(rin[x][1]), __uint_as_float(rin[x][2]),
                           __uint_as_float(rin[x][3])};
            if (!live)
                v4 = x == G_W ? f32x4{1.f, 1.f, 1.f, 1.f} : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sm.raw[x][s_tau][s_c4 + e] = v4[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            b.dout[s_tau][s_c4 + e] = live ? __uint_as_float(rdo[e]) : 0.f;
    };
    auto exact_of = [](const GchainBuf &b) { return (b.flag[0] | b.flag[1] | b.flag[2] | b.flag[3]) != 0; };

    // (chain) the factors of the staged chunk, and its A', R', B': lane (q, n) of chain
    // wave cw forms those of key 16 cw + n and writes its tokens 4 q .. 4 q + 3
    auto factors = [&](GchainBuf &b) {
        const int i = col;
        float wc[CC], ra[4], rr[4], rb[4];
        // every read before the first write (LDS writes the compiler cannot tell apart
        // from the reads would make each read wait for the write before it)
#pragma unroll
        for (int tau = 0; tau < CC; ++tau)
            wc[tau] = sm.raw[G_W][tau][i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ra[e] = sm.raw[G_A][4 * q + e][i];
            rr[e] = sm.raw[G_R][4 * q + e][i];
            rb[e] = sm.raw[G_B][4 * q + e][i];
        }
        bool tiny = false;
#pragma unroll
        for (int tau = 0; tau < CC; ++tau)
            tiny = tiny || !(fabsf(wc[tau]) >= kExactBelow);  // NaN included
        const bool any_tiny = __ballot(tiny) != 0ull;
        if (lane == 0)
            b.flag[w4] = any_tiny ? 1 : 0;
        float d[CC];
        d[REF] = 1.0f;
#pragma unroll
        for (int tau = REF + 1; tau < CC; ++tau)
            d[tau] = d[tau - 1] * wc[tau];
#pragma unroll
        for (int tau = REF - 1; tau >= 0; --tau)
            d[tau] = d[tau + 1] * __builtin_amdgcn_rcpf(wc[tau + 1]);
        float pr = wc[0];
#pragma unroll
        for (int tau = 1; tau <= REF; ++tau)
            pr *= wc[tau];
        if (q == 0) {
            b.p7[i] = pr;
            b.d15[i] = d[CC - 1];
        }
        const float dm1 = d[0] * __builtin_amdgcn_rcpf(wc[0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tau = 4 * q + e;
            const float dq = sel4(q, d[e], d[4 + e], d[8 + e], d[12 + e]);
            const float dp = sel4(q, e == 0 ? dm1 : d[e - 1], d[3 + e], d[7 + e], d[11 + e]);
            b.der[D_A][tau][i] = ra[e] * dp;
            b.der[D_R][tau][i] = rr[e] * dq;
            b.der[D_B][tau][i] = rb[e] * __builtin_amdgcn_rcpf(dq);
        }
    };
    // (prep) the exact path keeps the raw rows: this thread copies the elements it
    // staged (and is the one to overwrite them next)
    auto copy_raw = [&](GchainBuf &b) {
        float v[4][4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[0][e] = sm.raw[G_A][s_tau][s_c4 + e];
            v[1][e] = sm.raw[G_R][s_tau][s_c4 + e];
            v[2][e] = sm.raw[G_B][s_tau][s_c4 + e];
            v[3][e] = sm.raw[G_W][s_tau][s_c4 + e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            b.der[D_A][s_tau][s_c4 + e] = v[0][e];
            b.der[D_R][s_tau][s_c4 + e] = v[1][e];
            b.der[D_B][s_tau][s_c4 + e] = v[2][e];
            b.der[D_W][s_tau][s_c4 + e] = v[3][e];
        }
    };
    // (prep) M_ab = tril(A' B'^T, -1) (wave 4), M_rb = tril(R' B'^T) (wave 5)
    auto mprod = [&](GchainBuf &b) {
        if (w4 < 2) {
            const int xa = w4 == 0 ? D_A : D_R;
            f32x4 acc = zero4;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                acc = mfma4(b.der[xa][n][16 * q + i], b.der[D_B][n][16 * q + i], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tau = 4 * q + e;
                const bool keep = w4 == 0 ? n < tau : n <= tau;  // entries above are dropped
                b.sm[w4 == 0 ? S_AB : S_RB][tau][n] = keep ? acc[e] : 0.f;
            }
        }
    };
    // (prep, wave 7) T = (I - M_ab)^{-1} (over M_ab, read no more)
    auto tsolve = [&](GchainBuf &b) { unit_lower_inverse(b.sm[S_AB], b.sm[S_T], lane); };
    // (prep) R'^T dO at chain wave cw's columns, tile by tile (keys 16 pt ..), in its
    // accumulator layout
    auto qprod = [&](GchainBuf &b, int cw) {
        const int qc = 16 * cw + n;
        float dob[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dob[i] = b.dout[4 * q + i][qc];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            f32x4 acc = zero4;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc = mfma4(b.der[D_R][4 * q + i][16 * pt + n], dob[i], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                b.qd[cw][4 * pt + e][lane] = acc[e];
        }
    };

    // ---- prologue: the last chunk prepared in buffer 0, the one before it staged
    int c = nck - 1;
    if (!chain) {
        stage_load(c);
        stage_store(c, sm.buf[0]);
        if (c > 0)
            stage_load(c - 1);
    }
    __syncthreads();
    if (chain)
        factors(sm.buf[0]);
    __syncthreads();
    if (!chain) {
        if (exact_of(sm.buf[0]))
            copy_raw(sm.buf[0]);
        else
            mprod(sm.buf[0]);
        if (c > 0) {
            stage_store(c - 1, sm.buf[1]);
            if (c > 1)
                stage_load(c - 2);
        }
    }
    __syncthreads();

    // The chain waves and the prep waves run loops of their own with the same barriers
    // (two per chunk), so that neither waits on the other's memory operations.
    if (chain) {
        // G_end of chunk c - 1, key row 16 pt + 4 q + e, goes to token 16 (c - 1) + 4 q + e
        // of tensor pt (dr, dk, da, db): byte offsets from this lane's row of token 0
        const u64 e_step = 4ull * tok_e;
        const u64 row0 = 4ull * (head_e + static_cast<size_t>(4 * q) * tok_e + col);
        for (int k = 0; c >= 0; ++k, --c) {
            GchainBuf &cur = sm.buf[k & 1], &nxt = sm.buf[(k & 1) ^ 1];
            // ---- phase 1: G^ = diag(d_15) G;  dZ = B' G^ (keys in the accumulator order)
            // + M_rb^T dO;  then chunk c - 1's factors
            const bool ex = exact_of(cur);
            float gh[4][4], ap[4][4], p7v[4][4];
            f32x4 dz = zero4;
            if (ex) {
                // the recurrence over the chunk's tokens, wave-local: c = G^T b sums the
                // lane's sixteen keys, then the four lanes of the column (lanes n + 16 q)
                const int L = min(CC, T - c * CC);
                for (int t = L - 1; t >= 0; --t) {
                    const float dj = cur.dout[t][col];
                    float cs = 0.f;
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int key = 16 * pt + 4 * q + e;
                            g[pt][e] = fmaf(cur.der[D_R][t][key], dj, g[pt][e]);
                            cs = fmaf(cur.der[D_B][t][key], g[pt][e], cs);
                        }
                    cs += __shfl_xor(cs, 16);
                    cs += __shfl_xor(cs, 32);
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int key = 16 * pt + 4 * q + e;
                            g[pt][e] = fmaf(cur.der[D_W][t][key], g[pt][e], cur.der[D_A][t][key] * cs);
                        }
                }
                factors(nxt);
            } else {
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&cur.d15[16 * pt + 4 * q]);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        gh[pt][e] = g[pt][e] * d4[e];
                }
                f32x4 dz0 = zero4, dz1 = zero4, dzy = zero4;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dzy = mfma4(cur.sm[S_RB][4 * q + i][n], cur.dout[4 * q + i][col], dzy);
#pragma unroll
                for (int pt = 0; pt < 4; ++pt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float a = cur.der[D_B][n][16 * pt + 4 * q + e];
                        if (pt & 1)
                            dz1 = mfma4(a, gh[pt][e], dz1);
                        else
                            dz0 = mfma4(a, gh[pt][e], dz0);
                    }
                // the next chunk's factors while the products run (with no chunk left,
                // harmlessly over the idle buffer: nothing reads it again)
                factors(nxt);
                dz = (dz0 + dz1) + dzy;
                // the operands of phase 2 that are ready now
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const f32x4 p4 = *reinterpret_cast<const f32x4 *>(&cur.p7[16 * pt + 4 * q]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        ap[pt][i] = cur.der[D_A][4 * q + i][16 * pt + n];
                        p7v[pt][i] = p4[i];
                    }
                }
            }
            __syncthreads();
            // ---- phase 2: dX = T^T dZ (the B operand is this lane's own rows of dZ);
            // G_end of the chunk before = diag(P_7) (G^ + R'^T dO + A'^T dX), tile by tile
            if (!ex) {
                f32x4 dx = zero4;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dx = mfma4(cur.sm[S_T][4 * q + i][n], dz[i], dx);
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    f32x4 acc;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[e] = gh[pt][e] + cur.qd[w4][4 * pt + e][lane];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc = mfma4(ap[pt][i], dx[i], acc);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        g[pt][e] = acc[e] * p7v[pt][e];
                }
            }
            if (c > 0) {
                const u64 rowc = row0 + static_cast<u64>((c - 1) * CC) * e_step;
                float *const outs[4] = {p.dr, p.dk, p.da, p.db};
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const u64 at = reinterpret_cast<u64>(outs[pt]) + rowc;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        *reinterpret_cast<GLOBAL_AS float *>(at + e * e_step) = g[pt][e];
                }
            }
            __syncthreads();
        }
        put_state(p.d_state_in);
    } else {
        for (int k = 0; c >= 0; ++k, --c) {
            GchainBuf &cur = sm.buf[k & 1], &nxt = sm.buf[(k & 1) ^ 1];
            // ---- phase 1: T of chunk c (wave 7); R'^T dO of chunk c at the chain waves'
            // columns (wave 4 for chain waves 0 and 3, waves 5 and 6 for 1 and 2)
            if (!exact_of(cur)) {
                if (w4 == 3) {
                    tsolve(cur);
                } else {
                    qprod(cur, w4);
                    if (w4 == 0)
                        qprod(cur, 3);
                }
            }
            __syncthreads();
            // ---- phase 2: chunk c - 1's matrices (its raw rows are still staged), then
            // chunk c - 2 staged (over chunk c's dO, read no more)
            if (c > 0) {
                if (exact_of(nxt))
                    copy_raw(nxt);
                else
                    mprod(nxt);
                if (c > 1) {
                    stage_store(c - 2, cur);
                    if (c > 2)
                        stage_load(c - 3);
                }
            }
            __syncthreads();
        }
    }
}

template <typename Tin>
hipError_t launch_bwdc_t(const BwdArgs &p, hipStream_t stream)
{
    const int nbh = p.B * p.H;
    const int nck = (p.T + CC - 1) / CC;
    if (nck > 0)  // every head's last chunk: G_end is d_state_out
        hipLaunchKernelGGL(wkv7_bwdc_chunk_kernel<Tin>, dim3(static_cast<unsigned>(nbh)), dim3(256), 0, stream, p,
                           nck - 1, nbh);
    // the chain: with few heads, the token recurrence in two workgroups per head (more
    // waves in flight); otherwise the chunk form on the matrix cores, a workgroup per head
    if (2 * nbh <= kCUs) {
        const dim3 cgrid(2 * static_cast<unsigned>(nbh));
        if (p.d_state_out)
            hipLaunchKernelGGL((wkv7_bwdc_chain_kernel<Tin, true>), cgrid, dim3(GNW * 64), 0, stream, p);
        else
            hipLaunchKernelGGL((wkv7_bwdc_chain_kernel<Tin, false>), cgrid, dim3(GNW * 64), 0, stream, p);
    } else if (p.d_state_out) {
        hipLaunchKernelGGL((wkv7_bwdc_gchain_kernel<Tin, true>), dim3(static_cast<unsigned>(nbh)), dim3(512), 0,
                           stream, p);
    } else {
        hipLaunchKernelGGL((wkv7_bwdc_gchain_kernel<Tin, false>), dim3(static_cast<unsigned>(nbh)), dim3(512), 0,
                           stream, p);
    }
    // the other chunks, fewer than 2^32 threads (2^24 workgroups) per launch
    const int per = static_cast<int>(std::max<long long>(1, ((1ll << 24) - 1) / nbh));
    for (int c0 = 0; c0 < nck - 1; c0 += per) {
        const int n = std::min(per, nck - 1 - c0);
        hipLaunchKernelGGL(wkv7_bwdc_chunk_kernel<Tin>, dim3(static_cast<unsigned>(n) * static_cast<unsigned>(nbh)),
                           dim3(256), 0, stream, p, c0, nbh);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_chunked(const BwdArgs &p, hipStream_t stream)
{
    return p.in_bf16 ? launch_bwdc_t<uint16_t>(p, stream) : launch_bwdc_t<float>(p, stream);
}

}  // namespace wkv7
