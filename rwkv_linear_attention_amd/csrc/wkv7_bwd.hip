// wkv7_bwd.hip -- the backward pass of the WKV-7 recurrence (gradients).
//
// The SwiftRWKV Inference guide (its `.rwkvq` backend section) keeps a trainable
// WKV kernel whose backward pass rebuilds the state chunk by chunk.  The
// recurrence (RWKV-X Architecture page, section "WKV-7 Kernel (Generalized Delta
// Rule)") is
//     S_t = diag(w_t) S_{t-1} + b_t (a_t^T S_{t-1}) + k_t v_t^T,   o_t = S_t^T r_t.
// Its reverse-mode adjoint, with G the gradient with respect to S_t (G starts
// as the gradient of the final state), runs backward in t:
//     G    += r_t do_t^T
//     dr_t  = S_t do_t            dk_t = G v_t             dv_t = G^T k_t
//     dw_t  = rowsum(G * S_{t-1}) db_t = G (S_{t-1}^T a_t)
//     c     = G^T b_t             da_t = S_{t-1} c
//     G     = diag(w_t) G + a_t c^T
// and the gradient of the input state is the last G.  The states S_t are an
// input (the per-position states the step kernel writes), so nothing is
// rebuilt: with 288 GB of HBM the states of long sequences fit.  (The backward
// from chunk checkpoints, which rebuilds them, is wkv7_bwdc.hip.)
//
// The columns of G evolve independently (column j needs only c_j, a sum over
// the rows of column j); only the outputs dr, dk, dw, db, da sum over columns.
//
// MAPPING (gfx950).  SPLIT workgroups of eight waves per (batch, head), each
// with 64 / SPLIT value columns: SPLIT = 2 when the heads alone would leave most
// of the 256 compute units idle, else 1.  Lane i of every wave is key row i;
// wave g keeps CW = 8 / SPLIT value columns of G, S_t and S_{t-1} in registers.
//  * Sums over the value columns (dr, dk, dw, db, da) are a CW-term sum in each
//    lane and a sum of the eight waves' partials through LDS, once per four
//    tokens (one barrier; the partials double-buffered).  With SPLIT = 2 the two
//    workgroups' sums meet in an atomic add onto zeroed outputs: two terms, so
//    the result does not depend on their order.
//  * Sums over the key rows (c, S_{t-1}^T a, dv) stay inside a wave: the lanes
//    write their CW terms of each to LDS, a group of lanes adds each (quantity,
//    column) pair over the rows, and quad exchanges in the vector ALU finish
//    it; lane reads hand c and S_{t-1}^T a to every lane (ColSum below).
// Each token's inputs and S_{t-1} are loaded three tokens ahead.  All arithmetic
// is fp32; gradients are written as fp32.
#include "wkv7_device.h"
#include "wkv7_launch.h"

namespace wkv7 {
namespace {

#define GLOBAL_AS __attribute__((address_space(1)))
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int NWB = 8;               // waves per workgroup
constexpr int NSET = 4;              // tokens of inputs in flight (loaded NSET-1 ahead)
constexpr int TB = NSET;             // tokens whose row partials are summed together
constexpr int kCUs = 256;            // compute units of the MI355X

// The column sums over the 64 key rows (c = G^T b, sa = S_{t-1}^T a, dv = G^T k)
// go through LDS.  There are 3 CW (quantity, column) pairs; pair P is summed by
// the L lanes L P .. L P + L - 1 (lane L P + h adds rows RPL h .. RPL h + RPL - 1),
// and one or two quad exchanges finish it.  Lanes past the 3 CW pairs repeat
// pairs of the third quantity.
template <int CW>
struct ColSum {
    static constexpr int L = CW == 4 ? 4 : 2;   // lanes per pair (3 CW pairs in 64 / L slots)
    static constexpr int RPL = kN / L;           // key rows per lane
    // Storage: quantity q, row block h (RPL rows), row rr, column jj at
    // q QS + h BS + rr CW + jj.  The padding (CW per block) makes the 32 lanes of
    // a half wave, which read one row rr at a time, fall in 32 different banks:
    // jj in the low bits, and (q, h) in distinct groups of CW banks.
    static constexpr int BS = RPL * CW + CW;
    static constexpr int QS = L * BS;
    static_assert(3 * CW <= kN / L && kN / L - 3 * CW <= CW, "pairs and their repeats fit the lanes");
};

template <int CW>
struct alignas(16) BwdSmem {
    float x[NWB][3 * ColSum<CW>::QS];  // per-wave column-sum terms
    float part[2][TB][5][NWB][kN];     // per-wave row partials (dr, dk, dw, db, da) of TB tokens
};

// x plus its value in lane l ^ m (m = 1 or 2: within groups of four lanes)
template <int M>
__device__ __forceinline__ float add_quad_xor(float x)
{
    constexpr int ctrl = M == 1 ? 0xB1 /* quad_perm [1,0,3,2] */ : 0x4E /* quad_perm [2,3,0,1] */;
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xf, 0xf, false));
}

// an input element as loaded (fp32, or the upper half of an fp32 for bf16)
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return __uint_as_float(static_cast<unsigned>(x) << 16); }

// Zeroes n floats (n % 4 == 0, 16-byte aligned) in each of five buffers: the
// outputs that the SPLIT = 2 workgroups add into.
__global__ __launch_bounds__(256) void zero5_kernel(float *p0, float *p1, float *p2, float *p3, float *p4, size_t n4)
{
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (size_t e = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; e < n4; e += static_cast<size_t>(gridDim.x) * 256) {
        reinterpret_cast<f32x4 *>(p0)[e] = z;
        reinterpret_cast<f32x4 *>(p1)[e] = z;
        reinterpret_cast<f32x4 *>(p2)[e] = z;
        reinterpret_cast<f32x4 *>(p3)[e] = z;
        reinterpret_cast<f32x4 *>(p4)[e] = z;
    }
}

template <typename Tin, bool HAS_STATE_IN, bool HAS_DOUT, int SPLIT>
__global__ __launch_bounds__(NWB * 64) void wkv7_bwd_kernel(BwdArgs p)
{
    constexpr int CW = kN / (NWB * SPLIT);  // value columns per wave
    using CS = ColSum<CW>;
    __shared__ BwdSmem<CW> sm;
    const int i = threadIdx.x & 63;                                   // key row of this lane
    const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // column block of this wave
    // workgroups are dealt to the 8 XCDs in turn: with SPLIT = 2, workgroups x
    // and x + 8 of each group of 16 are the two halves of one head, so that both
    // run on one XCD and share its L2 (the head's inputs, the adds into dr .. da)
    const int x = blockIdx.x;
    const int bh = SPLIT == 1 ? x : (x / 16) * 8 + x % 8;
    const int half = SPLIT == 1 ? 0 : (x / 8) % 2;
    if (bh >= p.B * p.H)
        return;  // (the last group of 16 can be partly empty)
    const int j0 = (half * NWB + g) * CW;
    const int H = p.H, T = p.T;
    const int bb = bh / H, hh = bh - bb * H;
    const Tin *__restrict__ r = static_cast<const Tin *>(p.r);
    const Tin *__restrict__ w = static_cast<const Tin *>(p.w);
    const Tin *__restrict__ k = static_cast<const Tin *>(p.k);
    const Tin *__restrict__ v = static_cast<const Tin *>(p.v);
    const Tin *__restrict__ a = static_cast<const Tin *>(p.a);
    const Tin *__restrict__ b = static_cast<const Tin *>(p.b);
    const size_t sbase = static_cast<size_t>(bh) * (kN * kN) + static_cast<size_t>(i) * kN + j0;
    // Offsets by token: element (b, t, h, 0) of the [B, T, H, N] tensors is
    // e_of(t) = base_e + t tok_e, and state (b, t, h) in state_pos starts at
    // spos_h + t tok_s.  The loop walks them with running offsets.  Addresses are
    // a per-wave base plus a 32-bit lane offset (iu, soff), which the loads take
    // as they are (a scalar base register and a vector offset).
    const size_t tok_e = static_cast<size_t>(H) * kN, tok_s = tok_e * kN;
    const size_t base_e = static_cast<size_t>(bb) * T * tok_e + static_cast<size_t>(hh) * kN;
    const float *const spos_h = p.state_pos + base_e * kN;
    const unsigned iu = static_cast<unsigned>(i), soff = iu * kN + j0;

    // Everything a token reads (its six inputs, d_o and S_{t-1}) is loaded ahead
    // into a ring of NSET register sets: each token's work is short next to the
    // HBM latency.
    // d_o and v of the wave's columns are the same for every lane: every lane
    // loads all CW of them (one address for the wave).  The address carries a
    // zero that the compiler takes as varying by lane: else it moves the values
    // into scalar registers and waits for the load at the time of the next one.
    // A set holds the values as loaded; conversion and the zero state happen in
    // the step, so that nothing waits for a load at the time it is issued.
    const int lane_zero = static_cast<int>(__builtin_amdgcn_mbcnt_lo(0u, 0u));
    constexpr int VW = CW * static_cast<int>(sizeof(Tin)) / 4;  // 32-bit words of v's CW values
    struct StepIn {
        Tin ri, wi, ki, ai, bi;
        f32x4 dO4[CW / 4];
        uint32_t vw[VW];
        f32x4 Sp4[CW / 4];
        bool live;
    };
    // The byte addresses of one token: its (b, t, h) rows of the six inputs and
    // of d_o (v and d_o at the wave's columns), and the state S_{t-1}.  They are
    // typed as global memory: in the loop they pass through an empty asm, after
    // which the compiler could no longer tell.
    typedef const GLOBAL_AS char *gchar;
    struct TokPtrs {
        gchar r, w, k, a, b, v, d_o, s;
    };
    // One token's loads into a set; live: S_{t-1} is not the zero state.  The
    // same loads on every path keep the compiler's count of loads in flight
    // exact.  (The lane offsets, in bytes, pass through an empty asm, so that the
    // compiler keeps them apart from the bases instead of holding 64-bit
    // addresses per load in vector registers.)
    auto load_ptrs = [&](const TokPtrs &q, bool live, StepIn &s) {
        unsigned lo = iu * sizeof(Tin), lz = static_cast<unsigned>(lane_zero), so = soff * 4u;
        asm volatile("" : "+v"(lo), "+v"(lz), "+v"(so));
        s.ri = *reinterpret_cast<const GLOBAL_AS Tin *>(q.r + lo);
        s.wi = *reinterpret_cast<const GLOBAL_AS Tin *>(q.w + lo);
        s.ki = *reinterpret_cast<const GLOBAL_AS Tin *>(q.k + lo);
        s.ai = *reinterpret_cast<const GLOBAL_AS Tin *>(q.a + lo);
        s.bi = *reinterpret_cast<const GLOBAL_AS Tin *>(q.b + lo);
#pragma unroll
        for (int qq = 0; qq < CW / 4; ++qq)
            s.dO4[qq] = *reinterpret_cast<const GLOBAL_AS f32x4 *>(q.d_o + 16 * qq + lz);
        if (VW % 4 == 0) {
#pragma unroll
            for (int qq = 0; qq < VW; qq += 4) {
                const u32x4 x = *reinterpret_cast<const GLOBAL_AS u32x4 *>(q.v + 4 * qq + lz);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s.vw[qq + e] = x[e];
            }
        } else {
            const u32x2 x = *reinterpret_cast<const GLOBAL_AS u32x2 *>(q.v + lz);
            s.vw[0] = x[0];
            s.vw[VW > 1 ? 1 : 0] = x[1];
        }
        s.live = live;
#pragma unroll
        for (int qq = 0; qq < CW / 4; ++qq)
            s.Sp4[qq] = *reinterpret_cast<const GLOBAL_AS f32x4 *>(q.s + 16 * qq + so);
    };
    auto gb = [](const void *x) { return (gchar)(static_cast<const char *>(x)); };
    // the addresses of token t; its S_{t-1} is the input state for t = 0 (or,
    // without one, a valid state that is read and not used)
    auto ptrs_of = [&](int t) {
        const size_t e = base_e + static_cast<size_t>(t) * tok_e;
        const float *src = t > 0 ? spos_h + static_cast<size_t>(t - 1) * tok_s
                                 : HAS_STATE_IN ? p.state_in + static_cast<size_t>(bh) * (kN * kN) : spos_h;
        return TokPtrs{gb(r + e), gb(w + e), gb(k + e), gb(a + e), gb(b + e), gb(v + e + j0), gb(p.d_o + e + j0), gb(src)};
    };
    auto load_token = [&](int t, StepIn &s) { load_ptrs(ptrs_of(t), t > 0 || HAS_STATE_IN, s); };

    float G[CW], St[CW];
#pragma unroll
    for (int jj = 0; jj < CW; ++jj)
        G[jj] = HAS_DOUT ? p.d_state_out[sbase + jj] : 0.0f;
    if (T == 0) {  // no tokens: the gradient passes through
#pragma unroll
        for (int jj = 0; jj < CW; jj += 4)
            *reinterpret_cast<f32x4 *>(&p.d_state_in[sbase + jj]) = f32x4{G[jj], G[jj + 1], G[jj + 2], G[jj + 3]};
        return;
    }
#pragma unroll
    for (int jj = 0; jj < CW; jj += 4) {
        const f32x4 x4 = *reinterpret_cast<const f32x4 *>((spos_h + static_cast<size_t>(T - 1) * tok_s) + (soff + jj));
#pragma unroll
        for (int e = 0; e < 4; ++e)
            St[jj + e] = x4[e];
    }
    // lane roles in the column sums: this lane writes key row i at x_w; it adds
    // pair P (quantity P / CW, column P % CW), rows RPL h .. RPL h + RPL - 1, from
    // x_r; after the half-wave swap it holds dv of column dv_col
    const int x_w = (i / CS::RPL) * CS::BS + (i % CS::RPL) * CW;
    const int P0 = i / CS::L, P = P0 < 3 * CW ? P0 : P0 - CW, h = i % CS::L;
    const int x_r = (P / CW) * CS::QS + h * CS::BS + P % CW;
    const int Pu = (i | 32) / CS::L, dv_col = (Pu < 3 * CW ? Pu : Pu - CW) % CW;

    // The row partials of a batch of TB tokens (fewer in the last) are written
    // by every wave, and after one barrier the 5 x TB sums are spread over the
    // waves: sum m of wave g is pair g + NWB m = 5 slot + quantity.  Every wave
    // stores the same number of sums (no branch, so that the compiler's count of
    // stores in flight stays exact): a wave with fewer pairs, or a pair past the
    // batch's last slot, repeats one it has (and adds zero with it when the sums
    // are added into the outputs).
    constexpr int NM = (5 * TB + NWB - 1) / NWB;
    int sl0[NM];
    bool extra[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int pi0 = g + NWB * m, pi = pi0 < 5 * TB ? pi0 : pi0 - NWB;
        sl0[m] = pi / 5;
        extra[m] = pi0 >= 5 * TB;
    }
    // e_end: e_of the batch's last token, whose slot is slot_end
    auto finish_batch = [&](size_t e_end, int slot_end, int pb) {
        // a barrier for the LDS partials only: waiting here for this wave's LDS
        // writes (not for its global loads and stores, which a full fence would
        // include, and with them the loads issued for the tokens ahead)
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const int sl = min(sl0[m], slot_end);
            const int qn = (g + NWB * m - (extra[m] ? NWB : 0)) - 5 * sl0[m];
            float sum = 0.f;
#pragma unroll
            for (int gg = 0; gg < NWB; ++gg)
                sum += sm.part[pb][sl][qn][gg][i];
            // (a select, not an indexed array, keeps the pointer's address space known)
            float *const dst = qn == 0 ? p.dr : qn == 1 ? p.dk : qn == 2 ? p.dw : qn == 3 ? p.db : p.da;
            float *const at = (dst + e_end + static_cast<size_t>(slot_end - sl) * tok_e) + iu;
            if (SPLIT == 1)
                *at = sum;
            else
                unsafeAtomicAdd(at, !extra[m] && sl0[m] <= slot_end ? sum : 0.0f);
        }
    };

    // one token of the adjoint (e0 = e_of(t)), from its loaded inputs; slot is its
    // place in its batch of TB tokens, pb the batch's partial buffer; live_known:
    // S_{t-1} is known to be a loaded state (t > 0 or an input state)
    auto step = [&](size_t e0, const StepIn &s, int slot, int pb, bool live_known) {
        const float ri = to_f32(s.ri), wi = to_f32(s.wi), ki = to_f32(s.ki), ai = to_f32(s.ai), bi = to_f32(s.bi);
        float dO[CW], vv[CW], Sp[CW];
#pragma unroll
        for (int jj = 0; jj < CW; ++jj) {
            dO[jj] = s.dO4[jj / 4][jj % 4];
            if (sizeof(Tin) == 4)
                vv[jj] = __uint_as_float(s.vw[jj]);
            else  // two bf16 per word, the lower one first
                vv[jj] = __uint_as_float(jj % 2 == 0 ? s.vw[jj / 2] << 16 : s.vw[jj / 2] & 0xffff0000u);
            Sp[jj] = live_known || s.live ? s.Sp4[jj / 4][jj % 4] : 0.0f;
        }

        // G += r_t do_t^T, then the row partials that need only G, S_t, S_{t-1}
        float p_dr = 0.f, p_dk = 0.f, p_dw = 0.f;
#pragma unroll
        for (int jj = 0; jj < CW; ++jj) {
            G[jj] += ri * dO[jj];
            p_dr += St[jj] * dO[jj];
            p_dk += G[jj] * vv[jj];
            p_dw += G[jj] * Sp[jj];
        }

        // column sums over the 64 key rows: c = G^T b, sa = S_{t-1}^T a, dv = G^T k
        float *const xw = sm.x[g];
#pragma unroll
        for (int jj = 0; jj < CW; jj += 4) {
            f32x4 xc, xs, xv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xc[e] = bi * G[jj + e];
                xs[e] = ai * Sp[jj + e];
                xv[e] = ki * G[jj + e];
            }
            *reinterpret_cast<f32x4 *>(&xw[x_w + jj]) = xc;
            *reinterpret_cast<f32x4 *>(&xw[CS::QS + x_w + jj]) = xs;
            *reinterpret_cast<f32x4 *>(&xw[2 * CS::QS + x_w + jj]) = xv;
        }
        // (four running sums, added as a tree: a short chain)
        float c4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rr = 0; rr < CS::RPL; ++rr)
            c4[rr % 4] += xw[x_r + rr * CW];
        float cs = (c4[0] + c4[1]) + (c4[2] + c4[3]);
        cs = add_quad_xor<1>(cs);
        if (CS::L == 4)
            cs = add_quad_xor<2>(cs);
        // lane L P holds pair P: c and sa read back by lane reads; dv sits in the
        // upper half-wave, and the half-wave swap gives it to every lane (the
        // lanes of a column store the same value)
        float c[CW], sa[CW];
#pragma unroll
        for (int jj = 0; jj < CW; ++jj) {
            c[jj] = lane_bcast(cs, CS::L * jj);
            sa[jj] = lane_bcast(cs, CS::L * (CW + jj));
        }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(cs), __float_as_uint(cs), false, false);
        (p.dv + e0 + j0)[static_cast<unsigned>(dv_col)] = __uint_as_float(sw[1]);

        // row partials that need c and sa, then G for the previous token
        float p_db = 0.f, p_da = 0.f;
#pragma unroll
        for (int jj = 0; jj < CW; ++jj) {
            p_db += G[jj] * sa[jj];
            p_da += Sp[jj] * c[jj];
            G[jj] = wi * G[jj] + ai * c[jj];
            St[jj] = Sp[jj];
        }

        // this wave's row partials, summed over the waves once per batch
        sm.part[pb][slot][0][g][i] = p_dr;
        sm.part[pb][slot][1][g][i] = p_dk;
        sm.part[pb][slot][2][g][i] = p_dw;
        sm.part[pb][slot][3][g][i] = p_db;
        sm.part[pb][slot][4][g][i] = p_da;
    };

    // Tokens T-1, T-2, ... ; the n-th (n = T-1-t) uses set n % NSET and is slot
    // n % TB of batch n / TB.  Its S_{t-1} is the next token's S_t, so the set stays
    // live one token more: after token t runs, the set of token t+1 is refilled
    // with token t+1-NSET (NSET-1 tokens ahead).  The loop holds whole rounds
    // whose loads are all real and of tokens t > 0 (so the compiler's wait
    // analysis sees one steady state and waits only for loads a round old) and
    // whose batch ends at a fixed place; the last rounds follow it.
    static_assert(TB == NSET, "a round of the loop is one batch");
    StepIn ring[NSET];
#pragma unroll
    for (int u = 0; u < NSET; ++u)
        load_token(max(T - 1 - u, 0), ring[u]);  // (a set past token 0 is never used)
    step(base_e + static_cast<size_t>(T - 1) * tok_e, ring[0], 0, 0, false);
    int t0 = T - 2, kb = 0;  // batch of the round's first token (n = 4 kb + 1)
    if (t0 >= 2 * NSET - 1) {
        size_t er = base_e + static_cast<size_t>(t0) * tok_e;  // e_of(t0)
        // the next token to load, t0 + 1 - NSET: running per-tensor addresses, one
        // token back after each load (through an empty asm, so that the compiler
        // keeps eight scalar pointers, not an address per tensor and token, which
        // ran out of scalar registers)
        TokPtrs lp = ptrs_of(t0 + 1 - NSET);
        const size_t tb_in = tok_e * sizeof(Tin), tb_f = tok_e * 4, tb_s = tok_s * 4;  // bytes per token
        for (; t0 >= 2 * NSET - 1; t0 -= NSET, ++kb, er -= NSET * tok_e) {
#pragma unroll
            for (int u = 0; u < NSET; ++u) {
                // token t0 - u (t >= NSET, its S_{t-1} loaded), then the load of
                // token t0 - u + 1 - NSET (>= 1), whose S_{t-1} is state t0 - u - NSET
                step(er - u * tok_e, ring[(u + 1) % NSET], (u + 1) % TB, (kb + (u + 1) / TB) & 1, true);
                load_ptrs(lp, true, ring[u]);
                lp.r -= tb_in; lp.w -= tb_in; lp.k -= tb_in; lp.a -= tb_in; lp.b -= tb_in; lp.v -= tb_in;
                lp.d_o -= tb_f; lp.s -= tb_s;
                asm volatile("" : "+s"(lp.r), "+s"(lp.w), "+s"(lp.k), "+s"(lp.a), "+s"(lp.b), "+s"(lp.v),
                             "+s"(lp.d_o), "+s"(lp.s));
                if (u == TB - 2)
                    finish_batch(er - u * tok_e, TB - 1, kb & 1);
            }
        }
    }
    for (; t0 >= 0; t0 -= NSET, ++kb) {
#pragma unroll
        for (int u = 0; u < NSET; ++u) {
            const int t = t0 - u;
            if (t >= 0) {
                const int pb = (kb + (u + 1) / TB) & 1;
                const size_t e0 = base_e + static_cast<size_t>(t) * tok_e;
                step(e0, ring[(u + 1) % NSET], (u + 1) % TB, pb, false);
                load_token(max(t + 1 - NSET, 0), ring[u]);
                if (u == TB - 2 || t == 0)
                    finish_batch(e0, (u + 1) % TB, pb);
            }
        }
    }
    if (T == 1)
        finish_batch(base_e, 0, 0);
#pragma unroll
    for (int jj = 0; jj < CW; jj += 4)
        *reinterpret_cast<f32x4 *>(&p.d_state_in[sbase + jj]) = f32x4{G[jj], G[jj + 1], G[jj + 2], G[jj + 3]};
}

template <typename Tin, int SPLIT>
hipError_t launch_bwd_split(const BwdArgs &p, hipStream_t stream)
{
    const size_t heads = static_cast<size_t>(p.B) * static_cast<size_t>(p.H);
    if (SPLIT > 1 && p.T > 0) {
        const size_t n4 = heads * static_cast<size_t>(p.T) * (kN / 4);
        const unsigned zblocks = static_cast<unsigned>(std::min<size_t>((n4 + 255) / 256, 4 * kCUs));
        hipLaunchKernelGGL(zero5_kernel, dim3(zblocks), dim3(256), 0, stream, p.dr, p.dk, p.dw, p.db, p.da, n4);
    }
    const size_t nwg = SPLIT == 1 ? heads : (heads + 7) / 8 * 16;
    const dim3 grid(static_cast<unsigned>(nwg)), block(NWB * 64);
    const bool sin = p.state_in != nullptr, dout = p.d_state_out != nullptr;
    if (sin && dout)
        hipLaunchKernelGGL((wkv7_bwd_kernel<Tin, true, true, SPLIT>), grid, block, 0, stream, p);
    else if (sin)
        hipLaunchKernelGGL((wkv7_bwd_kernel<Tin, true, false, SPLIT>), grid, block, 0, stream, p);
    else if (dout)
        hipLaunchKernelGGL((wkv7_bwd_kernel<Tin, false, true, SPLIT>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((wkv7_bwd_kernel<Tin, false, false, SPLIT>), grid, block, 0, stream, p);
    return hipGetLastError();
}

// one workgroup per compute unit (the LDS of a workgroup is more than half of a
// unit's): two per head while that still fits in one pass over the units
template <typename Tin>
hipError_t launch_bwd_t(const BwdArgs &p, hipStream_t stream)
{
    const int64_t heads = static_cast<int64_t>(p.B) * p.H;
    return heads * 2 <= kCUs ? launch_bwd_split<Tin, 2>(p, stream) : launch_bwd_split<Tin, 1>(p, stream);
}

}  // namespace

hipError_t launch_backward(const BwdArgs &p, hipStream_t stream)
{
    return p.in_bf16 ? launch_bwd_t<uint16_t>(p, stream) : launch_bwd_t<float>(p, stream);
}

}  // namespace wkv7
