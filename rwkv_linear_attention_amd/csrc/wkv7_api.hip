// wkv7_api.hip -- the C ABI of libwkv7 (declared in include/wkv7.h).
//
// Every argument is validated here, before any HIP call, so each error path
// can be exercised without a GPU.  The entry points only enqueue work on the
// caller's stream: no allocation, no synchronisation, no global state.
#include <stdint.h>

#include "../../include/wkv7.h"
#include "wkv7_launch.h"

namespace {

using wkv7::SeqArgs;

constexpr int64_t kN = 64;
// Sequences shorter than this go to the step kernel in wkv7_forward.
constexpr int kChunkMinT = 9;

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void *p, int64_t bytes)
{
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

bool overlap(const Range &x, const Range &y)
{
    return x.lo < y.hi && y.lo < x.hi && x.hi > x.lo && y.hi > y.lo;
}

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// B*T*H*N*N must fit in int64 (and every partial product with it).
// Largest B * H that one launch of a kernel covers.  A head is one workgroup of
// the step kernel (up to 512 threads) or up to J workgroups of the chunked kernel
// (up to 1024 threads each, J = 1 beyond 128 heads), and a launch holds fewer than
// 2^32 threads.
constexpr int64_t kMaxHeadsStep = WKV7_MAX_HEADS_STEP;
constexpr int64_t kMaxHeadsChunk = WKV7_MAX_HEADS_CHUNK;
// The chunked kernel stores a chunk's outputs at 32-bit byte offsets from the chunk's
// first row: (15 H N + 15) * 4 must stay below 2^32.
constexpr int64_t kMaxHChunk = WKV7_MAX_H_CHUNK;
static_assert((15 * kMaxHChunk * kN + 15) * 4 < (1ll << 32), "32-bit output offsets of the chunked kernel");
// Largest B * T * H of the time-mix tail pass (16 threads per row).
constexpr int64_t kMaxRowsTail = WKV7_MAX_ROWS_TAIL;
static_assert(kMaxHeadsStep * 512 < (1ll << 32) && kMaxHeadsChunk * 1024 < (1ll << 32) &&
                  kMaxRowsTail * 16 < (1ll << 32),
              "a launch must hold fewer than 2^32 threads");

bool shape_ok(int B, int T, int H, int64_t *tokens_out, int64_t max_heads = INT64_MAX)
{
    if (B < 1 || H < 1 || T < 0)
        return false;
    const int64_t lim = INT64_MAX / (kN * kN * 8);
    const int64_t bh = static_cast<int64_t>(B) * H;
    if (bh > max_heads)
        return false;
    if (T > 0 && bh > lim / T)
        return false;
    *tokens_out = bh * T;
    return true;
}

// state_out may be NULL only where the caller allows it (the recurrent pass with
// per-position states and T > 0: the last of those is the final state).
int check_seq(const void *r, const void *w, const void *k, const void *v, const void *a, const void *b,
              int in_dtype, const float *state_in, void *o, int o_dtype, float *state_out, float *state_pos,
              int B, int T, int H, int N, bool out_optional = false, bool step_only = true)
{
    int64_t tok = 0;
    if (N != kN)
        return WKV7_ERR_UNSUPPORTED;
    if ((in_dtype != WKV7_F32 && in_dtype != WKV7_BF16) || (o_dtype != WKV7_F32 && o_dtype != WKV7_BF16))
        return WKV7_ERR_UNSUPPORTED;
    // the parallel pass routes T >= kChunkMinT to the chunked kernel
    const bool chunked = !step_only && T >= kChunkMinT;
    if (!shape_ok(B, T, H, &tok, chunked ? kMaxHeadsChunk : kMaxHeadsStep) || (chunked && H > kMaxHChunk))
        return WKV7_ERR_SHAPE;
    if (!state_out && !(out_optional && state_pos && T > 0))
        return WKV7_ERR_NULL;
    if (T > 0 && (!r || !w || !k || !v || !a || !b || !o))
        return WKV7_ERR_NULL;
    const void *ptrs[] = {r, w, k, v, a, b, o, state_in, state_out, state_pos};
    for (const void *ptr : ptrs)
        if (ptr && misaligned(ptr))
            return WKV7_ERR_ALIGN;

    const int64_t ein = in_dtype == WKV7_BF16 ? 2 : 4, eo = o_dtype == WKV7_BF16 ? 2 : 4;
    const int64_t seq_elems = tok * kN, st_bytes = static_cast<int64_t>(B) * H * kN * kN * 4;
    Range ro{0, 0}, rpos{0, 0}, rin{0, 0}, rst{0, 0};
    if (state_out)
        rst = range_of(state_out, st_bytes);
    if (state_in)
        rin = range_of(state_in, st_bytes);
    if (T > 0)
        ro = range_of(o, seq_elems * eo);
    if (state_pos && T > 0)
        rpos = range_of(state_pos, seq_elems * kN * 4);

    // state_out may be state_in exactly; any other overlap is refused.
    if (state_in && state_out && state_in != state_out && overlap(rst, rin))
        return WKV7_ERR_ALIAS;
    Range ins[7] = {rin, {0, 0}, {0, 0}, {0, 0}, {0, 0}, {0, 0}, {0, 0}};
    if (T > 0) {
        const void *vin[6] = {r, w, k, v, a, b};
        for (int i = 0; i < 6; ++i)
            ins[i + 1] = range_of(vin[i], seq_elems * ein);
    }
    const Range outs[3] = {ro, rst, rpos};
    for (int x = 0; x < 3; ++x) {
        for (int y = 0; y < 7; ++y) {
            if (x == 1 && y == 0)
                continue;  // state_out vs state_in handled above
            if (overlap(outs[x], ins[y]))
                return WKV7_ERR_ALIAS;
        }
        for (int y = x + 1; y < 3; ++y)
            if (overlap(outs[x], outs[y]))
                return WKV7_ERR_ALIAS;
    }
    return WKV7_OK;
}

SeqArgs make_args(const void *r, const void *w, const void *k, const void *v, const void *a, const void *b,
                  int in_dtype, const float *state_in, void *o, int o_dtype, float *state_out,
                  float *state_pos, int B, int T, int H)
{
    SeqArgs s;
    s.r = r; s.w = w; s.k = k; s.v = v; s.a = a; s.b = b;
    s.state_in = state_in; s.o = o; s.state_out = state_out; s.state_pos = state_pos;
    s.ckpt = nullptr;
    s.lengths = nullptr;
    s.gate = nullptr;
    s.r_k = s.ln_w = s.ln_b = nullptr;
    s.eps = 0.f;
    s.B = B; s.T = T; s.H = H;
    s.in_bf16 = in_dtype == WKV7_BF16;
    s.o_bf16 = o_dtype == WKV7_BF16;
    return s;
}

// The tail's inputs: gate [B,T,H,N] of in_dtype and r_k, ln_w, ln_b [H,N] fp32 --
// present, aligned, and outside every output range given.
int check_tail_inputs(const void *gate, const float *r_k, const float *ln_w, const float *ln_b, int in_dtype,
                      int B, int T, int H, const Range *outs, int nouts)
{
    if (T > 0 && (!gate || !r_k || !ln_w || !ln_b))
        return WKV7_ERR_NULL;
    if (T == 0)
        return WKV7_OK;
    const void *ptrs[] = {gate, r_k, ln_w, ln_b};
    for (const void *ptr : ptrs)
        if (misaligned(ptr))
            return WKV7_ERR_ALIGN;
    const int64_t ein = in_dtype == WKV7_BF16 ? 2 : 4;
    const Range ins[4] = {range_of(gate, static_cast<int64_t>(B) * T * H * kN * ein), range_of(r_k, H * kN * 4),
                          range_of(ln_w, H * kN * 4), range_of(ln_b, H * kN * 4)};
    for (int x = 0; x < nouts; ++x)
        for (const Range &y : ins)
            if (overlap(outs[x], y))
                return WKV7_ERR_ALIAS;
    return WKV7_OK;
}

int empty_sequence(const float *state_in, float *state_out, int B, int H, hipStream_t stream)
{
    if (state_in == state_out)
        return WKV7_OK;
    const long long n = static_cast<long long>(B) * H * kN * kN;
    return wkv7::launch_state_copy(state_in, state_out, n, stream) == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

// Bytes of the chunk checkpoints [B, ceil(T/16), H, N, N] fp32 (within int64 once
// shape_ok has accepted B, T, H).
int64_t ckpt_bytes(int B, int T, int H)
{
    return static_cast<int64_t>(B) * ((T + 15) / 16) * H * kN * kN * 4;
}

// The backward passes' arguments: the per-position states (state_pos, with state_in)
// or the chunk checkpoints (ckpt: states is ckpt).  Fills *p when they are valid.
int check_backward(const void *r, const void *w, const void *k, const void *v, const void *a, const void *b,
                   int in_dtype, const float *state_in, const float *states, bool is_ckpt, const float *d_o,
                   const float *d_state_out, float *dr, float *dw, float *dk, float *dv, float *da, float *db,
                   float *d_state_in, int B, int T, int H, int N, wkv7::BwdArgs *p)
{
    int64_t tok = 0;
    if (N != kN)
        return WKV7_ERR_UNSUPPORTED;
    if (in_dtype != WKV7_F32 && in_dtype != WKV7_BF16)
        return WKV7_ERR_UNSUPPORTED;
    if (!shape_ok(B, T, H, &tok, kMaxHeadsStep))
        return WKV7_ERR_SHAPE;
    if (!d_state_in)
        return WKV7_ERR_NULL;
    const void *ins[] = {r, w, k, v, a, b, states, d_o};
    float *const grads[] = {dr, dw, dk, dv, da, db};
    if (T > 0) {
        for (const void *ptr : ins)
            if (!ptr)
                return WKV7_ERR_NULL;
        for (const float *ptr : grads)
            if (!ptr)
                return WKV7_ERR_NULL;
    }
    const void *all[] = {r, w, k, v, a, b, state_in, states, d_o, d_state_out,
                         dr, dw, dk, dv, da, db, d_state_in};
    for (const void *ptr : all)
        if (ptr && misaligned(ptr))
            return WKV7_ERR_ALIGN;
    // every output overlaps nothing else (d_state_in may be d_state_out itself)
    const int64_t ein = in_dtype == WKV7_BF16 ? 2 : 4;
    const int64_t vec = tok * kN, st_bytes = static_cast<int64_t>(B) * H * kN * kN * 4;
    Range in_r[11];
    int n_in = 0;
    if (T > 0) {
        for (int q = 0; q < 6; ++q)
            in_r[n_in++] = range_of(ins[q], vec * ein);
        in_r[n_in++] = range_of(states, is_ckpt ? ckpt_bytes(B, T, H) : vec * kN * 4);
        in_r[n_in++] = range_of(d_o, vec * 4);
    }
    if (state_in)
        in_r[n_in++] = range_of(state_in, st_bytes);
    // d_state_out is read by the pass: no gradient of an input may overlap it (d_state_in
    // may be d_state_out itself, checked below)
    if (d_state_out && d_state_out != d_state_in)
        in_r[n_in++] = range_of(d_state_out, st_bytes);
    const Range r_dsi = range_of(d_state_in, st_bytes);
    Range out_r[7];
    int n_out = 0;
    if (T > 0)
        for (const float *ptr : grads)
            out_r[n_out++] = range_of(ptr, vec * 4);
    out_r[n_out++] = r_dsi;
    for (int x = 0; x < n_out; ++x) {
        for (int y = 0; y < n_in; ++y)
            if (overlap(out_r[x], in_r[y]))
                return WKV7_ERR_ALIAS;
        for (int y = x + 1; y < n_out; ++y)
            if (overlap(out_r[x], out_r[y]))
                return WKV7_ERR_ALIAS;
    }
    if (d_state_out && d_state_out != d_state_in && overlap(r_dsi, range_of(d_state_out, st_bytes)))
        return WKV7_ERR_ALIAS;
    p->r = r; p->w = w; p->k = k; p->v = v; p->a = a; p->b = b;
    p->state_in = state_in;
    p->state_pos = is_ckpt ? nullptr : states;
    p->ckpt = is_ckpt ? states : nullptr;
    p->d_o = d_o; p->d_state_out = d_state_out;
    p->dr = dr; p->dw = dw; p->dk = dk; p->dv = dv; p->da = da; p->db = db; p->d_state_in = d_state_in;
    p->B = B; p->T = T; p->H = H;
    p->in_bf16 = in_dtype == WKV7_BF16;
    return WKV7_OK;
}

}  // namespace

extern "C" {

int wkv7_forward(const void *r, const void *w, const void *k, const void *v, const void *a, const void *b,
                 int in_dtype, const float *state_in, void *o, int o_dtype, float *state_out, int B, int T,
                 int H, int N, void *stream)
{
    int st = check_seq(r, w, k, v, a, b, in_dtype, state_in, o, o_dtype, state_out, nullptr, B, T, H, N,
                       false, false);
    if (st != WKV7_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0)
        return empty_sequence(state_in, state_out, B, H, s);
    const SeqArgs args = make_args(r, w, k, v, a, b, in_dtype, state_in, o, o_dtype, state_out, nullptr, B, T, H);
    const hipError_t e = T < kChunkMinT ? wkv7::launch_step(args, s) : wkv7::launch_chunk(args, s);
    return e == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

int wkv7_forward_varlen(const void *r, const void *w, const void *k, const void *v, const void *a,
                        const void *b, int in_dtype, const float *state_in, void *o, int o_dtype,
                        float *state_out, const int *lengths, int B, int T, int H, int N, void *stream)
{
    int st = check_seq(r, w, k, v, a, b, in_dtype, state_in, o, o_dtype, state_out, nullptr, B, T, H, N,
                       false, false);
    if (st != WKV7_OK)
        return st;
    if (!lengths)
        return WKV7_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(lengths) & 3u) != 0)
        return WKV7_ERR_ALIGN;
    // the lengths must not overlap an output
    const Range rl = range_of(lengths, static_cast<int64_t>(B) * 4);
    const int64_t eo = o_dtype == WKV7_BF16 ? 2 : 4;
    const int64_t st_bytes = static_cast<int64_t>(B) * H * kN * kN * 4;
    if (overlap(rl, range_of(state_out, st_bytes)) ||
        (T > 0 && overlap(rl, range_of(o, static_cast<int64_t>(B) * T * H * kN * eo))))
        return WKV7_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0)
        return empty_sequence(state_in, state_out, B, H, s);
    SeqArgs args = make_args(r, w, k, v, a, b, in_dtype, state_in, o, o_dtype, state_out, nullptr, B, T, H);
    args.lengths = lengths;
    const hipError_t e = T < kChunkMinT ? wkv7::launch_step(args, s) : wkv7::launch_chunk(args, s);
    return e == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

int wkv7_step(const void *r, const void *w, const void *k, const void *v, const void *a, const void *b,
              int in_dtype, const float *state_in, void *o, int o_dtype, float *state_out, float *state_pos,
              int B, int T, int H, int N, void *stream)
{
    int st = check_seq(r, w, k, v, a, b, in_dtype, state_in, o, o_dtype, state_out, state_pos, B, T, H, N, true);
    if (st != WKV7_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0)
        return empty_sequence(state_in, state_out, B, H, s);
    const SeqArgs args = make_args(r, w, k, v, a, b, in_dtype, state_in, o, o_dtype, state_out, state_pos, B, T, H);
    return wkv7::launch_step(args, s) == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

int wkv7_state_reset(float *state, int B, int H, int N, const unsigned char *row_mask, void *stream)
{
    int64_t tok = 0;
    if (N != kN)
        return WKV7_ERR_UNSUPPORTED;
    if (!shape_ok(B, 1, H, &tok))
        return WKV7_ERR_SHAPE;
    if (!state)
        return WKV7_ERR_NULL;
    if (misaligned(state))
        return WKV7_ERR_ALIGN;
    if (row_mask) {
        const Range rs = range_of(state, static_cast<int64_t>(B) * H * kN * kN * 4);
        if (overlap(rs, range_of(row_mask, B)))
            return WKV7_ERR_ALIAS;
    }
    return wkv7::launch_state_reset(state, B, H, row_mask, static_cast<hipStream_t>(stream)) == hipSuccess
               ? WKV7_OK
               : WKV7_ERR_HIP;
}

int wkv7_step_tail(const void *r, const void *w, const void *k, const void *v, const void *a, const void *b,
                   int in_dtype, const float *state_in, const void *gate, const float *r_k, const float *ln_w,
                   const float *ln_b, float eps, void *x, int x_dtype, float *state_out, float *state_pos, int B,
                   int T, int H, int N, void *stream)
{
    int st = check_seq(r, w, k, v, a, b, in_dtype, state_in, x, x_dtype, state_out, state_pos, B, T, H, N, true);
    if (st != WKV7_OK)
        return st;
    const int64_t tok = static_cast<int64_t>(B) * T * H;
    const int64_t ex = x_dtype == WKV7_BF16 ? 2 : 4;
    const Range outs[3] = {T > 0 ? range_of(x, tok * kN * ex) : Range{0, 0},
                           state_out ? range_of(state_out, static_cast<int64_t>(B) * H * kN * kN * 4) : Range{0, 0},
                           state_pos && T > 0 ? range_of(state_pos, tok * kN * kN * 4) : Range{0, 0}};
    st = check_tail_inputs(gate, r_k, ln_w, ln_b, in_dtype, B, T, H, outs, 3);
    if (st != WKV7_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0)
        return empty_sequence(state_in, state_out, B, H, s);
    SeqArgs args = make_args(r, w, k, v, a, b, in_dtype, state_in, x, x_dtype, state_out, state_pos, B, T, H);
    args.gate = gate;
    args.r_k = r_k;
    args.ln_w = ln_w;
    args.ln_b = ln_b;
    args.eps = eps;
    return wkv7::launch_step(args, s) == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

int wkv7_forward_tail(const void *r, const void *w, const void *k, const void *v, const void *a,
                      const void *b, int in_dtype, const float *state_in, const void *gate, const float *r_k,
                      const float *ln_w, const float *ln_b, float eps, void *x, int x_dtype, float *state_out,
                      int B, int T, int H, int N, void *stream)
{
    // fp32 inputs with an fp32 x (T >= kChunkMinT) finish with the tail pass, under its row limit
    const bool two_pass = in_dtype == WKV7_F32 && x_dtype == WKV7_F32 && T >= kChunkMinT;
    if (two_pass && B >= 1 && H >= 1 && static_cast<int64_t>(B) * T * H > kMaxRowsTail)
        return WKV7_ERR_SHAPE;
    int st = check_seq(r, w, k, v, a, b, in_dtype, state_in, x, x_dtype, state_out, nullptr, B, T, H, N, false,
                       false);
    if (st != WKV7_OK)
        return st;
    const int64_t tok = static_cast<int64_t>(B) * T * H;
    const int64_t ex = x_dtype == WKV7_BF16 ? 2 : 4;
    const Range outs[2] = {T > 0 ? range_of(x, tok * kN * ex) : Range{0, 0},
                           range_of(state_out, static_cast<int64_t>(B) * H * kN * kN * 4)};
    st = check_tail_inputs(gate, r_k, ln_w, ln_b, in_dtype, B, T, H, outs, 2);
    if (st != WKV7_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0)
        return empty_sequence(state_in, state_out, B, H, s);
    SeqArgs args = make_args(r, w, k, v, a, b, in_dtype, state_in, x, x_dtype, state_out, nullptr, B, T, H);
    args.gate = gate;
    args.r_k = r_k;
    args.ln_w = ln_w;
    args.ln_b = ln_b;
    args.eps = eps;
    hipError_t e;
    if (T < kChunkMinT || (in_dtype == WKV7_F32 && x_dtype == WKV7_BF16)) {
        e = wkv7::launch_step(args, s);  // the step kernel with its fused tail
    } else if (!two_pass) {
        e = wkv7::launch_chunk(args, s);  // bf16 inputs: one chunked kernel with the tail wave
    } else {
        // fp32 inputs: o (fp32) into x, then the tail pass over x in place
        args.gate = nullptr;
        e = wkv7::launch_chunk(args, s);
        if (e == hipSuccess) {
            wkv7::TailArgs t;
            t.o = x; t.r = r; t.k = k; t.v = v; t.gate = gate;
            t.r_k = r_k; t.ln_w = ln_w; t.ln_b = ln_b; t.eps = eps;
            t.x = x; t.rows = tok; t.H = H;
            t.in_bf16 = 0;
            t.o_bf16 = 0;
            t.x_bf16 = 0;
            e = wkv7::launch_tail(t, s);
        }
    }
    return e == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

int wkv7_tmix_tail(const void *o, int o_dtype, const void *r, const void *k, const void *v, const void *gate,
                   int in_dtype, const float *r_k, const float *ln_w, const float *ln_b, float eps, void *x,
                   int x_dtype, int B, int T, int H, int N, void *stream)
{
    int64_t tok = 0;
    if (N != kN)
        return WKV7_ERR_UNSUPPORTED;
    const int dts[3] = {o_dtype, in_dtype, x_dtype};
    for (int dt : dts)
        if (dt != WKV7_F32 && dt != WKV7_BF16)
            return WKV7_ERR_UNSUPPORTED;
    if (!shape_ok(B, T, H, &tok) || tok > kMaxRowsTail)
        return WKV7_ERR_SHAPE;
    if (T > 0 && (!o || !r || !k || !v || !x))
        return WKV7_ERR_NULL;
    if (T == 0)
        return check_tail_inputs(gate, r_k, ln_w, ln_b, in_dtype, B, T, H, nullptr, 0);
    const void *ptrs[] = {o, r, k, v, x};
    for (const void *ptr : ptrs)
        if (misaligned(ptr))
            return WKV7_ERR_ALIGN;
    const int64_t n = tok * kN;
    const int64_t eo = o_dtype == WKV7_BF16 ? 2 : 4, ein = in_dtype == WKV7_BF16 ? 2 : 4;
    const int64_t ex = x_dtype == WKV7_BF16 ? 2 : 4;
    const Range rx = range_of(x, n * ex);
    // x may be o itself when both have one type (each lane reads its element before writing it)
    if (overlap(rx, range_of(o, n * eo)) && !(x == o && x_dtype == o_dtype))
        return WKV7_ERR_ALIAS;
    const void *vin[3] = {r, k, v};
    for (const void *ptr : vin)
        if (overlap(rx, range_of(ptr, n * ein)))
            return WKV7_ERR_ALIAS;
    int st = check_tail_inputs(gate, r_k, ln_w, ln_b, in_dtype, B, T, H, &rx, 1);
    if (st != WKV7_OK)
        return st;
    wkv7::TailArgs t;
    t.o = o; t.r = r; t.k = k; t.v = v; t.gate = gate;
    t.r_k = r_k; t.ln_w = ln_w; t.ln_b = ln_b; t.eps = eps;
    t.x = x; t.rows = tok; t.H = H;
    t.in_bf16 = in_dtype == WKV7_BF16;
    t.o_bf16 = o_dtype == WKV7_BF16;
    t.x_bf16 = x_dtype == WKV7_BF16;
    return wkv7::launch_tail(t, static_cast<hipStream_t>(stream)) == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

int wkv7_state_commit(const float *state_pos, const int *accepted, const float *state_in, float *state_out,
                      int B, int T, int H, int N, void *stream)
{
    int64_t tok = 0;
    if (N != kN)
        return WKV7_ERR_UNSUPPORTED;
    if (!shape_ok(B, T, H, &tok, kMaxHeadsStep))
        return WKV7_ERR_SHAPE;
    if (!accepted || !state_out || (T > 0 && !state_pos))
        return WKV7_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(accepted) & 3u) != 0)
        return WKV7_ERR_ALIGN;
    const void *ptrs[] = {state_pos, state_in, state_out};
    for (const void *ptr : ptrs)
        if (ptr && misaligned(ptr))
            return WKV7_ERR_ALIGN;
    const int64_t st_bytes = static_cast<int64_t>(B) * H * kN * kN * 4;
    const Range rst = range_of(state_out, st_bytes);
    const Range racc = range_of(accepted, static_cast<int64_t>(B) * 4);
    Range rpos{0, 0}, rin{0, 0};
    if (T > 0)
        rpos = range_of(state_pos, tok * kN * kN * 4);
    if (state_in)
        rin = range_of(state_in, st_bytes);
    if (overlap(rst, rpos) || overlap(rst, racc) || (state_in && state_in != state_out && overlap(rst, rin)))
        return WKV7_ERR_ALIAS;
    return wkv7::launch_state_commit(state_pos, accepted, state_in, state_out, B, T, H,
                                     static_cast<hipStream_t>(stream)) == hipSuccess
               ? WKV7_OK
               : WKV7_ERR_HIP;
}

int wkv7_backward(const void *r, const void *w, const void *k, const void *v, const void *a, const void *b,
                  int in_dtype, const float *state_in, const float *state_pos, const float *d_o,
                  const float *d_state_out, float *dr, float *dw, float *dk, float *dv, float *da, float *db,
                  float *d_state_in, int B, int T, int H, int N, void *stream)
{
    wkv7::BwdArgs p{};
    const int st = check_backward(r, w, k, v, a, b, in_dtype, state_in, state_pos, false, d_o, d_state_out, dr, dw,
                                  dk, dv, da, db, d_state_in, B, T, H, N, &p);
    if (st != WKV7_OK)
        return st;
    return wkv7::launch_backward(p, static_cast<hipStream_t>(stream)) == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

int wkv7_forward_ckpt(const void *r, const void *w, const void *k, const void *v, const void *a, const void *b,
                      int in_dtype, const float *state_in, float *o, float *state_out, float *ckpt, int B, int T,
                      int H, int N, void *stream)
{
    int st = check_seq(r, w, k, v, a, b, in_dtype, state_in, o, WKV7_F32, state_out, nullptr, B, T, H, N,
                       false, false);
    if (st != WKV7_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0)
        return empty_sequence(state_in, state_out, B, H, s);
    if (!ckpt)
        return WKV7_ERR_NULL;
    if (misaligned(ckpt))
        return WKV7_ERR_ALIGN;
    // the checkpoints overlap no input and no other output
    const int64_t ein = in_dtype == WKV7_BF16 ? 2 : 4;
    const int64_t vec = static_cast<int64_t>(B) * T * H * kN, st_bytes = static_cast<int64_t>(B) * H * kN * kN * 4;
    const Range rc = range_of(ckpt, ckpt_bytes(B, T, H));
    const void *seq[] = {r, w, k, v, a, b};
    for (const void *ptr : seq)
        if (overlap(rc, range_of(ptr, vec * ein)))
            return WKV7_ERR_ALIAS;
    if (overlap(rc, range_of(o, vec * 4)) || overlap(rc, range_of(state_out, st_bytes)) ||
        (state_in && overlap(rc, range_of(state_in, st_bytes))))
        return WKV7_ERR_ALIAS;
    SeqArgs args = make_args(r, w, k, v, a, b, in_dtype, state_in, o, WKV7_F32, state_out, nullptr, B, T, H);
    if (T >= kChunkMinT) {
        args.ckpt = ckpt;
        return wkv7::launch_chunk(args, s) == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
    }
    // one chunk: its checkpoint is the input state, taken before the pass (which may
    // update that state in place)
    if (wkv7::launch_ckpt_from_state(state_in, ckpt, B, H, s) != hipSuccess)
        return WKV7_ERR_HIP;
    return wkv7::launch_step(args, s) == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

int wkv7_backward_ckpt(const void *r, const void *w, const void *k, const void *v, const void *a,
                       const void *b, int in_dtype, const float *ckpt, const float *d_o, const float *d_state_out,
                       float *dr, float *dw, float *dk, float *dv, float *da, float *db, float *d_state_in, int B,
                       int T, int H, int N, void *stream)
{
    wkv7::BwdArgs p{};
    const int st = check_backward(r, w, k, v, a, b, in_dtype, nullptr, ckpt, true, d_o, d_state_out, dr, dw, dk,
                                  dv, da, db, d_state_in, B, T, H, N, &p);
    if (st != WKV7_OK)
        return st;
    return wkv7::launch_backward_chunked(p, static_cast<hipStream_t>(stream)) == hipSuccess ? WKV7_OK
                                                                                             : WKV7_ERR_HIP;
}

const char *wkv7_status_string(int status)
{
    switch (status) {
    case WKV7_OK: return "WKV7_OK: success";
    case WKV7_ERR_NULL: return "WKV7_ERR_NULL: a required pointer is NULL";
    case WKV7_ERR_SHAPE: return "WKV7_ERR_SHAPE: B and H must be >= 1, T >= 0, and sizes must fit in int64";
    case WKV7_ERR_UNSUPPORTED: return "WKV7_ERR_UNSUPPORTED: N must be 64 and dtypes WKV7_F32 or WKV7_BF16";
    case WKV7_ERR_ALIGN: return "WKV7_ERR_ALIGN: every buffer must be 16-byte aligned";
    case WKV7_ERR_ALIAS: return "WKV7_ERR_ALIAS: an output overlaps another buffer (only state_out == state_in is allowed)";
    case WKV7_ERR_HIP: return "WKV7_ERR_HIP: the HIP runtime refused a launch";
    default: return "unknown wkv7 status";
    }
}

int wkv7_abi_version(void) { return WKV7_ABI_VERSION; }

}  // extern "C"
