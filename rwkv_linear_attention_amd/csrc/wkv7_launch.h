// wkv7_launch.h -- internal launch entry points of the libwkv7 kernels.
// Arguments are validated by the C-ABI layer (wkv7_api.hip) before these run.
#pragma once

#include <hip/hip_runtime.h>

namespace wkv7 {

// Offset of element (i, j) (key row i, value column j) of one head's 64 x 64 state
// within a checkpoint: the state is kept as 16 x 16 tiles, the tiles of one block of
// 16 value columns together (row tiles inside), and within a tile as four groups of
// four rows, each column's four values of a group in one 16-byte unit.
__host__ __device__ constexpr int ckpt_offset(int i, int j)
{
    return (j >> 4) * 1024 + (i >> 4) * 256 + ((i >> 2) & 3) * 64 + (j & 15) * 4 + (i & 3);
}

struct SeqArgs {
    const void *r, *w, *k, *v, *a, *b;  // [B,T,H,64], in_dtype
    const float *state_in;              // [B,H,64,64] or nullptr (zeros)
    void *o;                            // [B,T,H,64], o_dtype
    float *state_out;                   // [B,H,64,64]
    float *state_pos;                   // [B,T,H,64,64] or nullptr
    float *ckpt;                        // [B,ceil(T/16),H,64*64]: state entering each 16-token chunk
                                        // (element order ckpt_offset), or nullptr
    const int *lengths;                 // [B] tokens of each row (clamped to [0, T]), or nullptr: all T
    int B, T, H;
    int in_bf16, o_bf16;                // dtype flags
    // the fused time-mix tail (o then holds x): gate [B,T,H,64] in_dtype, r_k / ln_w / ln_b [H,64]
    const void *gate;                   // nullptr: no tail
    const float *r_k, *ln_w, *ln_b;
    float eps;
};

struct TailArgs {
    const void *o, *r, *k, *v, *gate;   // [B,T,H,64]; o of o_dtype, the rest of in_dtype
    const float *r_k, *ln_w, *ln_b;     // [H,64]
    float eps;
    void *x;                            // [B,T,H,64] of x_dtype
    long long rows;                     // B*T*H
    int H;
    int in_bf16, o_bf16, x_bf16;
};

// the backward pass: gradients of the recurrence given its per-position states
struct BwdArgs {
    const void *r, *w, *k, *v, *a, *b;  // [B,T,H,64], in_dtype
    const float *state_in;              // [B,H,64,64] or nullptr (zeros)
    const float *state_pos;             // [B,T,H,64,64]: the state after each token (wkv7_backward)
    const float *ckpt;                  // [B,ceil(T/16),H,64*64]: the state entering each chunk (ckpt_offset)
    const float *d_o;                   // [B,T,H,64]: gradient of o
    const float *d_state_out;           // [B,H,64,64] or nullptr (zeros)
    float *dr, *dw, *dk, *dv, *da, *db; // [B,T,H,64]
    float *d_state_in;                  // [B,H,64,64]
    int B, T, H;
    int in_bf16;
};

hipError_t launch_step(const SeqArgs &a, hipStream_t stream);
hipError_t launch_chunk(const SeqArgs &a, hipStream_t stream);
hipError_t launch_ckpt_from_state(const float *state, float *ckpt, int B, int H, hipStream_t stream);
hipError_t launch_state_copy(const float *src, float *dst, long long n_floats, hipStream_t stream);
hipError_t launch_state_reset(float *state, int B, int H, const unsigned char *row_mask,
                              hipStream_t stream);
hipError_t launch_tail(const TailArgs &a, hipStream_t stream);
hipError_t launch_backward(const BwdArgs &a, hipStream_t stream);
hipError_t launch_backward_chunked(const BwdArgs &a, hipStream_t stream);
hipError_t launch_state_commit(const float *state_pos, const int *accepted, const float *state_in,
                               float *state_out, int B, int T, int H, hipStream_t stream);

}  // namespace wkv7
