/*
 * wkv7.h -- libwkv7: the WKV-7 recurrence (RWKV-7 "generalized delta rule")
 * on AMD Instinct MI355X (gfx950).
 *
 * THE OPERATION.  Per batch row b and head h the library carries an N x N fp32
 * state S (N = 64).  Row i of S is a key channel, column j a value channel
 * (S = [K,V], as in the Core AI RWKV-7 note, section 1, and the head_size x
 * head_size state of the RWKV-X Architecture page, section "WKV-7 Kernel
 * (Generalized Delta Rule)").  For each token t:
 *
 *     sa[j]   = sum_i a_t[i] * S[i][j]                 (state before the step)
 *     S[i][j] = w_t[i]*S[i][j] + b_t[i]*sa[j] + k_t[i]*v_t[j]
 *     o_t[j]  = sum_i r_t[i] * S[i][j]                 (state after the step)
 *
 * i.e. S_t = diag(w_t) S_{t-1} + b_t (a_t^T S_{t-1}) + k_t v_t^T, o_t = S_t^T r_t.
 * RWKV-7 feeds a = -kk and b = kk*a_gate (the Core AI note writes the rank-1
 * term as -(kk*a)(kk^T S)); the library takes a and b as two general vectors.
 * w is the decay MULTIPLIER (RWKV-7 keeps it in (0.545, 1)), not its log.
 *
 * The SwiftRWKV Inference guide describes the two passes this library
 * provides: a parallel pass over a whole prompt (wkv7_forward, prefill) and a
 * recurrent pass one token at a time (wkv7_step, decode).  They compute the
 * same function and differ only in summation order.  wkv7_step also serves the
 * verify pass of speculative decoding (RWKV7-MTP-Exp model card, section
 * "Inference": the base model runs [t, d1..dK] in one forward and its recurrent
 * state is rolled back to the accepted prefix), for which it can emit the
 * state after every position.
 *
 * LAYOUTS (all row-major, contiguous, no padding):
 *   r, w, k, v, a, b, o : [B, T, H, N]      element (b,t,h,n) at ((b*T+t)*H+h)*N+n
 *   state_in, state_out : [B, H, N, N] fp32 element (b,h,i,j) at ((b*H+h)*N+i)*N+j
 *   state_pos           : [B, T, H, N, N] fp32, [b,t,h] = S after token t
 *   ckpt                : [B, ceil(T/16), H, N*N] fp32, [b,c,h] = S before token 16c,
 *                         its element (i,j) at (j/16)*1024 + (i/16)*256 + (i/4%4)*64
 *                         + (j%16)*4 + i%4 (tile order, see wkv7_forward_ckpt)
 *
 * MEMORY.  Every pointer is a DEVICE pointer on the current HIP device,
 * 16-byte aligned.  The caller owns every buffer; the library never
 * allocates, frees or synchronises, and keeps no global mutable state.
 *
 * ASYNCHRONY.  Calls enqueue on `stream` (a hipStream_t; NULL = the default
 * stream) and return.  Argument errors are detected before any HIP call and
 * reported synchronously; nothing is enqueued then.  WKV7_ERR_HIP reports a
 * failed launch; faults inside a kernel surface at the caller's next
 * synchronisation.
 *
 * ALIASING.  state_out may equal state_in exactly (update in place).  Any
 * other overlap between an output (o, state_out, state_pos) and any other
 * buffer of the call is refused with WKV7_ERR_ALIAS.
 *
 * NUMERICS.  The state and every accumulation are fp32.  bf16 inputs are
 * widened exactly.  NaN / Inf propagate as the arithmetic dictates: value
 * channels stay independent (a NaN in v[b,t,h,j] reaches only column j of that
 * head, from token t on), except that the chunked kernel of wkv7_forward forms
 * the outputs of 16 tokens together, so there it can also reach the earlier
 * tokens of the same 16-token chunk.  Results
 * match an fp64 evaluation of the definition to a relative L2 error of about
 * 1e-6 (fp32 inputs) and well under 2e-3 (bf16 inputs, fp32 state).
 */
#ifndef WKV7_H
#define WKV7_H

#ifdef __cplusplus
extern "C" {
#endif

/* 2: commit and variable-length rows; 3: the two tail entry points; 4: the
 * backward pass; 5: wkv7_forward_tail (and the chunked kernel exact for every
 * decay); 6: wkv7_forward_ckpt and wkv7_backward_ckpt; 7: the checkpoints in
 * tile order (version 6 kept each checkpoint state row-major).  No other entry
 * point's meaning changed in any of these. */
#define WKV7_ABI_VERSION 7

/* Element types of r, w, k, v, a, b (in_dtype) and of o (o_dtype). */
enum wkv7_dtype {
    WKV7_F32 = 0,  /* IEEE binary32 */
    WKV7_BF16 = 1  /* bfloat16; o is rounded to nearest even when requested */
};

/* Return codes.  Every entry point returns one of these. */
enum wkv7_status {
    WKV7_OK = 0,
    WKV7_ERR_NULL = -1,        /* a required pointer is NULL                          */
    WKV7_ERR_SHAPE = -2,       /* B, H < 1, T < 0, a size overflows int64, or a call
                                  exceeds what one launch covers (WKV7_MAX_* below)   */
    WKV7_ERR_UNSUPPORTED = -3, /* N != 64, or an unknown dtype                         */
    WKV7_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned                     */
    WKV7_ERR_ALIAS = -5,       /* an output overlaps another buffer (see ALIASING)     */
    WKV7_ERR_HIP = -6          /* the HIP runtime refused a launch or a query          */
};

/*
 * Size limits (WKV7_ERR_SHAPE beyond them).  Each head runs as one or a few
 * workgroups of one launch, and a launch holds fewer than 2^32 threads:
 *   B * H <= WKV7_MAX_HEADS_STEP   for wkv7_step, wkv7_step_tail, wkv7_state_commit, wkv7_backward,
 *                                  wkv7_backward_ckpt, and wkv7_forward[_varlen] with T < 9;
 *   B * H <= WKV7_MAX_HEADS_CHUNK  for wkv7_forward[_varlen] with T >= 9;
 *   H <= WKV7_MAX_H_CHUNK           for wkv7_forward[_varlen] with T >= 9 (a lane of the
 *                                  chunked kernel addresses its 16 tokens' outputs with 32-bit
 *                                  byte offsets from the chunk's first output row);
 *   B * T * H <= WKV7_MAX_ROWS_TAIL for wkv7_tmix_tail.
 * Tensor offsets are 64-bit: tensors of more than 2^32 elements are supported
 * within these limits.
 */
#define WKV7_MAX_HEADS_STEP 8000000
#define WKV7_MAX_HEADS_CHUNK 4000000
#define WKV7_MAX_H_CHUNK 1048576
#define WKV7_MAX_ROWS_TAIL 200000000

/*
 * wkv7_forward -- the parallel (prefill) pass over T tokens.
 *
 *   r, w, k, v, a, b : [B,T,H,N] inputs of type in_dtype (WKV7_F32 | WKV7_BF16).
 *   state_in         : [B,H,N,N] fp32 state entering token 0; NULL = all zeros.
 *   o                : [B,T,H,N] outputs of type o_dtype (WKV7_F32 | WKV7_BF16).
 *   state_out        : [B,H,N,N] fp32 state after token T-1 (may == state_in).
 *   B, T, H, N       : batch, tokens, heads, head size (N must be 64).
 *   stream           : hipStream_t to enqueue on, or NULL.
 *
 * Long sequences run a chunked-parallel kernel (chunks of 16 tokens, a
 * triangular solve for the rank-1 terms inside a chunk, matrix-core products,
 * and the state carried from chunk to chunk in order); short ones run the
 * step kernel.  T = 0 copies state_in to state_out (zeros if state_in is NULL)
 * and leaves o untouched.  Every decay in [0, 1] is taken exactly: a chunk of
 * 16 tokens that holds a decay below 2^-15 (where the chunk form's decay
 * factors would leave the fp32 range) is evaluated token by token instead,
 * which costs that chunk several times its usual time; RWKV-7's decays
 * (>= 0.545) never come near that bound.
 */
int wkv7_forward(const void *r, const void *w, const void *k, const void *v,
                 const void *a, const void *b, int in_dtype,
                 const float *state_in, void *o, int o_dtype, float *state_out,
                 int B, int T, int H, int N, void *stream);

/*
 * wkv7_forward_varlen -- wkv7_forward over right-padded rows of their own lengths
 * (batched prefill of prompts of different lengths).
 *
 * Arguments as for wkv7_forward, plus
 *   lengths : [B] int32 on the device (4-byte aligned).  Row b runs its first
 *             L_b = lengths[b] tokens, L_b clamped to [0, T]: o[b, t] for
 *             t < L_b and state_out[b] (the state after those L_b tokens;
 *             state_in[b], or zeros, when L_b = 0) are written, and o[b, t]
 *             for t >= L_b is left untouched.  The inputs keep the [B,T,H,N]
 *             layout with row stride T; the values past L_b are not read.
 * A NULL lengths is refused (WKV7_ERR_NULL); lengths may not overlap o or
 * state_out (WKV7_ERR_ALIAS).  The lengths are device values, so they are not
 * checked here: values outside [0, T] are clamped by the kernels.
 */
int wkv7_forward_varlen(const void *r, const void *w, const void *k, const void *v,
                        const void *a, const void *b, int in_dtype,
                        const float *state_in, void *o, int o_dtype, float *state_out,
                        const int *lengths, int B, int T, int H, int N, void *stream);

/*
 * wkv7_step -- the recurrent (decode / speculative-verify) pass, token by token.
 *
 * Arguments as for wkv7_forward, plus
 *   state_pos : [B,T,H,N,N] fp32, or NULL.  When given, state_pos[b,t,h] is the
 *               state after token t, so a caller can keep the state after any
 *               accepted prefix of a speculative step (state_pos[:,T-1] equals
 *               state_out).  With state_pos given and T > 0, state_out may be
 *               NULL: the final state is then only in state_pos (a verify step
 *               followed by wkv7_state_commit needs no separate copy).
 * Meant for small T (1 for decode, K+1 for a verify step), but correct for
 * any T >= 0.  Exact for every decay in [0, 1].
 */
int wkv7_step(const void *r, const void *w, const void *k, const void *v,
              const void *a, const void *b, int in_dtype,
              const float *state_in, void *o, int o_dtype, float *state_out,
              float *state_pos, int B, int T, int H, int N, void *stream);

/*
 * wkv7_state_reset -- zero the recurrent state (the RWKV-X Architecture page,
 * section "Dual State": a reset zeros the recurrent state).
 *
 *   state    : [B,H,N,N] fp32.
 *   row_mask : [B] bytes on the device, or NULL.  NULL zeros every batch row;
 *              otherwise row b is zeroed iff row_mask[b] != 0 and the other rows
 *              are left untouched.  (The mask itself needs no alignment.)
 */
int wkv7_state_reset(float *state, int B, int H, int N, const unsigned char *row_mask,
                     void *stream);

/*
 * THE TIME-MIX TAIL.  The SwiftRWKV Inference guide (its decode-path list and
 * the fused frozen pass) fuses the three steps that follow WKV in an RWKV-7
 * block -- group norm, bonus and gate -- and names only those parts.  The
 * reading taken here, per (b, t, h) over the N value channels j of o:
 *     mu   = mean_j o[j],  var = mean_j (o[j] - mu)^2                (biased)
 *     y[j] = (o[j] - mu) / sqrt(var + eps) * ln_w[h,j] + ln_b[h,j]
 *     x[j] = (y[j] + (sum_i r[i] k[i] r_k[h,i]) * v[j]) * g[j]
 * with r, k, v the WKV inputs of the same token, g the gate, and r_k, ln_w,
 * ln_b [H,N] fp32 per-head parameters (16-byte aligned).  The arithmetic is
 * fp32; eps is taken as given (eps <= 0 with a constant row gives Inf / NaN).
 */

/*
 * wkv7_step_tail -- wkv7_step with the time-mix tail fused into its epilogue:
 * each token's o never leaves the kernel, and x (type x_dtype, layout of o) is
 * written instead.
 *   gate : [B,T,H,N] of in_dtype;  r_k, ln_w, ln_b : [H,N] fp32;  eps : as above.
 * Every other argument as for wkv7_step (x in the place of o).  gate, r_k,
 * ln_w and ln_b may not overlap x, state_out or state_pos.
 */
int wkv7_step_tail(const void *r, const void *w, const void *k, const void *v,
                   const void *a, const void *b, int in_dtype, const float *state_in,
                   const void *gate, const float *r_k, const float *ln_w, const float *ln_b,
                   float eps, void *x, int x_dtype, float *state_out, float *state_pos,
                   int B, int T, int H, int N, void *stream);

/*
 * wkv7_forward_tail -- wkv7_forward with the time-mix tail fused: the parallel
 * (prefill) pass writes x (type x_dtype, layout of o) instead of o, and o never
 * reaches memory.  The SwiftRWKV Inference guide runs this tail over the B*T rows
 * of its parallel pass (the fused frozen pass).
 *   gate : [B,T,H,N] of in_dtype;  r_k, ln_w, ln_b : [H,N] fp32;  eps : as above.
 * Every other argument as for wkv7_forward (x in the place of o); gate, r_k,
 * ln_w and ln_b may not overlap x or state_out.  With bf16 inputs and T >= 9 one
 * chunked kernel computes both (a head per workgroup; o stays in LDS); shorter
 * sequences take the step kernel with its fused tail.  With fp32 inputs and an fp32
 * x, the chunked kernel writes o into x and the tail pass then runs in place; with
 * fp32 inputs and a bf16 x, the step kernel with its fused tail runs the whole
 * sequence (exact, slower).
 */
int wkv7_forward_tail(const void *r, const void *w, const void *k, const void *v,
                      const void *a, const void *b, int in_dtype, const float *state_in,
                      const void *gate, const float *r_k, const float *ln_w, const float *ln_b,
                      float eps, void *x, int x_dtype, float *state_out,
                      int B, int T, int H, int N, void *stream);

/*
 * wkv7_tmix_tail -- the time-mix tail as a pass of its own, for the output of
 * wkv7_forward / wkv7_forward_varlen (whose chunked kernel spreads one token's
 * outputs over several waves).
 *   o          : [B,T,H,N] of o_dtype (WKV7_F32 | WKV7_BF16).
 *   r, k, v, g : [B,T,H,N] of in_dtype.
 *   r_k, ln_w, ln_b : [H,N] fp32;  eps : as above.
 *   x          : [B,T,H,N] of x_dtype; may be o itself when x_dtype == o_dtype,
 *                otherwise it may not overlap any input.
 * T = 0 does nothing.
 */
int wkv7_tmix_tail(const void *o, int o_dtype, const void *r, const void *k, const void *v,
                   const void *g, int in_dtype, const float *r_k, const float *ln_w,
                   const float *ln_b, float eps, void *x, int x_dtype,
                   int B, int T, int H, int N, void *stream);

/*
 * wkv7_state_commit -- keep the state after each row's accepted prefix of a
 * speculative verify step (RWKV7-MTP-Exp model card, section "Inference": the
 * recurrent state is rolled back to the accepted prefix).
 *
 *   state_pos : [B,T,H,N,N] fp32, the per-position states of wkv7_step
 *               (state_pos[b,t] = state after token t); may be NULL when T = 0.
 *   accepted  : [B] int32 on the device (4-byte aligned): n_b tokens of row b
 *               are accepted.
 *   state_in  : [B,H,N,N] fp32, the state before the step, or NULL (zeros).
 *   state_out : [B,H,N,N] fp32; may equal state_in exactly.
 * Row b of state_out becomes state_pos[b, n_b - 1] for 1 <= n_b <= T and
 * state_in[b] for n_b = 0; a row with n_b outside [0, T] is left untouched
 * (device values are not checked here).  state_out may not overlap state_pos
 * or accepted, and may overlap state_in only by being equal to it.
 */
int wkv7_state_commit(const float *state_pos, const int *accepted, const float *state_in,
                      float *state_out, int B, int T, int H, int N, void *stream);

/*
 * wkv7_backward -- gradients of the recurrence (the backward pass of a trainable
 * WKV layer; the SwiftRWKV Inference guide, its `.rwkvq` backend section, keeps
 * such a kernel).  For a loss L with dL/do = d_o and dL/dS_T = d_state_out it
 * returns dL/d(r, w, k, v, a, b) and dL/d(state_in): the reverse-mode adjoint of
 * the loop of wkv7_forward (RWKV-X Architecture page, section "WKV-7 Kernel
 * (Generalized Delta Rule)").
 *
 *   r, w, k, v, a, b : [B,T,H,N] inputs of the forward pass, of in_dtype.
 *   state_in    : [B,H,N,N] fp32 state before token 0, or NULL (zeros).
 *   state_pos   : [B,T,H,N,N] fp32, the state after each token, as wkv7_step
 *                 writes it (these are read, not rebuilt).
 *   d_o         : [B,T,H,N] fp32 gradient of o.
 *   d_state_out : [B,H,N,N] fp32 gradient of the final state, or NULL (zeros).
 *   dr .. db    : [B,T,H,N] fp32 gradients of the six inputs.
 *   d_state_in  : [B,H,N,N] fp32 gradient of state_in; may equal d_state_out.
 * The inputs may be NULL when T = 0 (then d_state_in becomes d_state_out, or
 * zeros).  No output may overlap another buffer, except d_state_in ==
 * d_state_out.  B * H <= WKV7_MAX_HEADS_STEP.
 * With B * H <= 128 a head runs as two workgroups of 32 value columns each, and
 * the call launches two kernels on the stream: a fill that zeroes dr, dk, dw,
 * db, da, then the pass, whose two workgroups per head add their row sums into
 * them with hardware float atomics (two terms, so the order of the adds does
 * not change the sum).  Those five outputs must then be ordinary device memory
 * (hipMalloc), where such atomics are supported.
 */
int wkv7_backward(const void *r, const void *w, const void *k, const void *v,
                  const void *a, const void *b, int in_dtype, const float *state_in,
                  const float *state_pos, const float *d_o, const float *d_state_out,
                  float *dr, float *dw, float *dk, float *dv, float *da, float *db,
                  float *d_state_in, int B, int T, int H, int N, void *stream);

/*
 * wkv7_forward_ckpt -- the forward pass of training: wkv7_forward (fp32 o) that
 * also keeps the state entering every chunk of 16 tokens, the checkpoints from
 * which wkv7_backward_ckpt rebuilds the rest.  The SwiftRWKV Inference guide
 * (its `.rwkvq` backend section) describes this trainable kernel: it chunks, and
 * its backward pass rebuilds the state chunk by chunk.
 *
 *   ckpt : [B, ceil(T/16), H, N*N] fp32; ckpt[b, c, h] = the state of head h of
 *          row b before token 16 c (state_in, or zeros, for c = 0), in tile
 *          order: element (i, j) (key row i, value column j) at
 *          (j/16)*1024 + (i/16)*256 + (i/4 % 4)*64 + (j % 16)*4 + i % 4.  The
 *          16 x 16 tiles of one block of 16 value columns lie together, and in
 *          a tile each column's values of a group of four rows form one
 *          16-byte unit: the chunked kernel keeps its state in that order, so
 *          each of its stores writes whole contiguous kilobytes.
 * Everything else as wkv7_forward with o_dtype = WKV7_F32.  ckpt may be NULL
 * only when T = 0, and overlaps no other buffer.  For 1 <= T <= 8 (one chunk)
 * the call enqueues a copy of state_in in tile order (or a fill of zeros) into
 * ckpt, then the step kernel; from T = 9 on, the chunked kernel writes the
 * checkpoints itself.
 * The checkpoints carry the chunked kernel's fp32 state: within about 1e-6
 * (relative L2) of the states of the definition.
 */
int wkv7_forward_ckpt(const void *r, const void *w, const void *k, const void *v,
                      const void *a, const void *b, int in_dtype, const float *state_in,
                      float *o, float *state_out, float *ckpt, int B, int T, int H, int N,
                      void *stream);

/*
 * wkv7_backward_ckpt -- wkv7_backward from the checkpoints of wkv7_forward_ckpt
 * instead of per-position states.  The gradient for the state is carried back
 * over the tokens on its own (it needs no states); the gradients of each chunk of
 * 16 tokens then follow from the chunk's checkpoint and that gradient at the
 * chunk's end, in the chunk form of the recurrence (matrix products), for all
 * chunks at once.  A chunk with a decay below 2^-15 in magnitude (w = 0
 * included) runs the recurrence token by token instead.  It reads 1/16 of the
 * state bytes that wkv7_backward reads, and no state_in (ckpt[:, 0] is the input
 * state).
 *
 *   ckpt : [B, ceil(T/16), H, N*N] fp32 in tile order, as wkv7_forward_ckpt
 *          wrote it from the same inputs and state_in.
 * Everything else (d_o, d_state_out, the gradients, NULL rules, aliasing, the
 * limit B * H <= WKV7_MAX_HEADS_STEP) as wkv7_backward.  While the call runs,
 * dr, dk, da and db also hold the gradient for the state at each chunk's end
 * (16 rows of each per chunk) before the gradients replace it.
 */
int wkv7_backward_ckpt(const void *r, const void *w, const void *k, const void *v,
                       const void *a, const void *b, int in_dtype, const float *ckpt,
                       const float *d_o, const float *d_state_out, float *dr, float *dw,
                       float *dk, float *dv, float *da, float *db, float *d_state_in,
                       int B, int T, int H, int N, void *stream);

/* A static, human-readable name for a status code (never NULL). */
const char *wkv7_status_string(int status);

/* WKV7_ABI_VERSION of the built library. */
int wkv7_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WKV7_H */
