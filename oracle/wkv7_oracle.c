/*
 * wkv7_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The plain, slow fp64 CPU definition of the WKV-7 recurrence (the RWKV-7
 * "generalized delta rule").  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may call it.  It shares no code, header,
 * table or helper with the GPU library and must never be reached from it.
 *
 * What it computes, per (batch b, head h) independently, with the state
 * S[i][j] held as an N x N fp64 matrix whose row i is a KEY channel and whose
 * column j is a VALUE channel:
 *
 *   for t = 0 .. T-1:
 *     sa[j]   = sum_i a_t[i] * S[i][j]                (uses S before this step)
 *     S[i][j] = w_t[i]*S[i][j] + b_t[i]*sa[j] + k_t[i]*v_t[j]
 *     o_t[j]  = sum_i r_t[i] * S[i][j]                (reads S after the update)
 *
 * Passages followed:
 *  - "RWKV-X Architecture" (Pantheon docs), section "WKV-7 Kernel (Generalized
 *    Delta Rule)": one step per timestep and head -- decay, rank-1 delta term,
 *    key-value write, readout, in that order; state is head_size x head_size.
 *  - "Recurrent / linear-attention LLMs on Core AI (RWKV-7, and the no-KV
 *    playbook)", section 1: the state is S = [K,V]; the key-value write is the
 *    outer product k (x) v; the readout is r^T S; the decay and the rank-1 term
 *    both act on the state the step started from.
 *  - The same section 1 writes the rank-1 term as -(kk*a)(kk^T S); with the
 *    inputs a = -kk and b = kk*a_gate that is exactly b (a^T S), the general
 *    form used here (a and b are taken as two independent vectors).
 *  - SwiftRWKV Inference guide, the passage on the recurrent and parallel
 *    passes: the token-by-token loop is the reference the fast path is checked
 *    against; both passes compute the same function.
 *
 * Sums run over ascending i.  The file is compiled with -ffp-contract=off so
 * that no multiply-add is fused and the result does not depend on the
 * compiler.  Inputs arrive as fp32 or fp64; bf16 and fp32 values convert to
 * fp64 exactly, so the oracle sees the same numbers the GPU path sees.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    const void *r, *w, *k, *v, *a, *b; /* [B,T,H,N] */
    int in_is_f64;                      /* 0: float inputs, 1: double inputs */
    const double *state_in;             /* [B,H,N,N] or NULL (zeros)        */
    double *o;                          /* [B,T,H,N]                        */
    double *state_out;                  /* [B,H,N,N]                        */
    double *state_pos;                  /* [B,T,H,N,N] or NULL              */
    int64_t B, T, H, N;
    int64_t next;                       /* next (b,h) pair to take          */
    pthread_mutex_t lock;
    int failed;
} oracle_job;

static double ld(const void *p, int is_f64, int64_t idx)
{
    return is_f64 ? ((const double *)p)[idx] : (double)((const float *)p)[idx];
}

/* One head over the whole sequence: the definition above, written out. */
static int run_one_head(oracle_job *J, int64_t bb, int64_t hh)
{
    const int64_t N = J->N, T = J->T, H = J->H;
    double *S = (double *)malloc((size_t)(N * N) * sizeof(double));
    double *sa = (double *)malloc((size_t)N * sizeof(double));
    double *rt = (double *)malloc((size_t)N * 6 * sizeof(double));
    if (!S || !sa || !rt) {
        free(S); free(sa); free(rt);
        return -1;
    }
    double *wt = rt + N, *kt = rt + 2 * N, *vt = rt + 3 * N, *at = rt + 4 * N, *bt = rt + 5 * N;
    const int64_t sbase = (bb * H + hh) * N * N;
    for (int64_t e = 0; e < N * N; ++e)
        S[e] = J->state_in ? J->state_in[sbase + e] : 0.0;

    for (int64_t t = 0; t < T; ++t) {
        const int64_t base = ((bb * T + t) * H + hh) * N;
        for (int64_t i = 0; i < N; ++i) {
            rt[i] = ld(J->r, J->in_is_f64, base + i);
            wt[i] = ld(J->w, J->in_is_f64, base + i);
            kt[i] = ld(J->k, J->in_is_f64, base + i);
            vt[i] = ld(J->v, J->in_is_f64, base + i);
            at[i] = ld(J->a, J->in_is_f64, base + i);
            bt[i] = ld(J->b, J->in_is_f64, base + i);
        }
        /* sa = S^T a over the state before this step */
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < N; ++i)
                acc += at[i] * S[i * N + j];
            sa[j] = acc;
        }
        /* decay the rows, add the rank-1 delta term and the key-value write */
        for (int64_t i = 0; i < N; ++i)
            for (int64_t j = 0; j < N; ++j)
                S[i * N + j] = wt[i] * S[i * N + j] + bt[i] * sa[j] + kt[i] * vt[j];
        /* read out after the update: o = S^T r */
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < N; ++i)
                acc += rt[i] * S[i * N + j];
            J->o[base + j] = acc;
        }
        if (J->state_pos) {
            double *dst = J->state_pos + (((bb * T + t) * H + hh) * N * N);
            memcpy(dst, S, (size_t)(N * N) * sizeof(double));
        }
    }
    memcpy(J->state_out + sbase, S, (size_t)(N * N) * sizeof(double));
    free(S); free(sa); free(rt);
    return 0;
}

static void *worker(void *arg)
{
    oracle_job *J = (oracle_job *)arg;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t p = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (p >= J->B * J->H)
            break;
        if (run_one_head(J, p / J->H, p % J->H) != 0) {
            pthread_mutex_lock(&J->lock);
            J->failed = 1;
            pthread_mutex_unlock(&J->lock);
        }
    }
    return NULL;
}

/* Number of threads a call with nthreads <= 0 would use. */
int wkv7_oracle_default_threads(void)
{
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/*
 * Runs the recurrence.  Returns 0 on success, -1 on a bad argument, -2 when
 * memory runs out.  o, state_out (and state_pos if given) are written in full.
 */
int wkv7_oracle_forward(const void *r, const void *w, const void *k, const void *v,
                        const void *a, const void *b, int in_is_f64,
                        const double *state_in, double *o, double *state_out,
                        double *state_pos, int64_t B, int64_t T, int64_t H, int64_t N,
                        int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || N <= 0 || !state_out || (T > 0 && (!o || !r || !w || !k || !v || !a || !b)))
        return -1;
    oracle_job J;
    memset(&J, 0, sizeof(J));
    J.r = r; J.w = w; J.k = k; J.v = v; J.a = a; J.b = b;
    J.in_is_f64 = in_is_f64;
    J.state_in = state_in; J.o = o; J.state_out = state_out; J.state_pos = state_pos;
    J.B = B; J.T = T; J.H = H; J.N = N;
    pthread_mutex_init(&J.lock, NULL);
    int64_t pairs = B * H;
    if (nthreads <= 0)
        nthreads = wkv7_oracle_default_threads();
    if (nthreads > pairs)
        nthreads = (int)(pairs > 0 ? pairs : 1);
    if (nthreads <= 1) {
        worker(&J);
    } else {
        pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
        if (!th) {
            worker(&J);
        } else {
            int started = 0;
            for (int i = 0; i < nthreads; ++i)
                if (pthread_create(&th[i], NULL, worker, &J) == 0)
                    ++started;
            if (started == 0)
                worker(&J);
            for (int i = 0; i < started; ++i)
                pthread_join(th[i], NULL);
            free(th);
        }
    }
    pthread_mutex_destroy(&J.lock);
    return J.failed ? -2 : 0;
}
