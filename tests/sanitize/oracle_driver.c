/*
 * Runs the C oracle (oracle/wkv7_oracle.c) over a spread of shapes under
 * AddressSanitizer and UndefinedBehaviorSanitizer: float and double carriers, with
 * and without an input state and per-position states, one and several threads,
 * T = 0, N = 1 and a head size other than 64.  Buffers are heap blocks of exactly
 * the documented sizes, so any read or write past them aborts the run.  Also checks
 * the argument errors and one exact value (N = 1: o_t = r_t S_t with scalar S).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int wkv7_oracle_forward(const void *r, const void *w, const void *k, const void *v, const void *a, const void *b,
                        int in_is_f64, const double *state_in, double *o, double *state_out, double *state_pos,
                        int64_t B, int64_t T, int64_t H, int64_t N, int nthreads);

static unsigned long long rng = 88172645463325252ull;
static double urand(void)
{
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0 - 0.5;
}

static int run(int64_t B, int64_t T, int64_t H, int64_t N, int f64, int with_state, int with_pos, int threads)
{
    const size_t nin = (size_t)(B * T * H * N), nst = (size_t)(B * H * N * N);
    const size_t es = f64 ? sizeof(double) : sizeof(float);
    void *x[6];
    for (int q = 0; q < 6; ++q) {
        x[q] = malloc(nin ? nin * es : 1);
        for (size_t e = 0; e < nin; ++e) {
            double val = q == 1 ? 0.5 + urand() : urand();
            if (f64)
                ((double *)x[q])[e] = val;
            else
                ((float *)x[q])[e] = (float)val;
        }
    }
    double *s_in = with_state ? malloc(nst * sizeof(double)) : NULL;
    for (size_t e = 0; with_state && e < nst; ++e)
        s_in[e] = urand();
    double *o = malloc(nin ? nin * sizeof(double) : 1);
    double *s_out = malloc(nst * sizeof(double));
    double *s_pos = with_pos ? malloc(nin * N ? nin * N * sizeof(double) : 1) : NULL;
    int rc = wkv7_oracle_forward(x[0], x[1], x[2], x[3], x[4], x[5], f64, s_in, o, s_out, s_pos, B, T, H, N, threads);
    if (rc == 0 && T == 0)
        for (size_t e = 0; e < nst; ++e)
            if (s_out[e] != (with_state ? s_in[e] : 0.0))
                rc = 100;
    for (int q = 0; q < 6; ++q)
        free(x[q]);
    free(s_in); free(o); free(s_out); free(s_pos);
    return rc;
}

int main(void)
{
    int bad = 0;
    const int64_t shapes[][4] = {{1, 1, 1, 64}, {2, 7, 3, 64}, {3, 0, 2, 64}, {1, 5, 1, 1}, {2, 4, 3, 5}, {4, 9, 5, 16}};
    for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s)
        for (int mode = 0; mode < 16; ++mode) {
            const int threads = (mode & 8) ? 4 : 1;
            const int rc = run(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], mode & 1, (mode >> 1) & 1,
                               (mode >> 2) & 1, threads);
            if (rc != 0) {
                fprintf(stderr, "oracle_driver: shape %zu mode %d returned %d\n", s, mode, rc);
                bad = 1;
            }
        }
    /* argument errors */
    double so[4];
    if (wkv7_oracle_forward(NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL, so, NULL, 1, 3, 1, 2, 1) != -1 ||
        wkv7_oracle_forward(NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL, 1, 0, 1, 2, 1) != -1 ||
        wkv7_oracle_forward(NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL, so, NULL, 1, 0, 1, 0, 1) != -1) {
        fprintf(stderr, "oracle_driver: a bad argument was accepted\n");
        bad = 1;
    }
    /* N = 1 by hand: s' = w s + b a s + k v, o = r s' */
    {
        const double r[2] = {2, -1}, w[2] = {0.5, 0.25}, k[2] = {1, 3}, v[2] = {4, -2}, a[2] = {1, 2}, b[2] = {-1, 0.5};
        const double s0 = 3.0;
        double o[2], s1;
        const double e1 = 0.5 * 3 + (-1) * (1 * 3) + 1 * 4;      /* 2.5 */
        const double e2 = 0.25 * e1 + 0.5 * (2 * e1) + 3 * (-2); /* -2.875 */
        if (wkv7_oracle_forward(r, w, k, v, a, b, 1, &s0, o, &s1, NULL, 1, 2, 1, 1, 1) != 0 || o[0] != 2 * e1 ||
            o[1] != -e2 || s1 != e2) {
            fprintf(stderr, "oracle_driver: N = 1 by hand differs\n");
            bad = 1;
        }
    }
    if (!bad)
        printf("oracle_driver: all runs clean\n");
    return bad;
}
