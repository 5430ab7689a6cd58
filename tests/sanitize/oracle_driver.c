/*
 * The fp64 oracle's C code under sanitizers (test infrastructure): built
 * together with oracle/ssd_oracle.c with AddressSanitizer and
 * UndefinedBehaviorSanitizer, or with ThreadSanitizer, this driver runs every
 * oracle entry point on small random inputs with several worker threads
 * (more threads than units too), the edge cases (empty and one-token
 * sequences, a subset of units, snapshots, every option) and argument errors,
 * and checks that the outputs are finite. Exit status 0 when every check
 * holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const float *dt_bias;
    int dt_softplus;
    int dt_clamp;
    double dt_min, dt_max;
    int zoh;
} oracle_opts;  /* the oracle's own struct, restated */

int ssd_oracle_forward_ex(const float *x, const float *dt, const float *A, const float *B,
                          const float *C, const float *D, const double *init, int batch,
                          int seqlen, int nheads, int headdim, int ngroups, int dstate,
                          const int *units, int nunits, double *y, double *state, double *snaps,
                          int snap_every, int nthreads, const oracle_opts *opts);
int ssd_oracle_forward_varlen(const float *x, const float *dt, const float *A, const float *B,
                              const float *C, const float *D, int seqlen, int nheads, int headdim,
                              int ngroups, int dstate, const int *cu_seqlens, int nseq,
                              const int *units, int nunits, double *y, double *seq_states,
                              int nthreads, const oracle_opts *opts);
int ssd_oracle_step_ex(double *state, const float *x, const float *dt, const float *A,
                       const float *B, const float *C, const float *D, int batch, int nheads,
                       int headdim, int ngroups, int dstate, const int *units, int nunits,
                       double *y, int nthreads, const oracle_opts *opts);
int ssd_oracle_backward(const float *x, const float *dt, const float *A, const float *B,
                        const float *C, const float *D, const double *init, const float *dy,
                        const double *dfinal, int batch, int seqlen, int nheads, int headdim,
                        int ngroups, int dstate, const int *units, int nunits, double *dx,
                        double *ddt, double *dA, double *dB, double *dC, double *dD,
                        double *dinit, double *dbias, int nthreads, const oracle_opts *opts);

static int failures = 0;
#define EXPECT(cond)                                                                    \
    do {                                                                                \
        if (!(cond)) {                                                                  \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                                 \
        }                                                                               \
    } while (0)

static uint64_t rng = 88172645463325252ull;
static double unif(void) {  /* xorshift64, [0, 1) */
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0;
}
static float *randf(size_t n, double lo, double hi) {
    float *p = malloc((n ? n : 1) * sizeof *p);
    for (size_t i = 0; i < n; ++i) p[i] = (float)(lo + (hi - lo) * unif());
    return p;
}
static double *randd(size_t n, double s) {
    double *p = malloc((n ? n : 1) * sizeof *p);
    for (size_t i = 0; i < n; ++i) p[i] = s * (2 * unif() - 1);
    return p;
}
static double *zerod(size_t n) { return calloc(n ? n : 1, sizeof(double)); }
static int finite_all(const double *p, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

static void run_case(int Bt, int L, int H, int P, int G, int N, int threads, int use_opts) {
    const size_t nx = (size_t)Bt * L * H * P, nbc = (size_t)Bt * L * G * N, nst = (size_t)Bt * H * P * N;
    float *x = randf(nx, -1, 1), *dt = randf((size_t)Bt * L * H, 0.01, 0.2), *A = randf(H, -2, -0.1);
    float *B = randf(nbc, -0.5, 0.5), *C = randf(nbc, -0.5, 0.5), *D = randf(H, -1, 1);
    float *bias = randf(H, -0.1, 0.1), *dy = randf(nx, -1, 1);
    double *init = randd(nst, 0.3), *dfinal = randd(nst, 0.3);
    oracle_opts o = {bias, 1, 1, 0.02, 0.5, 1};
    const oracle_opts *op = use_opts ? &o : NULL;
    const int U = Bt * H;

    /* forward over every unit, with states and snapshots every 3 tokens */
    double *y = zerod(nx), *st = zerod(nst), *snaps = zerod((size_t)U * ((L + 2) / 3 + 1) * P * N);
    EXPECT(ssd_oracle_forward_ex(x, dt, A, B, C, D, init, Bt, L, H, P, G, N, NULL, 0, y, st, snaps, 3,
                                 threads, op) == 0);
    EXPECT(finite_all(y, nx) && finite_all(st, nst));
    /* a subset of units, no D, no initial state */
    int units[3] = {U - 1, 0, U / 2};
    const int nu = U < 3 ? U : 3;
    double *ys = zerod((size_t)nu * L * P);
    EXPECT(ssd_oracle_forward_ex(x, dt, A, B, C, NULL, NULL, Bt, L, H, P, G, N, units, nu, ys, NULL, NULL,
                                 0, threads, op) == 0);
    EXPECT(finite_all(ys, (size_t)nu * L * P));

    /* packed sequences over batch row 0's tokens: an empty and a one-token sequence among them */
    if (L >= 3) {
        int cu[5] = {0, 0, 1, L / 2, L};
        double *yv = zerod((size_t)H * L * P), *sv = zerod((size_t)H * 4 * P * N);
        EXPECT(ssd_oracle_forward_varlen(x, dt, A, B, C, D, L, H, P, G, N, cu, 4, NULL, 0, yv, sv,
                                         threads, op) == 0);
        EXPECT(finite_all(yv, (size_t)H * L * P) && finite_all(sv, (size_t)H * 4 * P * N));
        int bad[3] = {0, 5, 2};  /* decreasing offsets */
        EXPECT(ssd_oracle_forward_varlen(x, dt, A, B, C, D, L, H, P, G, N, bad, 2, NULL, 0, yv, sv,
                                         threads, op) < 0);
        free(yv);
        free(sv);
    }

    /* decode steps from the forward's states */
    float *xs = randf((size_t)Bt * H * P, -1, 1), *dts = randf((size_t)Bt * H, 0.01, 0.2);
    float *Bs = randf((size_t)Bt * G * N, -0.5, 0.5), *Cs = randf((size_t)Bt * G * N, -0.5, 0.5);
    double *yst = zerod((size_t)Bt * H * P);
    for (int s = 0; s < 3; ++s)
        EXPECT(ssd_oracle_step_ex(st, xs, dts, A, Bs, Cs, D, Bt, H, P, G, N, NULL, 0, yst, threads, op) == 0);
    EXPECT(finite_all(yst, (size_t)Bt * H * P) && finite_all(st, nst));

    /* the backward with every optional gradient */
    if (L >= 1) {
        double *dx = zerod(nx), *ddt = zerod((size_t)U * L), *dA = zerod(U), *dB = zerod((size_t)U * L * N);
        double *dC = zerod((size_t)U * L * N), *dD = zerod(U), *dinit = zerod(nst), *dbias = zerod(U);
        EXPECT(ssd_oracle_backward(x, dt, A, B, C, D, init, dy, dfinal, Bt, L, H, P, G, N, NULL, 0, dx,
                                   ddt, dA, dB, dC, dD, dinit, dbias, threads, op) == 0);
        EXPECT(finite_all(dx, nx) && finite_all(ddt, (size_t)U * L) && finite_all(dA, U));
        EXPECT(finite_all(dB, (size_t)U * L * N) && finite_all(dC, (size_t)U * L * N));
        EXPECT(finite_all(dD, U) && finite_all(dinit, nst) && finite_all(dbias, U));
        free(dx), free(ddt), free(dA), free(dB), free(dC), free(dD), free(dinit), free(dbias);
    }

    /* argument errors */
    EXPECT(ssd_oracle_forward_ex(NULL, dt, A, B, C, D, NULL, Bt, L, H, P, G, N, NULL, 0, y, NULL, NULL, 0,
                                 threads, op) < 0);
    EXPECT(ssd_oracle_forward_ex(x, dt, A, B, C, D, NULL, Bt, L, H, P, H + 1, N, NULL, 0, y, NULL, NULL,
                                 0, threads, op) < 0);  /* heads not a multiple of the groups */
    int badu[1] = {U};
    EXPECT(ssd_oracle_forward_ex(x, dt, A, B, C, D, NULL, Bt, L, H, P, G, N, badu, 1, y, NULL, NULL, 0,
                                 threads, op) < 0);

    free(x), free(dt), free(A), free(B), free(C), free(D), free(bias), free(dy), free(init), free(dfinal);
    free(y), free(st), free(snaps), free(ys), free(xs), free(dts), free(Bs), free(Cs), free(yst);
}

int main(void) {
    /* batch, tokens, heads, head dim, groups, state size, threads, options */
    run_case(1, 1, 1, 4, 1, 2, 1, 0);
    run_case(2, 7, 4, 8, 2, 16, 3, 1);
    run_case(2, 33, 6, 16, 3, 8, 16, 0);  /* more threads than units */
    run_case(3, 20, 4, 4, 1, 32, 5, 1);
    run_case(1, 0, 2, 4, 1, 4, 2, 0);     /* no tokens */
    if (failures) fprintf(stderr, "%d expectation(s) failed\n", failures);
    else printf("oracle driver: every check passed\n");
    return failures ? 1 : 0;
}
