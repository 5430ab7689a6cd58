/*
 * Plain fp64 CPU oracle for the selective state-space (SSD) layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls
 * this file; it is used by the tests, by the smoke check and by the benchmark's
 * CPU-baseline leg. It shares no code with the HIP library.
 *
 * What it computes is the token-by-token recurrence, written out directly:
 *
 *   per head h (B/C group g = h / (H/G)), state hs in R^{P x N}, for t = 0..L-1:
 *     a        = exp(dt_t * A_h)                       decay of the step
 *     hs[p][n] = a * hs[p][n] + dt_t * x_t[p] * B_t[n] input enters the state
 *     y_t[p]   = sum_n C_t[n] * hs[p][n] + D_h * x_t[p] output read after update
 *
 * Sources (titles and sections of the pages):
 *   - "从Transformer到Mamba" tutorial, section 2.2 (discretisation): the
 *     discrete recurrence x_k = Abar x_{k-1} + Bbar u_k, y_k = C x_k with
 *     Abar = exp(dt A); the output is taken from the updated state.
 *   - same page, section 2.1, and "深挖-Mamba", core concept 1 (SSM): the
 *     D x feed-through term.
 *   - "深挖-Mamba", core concept 3 (selective scan), and the tutorial's
 *     section 3.2: dt, B and C are per token, A is shared (one scalar per
 *     head here, as in the Mamba-2 "Draft:Mamba2" page's SSD section).
 *   - The input is scaled by dt (Bbar = dt * B), the Euler form the layer is
 *     defined with. Optionally (the _ex entry points) the input weight is the
 *     zero-order hold of the tutorial's section 2.2 and "Mamba 模型" section
 *     2.3.1, Bbar = (dA)^-1 (exp(dA) - 1) dB, which for a scalar A is
 *     (exp(dt A) - 1) / A * B (and dt * B at A = 0).
 *   - Optionally dt is preprocessed. The tutorial's section 3.2 makes the
 *     step size a linear projection of the input made positive by softplus
 *     (log(1 + e^v)); the projection's constant term is taken as a per-head
 *     bias added before softplus. Its section 8.2 speaks of adjusting the
 *     range the step sizes are produced in; that is read as an optional clamp
 *     to [dt_min, dt_max] after softplus.
 *   - Packed variable-length sequences (ssd_oracle_forward_varlen): several
 *     sequences concatenated along the token axis, each with its own
 *     recurrence. The state is reset to zero where a sequence begins, and
 *     each sequence's state after its last token is kept (the dynamic packing
 *     of variable-length sequences on the "Mamba-2架构深度解析" page, section 5).
 * The state is stored transposed to the usual N x P: hs[p][n], n fastest.
 *
 * All token inputs arrive as float32 arrays holding the exact values the GPU
 * reads (bf16 values are exact in float32) and are promoted to double; the
 * optional initial state is double.
 *
 * Work is split over independent (batch, head) units with POSIX threads; each
 * unit runs its tokens strictly in order.
 */
#include <math.h>
#include <pthread.h>
#include <stdatomic.h>
#include <stdlib.h>
#include <string.h>

/* Preprocessing of dt and the input discretisation (all off when NULL). */
typedef struct {
    const float *dt_bias; /* [nheads] or NULL: added to dt first */
    int dt_softplus;      /* nonzero: dt <- log(1 + exp(dt)) */
    int dt_clamp;         /* nonzero: dt <- min(max(dt, dt_min), dt_max) */
    double dt_min, dt_max;
    int zoh;              /* nonzero: input weight (exp(dt A) - 1) / A instead of dt */
} oracle_opts;

/* The step size the recurrence uses for raw dt value v of head h. */
static double step_size(const oracle_opts *o, double v, int h)
{
    if (!o) return v;
    if (o->dt_bias) v += (double)o->dt_bias[h];
    if (o->dt_softplus) v = fmax(v, 0.0) + log1p(exp(-fabs(v))); /* log(1 + e^v), no overflow */
    if (o->dt_clamp) v = fmin(fmax(v, o->dt_min), o->dt_max);
    return v;
}

/* The weight of the input term for step size d: dt (Euler) or the zero-order
 * hold (exp(d A) - 1) / A, with expm1 so that small d A keeps its digits. */
static double input_weight(const oracle_opts *o, double d, double A)
{
    if (o && o->zoh) return A != 0.0 ? expm1(d * A) / A : d;
    return d;
}

typedef struct {
    const float *x, *dt, *A, *B, *C, *D;
    const double *init;
    int batch, seqlen, nheads, headdim, ngroups, dstate;
    const int *units;
    int nunits;
    double *y;      /* [nunits][seqlen][headdim] */
    double *state;  /* [nunits][headdim][dstate] final state (may be NULL) */
    double *snaps;  /* [nunits][seqlen/snap_every][headdim][dstate] (may be NULL) */
    int snap_every;
    const oracle_opts *opts;
    const int *cu;       /* packed sequences: offsets [nseq + 1], or NULL */
    int nseq;
    double *seq_states;  /* [nunits][nseq][headdim][dstate]: state after each sequence */
    atomic_int next;
} fwd_job;

static void fwd_unit(fwd_job *j, int u, double *hs)
{
    const int H = j->nheads, P = j->headdim, N = j->dstate, L = j->seqlen;
    const int G = j->ngroups;
    const int bh = j->units ? j->units[u] : u;
    const int b = bh / H, h = bh % H;
    const int g = h / (H / G);
    const double A = j->A[h];
    const double D = j->D ? j->D[h] : 0.0;
    const size_t PN = (size_t)P * N;

    if (j->init) {
        const double *s0 = j->init + (size_t)bh * PN;
        for (size_t k = 0; k < PN; ++k) hs[k] = s0[k];
    } else {
        memset(hs, 0, PN * sizeof(double));
    }
    double *yu = j->y ? j->y + (size_t)u * L * P : NULL;
    int nsnap = 0;
    int k = 0;  /* packed sequences: the sequence token t belongs to */
    if (j->cu) memset(j->seq_states + (size_t)u * j->nseq * PN, 0, (size_t)j->nseq * PN * sizeof(double));
    for (int t = 0; t < L; ++t) {
        const size_t tok = (size_t)b * L + t;
        if (j->cu) {
            /* the last sequence that starts at or before t (empty ones are skipped) */
            while (k + 1 < j->nseq && j->cu[k + 1] <= t) ++k;
            if (k > 0 && j->cu[k] == t) memset(hs, 0, PN * sizeof(double)); /* a new sequence */
        }
        const double d = step_size(j->opts, j->dt[tok * H + h], h);
        const double a = exp(d * A);
        const double wi = input_weight(j->opts, d, A);
        const float *xt = j->x + (tok * H + h) * P;
        const float *Bt = j->B + (tok * G + g) * N;
        const float *Ct = j->C + (tok * G + g) * N;
        for (int p = 0; p < P; ++p) {
            double *row = hs + (size_t)p * N;
            const double dx = wi * (double)xt[p];
            double acc = 0.0;
            for (int n = 0; n < N; ++n) {
                row[n] = a * row[n] + dx * (double)Bt[n];
                acc += (double)Ct[n] * row[n];
            }
            if (yu) yu[(size_t)t * P + p] = acc + D * (double)xt[p];
        }
        if (j->cu && t == j->cu[k + 1] - 1)  /* the last token of sequence k */
            memcpy(j->seq_states + ((size_t)u * j->nseq + k) * PN, hs, PN * sizeof(double));
        if (j->snaps && j->snap_every > 0 && (t + 1) % j->snap_every == 0) {
            const int per = L / j->snap_every;
            memcpy(j->snaps + ((size_t)u * per + nsnap) * PN, hs, PN * sizeof(double));
            ++nsnap;
        }
    }
    if (j->state) memcpy(j->state + (size_t)u * PN, hs, PN * sizeof(double));
}

static void *fwd_worker(void *arg)
{
    fwd_job *j = (fwd_job *)arg;
    double *hs = (double *)malloc((size_t)j->headdim * j->dstate * sizeof(double));
    if (!hs) return (void *)1;
    for (;;) {
        int u = atomic_fetch_add(&j->next, 1);
        if (u >= j->nunits) break;
        fwd_unit(j, u, hs);
    }
    free(hs);
    return NULL;
}

static int run_threads(void *(*fn)(void *), void *job, int nthreads, int nunits)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nunits) nthreads = nunits;
    if (nthreads <= 1) return fn(job) == NULL ? 0 : -3;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tid) return -3;
    int started = 0, rc = 0;
    for (; started < nthreads; ++started)
        if (pthread_create(&tid[started], NULL, fn, job) != 0) break;
    if (started == 0) rc = (fn(job) == NULL) ? 0 : -3;
    for (int i = 0; i < started; ++i) {
        void *r = NULL;
        pthread_join(tid[i], &r);
        if (r != NULL) rc = -3;
    }
    free(tid);
    return rc;
}

/*
 * Forward over whole sequences.
 *   x [batch][seqlen][nheads][headdim], dt [batch][seqlen][nheads],
 *   B, C [batch][seqlen][ngroups][dstate], A, D [nheads] (D may be NULL: 0),
 *   init [batch][nheads][headdim][dstate] (may be NULL: zero state).
 *   units: flat (b*nheads + h) indices to compute, or NULL for all of them.
 *   y [nunits][seqlen][headdim]; state [nunits][headdim][dstate] (may be NULL);
 *   snaps: the state after every snap_every-th token (may be NULL).
 * Returns 0, or a negative value on bad arguments / allocation failure.
 */
int ssd_oracle_forward_ex(const float *x, const float *dt, const float *A, const float *B,
                          const float *C, const float *D, const double *init,
                          int batch, int seqlen, int nheads, int headdim, int ngroups,
                          int dstate, const int *units, int nunits, double *y, double *state,
                          double *snaps, int snap_every, int nthreads, const oracle_opts *opts)
{
    if (!x || !dt || !A || !B || !C) return -1;
    if (batch < 1 || seqlen < 0 || nheads < 1 || headdim < 1 || ngroups < 1 || dstate < 1) return -2;
    if (nheads % ngroups) return -2;
    if (!units) nunits = batch * nheads;
    if (nunits < 0) return -2;
    for (int u = 0; units && u < nunits; ++u)
        if (units[u] < 0 || units[u] >= batch * nheads) return -2;
    if (nunits == 0) return 0;
    fwd_job j = {x, dt, A, B, C, D, init, batch, seqlen, nheads, headdim, ngroups, dstate,
                 units, nunits, y, state, snaps, snap_every, opts, NULL, 0, NULL, 0};
    atomic_init(&j.next, 0);
    return run_threads(fwd_worker, &j, nthreads, nunits);
}

/*
 * Packed variable-length sequences: the token axis of x, dt, B, C (batch 1,
 * seqlen tokens in all) holds nseq sequences, sequence k being tokens
 * cu_seqlens[k] .. cu_seqlens[k+1]-1 (cu_seqlens[0] = 0, non-decreasing,
 * cu_seqlens[nseq] = seqlen; empty sequences allowed). Every sequence starts
 * from the zero state.
 *   units: head indices (0 .. nheads-1) to compute, or NULL for all.
 *   y [nunits][seqlen][headdim];
 *   seq_states [nunits][nseq][headdim][dstate]: each sequence's state after
 *   its last token (zero for an empty sequence).
 */
int ssd_oracle_forward_varlen(const float *x, const float *dt, const float *A, const float *B,
                              const float *C, const float *D, int seqlen, int nheads, int headdim,
                              int ngroups, int dstate, const int *cu_seqlens, int nseq,
                              const int *units, int nunits, double *y, double *seq_states,
                              int nthreads, const oracle_opts *opts)
{
    if (!x || !dt || !A || !B || !C || !cu_seqlens || !seq_states) return -1;
    if (seqlen < 0 || nheads < 1 || headdim < 1 || ngroups < 1 || dstate < 1 || nseq < 1) return -2;
    if (nheads % ngroups) return -2;
    if (cu_seqlens[0] != 0 || cu_seqlens[nseq] != seqlen) return -2;
    for (int k = 0; k < nseq; ++k)
        if (cu_seqlens[k + 1] < cu_seqlens[k]) return -2;
    if (!units) nunits = nheads;
    if (nunits < 0) return -2;
    for (int u = 0; units && u < nunits; ++u)
        if (units[u] < 0 || units[u] >= nheads) return -2;
    if (nunits == 0) return 0;
    fwd_job j = {x, dt, A, B, C, D, NULL, 1, seqlen, nheads, headdim, ngroups, dstate,
                 units, nunits, y, NULL, NULL, 0, opts, cu_seqlens, nseq, seq_states, 0};
    atomic_init(&j.next, 0);
    return run_threads(fwd_worker, &j, nthreads, nunits);
}

/* The plain layer: Euler input weight, dt used as given. */
int ssd_oracle_forward(const float *x, const float *dt, const float *A, const float *B,
                       const float *C, const float *D, const double *init,
                       int batch, int seqlen, int nheads, int headdim, int ngroups, int dstate,
                       const int *units, int nunits, double *y, double *state,
                       double *snaps, int snap_every, int nthreads)
{
    return ssd_oracle_forward_ex(x, dt, A, B, C, D, init, batch, seqlen, nheads, headdim,
                                 ngroups, dstate, units, nunits, y, state, snaps, snap_every,
                                 nthreads, NULL);
}

typedef struct {
    double *state;  /* [nunits][headdim][dstate] */
    const float *x, *dt, *A, *B, *C, *D;
    int batch, nheads, headdim, ngroups, dstate;
    const int *units;
    int nunits;
    double *y;      /* [nunits][headdim] */
    const oracle_opts *opts;
    atomic_int next;
} step_job;

static void *step_worker(void *arg)
{
    step_job *j = (step_job *)arg;
    const int H = j->nheads, P = j->headdim, N = j->dstate, G = j->ngroups;
    for (;;) {
        int u = atomic_fetch_add(&j->next, 1);
        if (u >= j->nunits) break;
        const int bh = j->units ? j->units[u] : u;
        const int b = bh / H, h = bh % H, g = h / (H / G);
        const double d = step_size(j->opts, j->dt[bh], h);
        const double a = exp(d * (double)j->A[h]);
        const double wi = input_weight(j->opts, d, (double)j->A[h]);
        const double D = j->D ? j->D[h] : 0.0;
        const float *xt = j->x + (size_t)bh * P;
        const float *Bt = j->B + ((size_t)b * G + g) * N;
        const float *Ct = j->C + ((size_t)b * G + g) * N;
        double *hs = j->state + (size_t)u * P * N;
        for (int p = 0; p < P; ++p) {
            double *row = hs + (size_t)p * N;
            const double dx = wi * (double)xt[p];
            double acc = 0.0;
            for (int n = 0; n < N; ++n) {
                row[n] = a * row[n] + dx * (double)Bt[n];
                acc += (double)Ct[n] * row[n];
            }
            j->y[(size_t)u * P + p] = acc + D * (double)xt[p];
        }
    }
    return NULL;
}

/*
 * One recurrent step for every selected (b, h) unit: the loop body above for a
 * single token.
 *   state [nunits][headdim][dstate] (in/out, double),
 *   x [batch][nheads][headdim], dt [batch][nheads], B, C [batch][ngroups][dstate],
 *   y [nunits][headdim].
 */
int ssd_oracle_step_ex(double *state, const float *x, const float *dt, const float *A,
                       const float *B, const float *C, const float *D,
                       int batch, int nheads, int headdim, int ngroups, int dstate,
                       const int *units, int nunits, double *y, int nthreads,
                       const oracle_opts *opts)
{
    if (!state || !x || !dt || !A || !B || !C || !y) return -1;
    if (batch < 1 || nheads < 1 || headdim < 1 || ngroups < 1 || dstate < 1) return -2;
    if (nheads % ngroups) return -2;
    if (!units) nunits = batch * nheads;
    for (int u = 0; units && u < nunits; ++u)
        if (units[u] < 0 || units[u] >= batch * nheads) return -2;
    if (nunits <= 0) return 0;
    step_job j = {state, x, dt, A, B, C, D, batch, nheads, headdim, ngroups, dstate,
                  units, nunits, y, opts, 0};
    atomic_init(&j.next, 0);
    return run_threads(step_worker, &j, nthreads, nunits);
}

int ssd_oracle_step(double *state, const float *x, const float *dt, const float *A,
                    const float *B, const float *C, const float *D,
                    int batch, int nheads, int headdim, int ngroups, int dstate,
                    const int *units, int nunits, double *y, int nthreads)
{
    return ssd_oracle_step_ex(state, x, dt, A, B, C, D, batch, nheads, headdim, ngroups, dstate,
                              units, nunits, y, nthreads, NULL);
}

/* ------------------------------------------------------------------------- */
/* Gradients (reverse mode) of the forward above.                             */
/*                                                                            */
/* With loss = sum_t dy_t . y_t + <dfinal, h_{L-1}>, the adjoint of the state */
/* g_t = dloss/dh_t obeys g_t = dy_t C_t^T + a_{t+1} g_{t+1} (g_{L-1} starts  */
/* from dfinal), since h_{t+1} = a_{t+1} h_t + ... and y_t = h_t C_t + D x_t. */
/* Each token then gives, with hp = h_{t-1} and w the input weight:           */
/*   dx_t = w g_t B_t + D dy_t,   dB_t = w g_t^T x_t,   dC_t = h_t^T dy_t,    */
/*   dstep_t = (da/dstep) <g_t, hp> + (dw/dstep) x_t^T g_t B_t,               */
/*   dA += (da/dA) <g_t, hp> + (dw/dA) x_t^T g_t B_t,   dD += dy_t . x_t,     */
/* and d(raw dt) = dstep * d(step)/d(raw) through the options; dinit = a_0 g_0.*/
/* States are recomputed block by block from checkpoints every BWD_BLOCK     */
/* tokens.                                                                    */
/* ------------------------------------------------------------------------- */

#define BWD_BLOCK 64

/* d(step)/d(raw dt): 1, times sigmoid for softplus, times 0 outside the clamp
 * range (the bounds themselves pass the gradient). */
static double step_slope(const oracle_opts *o, double v, int h)
{
    if (!o) return 1.0;
    double slope = 1.0;
    if (o->dt_bias) v += (double)o->dt_bias[h];
    if (o->dt_softplus) {
        slope = 1.0 / (1.0 + exp(-v));
        v = fmax(v, 0.0) + log1p(exp(-fabs(v)));
    }
    if (o->dt_clamp && (v < o->dt_min || v > o->dt_max)) slope = 0.0;
    return slope;
}

/* Derivatives of the input weight w(d, A) with respect to d and A. For the
 * zero-order hold w = (e^z - 1)/A with z = d A: dw/dd = e^z and
 * dw/dA = (z e^z - (e^z - 1)) / A^2 = d^2 (1/2 + z/3 + z^2/8 + ...). */
static void weight_slopes(const oracle_opts *o, double d, double A, double *wd, double *wA)
{
    if (!(o && o->zoh)) {
        *wd = 1.0;
        *wA = 0.0;
        return;
    }
    const double z = d * A;
    *wd = exp(z);
    if (fabs(z) < 1e-3) *wA = d * d * (0.5 + z / 3.0 + z * z / 8.0);
    else *wA = (z * exp(z) - expm1(z)) / (A * A);
}

typedef struct {
    const float *x, *dt, *A, *B, *C, *D, *dy;
    const double *init, *dfinal;
    int batch, seqlen, nheads, headdim, ngroups, dstate;
    const int *units;
    int nunits;
    double *dx, *ddt, *dA, *dB, *dC, *dD, *dinit, *dbias;
    const oracle_opts *opts;
    atomic_int next;
} bwd_job;

/* State update of token t (global index tok) from prev into out. */
static void bwd_advance(const bwd_job *j, size_t tok, int h, int g, const double *prev, double *out)
{
    const int H = j->nheads, P = j->headdim, N = j->dstate, G = j->ngroups;
    const double A = j->A[h];
    const double d = step_size(j->opts, j->dt[tok * H + h], h);
    const double a = exp(d * A);
    const double wi = input_weight(j->opts, d, A);
    const float *xt = j->x + (tok * H + h) * P;
    const float *Bt = j->B + (tok * G + g) * N;
    for (int p = 0; p < P; ++p)
        for (int n = 0; n < N; ++n)
            out[(size_t)p * N + n] = a * prev[(size_t)p * N + n] + wi * (double)xt[p] * (double)Bt[n];
}

static void bwd_unit(bwd_job *j, int u, double *ckpt, double *blk, double *gs)
{
    const int H = j->nheads, P = j->headdim, N = j->dstate, L = j->seqlen;
    const int G = j->ngroups;
    const int bh = j->units ? j->units[u] : u;
    const int b = bh / H, h = bh % H;
    const int g = h / (H / G);
    const double A = j->A[h];
    const double D = j->D ? j->D[h] : 0.0;
    const size_t PN = (size_t)P * N;
    const int nb = (L + BWD_BLOCK - 1) / BWD_BLOCK;

    /* forward: the state entering every block */
    double *hs = blk;
    if (j->init) memcpy(hs, j->init + (size_t)bh * PN, PN * sizeof(double));
    else memset(hs, 0, PN * sizeof(double));
    for (int t = 0; t < L; ++t) {
        if (t % BWD_BLOCK == 0) memcpy(ckpt + (size_t)(t / BWD_BLOCK) * PN, hs, PN * sizeof(double));
        bwd_advance(j, (size_t)b * L + t, h, g, hs, blk + PN);
        memcpy(hs, blk + PN, PN * sizeof(double));
    }

    /* backward */
    if (j->dfinal) memcpy(gs, j->dfinal + (size_t)bh * PN, PN * sizeof(double));
    else memset(gs, 0, PN * sizeof(double));
    double dA = 0.0, dD = 0.0, dbias = 0.0;
    for (int kb = nb - 1; kb >= 0; --kb) {
        const int t0 = kb * BWD_BLOCK, t1 = t0 + BWD_BLOCK < L ? t0 + BWD_BLOCK : L;
        memcpy(blk, ckpt + (size_t)kb * PN, PN * sizeof(double));  /* h_{t0-1} */
        for (int t = t0; t < t1; ++t)
            bwd_advance(j, (size_t)b * L + t, h, g, blk + (size_t)(t - t0) * PN,
                        blk + (size_t)(t - t0 + 1) * PN);
        for (int t = t1 - 1; t >= t0; --t) {
            const size_t tok = (size_t)b * L + t;
            const double raw = j->dt[tok * H + h];
            const double d = step_size(j->opts, raw, h);
            const double a = exp(d * A);
            const double wi = input_weight(j->opts, d, A);
            double wd, wA;
            weight_slopes(j->opts, d, A, &wd, &wA);
            const float *xt = j->x + (tok * H + h) * P;
            const float *dyt = j->dy + (tok * H + h) * P;
            const float *Bt = j->B + (tok * G + g) * N;
            const float *Ct = j->C + (tok * G + g) * N;
            const double *hcur = blk + (size_t)(t - t0 + 1) * PN;
            const double *hprev = blk + (size_t)(t - t0) * PN;
            /* g_t: the output of token t reads h_t */
            for (int p = 0; p < P; ++p)
                for (int n = 0; n < N; ++n) gs[(size_t)p * N + n] += (double)dyt[p] * (double)Ct[n];
            double gh = 0.0, gx = 0.0;
            double *dxt = j->dx + ((size_t)u * L + t) * P;
            double *dBt = j->dB + ((size_t)u * L + t) * N;
            double *dCt = j->dC + ((size_t)u * L + t) * N;
            for (int n = 0; n < N; ++n) dBt[n] = dCt[n] = 0.0;
            for (int p = 0; p < P; ++p) {
                const double *gr = gs + (size_t)p * N;
                double gB = 0.0;
                for (int n = 0; n < N; ++n) {
                    gh += gr[n] * hprev[(size_t)p * N + n];
                    gB += gr[n] * (double)Bt[n];
                    dBt[n] += wi * gr[n] * (double)xt[p];
                    dCt[n] += (double)dyt[p] * hcur[(size_t)p * N + n];
                }
                gx += (double)xt[p] * gB;
                dxt[p] = wi * gB + D * (double)dyt[p];
                dD += (double)dyt[p] * (double)xt[p];
            }
            const double dstep = A * a * gh + wd * gx;
            dA += d * a * gh + wA * gx;
            const double draw = dstep * step_slope(j->opts, raw, h);
            j->ddt[(size_t)u * L + t] = draw;
            dbias += draw;
            for (size_t k = 0; k < PN; ++k) gs[k] *= a;  /* to h_{t-1} */
        }
    }
    j->dA[u] = dA;
    if (j->dD) j->dD[u] = dD;
    if (j->dbias) j->dbias[u] = dbias;
    if (j->dinit) memcpy(j->dinit + (size_t)u * PN, gs, PN * sizeof(double));
}

static void *bwd_worker(void *arg)
{
    bwd_job *j = (bwd_job *)arg;
    const size_t PN = (size_t)j->headdim * j->dstate;
    const int nb = (j->seqlen + BWD_BLOCK - 1) / BWD_BLOCK;
    double *ckpt = (double *)malloc((size_t)(nb > 0 ? nb : 1) * PN * sizeof(double));
    double *blk = (double *)malloc((size_t)(BWD_BLOCK + 1) * PN * sizeof(double));
    double *gs = (double *)malloc(PN * sizeof(double));
    void *rc = NULL;
    if (!ckpt || !blk || !gs) rc = (void *)1;
    for (; rc == NULL;) {
        int u = atomic_fetch_add(&j->next, 1);
        if (u >= j->nunits) break;
        bwd_unit(j, u, ckpt, blk, gs);
    }
    free(ckpt);
    free(blk);
    free(gs);
    return rc;
}

/*
 * Gradients of loss = sum dy . y + <dfinal, final state> (dfinal may be NULL)
 * for the forward of ssd_oracle_forward_ex with the same arguments and options.
 * Per unit u = (b, h) (units: flat b*nheads + h, or NULL for all):
 *   dx [U][L][P]; ddt [U][L] (with respect to the raw dt); dA [U];
 *   dB, dC [U][L][N] (this head's share: a group's gradient is the sum over
 *   its heads); dD [U] (may be NULL); dinit [U][P][N] (may be NULL);
 *   dbias [U] (may be NULL; the gradient of opts->dt_bias[h] from this unit).
 * dy has x's layout; dfinal [batch][nheads][P][N].
 */
int ssd_oracle_backward(const float *x, const float *dt, const float *A, const float *B,
                        const float *C, const float *D, const double *init, const float *dy,
                        const double *dfinal, int batch, int seqlen, int nheads, int headdim,
                        int ngroups, int dstate, const int *units, int nunits, double *dx,
                        double *ddt, double *dA, double *dB, double *dC, double *dD,
                        double *dinit, double *dbias, int nthreads, const oracle_opts *opts)
{
    if (!x || !dt || !A || !B || !C || !dy || !dx || !ddt || !dA || !dB || !dC) return -1;
    if (batch < 1 || seqlen < 1 || nheads < 1 || headdim < 1 || ngroups < 1 || dstate < 1) return -2;
    if (nheads % ngroups) return -2;
    if (!units) nunits = batch * nheads;
    if (nunits < 0) return -2;
    for (int u = 0; units && u < nunits; ++u)
        if (units[u] < 0 || units[u] >= batch * nheads) return -2;
    if (nunits == 0) return 0;
    bwd_job j = {x, dt, A, B, C, D, dy, init, dfinal, batch, seqlen, nheads, headdim, ngroups,
                 dstate, units, nunits, dx, ddt, dA, dB, dC, dD, dinit, dbias, opts, 0};
    atomic_init(&j.next, 0);
    return run_threads(bwd_worker, &j, nthreads, nunits);
}
