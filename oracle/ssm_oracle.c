/*
 * Plain fp64 CPU oracle of the Mamba (S6) selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the package's smoke check and the bench's
 * CPU-baseline leg use it.  It shares no code with the GPU library.
 *
 * What it computes (one independent channel (b, d) at a time, state size N):
 *
 *   h[n] = h0[n] (or 0)
 *   for t = 0 .. L-1:
 *       dt   = delta[t]                 (or log(1 + exp(delta[t])) in softplus mode)
 *       h[n] = exp(dt * A[d, n]) * h[n] + dt * B[b, t, n] * x[t]     for every n
 *       y[t] = sum_n C[b, t, n] * h[n] + Dskip[d] * x[t]
 *       y[t] = y[t] * z[t] / (1 + exp(-z[t]))       (only when a gate z is given)
 *   h_last = h
 *
 * Sources (the five web pages on state space models / Mamba):
 *  - discretisation A_bar = exp(delta A), B_bar = delta B: "State Space
 *    Models Mamba" skill page, section "Discretization" and the
 *    MambaBlock._selective_scan listing; managen.ai "Mamba: State Space
 *    Models Challenge Transformers", section "Selective Scan Algorithm";
 *  - recurrence, readout through C after the update, skip term D x: the same
 *    two listings; brentwoodlivery "State-space models (Mamba, S4)" section
 *    "Training vs Inference Modes" (inference update h_k, output y_k);
 *  - output gate y * silu(z): managen.ai page, MambaBlock.forward;
 *  - delta = softplus(Linear(x)): dileepadev "State Space Models and Mamba",
 *    section "Mamba: Selective State Spaces".
 *
 * Every value is double precision; the caller widens stored bf16/fp32 inputs
 * to double exactly before the call.  No blocking, no reordering: time runs
 * forward one step at a time.  Threads only split the independent channels.
 *
 * Layouts (all row-major, double):
 *   x, delta, z : [nchan][L]       series of each listed channel
 *   Bm, Cm      : [nb][L][N]       per-token input/output vectors, indexed by ch_b
 *   A           : [nd][N]          indexed by ch_d
 *   Dskip       : [nd] or NULL (no skip term)
 *   h0          : [nchan][N] or NULL (start from zero)
 *   y           : [nchan][L]       output, unrounded
 *   h_last      : [nchan][N] or NULL; may alias h0 (single-token state update)
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t L, N, nchan;
    const int64_t *ch_b, *ch_d;
    const double *x, *delta, *z;
    int delta_softplus;
    const double *Bm, *Cm, *A, *Dskip, *h0;
    double *y, *h_last;
    int64_t next;            /* next channel to take (guarded by lock) */
    pthread_mutex_t lock;
} job_t;

/* softplus(u) = log(1 + exp(u)); the second branch is the same function
 * written so that exp does not overflow for large u. */
static double softplus(double u)
{
    if (u <= 30.0)
        return log1p(exp(u));
    return u + log1p(exp(-u));
}

static void one_channel(const job_t *J, int64_t c)
{
    const int64_t L = J->L, N = J->N;
    const int64_t b = J->ch_b[c], d = J->ch_d[c];
    double *h = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    for (int64_t n = 0; n < N; ++n)
        h[n] = J->h0 ? J->h0[c * N + n] : 0.0;

    for (int64_t t = 0; t < L; ++t) {
        double dt = J->delta[c * L + t];
        if (J->delta_softplus)
            dt = softplus(dt);
        const double xt = J->x[c * L + t];
        const double *Bt = J->Bm + (b * L + t) * N;
        const double *Ct = J->Cm + (b * L + t) * N;
        double y = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double a_bar = exp(dt * J->A[d * N + n]);
            const double b_bar = dt * Bt[n];
            h[n] = a_bar * h[n] + b_bar * xt;
        }
        for (int64_t n = 0; n < N; ++n)
            y += Ct[n] * h[n];
        if (J->Dskip)
            y += J->Dskip[d] * xt;
        if (J->z) {
            const double zt = J->z[c * L + t];
            y = y * (zt / (1.0 + exp(-zt)));
        }
        J->y[c * L + t] = y;
    }
    if (J->h_last)
        for (int64_t n = 0; n < N; ++n)
            J->h_last[c * N + n] = h[n];
    free(h);
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int64_t c = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (c >= J->nchan)
            break;
        one_channel(J, c);
    }
    return NULL;
}

/* Returns 0 on success, -1 on bad arguments. */
int oracle_scan(int64_t L, int64_t N, int64_t nchan, const int64_t *ch_b, const int64_t *ch_d,
                const double *x, const double *delta, const double *z, int delta_softplus,
                const double *Bm, const double *Cm, const double *A, const double *Dskip,
                const double *h0, double *y, double *h_last, int nthreads)
{
    if (L < 0 || N < 0 || nchan < 0)
        return -1;
    if (nchan > 0 && (!ch_b || !ch_d || !y || (L > 0 && (!x || !delta || !Bm || !Cm)) || (N > 0 && !A)))
        return -1;
    job_t J;
    memset(&J, 0, sizeof(J));
    J.L = L; J.N = N; J.nchan = nchan; J.ch_b = ch_b; J.ch_d = ch_d;
    J.x = x; J.delta = delta; J.z = z; J.delta_softplus = delta_softplus;
    J.Bm = Bm; J.Cm = Cm; J.A = A; J.Dskip = Dskip; J.h0 = h0;
    J.y = y; J.h_last = h_last; J.next = 0;
    pthread_mutex_init(&J.lock, NULL);
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > nchan)
        nthreads = (int)(nchan > 0 ? nchan : 1);
    pthread_t tid[256];
    int started = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&tid[started], NULL, worker, &J) == 0)
            ++started;
    worker(&J);
    for (int i = 0; i < started; ++i)
        pthread_join(tid[i], NULL);
    pthread_mutex_destroy(&J.lock);
    return 0;
}

int oracle_abi_version(void) { return 1; }
