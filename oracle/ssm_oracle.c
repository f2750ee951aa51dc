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
 *       dt   = delta[t] + dbias[d]      (dbias optional; log(1 + exp(.)) of it in softplus mode)
 *       h[n] = A_bar(dt, A[d, n]) * h[n] + Bf(dt, A[d, n]) * B[b, t, n] * x[t]   for every n
 *       y[t] = sum_n C[b, t, n] * h[n] + Dskip[d] * x[t]
 *       y[t] = y[t] * z[t] / (1 + exp(-z[t]))       (only when a gate z is given)
 *   h_last = h
 *
 * Discretisations of the continuous (A, B) with step dt, A diagonal (A_bar,
 * B_bar = Bf * B):
 *   0 Mamba:    A_bar = exp(dt a),  Bf = dt  (the first-order B_bar of the Mamba listings)
 *   1 ZOH:      A_bar = exp(dt a),  Bf = (exp(dt a) - 1) / a, and dt where a = 0 (its
 *               limit), evaluated with expm1 so that small dt a keeps full precision
 *   2 bilinear: A_bar = (1 + dt a / 2) / (1 - dt a / 2),  Bf = dt / (1 - dt a / 2)
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
 *    section "Mamba: Selective State Spaces"; the linear map's bias added before
 *    the softplus: skill page, MambaBlock listing (dt_proj with bias, then softplus);
 *  - zero-order hold B_bar = (exp(dt A) - I) A^-1 B: the skill page's "Discretization"
 *    docstring and brentwoodlivery's section "From Continuous to Discrete" and its
 *    discretisation flashcard;
 *  - bilinear A_bar = (I + dt/2 A)(I - dt/2 A)^-1, B_bar = (I - dt/2 A)^-1 B dt:
 *    chipfoundryservices glossary "State Space Models & Mamba", Lab 1 and the
 *    section "Discretization Method".
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
    int delta_softplus, disc;
    const double *dbias;
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

/* A_bar and Bf (B_bar = Bf * B) of one state, for the discretisations listed above */
static void discretize(int disc, double dt, double a, double *a_bar, double *bf)
{
    if (disc == 2) {
        const double half = 0.5 * dt * a;
        *a_bar = (1.0 + half) / (1.0 - half);
        *bf = dt / (1.0 - half);
        return;
    }
    *a_bar = exp(dt * a);
    if (disc == 1)
        *bf = a == 0.0 ? dt : expm1(dt * a) / a;
    else
        *bf = dt;
}

/* The same A_bar and Bf with their partial derivatives with respect to dt and a:
 *   Mamba:    dA_bar/ddt = a e^u, dBf/ddt = 1, dA_bar/da = dt e^u, dBf/da = 0   (u = dt a)
 *   ZOH:      Bf = dt phi(u), phi(u) = (e^u - 1) / u:  dBf/ddt = e^u,
 *             dBf/da = dt^2 psi(u), psi = phi' = (u e^u - e^u + 1) / u^2, taken from its
 *             Taylor series 1/2 + u/3 + u^2/8 + u^3/30 + u^4/144 where |u| < 1e-2 (the
 *             closed form cancels there); A_bar's derivatives as Mamba's
 *   bilinear: r = 1 / (1 - u/2), A_bar = 2 r - 1, Bf = r dt:  dA_bar/ddt = r^2 a,
 *             dBf/ddt = r^2, dA_bar/da = r^2 dt, dBf/da = r^2 dt^2 / 2 */
static void discretize_grad(int disc, double dt, double a, double *a_bar, double *bf, double *da_dt,
                            double *dbf_dt, double *da_da, double *dbf_da)
{
    discretize(disc, dt, a, a_bar, bf);
    const double u = dt * a;
    if (disc == 2) {
        const double r = 1.0 / (1.0 - 0.5 * u);
        *da_dt = r * r * a;
        *dbf_dt = r * r;
        *da_da = r * r * dt;
        *dbf_da = r * r * dt * dt / 2.0;
        return;
    }
    *da_dt = a * *a_bar;
    *da_da = dt * *a_bar;
    if (disc == 1) {
        double psi;
        if (fabs(u) < 1e-2)
            psi = 0.5 + u * (1.0 / 3.0 + u * (1.0 / 8.0 + u * (1.0 / 30.0 + u / 144.0)));
        else
            psi = (u * exp(u) - expm1(u)) / (u * u);
        *dbf_dt = *a_bar;
        *dbf_da = dt * dt * psi;
    } else {
        *dbf_dt = 1.0;
        *dbf_da = 0.0;
    }
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
        if (J->dbias)
            dt += J->dbias[d];
        if (J->delta_softplus)
            dt = softplus(dt);
        const double xt = J->x[c * L + t];
        const double *Bt = J->Bm + (b * L + t) * N;
        const double *Ct = J->Cm + (b * L + t) * N;
        double y = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double a_bar, bf;
            discretize(J->disc, dt, J->A[d * N + n], &a_bar, &bf);
            const double b_bar = bf * Bt[n];
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
    /* channels are handed out in runs, so short series do not queue on the lock */
    const int64_t run = J->L * (J->N + 1) >= 4096 ? 1 : 256;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int64_t c0 = J->next;
        J->next += run;
        pthread_mutex_unlock(&J->lock);
        if (c0 >= J->nchan)
            break;
        for (int64_t c = c0; c < c0 + run && c < J->nchan; ++c)
            one_channel(J, c);
    }
    return NULL;
}

/* Returns 0 on success, -1 on bad arguments.  disc: 0 Mamba, 1 ZOH, 2 bilinear;
 * dbias: [nd] or NULL. */
int oracle_scan(int64_t L, int64_t N, int64_t nchan, const int64_t *ch_b, const int64_t *ch_d,
                const double *x, const double *delta, const double *z, int delta_softplus,
                int disc, const double *dbias,
                const double *Bm, const double *Cm, const double *A, const double *Dskip,
                const double *h0, double *y, double *h_last, int nthreads)
{
    if (L < 0 || N < 0 || nchan < 0 || disc < 0 || disc > 2)
        return -1;
    if (nchan > 0 && (!ch_b || !ch_d || !y || (L > 0 && (!x || !delta || !Bm || !Cm)) || (N > 0 && !A)))
        return -1;
    job_t J;
    memset(&J, 0, sizeof(J));
    J.L = L; J.N = N; J.nchan = nchan; J.ch_b = ch_b; J.ch_d = ch_d;
    J.x = x; J.delta = delta; J.z = z; J.delta_softplus = delta_softplus;
    J.disc = disc; J.dbias = dbias;
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

/*
 * Backward (adjoint) of the same scan (any of the three discretisations; dbias optional), for a loss whose gradients with respect
 * to the outputs are given: gy[t] = dLoss/dy[t] for every channel, and
 * g_last[n] = dLoss/dh_last[n] (or 0).  Plain reverse-mode differentiation of
 * the definition above, one channel at a time, no reordering:
 *
 *   forward, kept for the reverse sweep:  h_{t-1}[n], y0[t] = sum_n C[t,n] h_t[n] + D x[t]
 *   with a_t[n] = A_bar(dt_t, A[d,n]) and f_t[n] = Bf(dt_t, A[d,n]) (B_bar = f B) and their
 *   partial derivatives from discretize_grad
 *   lam[n] = g_last[n]                    (dLoss/dh_t[n] arriving from step t+1)
 *   for t = L-1 .. 0:
 *       gy0      = gy[t] * silu(z[t])     (gy[t] without a gate)
 *       dz[t]    = gy[t] * y0[t] * silu'(z[t]),  silu'(z) = s (1 + z (1 - s)), s = sigmoid(z)
 *       dD      += gy0 * x[t]
 *       dx[t]    = D gy0
 *       for n:  lam[n]    += C[t,n] gy0                          (now dLoss/dh_t[n])
 *               dC[t,n]   += gy0 h_t[n]
 *               dB[t,n]   += lam[n] f_t[n] x[t]
 *               dx[t]     += lam[n] f_t[n] B[t,n]
 *               ddt       += lam[n] (da/ddt h_{t-1}[n] + df/ddt B[t,n] x[t])
 *               dA[d,n]   += lam[n] (da/dA h_{t-1}[n] + df/dA B[t,n] x[t])
 *               lam[n]     = a_t[n] lam[n]                       (dLoss/dh_{t-1}[n])
 *       ddelta[t] = ddt (times sigmoid(delta[t] + dbias[d]) in softplus mode, the
 *                   derivative of softplus at the raw input; the gradient of the bias is
 *                   the sum of ddelta over the steps, which the caller forms)
 *   dh0[n] = lam[n]
 *
 * The per-channel contributions to the shared tensors are returned separately
 * (dB, dC per channel [nchan][L][N]; dA, dD per channel), and the caller sums
 * them over the channels that share a batch row (dB, dC) or a dim index (dA, dD).
 * Layouts: gy, dx, ddelta, dz [nchan][L]; g_last, dh0, dA_c [nchan][N]; dD_c [nchan].
 */
typedef struct {
    int64_t L, N, nchan;
    const int64_t *ch_b, *ch_d;
    const double *x, *delta, *z;
    int delta_softplus, disc;
    const double *dbias;
    const double *Bm, *Cm, *A, *Dskip, *h0, *gy, *g_last;
    double *dx, *ddelta, *dz, *dB_c, *dC_c, *dA_c, *dD_c, *dh0;
    int64_t next;
    pthread_mutex_t lock;
} bjob_t;

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

static void one_channel_bwd(const bjob_t *J, int64_t c)
{
    const int64_t L = J->L, N = J->N;
    const int64_t b = J->ch_b[c], d = J->ch_d[c];
    const int64_t NN = N > 0 ? N : 1;
    double *hs = (double *)malloc(sizeof(double) * (size_t)((L + 1) * NN));   /* h_{t-1} at row t */
    double *y0 = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    double *lam = (double *)malloc(sizeof(double) * (size_t)NN);

    for (int64_t n = 0; n < N; ++n)
        hs[n] = J->h0 ? J->h0[c * N + n] : 0.0;
    const double bias = J->dbias ? J->dbias[d] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        double dt = J->delta[c * L + t] + bias;
        if (J->delta_softplus)
            dt = softplus(dt);
        const double xt = J->x[c * L + t];
        const double *Bt = J->Bm + (b * L + t) * N;
        const double *Ct = J->Cm + (b * L + t) * N;
        double y = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double a_bar, bf;
            discretize(J->disc, dt, J->A[d * N + n], &a_bar, &bf);
            const double h = a_bar * hs[t * N + n] + bf * Bt[n] * xt;
            hs[(t + 1) * N + n] = h;
            y += Ct[n] * h;
        }
        if (J->Dskip)
            y += J->Dskip[d] * xt;
        y0[t] = y;
    }

    for (int64_t n = 0; n < N; ++n) {
        lam[n] = J->g_last ? J->g_last[c * N + n] : 0.0;
        J->dA_c[c * N + n] = 0.0;
    }
    double dD = 0.0;
    for (int64_t t = L - 1; t >= 0; --t) {
        const double raw = J->delta[c * L + t] + bias;
        const double dt = J->delta_softplus ? softplus(raw) : raw;
        const double xt = J->x[c * L + t];
        const double *Bt = J->Bm + (b * L + t) * N;
        const double *Ct = J->Cm + (b * L + t) * N;
        const double gy = J->gy[c * L + t];
        double gy0 = gy;
        if (J->z) {
            const double zt = J->z[c * L + t];
            const double s = sigmoid(zt);
            gy0 = gy * (zt * s);
            J->dz[c * L + t] = gy * y0[t] * (s * (1.0 + zt * (1.0 - s)));
        }
        dD += gy0 * xt;
        double gx = J->Dskip ? J->Dskip[d] * gy0 : 0.0;
        double gdt = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double a, f, da_dt, df_dt, da_da, df_da;
            discretize_grad(J->disc, dt, J->A[d * N + n], &a, &f, &da_dt, &df_dt, &da_da, &df_da);
            const double hprev = hs[t * N + n];
            lam[n] += Ct[n] * gy0;
            J->dC_c[(c * L + t) * N + n] = gy0 * hs[(t + 1) * N + n];
            J->dB_c[(c * L + t) * N + n] = lam[n] * f * xt;
            gx += lam[n] * f * Bt[n];
            gdt += lam[n] * (da_dt * hprev + df_dt * Bt[n] * xt);
            J->dA_c[c * N + n] += lam[n] * (da_da * hprev + df_da * Bt[n] * xt);
            lam[n] = a * lam[n];
        }
        J->dx[c * L + t] = gx;
        J->ddelta[c * L + t] = J->delta_softplus ? gdt * sigmoid(raw) : gdt;
    }
    J->dD_c[c] = dD;
    for (int64_t n = 0; n < N; ++n)
        J->dh0[c * N + n] = lam[n];
    free(hs);
    free(y0);
    free(lam);
}

static void *worker_bwd(void *arg)
{
    bjob_t *J = (bjob_t *)arg;
    const int64_t run = J->L * (J->N + 1) >= 4096 ? 1 : 256;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int64_t c0 = J->next;
        J->next += run;
        pthread_mutex_unlock(&J->lock);
        if (c0 >= J->nchan)
            break;
        for (int64_t c = c0; c < c0 + run && c < J->nchan; ++c)
            one_channel_bwd(J, c);
    }
    return NULL;
}

/* Returns 0 on success, -1 on bad arguments.  z may be NULL (no gate; dz is then
 * not written), Dskip, h0 and g_last may be NULL.  disc as for oracle_scan. */
int oracle_scan_bwd(int64_t L, int64_t N, int64_t nchan, const int64_t *ch_b, const int64_t *ch_d,
                    const double *x, const double *delta, const double *z, int delta_softplus,
                    int disc, const double *dbias, const double *Bm, const double *Cm, const double *A, const double *Dskip,
                    const double *h0, const double *gy, const double *g_last,
                    double *dx, double *ddelta, double *dz, double *dB_c, double *dC_c,
                    double *dA_c, double *dD_c, double *dh0, int nthreads)
{
    if (L < 0 || N < 0 || nchan < 0 || disc < 0 || disc > 2)
        return -1;
    if (nchan > 0 && (!ch_b || !ch_d || !dD_c || !dh0 || (N > 0 && (!A || !dA_c)) ||
                      (L > 0 && (!x || !delta || !Bm || !Cm || !gy || !dx || !ddelta || !dB_c || !dC_c)) ||
                      (z && !dz)))
        return -1;
    bjob_t J;
    memset(&J, 0, sizeof(J));
    J.L = L; J.N = N; J.nchan = nchan; J.ch_b = ch_b; J.ch_d = ch_d;
    J.x = x; J.delta = delta; J.z = z; J.delta_softplus = delta_softplus; J.disc = disc;
    J.dbias = dbias;
    J.Bm = Bm; J.Cm = Cm; J.A = A; J.Dskip = Dskip; J.h0 = h0; J.gy = gy; J.g_last = g_last;
    J.dx = dx; J.ddelta = ddelta; J.dz = dz; J.dB_c = dB_c; J.dC_c = dC_c; J.dA_c = dA_c;
    J.dD_c = dD_c; J.dh0 = dh0; J.next = 0;
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
        if (pthread_create(&tid[started], NULL, worker_bwd, &J) == 0)
            ++started;
    worker_bwd(&J);
    for (int i = 0; i < started; ++i)
        pthread_join(tid[i], NULL);
    pthread_mutex_destroy(&J.lock);
    return 0;
}

int oracle_abi_version(void) { return 5; }
