/*
 * ssm_oracle_bwd.c - fp64 CPU reference for the gradients of the selective scan
 * (TEST INFRASTRUCTURE; only the test suite loads it).
 *
 * The pages say the model trains with parallel scans but never state the
 * gradients, so this file is the reverse-mode derivative of the forward
 * definition in ssm_oracle.h, taken step by step (see the header for the
 * equations). Per row: one forward sweep that keeps every state h_t, then one
 * backward sweep over t = L-1..0 carrying G = dLoss/dh_t. Nothing is blocked or
 * reordered; sums over rows (dA, dD, dbias over batch and time, dB and dC over
 * channels) are accumulated per thread and added in thread order at the end.
 */
#include "ssm_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* sigma(v) = 1 / (1 + e^-v), on the side where the exponential cannot overflow */
static double sigmoid(double v)
{
    if (v >= 0.0)
        return 1.0 / (1.0 + exp(-v));
    double e = exp(v);
    return e / (1.0 + e);
}

typedef struct {
    int64_t r0, r1, L, N, batch, dim;
    const int64_t *row_b, *row_d;
    const double *x, *delta, *z, *A, *B, *C, *D, *bias, *h0, *dy, *dh_final;
    int softplus;
    double *dx, *ddelta, *dz, *dh0;
    /* this thread's sums */
    double *dA, *dB, *dC, *dD, *dbias;
    int status;
} bwd_job;

static void bwd_block(bwd_job* j)
{
    const int64_t L = j->L, N = j->N;
    double* H = (double*)malloc((size_t)(L + 1) * N * sizeof(double)); /* H[t+1] = h_t */
    double* a = (double*)malloc((size_t)L * N * sizeof(double));       /* exp(Delta_t A) */
    double* dl = (double*)malloc((size_t)L * sizeof(double));          /* Delta_t */
    double* sg = (double*)malloc((size_t)L * sizeof(double));          /* softplus'(v_t) */
    double* q = (double*)malloc((size_t)L * sizeof(double));           /* output before gate */
    double* G = (double*)malloc((size_t)N * sizeof(double));
    double* Gc = (double*)malloc((size_t)N * sizeof(double));
    int64_t r, t, n;
    if (!H || !a || !dl || !sg || !q || !G || !Gc) {
        free(H); free(a); free(dl); free(sg); free(q); free(G); free(Gc);
        j->status = -1;
        return;
    }
    for (r = j->r0; r < j->r1; ++r) {
        const int64_t b = j->row_b[r], d = j->row_d[r];
        const double* Ad = j->A + d * N;
        const double* xr = j->x + r * L;
        /* ---- forward sweep, as in ssm_oracle.c, keeping every state ---- */
        for (n = 0; n < N; ++n)
            H[n] = j->h0 ? j->h0[r * N + n] : 0.0;
        for (t = 0; t < L; ++t) {
            const double* Bt = j->B + (b * L + t) * N;
            const double* Ct = j->C + (b * L + t) * N;
            const double v = j->delta[r * L + t] + (j->bias ? j->bias[d] : 0.0);
            const double delta = j->softplus ? ssm_oracle_softplus(v) : v;
            double s = 0.0;
            dl[t] = delta;
            sg[t] = j->softplus ? sigmoid(v) : 1.0;
            for (n = 0; n < N; ++n) {
                a[t * N + n] = exp(delta * Ad[n]);
                H[(t + 1) * N + n] = a[t * N + n] * H[t * N + n] + (delta * xr[t]) * Bt[n];
            }
            for (n = 0; n < N; ++n)
                s += Ct[n] * H[(t + 1) * N + n];
            if (j->D)
                s += j->D[d] * xr[t];
            q[t] = s;
        }
        /* ---- backward sweep. Gc = the gradient reaching h_t from later tokens
         * (exp(Delta_{t+1} A) * G_{t+1}); it starts as dLoss/dh_final. ---- */
        for (n = 0; n < N; ++n)
            Gc[n] = j->dh_final ? j->dh_final[r * N + n] : 0.0;
        for (t = L - 1; t >= 0; --t) {
            const double* Bt = j->B + (b * L + t) * N;
            const double* Ct = j->C + (b * L + t) * N;
            const double dyt = j->dy[r * L + t];
            double dq = dyt, du = 0.0, ddel = 0.0;
            /* y = q * silu(z): dq = dy * silu(z), dz = dy * q * silu'(z) */
            if (j->z) {
                const double zt = j->z[r * L + t];
                const double sz = sigmoid(zt);
                dq = dyt * ssm_oracle_silu(zt);
                j->dz[r * L + t] = dyt * q[t] * (sz * (1.0 + zt * (1.0 - sz)));
            }
            /* q = sum_n C h + D x */
            j->dx[r * L + t] = j->D ? dq * j->D[d] : 0.0;
            if (j->D)
                j->dD[d] += dq * xr[t];
            for (n = 0; n < N; ++n) {
                G[n] = Gc[n] + dq * Ct[n];                        /* dLoss/dh_t */
                j->dC[(b * L + t) * N + n] += dq * H[(t + 1) * N + n];
            }
            /* h_t = a_t h_{t-1} + u_t B_t with u_t = Delta_t x_t, a_t = exp(Delta_t A) */
            for (n = 0; n < N; ++n) {
                const double gh = G[n] * H[t * N + n] * a[t * N + n];   /* through a_t */
                du += G[n] * Bt[n];
                j->dB[(b * L + t) * N + n] += G[n] * (dl[t] * xr[t]);
                ddel += gh * Ad[n];
                j->dA[d * N + n] += gh * dl[t];
                Gc[n] = a[t * N + n] * G[n];                        /* to h_{t-1} */
            }
            j->dx[r * L + t] += du * dl[t];
            ddel += du * xr[t];
            /* Delta = softplus(delta_raw + bias) */
            j->ddelta[r * L + t] = ddel * sg[t];
            j->dbias[d] += ddel * sg[t];
        }
        if (j->dh0)
            for (n = 0; n < N; ++n)
                j->dh0[r * N + n] = Gc[n];
    }
    free(H); free(a); free(dl); free(sg); free(q); free(G); free(Gc);
    j->status = 0;
}

static void* bwd_thread(void* p)
{
    bwd_block((bwd_job*)p);
    return NULL;
}

int ssm_oracle_scan_bwd_rows(int64_t nrows, int64_t seqlen, int64_t dstate,
                             const int64_t* row_b, const int64_t* row_d, int64_t batch,
                             int64_t dim, const double* x, const double* delta,
                             const double* z, const double* A, const double* B,
                             const double* C, const double* D, const double* delta_bias,
                             int delta_softplus, const double* h0, const double* dy,
                             const double* dh_final, double* dx, double* ddelta, double* dz,
                             double* dA, double* dB, double* dC, double* dD, double* dbias,
                             double* dh0, int nthreads)
{
    bwd_job* jobs;
    pthread_t* tids;
    int64_t per, i, k;
    int nt, rc = 0;
    const int64_t nA = dim * dstate, nBC = batch * seqlen * dstate;

    if (nrows < 0 || seqlen < 0 || dstate <= 0 || batch <= 0 || dim <= 0 || !row_b ||
        !row_d || !x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dA || !dB ||
        !dC || !dbias || (z && !dz) || (D && !dD))
        return -1;
    memset(dA, 0, (size_t)nA * sizeof(double));
    memset(dB, 0, (size_t)nBC * sizeof(double));
    memset(dC, 0, (size_t)nBC * sizeof(double));
    memset(dbias, 0, (size_t)dim * sizeof(double));
    if (dD)
        memset(dD, 0, (size_t)dim * sizeof(double));
    if (nrows == 0)
        return 0;
    nt = nthreads < 1 ? 1 : nthreads;
    if ((int64_t)nt > nrows)
        nt = (int)nrows;
    jobs = (bwd_job*)calloc((size_t)nt, sizeof(bwd_job));
    tids = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return -1;
    }
    per = (nrows + nt - 1) / nt;
    for (k = 0; k < nt; ++k) {
        bwd_job* j = &jobs[k];
        j->r0 = k * per;
        j->r1 = j->r0 + per < nrows ? j->r0 + per : nrows;
        j->L = seqlen;
        j->N = dstate;
        j->batch = batch;
        j->dim = dim;
        j->row_b = row_b;
        j->row_d = row_d;
        j->x = x;
        j->delta = delta;
        j->z = z;
        j->A = A;
        j->B = B;
        j->C = C;
        j->D = D;
        j->bias = delta_bias;
        j->softplus = delta_softplus;
        j->h0 = h0;
        j->dy = dy;
        j->dh_final = dh_final;
        j->dx = dx;
        j->ddelta = ddelta;
        j->dz = dz;
        j->dh0 = dh0;
        j->dA = (double*)calloc((size_t)nA, sizeof(double));
        j->dB = (double*)calloc((size_t)nBC, sizeof(double));
        j->dC = (double*)calloc((size_t)nBC, sizeof(double));
        j->dD = (double*)calloc((size_t)dim, sizeof(double));
        j->dbias = (double*)calloc((size_t)dim, sizeof(double));
        j->status = (j->dA && j->dB && j->dC && j->dD && j->dbias) ? 1 : -1;
    }
    for (k = 1; k < nt; ++k)
        if (jobs[k].status == 1 && pthread_create(&tids[k], NULL, bwd_thread, &jobs[k]) != 0)
            bwd_block(&jobs[k]), tids[k] = 0;
    if (jobs[0].status == 1)
        bwd_block(&jobs[0]);
    for (k = 1; k < nt; ++k)
        if (tids[k])
            pthread_join(tids[k], NULL);
    for (k = 0; k < nt; ++k) {
        bwd_job* j = &jobs[k];
        if (j->status != 0)
            rc = -1;
        if (j->dA && j->dB && j->dC && j->dD && j->dbias && rc == 0) {
            for (i = 0; i < nA; ++i) dA[i] += j->dA[i];
            for (i = 0; i < nBC; ++i) dB[i] += j->dB[i];
            for (i = 0; i < nBC; ++i) dC[i] += j->dC[i];
            for (i = 0; i < dim; ++i) dbias[i] += j->dbias[i];
            if (dD)
                for (i = 0; i < dim; ++i) dD[i] += j->dD[i];
        }
        free(j->dA); free(j->dB); free(j->dC); free(j->dD); free(j->dbias);
    }
    free(jobs);
    free(tids);
    return rc;
}
