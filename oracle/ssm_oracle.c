/*
 * ssm_oracle.c - fp64 CPU reference for the selective scan (TEST INFRASTRUCTURE).
 *
 * Only tests, the smoke check and the benchmark's CPU-baseline leg use this file.
 * The recurrence and its sources on the pages are stated in ssm_oracle.h. Every
 * row is a plain sequential loop over time, exactly in the order of the
 * definition; nothing is blocked, fused or reassociated.
 */
#include "ssm_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>

double ssm_oracle_softplus(double v)
{
    /* log(1 + e^v); for v > 0 rewrite as v + log(1 + e^-v) so e^v cannot overflow. */
    if (v > 0.0)
        return v + log1p(exp(-v));
    return log1p(exp(v));
}

double ssm_oracle_silu(double z)
{
    /* z * sigma(z) with sigma(z) = 1 / (1 + e^-z), taken on the side where the
     * exponential is at most 1. */
    double sig;
    if (z >= 0.0) {
        sig = 1.0 / (1.0 + exp(-z));
    } else {
        double e = exp(z);
        sig = e / (1.0 + e);
    }
    return z * sig;
}

/*
 * One token of one row: update the N states in place, return the output.
 * This single function is the whole method; the scan and the decode step both
 * call it, once per token.
 */
static double oracle_token(int64_t N, double* h, double x_t, double delta_raw_t,
                           const double* z_t, const double* a, const double* B_t,
                           const double* C_t, const double* D_d, const double* bias_d,
                           int delta_softplus)
{
    double v = delta_raw_t + (bias_d ? *bias_d : 0.0);
    double delta = delta_softplus ? ssm_oracle_softplus(v) : v;
    double s = 0.0;
    int64_t n;

    /* discretize and update: h = exp(Delta * A) * h + (Delta * x) * B */
    for (n = 0; n < N; ++n)
        h[n] = exp(delta * a[n]) * h[n] + (delta * x_t) * B_t[n];
    /* read out after the update: s = sum_n C[n] * h[n], ascending n */
    for (n = 0; n < N; ++n)
        s += C_t[n] * h[n];
    /* skip term D * x, then the gate silu(z) */
    if (D_d)
        s += (*D_d) * x_t;
    if (z_t)
        s *= ssm_oracle_silu(*z_t);
    return s;
}

typedef struct {
    int64_t r0, r1, L, N;
    const int64_t *row_b, *row_d;
    const double *x, *delta, *z, *A, *B, *C, *D, *bias, *h0;
    int softplus;
    double *y, *h_final;
    int status;
} scan_job;

static void scan_block(scan_job* j)
{
    const int64_t L = j->L, N = j->N;
    double* h = (double*)malloc((size_t)N * sizeof(double));
    int64_t r, t, n;
    if (!h) {
        j->status = -1;
        return;
    }
    for (r = j->r0; r < j->r1; ++r) {
        const int64_t b = j->row_b[r], d = j->row_d[r];
        const double* a = j->A + d * N;
        const double* Dd = j->D ? j->D + d : NULL;
        const double* bias = j->bias ? j->bias + d : NULL;
        for (n = 0; n < N; ++n)
            h[n] = j->h0 ? j->h0[r * N + n] : 0.0;
        for (t = 0; t < L; ++t) {
            const double* Bt = j->B + (b * L + t) * N;
            const double* Ct = j->C + (b * L + t) * N;
            const double* zt = j->z ? j->z + r * L + t : NULL;
            j->y[r * L + t] = oracle_token(N, h, j->x[r * L + t], j->delta[r * L + t], zt, a,
                                           Bt, Ct, Dd, bias, j->softplus);
        }
        if (j->h_final)
            for (n = 0; n < N; ++n)
                j->h_final[r * N + n] = h[n];
    }
    free(h);
    j->status = 0;
}

static void* scan_thread(void* p)
{
    scan_block((scan_job*)p);
    return NULL;
}

int ssm_oracle_scan_rows(int64_t nrows, int64_t seqlen, int64_t dstate,
                         const int64_t* row_b, const int64_t* row_d,
                         const double* x, const double* delta, const double* z,
                         const double* A, const double* B, const double* C,
                         const double* D, const double* delta_bias, int delta_softplus,
                         const double* h0, double* y, double* h_final, int nthreads)
{
    scan_job* jobs;
    pthread_t* tids;
    int64_t per, i;
    int k, nt, rc = 0;

    if (nrows < 0 || seqlen < 0 || dstate <= 0 || !row_b || !row_d || !x || !delta || !A ||
        !B || !C || !y)
        return -1;
    if (nrows == 0)
        return 0;
    nt = nthreads < 1 ? 1 : nthreads;
    if ((int64_t)nt > nrows)
        nt = (int)nrows;
    jobs = (scan_job*)calloc((size_t)nt, sizeof(scan_job));
    tids = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return -1;
    }
    per = (nrows + nt - 1) / nt;
    for (k = 0; k < nt; ++k) {
        scan_job* j = &jobs[k];
        j->r0 = (int64_t)k * per;
        j->r1 = j->r0 + per < nrows ? j->r0 + per : nrows;
        j->L = seqlen;
        j->N = dstate;
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
        j->h0 = h0;
        j->softplus = delta_softplus;
        j->y = y;
        j->h_final = h_final;
        j->status = -1;
    }
    /* thread 0's block runs on the calling thread */
    for (k = 1; k < nt; ++k)
        if (pthread_create(&tids[k], NULL, scan_thread, &jobs[k]) != 0)
            scan_block(&jobs[k]), tids[k] = 0;
    scan_block(&jobs[0]);
    for (k = 1; k < nt; ++k)
        if (tids[k])
            pthread_join(tids[k], NULL);
    for (i = 0; i < nt; ++i)
        if (jobs[i].status != 0)
            rc = -1;
    free(jobs);
    free(tids);
    return rc;
}

int ssm_oracle_step_rows(int64_t nrows, int64_t dstate,
                         const int64_t* row_b, const int64_t* row_d,
                         double* state, const double* x, const double* delta,
                         const double* z, const double* A, const double* B,
                         const double* C, const double* D, const double* delta_bias,
                         int delta_softplus, double* y)
{
    int64_t r;
    if (nrows < 0 || dstate <= 0 || !row_b || !row_d || !state || !x || !delta || !A || !B ||
        !C || !y)
        return -1;
    for (r = 0; r < nrows; ++r) {
        const int64_t b = row_b[r], d = row_d[r];
        y[r] = oracle_token(dstate, state + r * dstate, x[r], delta[r], z ? z + r : NULL,
                            A + d * dstate, B + b * dstate, C + b * dstate,
                            D ? D + d : NULL, delta_bias ? delta_bias + d : NULL,
                            delta_softplus);
    }
    return 0;
}
