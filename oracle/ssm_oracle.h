/*
 * ssm_oracle.h - fp64 CPU reference for the selective scan (TEST INFRASTRUCTURE).
 *
 * This is the oracle the HIP path is checked against. Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it. It shares no
 * code, header, table or constant with the GPU library.
 *
 * What it computes, per batch row b and channel d (a "row"), for t = 0..L-1 and
 * state index n = 0..N-1:
 *
 *   v        = delta_raw[t] + delta_bias[d]                 (bias 0 when absent)
 *   Delta_t  = softplus(v) = log(1 + e^v)                    (or v when softplus is off)
 *   h_t[n]   = exp(Delta_t * A[d,n]) * h_{t-1}[n] + (Delta_t * x_t) * B_t[n]
 *   s_t      = sum_n C_t[n] * h_t[n]  (+ D[d] * x_t when D is given)
 *   y_t      = s_t * silu(z_t)        (when z is given),  silu(z) = z / (1 + e^-z)
 *
 * with h_{-1} = h0 (zeros when absent). Sources on the pages:
 *  - the state and output equations h' = Ah + Bu, y = Ch + Du: "State-Space Models
 *    (SSMs) & Mamba" (aidatadrop), section "State-Space Models (SSMs): A
 *    Resurgent Paradigm for Sequence Modeling";
 *  - B, C and the step size Delta computed per token, A and D not: "Mamba: How
 *    Selective State Spaces Achieve 5x Faster Inference Than Transformers",
 *    section "The selective mechanism: input-dependent SSM parameters", and the
 *    aidatadrop page, section "The Magic of Selective Scan";
 *  - the discretized update (the pages call it discretized but print no
 *    formula; the zero-order-hold style exp(Delta*A) for the decay and Delta*B*x
 *    for the input is the plainest reading consistent with the continuous
 *    equations), the update-then-read order, and the gating of the scan output
 *    by SiLU of the second branch:
 *    "Mamba Architecture Explained: Why Transformers Aren't the Final Word",
 *    sections "The Mamba Innovation: Selective State Updates" and "The
 *    Architecture in Practice";
 *  - one token per step with a fixed-size state for inference: the promptingindex
 *    page, "The selective mechanism", and the aidatadrop page, "The Payoff".
 * softplus and dt_bias are not on the pages; they are the plainest Mamba reading
 * of a per-token step size that must stay positive.
 *
 * All arithmetic is plain fp64 in the order written above, one row after the
 * other; rows are independent, and the thread split only hands whole rows to
 * threads (no reordering inside a row).
 */
#ifndef SSM_ORACLE_H
#define SSM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* log(1 + e^v) evaluated without overflow: v + log1p(e^-v) for v > 0. */
double ssm_oracle_softplus(double v);
/* z * sigma(z), sigma evaluated on the side where e^(-|z|) cannot overflow. */
double ssm_oracle_silu(double z);

/*
 * Forward scan over `nrows` rows, each of `seqlen` tokens.
 *   row_b[r], row_d[r]  : batch index and channel index of row r
 *   x, delta            : [nrows][seqlen]  (delta is the raw value before the bias)
 *   z                   : [nrows][seqlen] or NULL (no gate)
 *   A                   : [dim][dstate]    (row r uses A[row_d[r]])
 *   B, C                : [batch][seqlen][dstate] (row r uses batch row_b[r])
 *   D, delta_bias       : [dim] or NULL
 *   h0                  : [nrows][dstate] or NULL (zeros)
 *   y                   : [nrows][seqlen] out
 *   h_final             : [nrows][dstate] out, or NULL
 *   nthreads            : worker threads (>= 1); rows are split into contiguous blocks
 * Returns 0, or -1 on a bad argument (nothing written).
 */
int ssm_oracle_scan_rows(int64_t nrows, int64_t seqlen, int64_t dstate,
                         const int64_t* row_b, const int64_t* row_d,
                         const double* x, const double* delta, const double* z,
                         const double* A, const double* B, const double* C,
                         const double* D, const double* delta_bias, int delta_softplus,
                         const double* h0, double* y, double* h_final, int nthreads);

/*
 * One decode step (one token per row), updating `state` in place.
 *   state               : [nrows][dstate] in: h_{t-1}, out: h_t
 *   x, delta, z         : [nrows] (z may be NULL)
 *   B, C                : [batch][dstate]
 *   y                   : [nrows] out
 * Same per-token arithmetic as ssm_oracle_scan_rows.
 */
int ssm_oracle_step_rows(int64_t nrows, int64_t dstate,
                         const int64_t* row_b, const int64_t* row_d,
                         double* state, const double* x, const double* delta,
                         const double* z, const double* A, const double* B,
                         const double* C, const double* D, const double* delta_bias,
                         int delta_softplus, double* y);

/*
 * Gradients of the scan (reverse mode; the pages give none, so this is the
 * derivative of the definition above). With q_t = sum_n C_t[n] h_t[n] + D x_t the
 * output before the gate, a_t[n] = exp(Delta_t A[n]), u_t = Delta_t x_t and
 * G_t = dLoss/dh_t, for t = L-1 down to 0:
 *   dq_t     = dy_t * silu(z_t)                 (dy_t without z)
 *   dz_t     = dy_t * q_t * silu'(z_t),   silu'(z) = s (1 + z (1 - s)), s = sigma(z)
 *   G_t[n]   = a_{t+1}[n] G_{t+1}[n] + dq_t C_t[n]     (the first term is dh_final at t = L-1)
 *   dC_t[n] += dq_t h_t[n]          dB_t[n] += G_t[n] u_t     (summed over channels)
 *   dx_t     = dq_t D + Delta_t sum_n G_t[n] B_t[n]
 *   dDelta_t = x_t sum_n G_t[n] B_t[n] + sum_n G_t[n] h_{t-1}[n] a_t[n] A[n]
 *   ddelta_t = dDelta_t * sigma(v_t)    (softplus' ; 1 without softplus),  dbias += ddelta_t
 *   dA[n]   += G_t[n] h_{t-1}[n] a_t[n] Delta_t     dD += dq_t x_t
 *   dh0[n]   = a_0[n] G_0[n]
 * Shapes as for ssm_oracle_scan_rows; dy [nrows][seqlen]; dh_final [nrows][dstate] or
 * NULL; outputs dx, ddelta, dz (when z is given) [nrows][seqlen]; dA [dim][dstate],
 * dD (when D is given), dbias [dim] and dB, dC [batch][seqlen][dstate] are the sums over
 * the given rows (overwritten); dh0 [nrows][dstate] or NULL. Returns 0 or -1.
 */
int ssm_oracle_scan_bwd_rows(int64_t nrows, int64_t seqlen, int64_t dstate,
                             const int64_t* row_b, const int64_t* row_d, int64_t batch,
                             int64_t dim, const double* x, const double* delta,
                             const double* z, const double* A, const double* B,
                             const double* C, const double* D, const double* delta_bias,
                             int delta_softplus, const double* h0, const double* dy,
                             const double* dh_final, double* dx, double* ddelta, double* dz,
                             double* dA, double* dB, double* dC, double* dD, double* dbias,
                             double* dh0, int nthreads);

#ifdef __cplusplus
}
#endif
#endif /* SSM_ORACLE_H */
