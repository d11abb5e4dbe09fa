/*
 * kdn_oracle.c -- plain sequential fp64 reference of the precision-tracking
 * memory recurrences.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the benchmark's CPU-baseline leg call it; the library never does.  It
 * shares no code, header or constant with the HIP path.
 *
 * Every loop runs in the order the recurrence is written: time outermost and
 * strictly sequential, one memory entry at a time, sums over j in ascending
 * order.  No blocking, reordering or algebraic rewriting.  Compile without
 * -ffast-math and with -ffp-contract=off so each line is plain IEEE double
 * arithmetic.
 *
 * Layouts are those of one head (b, h), row-major:
 *   q, k   [T][dk]      v, beta [T][dv]      d, a, p, Lam [T]
 *   I, mu  [dk][dv]     entry [j][i] couples key channel j with value channel i
 *   o, s   [T][dv]
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

/*
 * Diagonal-precision memory (Palimpsa: "Learning to Remember, Learn, and
 * Forget in Attention-Based Models", Metodologia items 1-2).
 *
 * Per token t:
 *   alpha_t = exp(-A d_t)                                   (forget gate, item 1)
 *   I_t  = alpha_t I_{t-1} + (1 - alpha_t) I_prior + beta_t (outer) k_t^2    (item 2)
 *   mu_t = alpha_t (I_{t-1} / I_t) . mu_{t-1}
 *          + (1 / I_t) . [(beta_t . v_t) (outer) k_t]                         (item 2)
 * with the outer products oriented [j][i] = (value-side i) x (key-side j),
 * then the read-out of the posterior mean by the query after the update
 * (Kalman Linear Attention summary, Metodologia 1, "Readout"):
 *   o_t[i] = sum_j q_t[j] mu_t[j][i]
 * s_t[i] = sum_j |q_t[j] mu_t[j][i]| is reported as the natural error scale of
 * that dot product (it bounds |o_t[i]|).
 *
 * I0 / mu0 may be NULL: then I_0 = I_prior and mu_0 = 0.  s, I_T, mu_T may be
 * NULL.  Returns 0, or -1 if scratch memory cannot be allocated.
 */
int oracle_diag_head(long T, long dk, long dv,
                     const double* q, const double* k, const double* v,
                     const double* beta, const double* d,
                     double A, double I_prior,
                     const double* I0, const double* mu0,
                     double* o, double* s, double* I_T, double* mu_T)
{
    const long n = dk * dv;
    double* I = (double*)malloc(sizeof(double) * n);
    double* mu = (double*)malloc(sizeof(double) * n);
    if (!I || !mu) { free(I); free(mu); return -1; }
    for (long e = 0; e < n; ++e) {
        I[e] = I0 ? I0[e] : I_prior;
        mu[e] = mu0 ? mu0[e] : 0.0;
    }

    for (long t = 0; t < T; ++t) {
        const double alpha = exp(-A * d[t]);
        const double* kt = k + t * dk;
        const double* qt = q + t * dk;
        const double* vt = v + t * dv;
        const double* bt = beta + t * dv;

        for (long j = 0; j < dk; ++j) {
            for (long i = 0; i < dv; ++i) {
                const long e = j * dv + i;
                const double I_old = I[e];
                const double I_new = alpha * I_old + (1.0 - alpha) * I_prior
                                   + bt[i] * kt[j] * kt[j];
                const double write = bt[i] * vt[i] * kt[j];
                mu[e] = alpha * (I_old / I_new) * mu[e] + (1.0 / I_new) * write;
                I[e] = I_new;
            }
        }

        for (long i = 0; i < dv; ++i) {
            double acc = 0.0, mag = 0.0;
            for (long j = 0; j < dk; ++j) {
                const double term = qt[j] * mu[j * dv + i];
                acc += term;
                mag += fabs(term);
            }
            o[t * dv + i] = acc;
            if (s) s[t * dv + i] = mag;
        }
    }

    if (I_T) memcpy(I_T, I, sizeof(double) * n);
    if (mu_T) memcpy(mu_T, mu, sizeof(double) * n);
    free(I);
    free(mu);
    return 0;
}

/*
 * Isotropic memory: one scalar precision lambda per head (Kalman Delta
 * Networks abstract, "Isotropic KDN"; Kalman Linear Attention summary,
 * Metodologia 1-3).  Written as the textbook scalar Kalman filter in
 * information form, predict then update:
 *
 *   predict  the latent mean decays by a_t and gains process noise of
 *            variance p_t:  variance 1/lambda -> a_t^2/lambda + p_t, so
 *            lambda_pred = 1 / (a_t^2 / lambda + p_t),   mean_pred = a_t mu
 *   update   add the observation's precision Lambda_t:
 *            lambda_t = lambda_pred + Lambda_t
 *            mu_t = (lambda_pred * mean_pred + Lambda_t * k_t v_t^T) / lambda_t
 *            (precision-weighted average of prediction and the token's write)
 *   read     o_t[i] = sum_j q_t[j] mu_t[j][i]
 *
 * lambda_out [T] (may be NULL) receives lambda_t.  mu0 NULL -> 0.  s, mu_T may
 * be NULL.  dk == 0 or dv == 0 runs the precision path only (q, k, v, o
 * ignored).  Returns 0, or -1 on allocation failure.
 */
int oracle_iso_head(long T, const double* a, const double* p, const double* Lam,
                    double lambda0, long dk, long dv,
                    const double* q, const double* k, const double* v,
                    const double* mu0, double* lambda_out,
                    double* o, double* s, double* mu_T)
{
    const long n = dk * dv;
    double* mu = NULL;
    if (n > 0) {
        mu = (double*)malloc(sizeof(double) * n);
        if (!mu) return -1;
        for (long e = 0; e < n; ++e) mu[e] = mu0 ? mu0[e] : 0.0;
    }

    double lambda = lambda0;
    for (long t = 0; t < T; ++t) {
        const double variance_pred = a[t] * a[t] / lambda + p[t];
        const double lambda_pred = 1.0 / variance_pred;
        const double lambda_new = lambda_pred + Lam[t];
        if (lambda_out) lambda_out[t] = lambda_new;

        if (n > 0) {
            const double* kt = k + t * dk;
            const double* qt = q + t * dk;
            const double* vt = v + t * dv;
            for (long j = 0; j < dk; ++j) {
                for (long i = 0; i < dv; ++i) {
                    const long e = j * dv + i;
                    const double mean_pred = a[t] * mu[e];
                    mu[e] = (lambda_pred * mean_pred + Lam[t] * kt[j] * vt[i]) / lambda_new;
                }
            }
            for (long i = 0; i < dv; ++i) {
                double acc = 0.0, mag = 0.0;
                for (long j = 0; j < dk; ++j) {
                    const double term = qt[j] * mu[j * dv + i];
                    acc += term;
                    mag += fabs(term);
                }
                o[t * dv + i] = acc;
                if (s) s[t * dv + i] = mag;
            }
        }
        lambda = lambda_new;
    }

    if (mu_T && n > 0) memcpy(mu_T, mu, sizeof(double) * n);
    free(mu);
    return 0;
}
