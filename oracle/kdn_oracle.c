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

/*
 * Reverse-mode gradient of the diagonal-precision memory above.  The pages
 * train these layers but print no gradient, so this is the mechanical adjoint
 * of the printed recurrence (Palimpsa summary, Metodologia items 1-2, in its
 * direct mu form), written entry by entry: every memory entry [j][i] follows
 * its own scalar recurrence (the update is elementwise), so for each entry
 * the forward values I_t, mu_t are recorded, then walked back in time.
 *
 * For the scalar loss
 *   L = sum_t sum_i dout[t][i] o_t[i] + sum_e dI_T[e] I_T[e] + sum_e dmu_T[e] mu_T[e]
 * (dI_T, dmu_T may be NULL = zero) it returns dL/d(input) in
 *   g[0] dq [T][dk]   g[1] dk [T][dk]   g[2] dv [T][dv]   g[3] dbeta [T][dv]
 *   g[4] dd [T]       g[5] dA [1]       g[6] dI_prior [1]
 *   g[7] dI0 [dk][dv] g[8] dmu0 [dk][dv]
 * With I0 == NULL the start is I_prior, whose path then feeds g[6] and g[7]
 * is not written; with mu0 == NULL the start mean is 0 and g[8] is not
 * written.
 *
 * scale (may be NULL, else 9 arrays shaped like g) receives the same
 * quantities computed with every term replaced by its absolute value: the
 * natural error scale of each gradient (it bounds |g|).
 *
 * Returns 0, or -1 if scratch memory cannot be allocated.
 */
int oracle_diag_head_bwd(long T, long dk, long dv,
                         const double* q, const double* k, const double* v,
                         const double* beta, const double* d,
                         double A, double I_prior,
                         const double* I0, const double* mu0,
                         const double* dout, const double* dI_T, const double* dmu_T,
                         double* const* g, double* const* scale)
{
    const long n = dk * dv;
    double* Ih = (double*)malloc(sizeof(double) * (T + 1));   /* I before/after each token */
    double* mh = (double*)malloc(sizeof(double) * (T + 1));   /* mu before/after each token */
    if (!Ih || !mh) { free(Ih); free(mh); return -1; }

    const long sizes[9] = {T * dk, T * dk, T * dv, T * dv, T, 1, 1, n, n};
    for (int a = 0; a < 9; ++a) {
        if ((a == 7 && !I0) || (a == 8 && !mu0)) continue;
        memset(g[a], 0, sizeof(double) * sizes[a]);
        if (scale) memset(scale[a], 0, sizeof(double) * sizes[a]);
    }

    for (long j = 0; j < dk; ++j) {
        for (long i = 0; i < dv; ++i) {
            const long e = j * dv + i;

            /* forward, recording the entry's history */
            Ih[0] = I0 ? I0[e] : I_prior;
            mh[0] = mu0 ? mu0[e] : 0.0;
            for (long t = 0; t < T; ++t) {
                const double alpha = exp(-A * d[t]);
                const double b = beta[t * dv + i], kk = k[t * dk + j], vv = v[t * dv + i];
                const double I_old = Ih[t];
                const double I_new = alpha * I_old + (1.0 - alpha) * I_prior + b * kk * kk;
                mh[t + 1] = alpha * (I_old / I_new) * mh[t] + (1.0 / I_new) * (b * vv * kk);
                Ih[t + 1] = I_new;
            }

            /* adjoints of the state after the last token, and their magnitudes */
            double gI = dI_T ? dI_T[e] : 0.0, gM = dmu_T ? dmu_T[e] : 0.0;
            double aI = fabs(gI), aM = fabs(gM);

            for (long t = T - 1; t >= 0; --t) {
                const double alpha = exp(-A * d[t]);
                const double b = beta[t * dv + i], kk = k[t * dk + j], vv = v[t * dv + i];
                const double qq = q[t * dk + j], go = dout[t * dv + i];
                const double Ip = Ih[t], In = Ih[t + 1], mp = mh[t], mn = mh[t + 1];

                /* read-out o_t[i] += q_t[j] mu_t[j][i] */
                gM += qq * go;
                aM += fabs(qq * go);
                g[0][t * dk + j] += mn * go;
                if (scale) scale[0][t * dk + j] += fabs(mn * go);

                /* mu_t = (alpha I_{t-1} mu_{t-1} + b v k) / I_t: its I_t dependence */
                const double gIn = gI - gM * mn / In;
                const double aIn = aI + aM * fabs(mn) / In;

                /* I_t = alpha I_{t-1} + (1 - alpha) I_prior + b k^2 and mu_t's own inputs */
                const double g_alpha = gM * Ip * mp / In + gIn * (Ip - I_prior);
                const double a_alpha = aM * fabs(Ip * mp) / In + aIn * fabs(Ip - I_prior);
                g[1][t * dk + j] += gM * b * vv / In + gIn * 2.0 * b * kk;
                g[2][t * dv + i] += gM * b * kk / In;
                g[3][t * dv + i] += gM * vv * kk / In + gIn * kk * kk;
                g[4][t] += g_alpha * (-A * alpha);
                g[5][0] += g_alpha * (-d[t] * alpha);
                g[6][0] += gIn * (1.0 - alpha);
                if (scale) {
                    scale[1][t * dk + j] += aM * fabs(b * vv) / In + aIn * 2.0 * fabs(b * kk);
                    scale[2][t * dv + i] += aM * fabs(b * kk) / In;
                    scale[3][t * dv + i] += aM * fabs(vv * kk) / In + aIn * kk * kk;
                    scale[4][t] += a_alpha * fabs(A * alpha);
                    scale[5][0] += a_alpha * fabs(d[t] * alpha);
                    scale[6][0] += aIn * (1.0 - alpha);
                }

                /* carry to the state before token t */
                const double gM_prev = gM * alpha * Ip / In;
                const double gI_prev = gM * alpha * mp / In + gIn * alpha;
                aI = aM * alpha * fabs(mp) / In + aIn * alpha;
                aM = aM * alpha * Ip / In;
                gM = gM_prev;
                gI = gI_prev;
            }

            if (I0) {
                g[7][e] = gI;
                if (scale) scale[7][e] = aI;
            } else {
                g[6][0] += gI;
                if (scale) scale[6][0] += aI;
            }
            if (mu0) {
                g[8][e] = gM;
                if (scale) scale[8][e] = aM;
            }
        }
    }
    free(Ih);
    free(mh);
    return 0;
}

/*
 * Diagonal KDN with process noise (Kalman Delta Networks abstract, "Diagonal
 * KDN": each one-step posterior is projected onto the diagonal Gaussian
 * family by online mean-field variational inference, and the Kalman gain
 * weights each residual write).  The memory column i is a latent vector
 * s_i in R^{d_k} observed through v_t[i] = k_t^T s_i + noise of precision
 * beta_t[i]; the state keeps one mean and one precision per entry [j][i].
 * Per token t, for every column i:
 *
 *   predict  (KLA summary, Metodologia 1: decay a_t, process noise p_t)
 *            variance_pred[j] = a_t^2 / lambda[j] + p_t,  mean_pred[j] = a_t mu[j]
 *   update   the exact one-step posterior from this diagonal prior is
 *            Gaussian with precision diag(1/variance_pred) + beta k k^T and mean
 *              mean_pred + variance_pred . k (v - k^T mean_pred) / S,
 *              S = sum_j k_j^2 variance_pred[j] + 1/beta
 *            (the Kalman gain on the residual); its mean-field projection
 *            keeps that mean and the diagonal of that precision:
 *            lambda[j] = 1/variance_pred[j] + beta k_j^2
 *   read     o_t[i] = sum_j q_t[j] mu_t[j][i]
 *
 * lam0 / mu0 may be NULL (then 1 and 0).  s (may be NULL) receives
 * sum_j |q_t[j] mu_t[j][i]|.  lam_T, mu_T may be NULL.  Returns 0 or -1.
 */
int oracle_diag_noise_head(long T, long dk, long dv,
                           const double* q, const double* k, const double* v,
                           const double* beta, const double* a, const double* p,
                           const double* lam0, const double* mu0,
                           double* o, double* s, double* lam_T, double* mu_T)
{
    const long n = dk * dv;
    double* lam = (double*)malloc(sizeof(double) * n);
    double* mu = (double*)malloc(sizeof(double) * n);
    double* var_pred = (double*)malloc(sizeof(double) * dk);
    double* mean_pred = (double*)malloc(sizeof(double) * dk);
    if (!lam || !mu || !var_pred || !mean_pred) {
        free(lam); free(mu); free(var_pred); free(mean_pred);
        return -1;
    }
    for (long e = 0; e < n; ++e) {
        lam[e] = lam0 ? lam0[e] : 1.0;
        mu[e] = mu0 ? mu0[e] : 0.0;
    }

    for (long t = 0; t < T; ++t) {
        const double* kt = k + t * dk;
        const double* qt = q + t * dk;
        const double* vt = v + t * dv;
        const double* bt = beta + t * dv;
        for (long i = 0; i < dv; ++i) {
            double S = 1.0 / bt[i];
            double prediction = 0.0;
            for (long j = 0; j < dk; ++j) {
                const long e = j * dv + i;
                var_pred[j] = a[t] * a[t] / lam[e] + p[t];
                mean_pred[j] = a[t] * mu[e];
                S += kt[j] * kt[j] * var_pred[j];
                prediction += kt[j] * mean_pred[j];
            }
            const double residual = vt[i] - prediction;
            for (long j = 0; j < dk; ++j) {
                const long e = j * dv + i;
                mu[e] = mean_pred[j] + var_pred[j] * kt[j] * residual / S;
                lam[e] = 1.0 / var_pred[j] + bt[i] * kt[j] * kt[j];
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
    if (lam_T) memcpy(lam_T, lam, sizeof(double) * n);
    if (mu_T) memcpy(mu_T, mu, sizeof(double) * n);
    free(lam);
    free(mu);
    free(var_pred);
    free(mean_pred);
    return 0;
}

/*
 * Exact KDN: the Kalman filter the diagonal and isotropic variants
 * approximate (Kalman Delta Networks abstract: exact tracking is a dense,
 * state-dependent Riccati recursion).  The memory is a d_k x d_v matrix whose
 * value column i is a latent vector s_i in R^{d_k}:
 *   transition   s_i <- a_t s_i + noise, covariance p_t Id   (KLA Metodologia 1)
 *   observation  v_t[i] = k_t^T s_i + noise, precision beta_t[i]
 * Each column keeps a full covariance P_i [d_k x d_k] and mean m_i; per token,
 * in covariance form:
 *   P- = a^2 P + p Id,  u = P- k,  S = k^T u + 1/beta,  K = u / S
 *   m  = a m + K (v_i - a k^T m),   P = P- - K u^T
 *   o_t[i] = q_t^T m_i
 * P0 [d_v][d_k][d_k] (may be NULL: Id / lambda0 with lambda0 = 1) and mu0
 * [d_k][d_v] (NULL: 0) give the start.  o is [T][d_v]; P_T (may be NULL)
 * receives the final covariances, mu_T (may be NULL) the means [d_k][d_v].
 * Returns 0 or -1.
 */
int oracle_kdn_exact_head(long T, long dk, long dv,
                          const double* q, const double* k, const double* v,
                          const double* beta, const double* a, const double* p,
                          const double* P0, const double* mu0,
                          double* o, double* P_T, double* mu_T)
{
    double* P = (double*)malloc(sizeof(double) * dv * dk * dk);
    double* m = (double*)malloc(sizeof(double) * dv * dk);
    double* u = (double*)malloc(sizeof(double) * dk);
    if (!P || !m || !u) { free(P); free(m); free(u); return -1; }
    for (long i = 0; i < dv; ++i) {
        for (long r = 0; r < dk; ++r) {
            m[i * dk + r] = mu0 ? mu0[r * dv + i] : 0.0;
            for (long c = 0; c < dk; ++c)
                P[(i * dk + r) * dk + c] = P0 ? P0[(i * dk + r) * dk + c] : (r == c ? 1.0 : 0.0);
        }
    }
    for (long t = 0; t < T; ++t) {
        const double* kt = k + t * dk;
        const double* qt = q + t * dk;
        const double a2 = a[t] * a[t];
        for (long i = 0; i < dv; ++i) {
            double* Pi = P + i * dk * dk;
            double* mi = m + i * dk;
            /* predict */
            for (long r = 0; r < dk; ++r) {
                for (long c = 0; c < dk; ++c) Pi[r * dk + c] *= a2;
                Pi[r * dk + r] += p[t];
                mi[r] *= a[t];
            }
            /* update with the scalar observation v_t[i] of k_t^T s_i */
            double S = 1.0 / beta[t * dv + i];
            double pred = 0.0;
            for (long r = 0; r < dk; ++r) {
                double acc = 0.0;
                for (long c = 0; c < dk; ++c) acc += Pi[r * dk + c] * kt[c];
                u[r] = acc;
                S += kt[r] * acc;
                pred += kt[r] * mi[r];
            }
            const double resid = v[t * dv + i] - pred;
            for (long r = 0; r < dk; ++r) mi[r] += u[r] / S * resid;
            for (long r = 0; r < dk; ++r)
                for (long c = 0; c < dk; ++c) Pi[r * dk + c] -= u[r] * u[c] / S;
            double acc = 0.0;
            for (long r = 0; r < dk; ++r) acc += qt[r] * mi[r];
            o[t * dv + i] = acc;
        }
    }
    if (P_T) memcpy(P_T, P, sizeof(double) * dv * dk * dk);
    if (mu_T)
        for (long i = 0; i < dv; ++i)
            for (long r = 0; r < dk; ++r) mu_T[r * dv + i] = m[i * dk + r];
    free(P);
    free(m);
    free(u);
    return 0;
}
