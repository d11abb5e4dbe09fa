/*
 * oracle_driver.c -- runs every function of the fp64 oracle (oracle/kdn_oracle.c)
 * on small seeded inputs held in exactly sized heap blocks, with optional
 * arguments both given and NULL, T = 0 and single-row/column heads.  Built
 * with AddressSanitizer and UndefinedBehaviorSanitizer on the CPU by the
 * sanitizer test: any out-of-bounds access, use after free, leak or
 * undefined operation in the oracle aborts the run with a report.  Exit
 * status 0 means every call returned 0 and produced finite results.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_diag_head(long T, long dk, long dv, const double* q, const double* k, const double* v,
                     const double* beta, const double* d, double A, double I_prior,
                     const double* I0, const double* mu0, double* o, double* s, double* I_T,
                     double* mu_T);
int oracle_iso_head(long T, const double* a, const double* p, const double* Lam, double lambda0,
                    long dk, long dv, const double* q, const double* k, const double* v,
                    const double* mu0, double* lambda_out, double* o, double* s, double* mu_T);
int oracle_diag_head_bwd(long T, long dk, long dv, const double* q, const double* k,
                         const double* v, const double* beta, const double* d, double A,
                         double I_prior, const double* I0, const double* mu0,
                         const double* dout, const double* dI_T, const double* dmu_T,
                         double* const* g, double* const* scale);
int oracle_diag_noise_head(long T, long dk, long dv, const double* q, const double* k,
                           const double* v, const double* beta, const double* a, const double* p,
                           const double* lam0, const double* mu0, double* o, double* s,
                           double* lam_T, double* mu_T);
int oracle_kdn_exact_head(long T, long dk, long dv, const double* q, const double* k,
                          const double* v, const double* beta, const double* a, const double* p,
                          const double* P0, const double* mu0, double* o, double* P_T,
                          double* mu_T);

static uint64_t g_state = 0x9e3779b97f4a7c15ull;

static double uniform(void) {   /* xorshift64*, in [0, 1) */
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (double)((g_state * 0x2545f4914f6cdd1dull) >> 11) / 9007199254740992.0;
}

/* n doubles in [lo, hi); n == 0 still returns a distinct heap block */
static double* fill(long n, double lo, double hi) {
    double* x = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!x) { fprintf(stderr, "out of memory\n"); exit(2); }
    for (long i = 0; i < n; ++i) x[i] = lo + (hi - lo) * uniform();
    return x;
}

static int g_fail = 0;

static void check(const char* what, int rc, const double* x, long n) {
    if (rc != 0) { fprintf(stderr, "%s: returned %d\n", what, rc); g_fail = 1; return; }
    for (long i = 0; i < n; ++i)
        if (!isfinite(x[i])) { fprintf(stderr, "%s: non-finite at %ld\n", what, i); g_fail = 1; return; }
}

static void diag_case(long T, long dk, long dv, int with_state, int with_opt) {
    double *q = fill(T * dk, -1, 1), *k = fill(T * dk, -1, 1), *v = fill(T * dv, -1, 1);
    double *beta = fill(T * dv, 0, 1), *d = fill(T, 0.1, 2);
    double *I0 = with_state ? fill(dk * dv, 0.5, 2) : NULL;
    double *mu0 = with_state ? fill(dk * dv, -1, 1) : NULL;
    double *o = fill(T * dv, 0, 0), *s = with_opt ? fill(T * dv, 0, 0) : NULL;
    double *IT = with_opt ? fill(dk * dv, 0, 0) : NULL, *muT = with_opt ? fill(dk * dv, 0, 0) : NULL;
    check("diag", oracle_diag_head(T, dk, dv, q, k, v, beta, d, 1.3, 0.7, I0, mu0, o, s, IT, muT), o, T * dv);

    /* gradient of the same head, every output array sized exactly */
    const long sz[9] = {T * dk, T * dk, T * dv, T * dv, T, 1, 1, dk * dv, dk * dv};
    double *g[9], *sc[9];
    for (int i = 0; i < 9; ++i) { g[i] = fill(sz[i], 0, 0); sc[i] = fill(sz[i], 0, 0); }
    double* dout = fill(T * dv, -1, 1);
    double* dIT = with_opt ? fill(dk * dv, -1, 1) : NULL;
    double* dmuT = with_opt ? fill(dk * dv, -1, 1) : NULL;
    const int rc = oracle_diag_head_bwd(T, dk, dv, q, k, v, beta, d, 1.3, 0.7, I0, mu0, dout, dIT, dmuT,
                                        g, with_opt ? sc : NULL);
    check("diag bwd dq", rc, g[0], sz[0]);
    check("diag bwd dA", rc, g[5], 1);
    for (int i = 0; i < 9; ++i) { free(g[i]); free(sc[i]); }
    free(dout); free(dIT); free(dmuT);
    free(q); free(k); free(v); free(beta); free(d); free(I0); free(mu0); free(o); free(s); free(IT); free(muT);
}

static void iso_case(long T, long dk, long dv, int with_opt) {
    double *a = fill(T, 0.2, 1), *p = fill(T, 0, 1), *L = fill(T, 0, 2);
    double *q = fill(T * dk, -1, 1), *k = fill(T * dk, -1, 1), *v = fill(T * dv, -1, 1);
    double *mu0 = with_opt ? fill(dk * dv, -1, 1) : NULL;
    double *lam = with_opt ? fill(T, 0, 0) : NULL;
    double *o = fill(T * dv, 0, 0), *s = with_opt ? fill(T * dv, 0, 0) : NULL;
    double *muT = with_opt ? fill(dk * dv, 0, 0) : NULL;
    check("iso", oracle_iso_head(T, a, p, L, 1.5, dk, dv, q, k, v, mu0, lam, o, s, muT), o, T * dv);
    free(a); free(p); free(L); free(q); free(k); free(v); free(mu0); free(lam); free(o); free(s); free(muT);
}

static void noise_case(long T, long dk, long dv, int with_opt) {
    double *q = fill(T * dk, -1, 1), *k = fill(T * dk, -1, 1), *v = fill(T * dv, -1, 1);
    double *beta = fill(T * dv, 0.1, 1), *a = fill(T, 0.2, 1), *p = fill(T, 0, 1);
    double *lam0 = with_opt ? fill(dk * dv, 0.5, 2) : NULL, *mu0 = with_opt ? fill(dk * dv, -1, 1) : NULL;
    double *o = fill(T * dv, 0, 0), *s = with_opt ? fill(T * dv, 0, 0) : NULL;
    double *lT = with_opt ? fill(dk * dv, 0, 0) : NULL, *mT = with_opt ? fill(dk * dv, 0, 0) : NULL;
    check("noise", oracle_diag_noise_head(T, dk, dv, q, k, v, beta, a, p, lam0, mu0, o, s, lT, mT), o, T * dv);
    /* the exact filter on the same head */
    double *P0 = with_opt ? fill(dv * dk * dk, 0, 0) : NULL;
    if (P0)
        for (long i = 0; i < dv; ++i)
            for (long j = 0; j < dk; ++j) P0[(i * dk + j) * dk + j] = 1.0 + uniform();
    double *PT = with_opt ? fill(dv * dk * dk, 0, 0) : NULL;
    check("exact", oracle_kdn_exact_head(T, dk, dv, q, k, v, beta, a, p, P0, mu0, o, PT, mT), o, T * dv);
    free(P0); free(PT);
    free(q); free(k); free(v); free(beta); free(a); free(p); free(lam0); free(mu0); free(o); free(s); free(lT); free(mT);
}

int main(void) {
    const long shapes[][3] = {{0, 4, 4}, {1, 1, 1}, {7, 1, 5}, {19, 4, 3}, {33, 8, 2}, {64, 16, 16}};
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i) {
        const long T = shapes[i][0], dk = shapes[i][1], dv = shapes[i][2];
        for (int st = 0; st < 2; ++st)
            for (int opt = 0; opt < 2; ++opt) diag_case(T, dk, dv, st, opt);
        for (int opt = 0; opt < 2; ++opt) {
            iso_case(T, dk, dv, opt);
            noise_case(T, dk, dv, opt);
        }
        iso_case(T, 0, 0, 0);   /* precision path only */
    }
    if (g_fail) return 1;
    printf("oracle sanitizer run: ok\n");
    return 0;
}
