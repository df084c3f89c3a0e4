/*
 * sanitize_check.c -- a driver that runs every entry point of efla_oracle.c
 * on exactly sized heap buffers, for a build with the address and
 * undefined-behaviour sanitizers (test infrastructure, like the oracle).
 *
 * Cases: forward, step and backward under both rules; zero and given
 * initial states and state gradients; L = 0, L = 1 and lengths that end in
 * a partial 64-token recompute segment; one and several threads; s_final
 * aliasing s0; the coefficient and its derivative at 0 and in the stiff
 * limit.  Exit status 0 when every call returns 0 and every result is finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_coeff_rule(const double *k, const double *beta, double *lam_out, double *alpha_out,
                      int64_t n, int dk, int rule);
int oracle_forward_rule(const double *q, const double *k, const double *v, const double *beta,
                        const double *s0, double *o, double *s_final, int B, int H, int64_t L, int dk,
                        int dv, int nthreads, int rule);
int oracle_step_rule(const double *q, const double *k, const double *v, const double *beta,
                     double *state, double *o, int N, int H, int dk, int dv, int rule);
int oracle_alpha_grad(double beta, double lam, int rule, double *out);
int oracle_backward_rule(const double *q, const double *k, const double *v, const double *beta,
                         const double *s0, const double *dO, const double *dSL, double *dq, double *dk,
                         double *dv, double *dbeta, double *dS0, int B, int H, int64_t L, int dk_,
                         int dv_, int nthreads, int rule);

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static double urand(void) { /* xorshift64*, uniform in [-1, 1) */
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return (double)((rng * 2685821657736338717ull) >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double *vec(size_t n, double scale) {
    double *p = (double *)malloc(n ? n * sizeof(double) : 1);
    if (!p) exit(3);
    for (size_t i = 0; i < n; ++i) p[i] = scale * urand();
    return p;
}
static int finite(const double *p, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}
static int failures = 0;
static void expect(int ok, const char *what) {
    if (!ok) { fprintf(stderr, "FAIL: %s\n", what); ++failures; }
}

static void run(int B, int H, int64_t L, int dk, int dv, int nthreads, int rule, int with_s0, int with_dsl) {
    const size_t nq = (size_t)(B * L * H) * dk, nv = (size_t)(B * L * H) * dv, nb = (size_t)(B * L * H);
    const size_t ns = (size_t)B * H * dk * dv;
    double *q = vec(nq, 1.0), *k = vec(nq, 1.0), *v = vec(nv, 1.0), *beta = vec(nb, 1.0);
    for (size_t i = 0; i < nb; ++i) beta[i] = fabs(beta[i]) * 3.0;
    double *s0 = with_s0 ? vec(ns, 0.1) : NULL;
    double *o = vec(nv, 0.0), *sf = vec(ns, 0.0);
    expect(oracle_forward_rule(q, k, v, beta, s0, o, sf, B, H, L, dk, dv, nthreads, rule) == 0, "forward");
    expect(finite(o, nv) && finite(sf, ns), "forward finite");
    if (s0) {  /* in place: s_final aliasing s0 */
        double *st = vec(ns, 0.0);
        for (size_t i = 0; i < ns; ++i) st[i] = s0[i];
        expect(oracle_forward_rule(q, k, v, beta, st, NULL, st, B, H, L, dk, dv, nthreads, rule) == 0,
               "forward in place");
        for (size_t i = 0; i < ns; ++i) expect(st[i] == sf[i], "in-place state equals the separate one");
        free(st);
    }
    double *dO = vec(nv, 1.0), *dsl = with_dsl ? vec(ns, 1.0) : NULL;
    double *dq = vec(nq, 0.0), *dkk = vec(nq, 0.0), *dvv = vec(nv, 0.0), *db = vec(nb, 0.0);
    double *ds0 = vec(ns, 0.0);
    expect(oracle_backward_rule(q, k, v, beta, s0, dO, dsl, dq, dkk, dvv, db, ds0, B, H, L, dk, dv, nthreads,
                                rule) == 0, "backward");
    expect(finite(dq, nq) && finite(dkk, nq) && finite(dvv, nv) && finite(db, nb) && finite(ds0, ns),
           "backward finite");
    expect(oracle_backward_rule(q, k, v, beta, s0, dO, dsl, dq, dkk, dvv, db, NULL, B, H, L, dk, dv, nthreads,
                                rule) == 0, "backward without ds0");
    double *lam = vec(nb, 0.0), *al = vec(nb, 0.0);
    expect(oracle_coeff_rule(k, beta, lam, al, (int64_t)nb, dk, rule) == 0, "coeff");
    expect(oracle_coeff_rule(k, beta, NULL, al, (int64_t)nb, dk, rule) == 0, "coeff without lambda");
    /* decode: B sequences of one token on the states reached above */
    if (L > 0) {
        const size_t n1 = (size_t)B * H;
        double *o1 = vec(n1 * dv, 0.0);
        expect(oracle_step_rule(q, k, v, beta, sf, o1, B, H, dk, dv, rule) == 0, "step");
        expect(oracle_step_rule(q, k, v, beta, sf, NULL, B, H, dk, dv, rule) == 0, "step without o");
        expect(finite(o1, n1 * dv) && finite(sf, ns), "step finite");
        free(o1);
    }
    free(q); free(k); free(v); free(beta); free(s0); free(o); free(sf); free(dO); free(dsl);
    free(dq); free(dkk); free(dvv); free(db); free(ds0); free(lam); free(al);
}

int main(void) {
    for (int rule = 0; rule < 2; ++rule) {
        run(1, 1, 0, 4, 3, 1, rule, 1, 1);      /* empty sequence */
        run(2, 3, 0, 4, 3, 2, rule, 0, 0);
        run(1, 2, 1, 5, 4, 1, rule, 1, 0);      /* one token */
        run(2, 3, 130, 6, 5, 3, rule, 1, 1);    /* two full recompute segments and a partial one */
        run(2, 3, 64, 8, 8, 4, rule, 0, 1);     /* exactly one segment, zero initial state */
        run(1, 5, 77, 3, 7, 8, rule, 0, 0);     /* more threads than some units */
    }
    const double grid[][2] = {{0.0, 0.0}, {1.0, 0.0}, {0.0, 2.0}, {0.5, 1e-30}, {3.0, 1e8}, {1e-3, 0.01}};
    for (int r = 0; r < 2; ++r)
        for (size_t i = 0; i < sizeof grid / sizeof grid[0]; ++i) {
            double out[2];
            expect(oracle_alpha_grad(grid[i][0], grid[i][1], r, out) == 0 && isfinite(out[0]) && isfinite(out[1]),
                   "alpha_grad");
        }
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("sanitize_check: all oracle entry points clean\n");
    return 0;
}
