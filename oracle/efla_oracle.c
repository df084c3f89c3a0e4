/*
 * efla_oracle.c -- fp64 CPU oracle for Exact Flow Linear Attention (EFLA).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline leg load it.  It shares no code, header, table or constant with the
 * HIP path.
 *
 * What it computes (source: "Exact Flow Linear Attention: Exact Solution from
 * Continuous-Time Dynamics", gist.science summary pages, Method section, steps
 * 2 and 3):
 *
 *   lambda_t = ||k_t||^2
 *   alpha_t  = (1 - exp(-beta_t * lambda_t)) / lambda_t         (Method step 3)
 *   S_t      = (I - alpha_t k_t k_t^T) S_{t-1} + alpha_t k_t v_t^T
 *   o_t      = S_t^T q_t                    (readout: post-update state)
 *
 * The _rule variants also run the other rule the pages discuss: one explicit
 * Euler step of length beta_t of the same ODE, which the pages identify with
 * the delta rule of DeltaNet (Problem statement; Key Contributions 1).  Its
 * coefficient is alpha_t = beta_t; everything else is identical.
 *   rule 0 = exact flow,  rule 1 = explicit Euler (delta rule)
 *
 * alpha is evaluated as beta * (-expm1(-x)/x) with x = beta*lambda: the same
 * quantity written without cancellation; at lambda == 0 it takes its limit,
 * beta.  The
 * pages print no readout; o_t = S_t^T q_t with the state after token t's update
 * is the reading used throughout this project.
 *
 * The recurrence is run token by token exactly as written above, in double
 * precision, one (batch, head) sequence at a time; independent sequences are
 * spread over POSIX threads.  No chunking, no blocking, no reordering.
 *
 * Layouts (all row-major, contiguous):
 *   q, k   [B, L, H, dk]      v, o  [B, L, H, dv]      beta [B, L, H]
 *   state  [B, H, dk, dv]     S[i][j]: i indexes key dims, j value dims.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/*
 * alpha_t from Method step 3.  With x = beta*lambda the coefficient
 * (1 - e^{-x})/lambda equals beta * (1 - e^{-x})/x; that form has no 0/0 at
 * lambda == 0 and survives x underflowing to zero (both give the limit beta).
 * x == +inf (beta or lambda infinite) gives the stiff limit 1/lambda.
 */
double oracle_alpha(double beta, double lam)
{
    const double x = beta * lam;
    if (x == 0.0)
        return beta;
    if (x == INFINITY)
        return 1.0 / lam;
    return beta * (-expm1(-x) / x);
}

/* alpha_t under a rule: the exact flow above, or the explicit Euler step of
 * length beta_t, whose coefficient is beta_t itself. */
static double rule_alpha(double beta, double lam, int rule)
{
    return rule == 1 ? beta : oracle_alpha(beta, lam);
}

/* lambda_t = ||k_t||^2 and alpha_t for n_tok tokens of dimension dk. */
int oracle_coeff_rule(const double *k, const double *beta, double *lam_out,
                      double *alpha_out, int64_t n_tok, int dk, int rule)
{
    if (n_tok < 0 || dk <= 0 || (rule != 0 && rule != 1))
        return 1;
    for (int64_t t = 0; t < n_tok; ++t) {
        const double *kt = k + t * (int64_t)dk;
        double lam = 0.0;
        for (int i = 0; i < dk; ++i)
            lam += kt[i] * kt[i];
        if (lam_out)
            lam_out[t] = lam;
        alpha_out[t] = rule_alpha(beta[t], lam, rule);
    }
    return 0;
}

int oracle_coeff(const double *k, const double *beta, double *lam_out,
                 double *alpha_out, int64_t n_tok, int dk)
{
    return oracle_coeff_rule(k, beta, lam_out, alpha_out, n_tok, dk, 0);
}

/*
 * One EFLA token update of one state, in place, followed by the readout.
 *   S  : dk x dv state (row-major), updated to S_t
 *   kS : scratch of length dv
 *   o  : output row of length dv (may be NULL)
 */
static void efla_token(double *S, double *kS, const double *q, const double *k,
                       const double *v, double beta, double *o, int dk, int dv,
                       int rule)
{
    double lam = 0.0;
    for (int i = 0; i < dk; ++i)
        lam += k[i] * k[i];
    const double a = rule_alpha(beta, lam, rule);

    /* k^T S_{t-1}  (a row vector over value dims) */
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i)
            acc += k[i] * S[(int64_t)i * dv + j];
        kS[j] = acc;
    }
    /* S_t = S_{t-1} - a k (k^T S_{t-1}) + a k v^T */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(int64_t)i * dv + j] += -a * k[i] * kS[j] + a * k[i] * v[j];

    /* o_t = S_t^T q_t */
    if (o) {
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += S[(int64_t)i * dv + j] * q[i];
            o[j] = acc;
        }
    }
}

typedef struct {
    const double *q, *k, *v, *beta, *s0;
    double *o, *s_final;
    int B, H, dk, dv;
    int64_t L;
    int nthreads, tid, rule;
} fwd_job;

static void *fwd_worker(void *arg)
{
    fwd_job *J = (fwd_job *)arg;
    const int64_t units = (int64_t)J->B * J->H;
    const int64_t sdim = (int64_t)J->dk * J->dv;
    double *S = (double *)malloc(sizeof(double) * (size_t)sdim);
    double *kS = (double *)malloc(sizeof(double) * (size_t)J->dv);
    if (!S || !kS) {
        free(S);
        free(kS);
        return (void *)1;
    }
    for (int64_t u = J->tid; u < units; u += J->nthreads) {
        const int64_t b = u / J->H, h = u % J->H;
        if (J->s0)
            memcpy(S, J->s0 + u * sdim, sizeof(double) * (size_t)sdim);
        else
            memset(S, 0, sizeof(double) * (size_t)sdim);
        for (int64_t t = 0; t < J->L; ++t) {
            const int64_t row = (b * J->L + t) * J->H + h;
            efla_token(S, kS, J->q + row * J->dk, J->k + row * J->dk,
                       J->v + row * J->dv, J->beta[row],
                       J->o ? J->o + row * J->dv : NULL, J->dk, J->dv, J->rule);
        }
        if (J->s_final)
            memcpy(J->s_final + u * sdim, S, sizeof(double) * (size_t)sdim);
    }
    free(S);
    free(kS);
    return NULL;
}

/*
 * Full forward pass over L tokens for every (b, h) sequence.
 * s0 may be NULL (zero initial state); o and s_final may be NULL.
 * s_final may alias s0.  Returns 0 on success.
 */
int oracle_forward_rule(const double *q, const double *k, const double *v,
                        const double *beta, const double *s0, double *o,
                        double *s_final, int B, int H, int64_t L, int dk, int dv,
                        int nthreads, int rule)
{
    if (B < 0 || H < 0 || L < 0 || dk <= 0 || dv <= 0 || (rule != 0 && rule != 1))
        return 1;
    const int64_t units = (int64_t)B * H;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > units)
        nthreads = units > 0 ? (int)units : 1;
    fwd_job *jobs = (fwd_job *)calloc((size_t)nthreads, sizeof(fwd_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return 2;
    }
    int rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        fwd_job J = {q, k, v, beta, s0, o, s_final, B, H, dk, dv, L, nthreads, i, rule};
        jobs[i] = J;
    }
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, fwd_worker, &jobs[i]) != 0) {
            rc = 3;
            break;
        }
        started = i;
    }
    if (rc == 0 && fwd_worker(&jobs[0]) != NULL)
        rc = 2;
    for (int i = 1; i <= started; ++i) {
        void *ret = NULL;
        pthread_join(th[i], &ret);
        if (ret != NULL)
            rc = 2;
    }
    free(jobs);
    free(th);
    return rc;
}

int oracle_forward(const double *q, const double *k, const double *v,
                   const double *beta, const double *s0, double *o,
                   double *s_final, int B, int H, int64_t L, int dk, int dv,
                   int nthreads)
{
    return oracle_forward_rule(q, k, v, beta, s0, o, s_final, B, H, L, dk, dv,
                               nthreads, 0);
}

/*
 * One decode step: a single token per (n, h) applied to the state in place.
 *   q, k [N, H, dk]   v, o [N, H, dv]   beta [N, H]   state [N, H, dk, dv]
 */
int oracle_step_rule(const double *q, const double *k, const double *v,
                     const double *beta, double *state, double *o, int N, int H,
                     int dk, int dv, int rule)
{
    if (N < 0 || H < 0 || dk <= 0 || dv <= 0 || (rule != 0 && rule != 1))
        return 1;
    double *kS = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!kS)
        return 2;
    const int64_t sdim = (int64_t)dk * dv;
    for (int64_t u = 0; u < (int64_t)N * H; ++u)
        efla_token(state + u * sdim, kS, q + u * dk, k + u * dk, v + u * dv,
                   beta[u], o ? o + u * dv : NULL, dk, dv, rule);
    free(kS);
    return 0;
}

int oracle_step(const double *q, const double *k, const double *v,
                const double *beta, double *state, double *o, int N, int H,
                int dk, int dv)
{
    return oracle_step_rule(q, k, v, beta, state, o, N, H, dk, dv, 0);
}
