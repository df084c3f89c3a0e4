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

/* ---------------------------------------------------------------------------
 * Backward pass.  The pages give none; this is plain reverse-mode calculus
 * through the token recurrence above, for a scalar loss with
 *   dO[t] = dLoss/do_t  and  dS_L = dLoss/dS_L (NULL: zero).
 * Outputs dq, dk, dv, dbeta (same layouts as the inputs) and dS_0 = dLoss/ds0
 * (NULL: not written).  Token by token, in reverse:
 *   o_t = S_t^T q_t:                 dq_t = S_t do_t;   dS_t += q_t do_t^T
 *   S_t = S_{t-1} + a k u^T with u = v - S_{t-1}^T k:
 *       da = k^T dS_t u;   du = a dS_t^T k;   dv_t = du
 *       dk_t = a dS_t u - S_{t-1} du + 2 dlambda k
 *       dS_{t-1} = dS_t - k du^T
 *   a(beta, lambda) of Method step 3, x = beta lambda:
 *       da/dbeta = e^{-x};   da/dlambda = beta^2 psi(x),
 *       psi(x) = -(1 - (1 + x) e^{-x}) / x^2   (-1/2 at x = 0)
 *   Euler rule (a = beta): da/dbeta = 1, da/dlambda = 0.
 * The states a segment of 64 tokens needs are recomputed forward from the
 * segment's start state, which one forward sweep keeps.
 * ------------------------------------------------------------------------- */

/* psi(x) for x >= 0 without cancellation: the series
 *   1 - (1 + x) e^{-x} = sum_{m >= 2} (-1)^m (m - 1) x^m / m!
 * below x = 0.05 (terms to m = 14), the closed form through expm1 above. */
static double oracle_psi(double x)
{
    if (x == INFINITY)
        return 0.0;
    if (x < 0.05) {
        double sum = 0.0, xp = 1.0, fact = 2.0; /* x^(m-2), m! */
        for (int m = 2; m <= 14; ++m) {
            if (m > 2) {
                xp *= x;
                fact *= m;
            }
            const double term = (double)(m - 1) * xp / fact;
            sum += (m % 2 == 0) ? term : -term;
        }
        return -sum;
    }
    return -((-expm1(-x)) - x * exp(-x)) / (x * x);
}

/* da/dbeta and da/dlambda under a rule */
static void rule_alpha_grad(double beta, double lam, int rule, double *da_db, double *da_dl)
{
    if (rule == 1) {
        *da_db = 1.0;
        *da_dl = 0.0;
        return;
    }
    const double x = beta * lam;
    *da_db = exp(-x);
    *da_dl = (x == INFINITY) ? -1.0 / (lam * lam) : beta * beta * oracle_psi(x);
}

/* exported for the pins: (da/dbeta, da/dlambda) into out[0], out[1] */
int oracle_alpha_grad(double beta, double lam, int rule, double *out)
{
    if (rule != 0 && rule != 1)
        return 1;
    rule_alpha_grad(beta, lam, rule, &out[0], &out[1]);
    return 0;
}

typedef struct {
    const double *q, *k, *v, *beta, *s0, *dO, *dSL;
    double *dq, *dk, *dv, *dbeta, *dS0;
    int B, H, dk_, dv_;
    int64_t L;
    int nthreads, tid, rule;
} bwd_job;

enum { SEG = 64 };

static void *bwd_worker(void *arg)
{
    bwd_job *J = (bwd_job *)arg;
    const int dk = J->dk_, dv = J->dv_;
    const int64_t units = (int64_t)J->B * J->H, sdim = (int64_t)dk * dv, L = J->L;
    const int64_t nseg = (L + SEG - 1) / SEG;
    double *starts = (double *)malloc(sizeof(double) * (size_t)((nseg > 0 ? nseg : 1) * sdim));
    double *seg = (double *)malloc(sizeof(double) * (size_t)((SEG + 1) * sdim));
    double *dS = (double *)malloc(sizeof(double) * (size_t)sdim);
    double *kS = (double *)malloc(sizeof(double) * (size_t)dv);
    double *u = (double *)malloc(sizeof(double) * (size_t)dv);
    double *du = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!starts || !seg || !dS || !kS || !u || !du) {
        free(starts); free(seg); free(dS); free(kS); free(u); free(du);
        return (void *)1;
    }
    for (int64_t w = J->tid; w < units; w += J->nthreads) {
        const int64_t b = w / J->H, h = w % J->H;
#define ROW(t) (((b) * L + (t)) * J->H + (h))
        /* forward sweep: the state at the start of every segment */
        double *S = seg; /* scratch */
        if (J->s0)
            memcpy(S, J->s0 + w * sdim, sizeof(double) * (size_t)sdim);
        else
            memset(S, 0, sizeof(double) * (size_t)sdim);
        for (int64_t t = 0; t < L; ++t) {
            if (t % SEG == 0)
                memcpy(starts + (t / SEG) * sdim, S, sizeof(double) * (size_t)sdim);
            const int64_t r = ROW(t);
            efla_token(S, kS, J->q + r * dk, J->k + r * dk, J->v + r * dv, J->beta[r], NULL, dk, dv,
                       J->rule);
        }
        /* dS_L */
        if (J->dSL)
            memcpy(dS, J->dSL + w * sdim, sizeof(double) * (size_t)sdim);
        else
            memset(dS, 0, sizeof(double) * (size_t)sdim);
        for (int64_t sg = nseg - 1; sg >= 0; --sg) {
            const int64_t t0 = sg * SEG, t1 = (t0 + SEG < L) ? t0 + SEG : L;
            /* seg[tau] = S_{t0 + tau - 1}, the state before token t0 + tau */
            memcpy(seg, starts + sg * sdim, sizeof(double) * (size_t)sdim);
            for (int64_t t = t0; t < t1; ++t) {
                double *next = seg + (t - t0 + 1) * sdim;
                memcpy(next, seg + (t - t0) * sdim, sizeof(double) * (size_t)sdim);
                const int64_t r = ROW(t);
                efla_token(next, kS, J->q + r * dk, J->k + r * dk, J->v + r * dv, J->beta[r], NULL,
                           dk, dv, J->rule);
            }
            for (int64_t t = t1 - 1; t >= t0; --t) {
                const int64_t r = ROW(t);
                const double *Sp = seg + (t - t0) * sdim, *St = seg + (t - t0 + 1) * sdim;
                const double *q = J->q + r * dk, *k = J->k + r * dk, *v = J->v + r * dv;
                const double *dO = J->dO + r * dv;
                double *dq = J->dq + r * dk, *dkk = J->dk + r * dk, *dvv = J->dv + r * dv;
                /* readout */
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        acc += St[(int64_t)i * dv + j] * dO[j];
                        dS[(int64_t)i * dv + j] += q[i] * dO[j];
                    }
                    dq[i] = acc;
                }
                /* the update */
                double lam = 0.0;
                for (int i = 0; i < dk; ++i)
                    lam += k[i] * k[i];
                const double a = rule_alpha(J->beta[r], lam, J->rule);
                for (int j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < dk; ++i)
                        acc += Sp[(int64_t)i * dv + j] * k[i];
                    u[j] = v[j] - acc;
                }
                double da = 0.0;
                for (int j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < dk; ++i)
                        acc += dS[(int64_t)i * dv + j] * k[i];
                    du[j] = a * acc;
                    da += acc * u[j];
                    dvv[j] = du[j];
                }
                double da_db, da_dl;
                rule_alpha_grad(J->beta[r], lam, J->rule, &da_db, &da_dl);
                J->dbeta[r] = da * da_db;
                const double dlam = da * da_dl;
                for (int i = 0; i < dk; ++i) {
                    double acc1 = 0.0, acc2 = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        acc1 += dS[(int64_t)i * dv + j] * u[j];
                        acc2 += Sp[(int64_t)i * dv + j] * du[j];
                    }
                    dkk[i] = a * acc1 - acc2 + 2.0 * dlam * k[i];
                }
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j)
                        dS[(int64_t)i * dv + j] -= k[i] * du[j];
            }
        }
        if (J->dS0)
            memcpy(J->dS0 + w * sdim, dS, sizeof(double) * (size_t)sdim);
#undef ROW
    }
    free(starts); free(seg); free(dS); free(kS); free(u); free(du);
    return NULL;
}

int oracle_backward_rule(const double *q, const double *k, const double *v,
                         const double *beta, const double *s0, const double *dO,
                         const double *dSL, double *dq, double *dk, double *dv,
                         double *dbeta, double *dS0, int B, int H, int64_t L, int dk_,
                         int dv_, int nthreads, int rule)
{
    if (B < 0 || H < 0 || L < 0 || dk_ <= 0 || dv_ <= 0 || (rule != 0 && rule != 1))
        return 1;
    const int64_t units = (int64_t)B * H;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > units)
        nthreads = units > 0 ? (int)units : 1;
    bwd_job *jobs = (bwd_job *)calloc((size_t)nthreads, sizeof(bwd_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return 2;
    }
    int rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        bwd_job J = {q, k, v, beta, s0, dO, dSL, dq, dk, dv, dbeta, dS0,
                     B, H, dk_, dv_, L, nthreads, i, rule};
        jobs[i] = J;
    }
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, bwd_worker, &jobs[i]) != 0) {
            rc = 3;
            break;
        }
        started = i;
    }
    if (rc == 0 && bwd_worker(&jobs[0]) != NULL)
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
