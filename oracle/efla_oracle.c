/*
 * efla_oracle.c -- plain, slow, fp64 CPU oracle for Error-Free Linear Attention (EFLA).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this file:
 * it exists so that tests, the smoke check and the CPU-baseline leg of the benchmark can
 * compare the HIP kernels against an obviously correct token-by-token recurrence.  It shares
 * no code, header, table or constant with the HIP library.
 *
 * What it computes (all in double precision, one token at a time, no chunking, no blocking):
 *
 *   per token t, with key k_t, value v_t, query q_t and step beta_t
 *     lambda_t = ||k_t||^2
 *     alpha_t  = (1 - e^{-beta_t lambda_t}) / lambda_t            (and alpha_t = beta_t if lambda_t = 0)
 *     S_t      = (I - alpha_t k_t k_t^T) S_{t-1} + alpha_t k_t v_t^T
 *     o_t      = S_t^T q_t                                          (read after the update)
 *
 *   Sources: "Exact Flow Linear Attention: Exact Solution from Continuous-Time Dynamics"
 *   (gist.science), section Metodologia, item 2 (closed-form exponential) and item 3 (update rule
 *   and coefficient); "Error-Free Linear Attention is a Free Lunch" (howistudyai.com), Step 1
 *   (alpha from lambda = ||k||^2), Step 2 (exact memory update), Step 3 (readout o_t = S_t^T q_t)
 *   and "Putting it all together (pipeline)" (update first, then emit o = S^T q).
 *
 * Readings taken where the pages are silent:
 *   - 1 - e^{-x} is evaluated as -expm1(-x): the same quantity, without cancellation for small x.
 *   - lambda = 0 (k = 0): the 0/0 in the coefficient is replaced by its limit beta; the state update
 *     is a no-op in that case because k = 0.
 *   - S is d_k x d_v (k v^T is d_k x d_v and o = S^T q has d_v entries); an absent initial state is 0.
 *
 * The product (alpha k k^T) S_{t-1} is evaluated as alpha k (k^T S_{t-1}), which is the same matrix by
 * associativity; both the erase term and the write term of the update are kept as written.
 *
 * A second function, efla_oracle_ut, gives the intra-chunk transform of the chunked form by its
 * definition (used to check the GPU's UT output; see its own comment).
 *
 * Gates.  Every entry point takes `gate`: 0 is the exact coefficient above; p >= 1 replaces alpha_t by
 * the coefficient of one p-th order Runge-Kutta step of the same per-token ODE over [0, beta_t]
 * (see oracle_alpha_rk).  "Error-Free Linear Attention guida completa" (mauroscia.it), section on
 * RK-infinity (Euler and Runge-Kutta schemes of rising order approach the exact solution, which is the
 * infinite-order limit); "Error-Free Linear Attention is a Free Lunch" (howistudyai.com), building blocks
 * "Delta Rule" (S <- (I - beta k k^T) S + beta k v^T, the Euler step) and "Runge-Kutta Methods".
 *
 * Layouts (all contiguous, row-major):
 *   q, k [B,H,L,d_k]; v [B,H,L,d_v]; beta [B,H,L]; o [B,H,L,d_v]; state [B,H,d_k,d_v].
 * Parallelism: OpenMP over independent (b, h) pairs only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One step of a p-th order Runge-Kutta method for dS/dt = -A S + k v^T (A = k k^T) over [0, beta]
 * multiplies S by the degree-p Taylor polynomial of e^{-beta A}, sum_{n=0}^{p} (-beta A)^n / n!, and adds
 * the matching truncation of the input integral.  With A^n = lambda^{n-1} A (n >= 1) both collapse to the
 * rank-1 form (I - alpha_p A) S + alpha_p k v^T with
 *   alpha_p = sum_{n=1}^{p} (-1)^{n-1} beta^n lambda^{n-1} / n!
 * (p = 1: alpha = beta, the delta rule).  Written out term by term. */
static double oracle_alpha_rk(double beta, double lambda, int p)
{
    double alpha = 0.0;
    double factorial = 1.0;
    for (int n = 1; n <= p; ++n) {
        factorial *= n;
        const double sign = (n % 2 == 1) ? 1.0 : -1.0;   /* (-1)^{n-1} */
        alpha += sign * pow(beta, n) * pow(lambda, n - 1) / factorial;
    }
    return alpha;
}

/* gate 0: alpha_t = (1 - e^{-beta lambda}) / lambda, lambda = ||k||^2, with the lambda = 0 limit beta;
 * gate p >= 1: oracle_alpha_rk. */
static double oracle_alpha_one(const double *k, double beta, int d_k, int gate)
{
    double lambda = 0.0;
    for (int i = 0; i < d_k; ++i)
        lambda += k[i] * k[i];
    if (gate > 0)
        return oracle_alpha_rk(beta, lambda, gate);
    if (lambda == 0.0 || beta * lambda == 0.0)
        return beta;
    return -expm1(-beta * lambda) / lambda;
}

/* One exact EFLA token update applied to S (d_k x d_v), followed by the readout o = S^T q.
 * kS is caller-provided scratch of d_v doubles. */
static void oracle_token(double *S, const double *q, const double *k, const double *v, double beta,
                         double *o, double *kS, int d_k, int d_v, int gate)
{
    const double alpha = oracle_alpha_one(k, beta, d_k, gate);
    /* kS = k^T S_{t-1} (a row vector of length d_v) */
    for (int j = 0; j < d_v; ++j)
        kS[j] = 0.0;
    for (int i = 0; i < d_k; ++i)
        for (int j = 0; j < d_v; ++j)
            kS[j] += k[i] * S[(size_t)i * d_v + j];
    /* S_t = S_{t-1} - alpha k (k^T S_{t-1}) + alpha k v^T */
    for (int i = 0; i < d_k; ++i)
        for (int j = 0; j < d_v; ++j)
            S[(size_t)i * d_v + j] = S[(size_t)i * d_v + j] - alpha * k[i] * kS[j] + alpha * k[i] * v[j];
    /* o_t = S_t^T q_t */
    if (o) {
        for (int j = 0; j < d_v; ++j)
            o[j] = 0.0;
        for (int i = 0; i < d_k; ++i)
            for (int j = 0; j < d_v; ++j)
                o[j] += S[(size_t)i * d_v + j] * q[i];
    }
}

static int oracle_threads(int requested)
{
#ifdef _OPENMP
    if (requested > 0)
        return requested;
    return omp_get_max_threads();
#else
    (void)requested;
    return 1;
#endif
}

/* alpha for n_tokens keys of length d_k. */
void efla_oracle_alpha(const double *k, const double *beta, double *alpha, int64_t n_tokens, int d_k, int gate)
{
    for (int64_t t = 0; t < n_tokens; ++t)
        alpha[t] = oracle_alpha_one(k + t * d_k, beta[t], d_k, gate);
}

/* Full-sequence recurrence for every (b, h).  initial_state may be NULL (zeros); final_state may
 * be NULL (not written); o may be NULL (not written).  Returns the number of threads used. */
int efla_oracle_fwd(const double *q, const double *k, const double *v, const double *beta,
                    const double *initial_state, double *o, double *final_state,
                    int B, int H, int L, int d_k, int d_v, int gate, int n_threads)
{
    const int64_t BH = (int64_t)B * H;
    const int nt = oracle_threads(n_threads);
    int used = 1;
#ifdef _OPENMP
#pragma omp parallel num_threads(nt)
#endif
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double *S = (double *)malloc(sizeof(double) * (size_t)d_k * d_v);
        double *kS = (double *)malloc(sizeof(double) * (size_t)d_v);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t bh = 0; bh < BH; ++bh) {
            const size_t ssz = (size_t)d_k * d_v;
            if (initial_state)
                memcpy(S, initial_state + bh * ssz, sizeof(double) * ssz);
            else
                memset(S, 0, sizeof(double) * ssz);
            for (int t = 0; t < L; ++t) {
                const int64_t tok = bh * L + t;
                oracle_token(S, q + tok * d_k, k + tok * d_k, v + tok * d_v, beta[tok],
                             o ? o + tok * d_v : NULL, kS, d_k, d_v, gate);
            }
            if (final_state)
                memcpy(final_state + bh * ssz, S, sizeof(double) * ssz);
        }
        free(S);
        free(kS);
    }
    (void)nt;
    return used;
}

/* One decode step for NH independent (sequence, head) states, updated in place.
 * q, k [NH,d_k]; v [NH,d_v]; beta [NH]; state [NH,d_k,d_v]; o [NH,d_v]. Returns threads used. */
int efla_oracle_step(const double *q, const double *k, const double *v, const double *beta,
                     double *state, double *o, int64_t NH, int d_k, int d_v, int gate, int n_threads)
{
    const int nt = oracle_threads(n_threads);
    int used = 1;
#ifdef _OPENMP
#pragma omp parallel num_threads(nt)
#endif
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double *kS = (double *)malloc(sizeof(double) * (size_t)d_v);
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t n = 0; n < NH; ++n)
            oracle_token(state + n * (int64_t)d_k * d_v, q + n * d_k, k + n * d_k, v + n * d_v, beta[n],
                         o ? o + n * d_v : NULL, kS, d_k, d_v, gate);
        free(kS);
    }
    (void)nt;
    return used;
}

/* The intra-chunk UT transform of the chunked form, by its definition.  For every (b, h) and every
 * chunk of C consecutive tokens (the last chunk may hold n < C tokens), with alpha_i the gate of token i
 * of the chunk and k_i its key:
 *   A[i][j] = alpha_i k_i . k_j  for j < i, else 0        (strict lower part of diag(alpha) K K^T)
 *   T       = (I + A)^{-1}                                 (unit lower triangular)
 *   out     = T diag(alpha)                                (column j of T scaled by alpha_j)
 * Sources: "Error-Free Linear Attention is a Free Lunch" (howistudyai.com), Step 4 (chunkwise-parallel
 * form: the within-chunk transforms are computed in parallel and the chunks are joined by passing the
 * state); "Exact Flow Linear Attention" (gist.science), Metodologia item 3 (the update keeps the
 * delta-rule rank-1 form, which is what makes the WY/UT representation apply).  Column j of T solves
 * (I + A) x = e_j, taken by forward substitution: x_i = [i == j] - sum_{m < i} A[i][m] x_m.
 * Output: tout[bh][c][i][j], a C x C row-major block per chunk; rows and columns n .. C-1 of a short
 * last chunk are zero.  Returns the number of threads used. */
int efla_oracle_ut(const double *k, const double *beta, double *tout, int B, int H, int L, int d_k, int C,
                   int gate, int n_threads)
{
    const int64_t BH = (int64_t)B * H;
    const int64_t NC = (L + C - 1) / C;
    const int nt = oracle_threads(n_threads);
    int used = 1;
#ifdef _OPENMP
#pragma omp parallel num_threads(nt)
#endif
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double *A = (double *)malloc(sizeof(double) * (size_t)C * C);
        double *alpha = (double *)malloc(sizeof(double) * (size_t)C);
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t u = 0; u < BH * NC; ++u) {
            const int64_t bh = u / NC;
            const int t0 = (int)(u % NC) * C;
            const int n = L - t0 < C ? L - t0 : C;
            const double *kc = k + (bh * L + t0) * d_k;
            double *T = tout + u * (int64_t)C * C;
            memset(T, 0, sizeof(double) * (size_t)C * C);
            memset(A, 0, sizeof(double) * (size_t)C * C);
            for (int i = 0; i < n; ++i)
                alpha[i] = oracle_alpha_one(kc + (size_t)i * d_k, beta[bh * L + t0 + i], d_k, gate);
            for (int i = 0; i < n; ++i)
                for (int j = 0; j < i; ++j) {
                    double dot = 0.0;
                    for (int e = 0; e < d_k; ++e)
                        dot += kc[(size_t)i * d_k + e] * kc[(size_t)j * d_k + e];
                    A[(size_t)i * C + j] = alpha[i] * dot;
                }
            for (int j = 0; j < n; ++j)
                for (int i = 0; i < n; ++i) {
                    double x = (i == j) ? 1.0 : 0.0;
                    for (int m = 0; m < i; ++m)
                        x -= A[(size_t)i * C + m] * T[(size_t)m * C + j];
                    T[(size_t)i * C + j] = x;
                }
            for (int i = 0; i < n; ++i)
                for (int j = 0; j < n; ++j)
                    T[(size_t)i * C + j] *= alpha[j];
        }
        free(A);
        free(alpha);
    }
    (void)nt;
    return used;
}

/* ------------------------------------------------------------------------------------------------
 * Gradients (reverse mode) of the token recurrence.  The pages train every model they report, but print
 * no backward pass ("Exact Flow Linear Attention" (gist.science), Risultati Sperimentali item 4: training
 * throughput matches DeltaNet; "Error-Free Linear Attention is a Free Lunch" (howistudyai.com), the language
 * modelling results at 340M and 1.3B parameters), so this is the adjoint of the forward above, derived term
 * by term from the update as written:
 *   S_t = S_{t-1} - alpha k a^T + alpha k v^T,  a = S_{t-1}^T k,   o_t = S_t^T q_t,
 *   alpha = f(beta, lambda),  lambda = k^T k.
 * Going backwards over the tokens with G = dLoss/dS_t (the gradient of the final state, or 0, at the end):
 *   readout:  dq_t = S_t do_t;                      G += q_t do_t^T
 *   update:   w = G^T k;  e = v - a
 *             dv_t = alpha w;   da = -alpha w;   dalpha = w . e
 *             dk_t = alpha G e + S_{t-1} da + 2 k dlambda,   dlambda = dalpha df/dlambda
 *             dbeta_t = dalpha df/dbeta;   G <- G + k da^T   (the gradient of S_{t-1})
 * and the gradient of the initial state is the G left after token 0.
 * ------------------------------------------------------------------------------------------------ */

/* d alpha / d beta and d alpha / d lambda of the gate.
 * gate 0: alpha = (1 - e^{-x}) / lambda, x = beta lambda:  d/dbeta = e^{-x};
 *         d/dlambda = beta^2 g(x),  g(x) = (x e^{-x} - (1 - e^{-x})) / x^2 = sum_{m>=2} (-1)^{m-1} (m-1)/m! x^{m-2}
 *         (the series below x = 1/2, where the closed form cancels; g(0) = -1/2).
 * gate p: the derivatives of sum_{n=1}^{p} (-1)^{n-1} beta^n lambda^{n-1} / n!, term by term. */
static void oracle_alpha_grad(double beta, double lambda, int gate, double *da_dbeta, double *da_dlambda)
{
    if (gate > 0) {
        double db = 0.0, dl = 0.0, nfact = 1.0;   /* n! */
        for (int n = 1; n <= gate; ++n) {
            nfact *= n;
            const double sgn = (n & 1) ? 1.0 : -1.0;   /* (-1)^{n-1} */
            db += sgn * n * pow(beta * lambda, n - 1) / nfact;
            if (n >= 2)
                dl += sgn * (n - 1) * pow(beta, n) * pow(lambda, n - 2) / nfact;
        }
        *da_dbeta = db;
        *da_dlambda = dl;
        return;
    }
    const double x = beta * lambda;
    *da_dbeta = exp(-x);
    double g;
    if (x < 0.5) {
        g = 0.0;
        double xp = 1.0, factorial = 2.0;   /* x^{m-2}, m! */
        for (int m = 2; m < 40; ++m) {
            if (m > 2) {
                xp *= x;
                factorial *= m;
            }
            const double sign = (m % 2 == 1) ? 1.0 : -1.0;   /* (-1)^{m-1} */
            g += sign * (m - 1) * xp / factorial;
        }
    } else {
        g = (x * exp(-x) + expm1(-x)) / (x * x);
    }
    *da_dlambda = beta * beta * g;
}

/* Gradients of sum(o * d_o) + sum(S_L * d_final) with respect to q, k, v, beta and the initial state,
 * for the recurrence of efla_oracle_fwd (same layouts; d_o [B,H,L,d_v]; d_final and d_initial
 * [B,H,d_k,d_v]; initial_state, d_final may be NULL = 0; d_initial may be NULL = not written).
 * Every state S_0 .. S_L of a (b, h) is kept (L + 1 blocks of d_k x d_v).  Returns the threads used. */
int efla_oracle_bwd(const double *q, const double *k, const double *v, const double *beta,
                    const double *initial_state, const double *d_o, const double *d_final,
                    double *dq, double *dk, double *dv, double *dbeta, double *d_initial,
                    int B, int H, int L, int d_k, int d_v, int gate, int n_threads)
{
    const int64_t BH = (int64_t)B * H;
    const int nt = oracle_threads(n_threads);
    int used = 1;
#ifdef _OPENMP
#pragma omp parallel num_threads(nt)
#endif
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        const size_t ssz = (size_t)d_k * d_v;
        double *Sall = (double *)malloc(sizeof(double) * ssz * (size_t)(L + 1));
        double *G = (double *)malloc(sizeof(double) * ssz);
        double *kS = (double *)malloc(sizeof(double) * (size_t)d_v);
        double *w = (double *)malloc(sizeof(double) * (size_t)d_v);
        double *e = (double *)malloc(sizeof(double) * (size_t)d_v);
        double *da = (double *)malloc(sizeof(double) * (size_t)d_v);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t bh = 0; bh < BH; ++bh) {
            /* forward, keeping every state */
            if (initial_state)
                memcpy(Sall, initial_state + bh * ssz, sizeof(double) * ssz);
            else
                memset(Sall, 0, sizeof(double) * ssz);
            for (int t = 0; t < L; ++t) {
                const int64_t tok = bh * L + t;
                memcpy(Sall + (size_t)(t + 1) * ssz, Sall + (size_t)t * ssz, sizeof(double) * ssz);
                oracle_token(Sall + (size_t)(t + 1) * ssz, q + tok * d_k, k + tok * d_k, v + tok * d_v, beta[tok],
                             NULL, kS, d_k, d_v, gate);
            }
            /* backward */
            if (d_final)
                memcpy(G, d_final + bh * ssz, sizeof(double) * ssz);
            else
                memset(G, 0, sizeof(double) * ssz);
            for (int t = L - 1; t >= 0; --t) {
                const int64_t tok = bh * L + t;
                const double *St = Sall + (size_t)(t + 1) * ssz;
                const double *Sp = Sall + (size_t)t * ssz;
                const double *qt = q + tok * d_k, *kt = k + tok * d_k, *vt = v + tok * d_v, *dot = d_o + tok * d_v;
                /* readout o_t = S_t^T q_t */
                for (int i = 0; i < d_k; ++i) {
                    double s = 0.0;
                    for (int j = 0; j < d_v; ++j)
                        s += St[(size_t)i * d_v + j] * dot[j];
                    dq[tok * d_k + i] = s;
                }
                for (int i = 0; i < d_k; ++i)
                    for (int j = 0; j < d_v; ++j)
                        G[(size_t)i * d_v + j] += qt[i] * dot[j];
                /* update S_t = S_{t-1} - alpha k a^T + alpha k v^T */
                double lambda = 0.0;
                for (int i = 0; i < d_k; ++i)
                    lambda += kt[i] * kt[i];
                const double alpha = oracle_alpha_one(kt, beta[tok], d_k, gate);
                for (int j = 0; j < d_v; ++j) {
                    double a = 0.0, s = 0.0;
                    for (int i = 0; i < d_k; ++i) {
                        a += kt[i] * Sp[(size_t)i * d_v + j];
                        s += G[(size_t)i * d_v + j] * kt[i];
                    }
                    e[j] = vt[j] - a;
                    w[j] = s;
                }
                double dalpha = 0.0;
                for (int j = 0; j < d_v; ++j) {
                    dalpha += w[j] * e[j];
                    dv[tok * d_v + j] = alpha * w[j];
                    da[j] = -alpha * w[j];
                }
                double da_db, da_dl;
                oracle_alpha_grad(beta[tok], lambda, gate, &da_db, &da_dl);
                const double dlambda = dalpha * da_dl;
                dbeta[tok] = dalpha * da_db;
                for (int i = 0; i < d_k; ++i) {
                    double s = 0.0;
                    for (int j = 0; j < d_v; ++j)
                        s += alpha * G[(size_t)i * d_v + j] * e[j] + Sp[(size_t)i * d_v + j] * da[j];
                    dk[tok * d_k + i] = s + 2.0 * kt[i] * dlambda;
                }
                for (int i = 0; i < d_k; ++i)
                    for (int j = 0; j < d_v; ++j)
                        G[(size_t)i * d_v + j] += kt[i] * da[j];
            }
            if (d_initial)
                memcpy(d_initial + bh * ssz, G, sizeof(double) * ssz);
        }
        free(Sall);
        free(G);
        free(kS);
        free(w);
        free(e);
        free(da);
    }
    (void)nt;
    return used;
}
