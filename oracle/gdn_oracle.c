/*
 * gdn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU implementation of the gated delta rule.  It exists
 * so that tests, the smoke check and the benchmark's CPU-baseline leg can
 * check and time the GPU library against an independent definition.  The GPU
 * product path never links, loads or calls anything in this directory, and
 * this file includes nothing from the GPU library.
 *
 * What it computes (source: the explainer page "論文解説: Qwen3.8-Next の設計"
 * on ta-paperlens.web.app, section "GDNの中身: 足すのではなく、消してから書く",
 * Eq. (1) and the concept code that follows it):
 *
 *   each head keeps a matrix state S (dk x dv) mapping keys to values;
 *   per token t:   S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *                  o_t = scale * S_t^T q_t          (read after the update)
 *
 * Readings where the page leaves a step open (each one pinned by a test):
 *   - S is dk x dv, stored row-major with dv contiguous; the read-out contracts
 *     over dk (Eq. (1) writes k v^T, so rows are indexed by the key).
 *   - alpha multiplies the whole product (Eq. (1)); the concept code's line
 *     order, which takes the difference from the undecayed state, is not used.
 *   - alpha is passed in log space: alpha_t = exp(g_t), evaluated here in fp64.
 *   - q/k heads are shared by groups of G = Hv/Hk consecutive value heads:
 *     value head hv reads q/k head hv / G.  beta and g are per value head.
 *   - a NULL initial state means zeros; the output state is the state after
 *     the last token.
 *
 * Arithmetic: every input value (fp32, or bf16 widened exactly to fp32 by the
 * caller) is widened to double; sums run over the contracted index in
 * ascending order; nothing is blocked, fused or reordered.  Build without
 * -ffast-math and with -ffp-contract=off.
 *
 * Parity status: pinned by the CPU tests (closed forms for beta = 0 and
 * beta = 1, orthonormal-key retrieval, exact rational brute force on tiny
 * sizes, dense transition-matrix products, an independently derived chunked
 * form, linearity, split/resume and GQA equivalence).  The packed-sequence
 * entry point with its input prologue is pinned by reduction to per-sequence
 * runs, by scale invariance of the normalisation and by the closed forms
 * sigmoid(0) = 1/2 and pure decay products.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Apply one token of Eq. (1) to the state S (dk x dv, row-major) and write
 * o = scale * S^T q for the updated state.  e and f are dv-long scratch. */
static void gdn_oracle_token(double *S, const double *q, const double *k,
                             const double *v, double alpha, double beta,
                             double scale, int dk, int dv, double *e,
                             double *f, double *o)
{
    /* e = S^T k : what the state currently stores under key k. */
    for (int j = 0; j < dv; ++j)
        e[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        const double ki = k[i];
        const double *row = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j)
            e[j] += ki * row[j];
    }
    /* S = alpha * (S - beta k e^T) + beta k v^T  ==  alpha (I - beta k k^T) S + beta k v^T */
    for (int i = 0; i < dk; ++i) {
        const double ki = k[i];
        double *row = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j)
            row[j] = alpha * (row[j] - beta * ki * e[j]) + beta * ki * v[j];
    }
    /* o = scale * S^T q, read from the updated state. */
    for (int j = 0; j < dv; ++j)
        f[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        const double qi = q[i];
        const double *row = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j)
            f[j] += qi * row[j];
    }
    for (int j = 0; j < dv; ++j)
        o[j] = scale * f[j];
}

/* Widen n stored values to double. */
static void gdn_oracle_widen(const float *x, int n, double *y)
{
    for (int i = 0; i < n; ++i)
        y[i] = (double)x[i];
}

/* The input prologue (plain definitions, fp64; flag values as in the library's header):
 *   1: q, k -> x / max(||x||_2, 1e-6)     2: beta = sigmoid(x)     4: log alpha = log sigmoid(x) */
#define GDN_ORACLE_QK_L2NORM 1u
#define GDN_ORACLE_BETA_LOGIT 2u
#define GDN_ORACLE_G_LOGIT 4u

static void gdn_oracle_l2normalise(double *x, int n)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i)
        ss += x[i] * x[i];
    double nrm = sqrt(ss);
    if (nrm < 1e-6)
        nrm = 1e-6;
    for (int i = 0; i < n; ++i)
        x[i] = x[i] / nrm;
}

static double gdn_oracle_sigmoid(double x)
{
    return 1.0 / (1.0 + exp(-x));
}

static double gdn_oracle_log_sigmoid(double x)
{
    /* log(1 / (1 + e^-x)), written so that neither branch overflows */
    return x >= 0.0 ? -log1p(exp(-x)) : x - log1p(exp(x));
}

static int gdn_oracle_dims_ok(int B, int T, int Hk, int Hv, int dk, int dv)
{
    if (B < 0 || T < 0 || Hk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0)
        return 0;
    if (Hv % Hk != 0)
        return 0;
    return 1;
}

/*
 * Run the recurrence over T tokens for the chains listed in `chains`
 * (chain id = b * Hv + hv; NULL means all B*Hv chains in order).
 *
 * Layouts (row-major, innermost last):
 *   q, k  [B, T, Hk, dk]      v    [B, T, Hv, dv]
 *   beta, g [B, T, Hv]        s0   [B, Hv, dk, dv] fp64, or NULL (zeros)
 *   o     [n_chains, T, dv]   sT   [n_chains, dk, dv] or NULL (not written)
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 */
int gdn_oracle_run(const float *q, const float *k, const float *v,
                   const float *beta, const float *g, const double *s0,
                   int B, int T, int Hk, int Hv, int dk, int dv, double scale,
                   const int64_t *chains, int64_t n_chains, double *o,
                   double *sT, int nthreads)
{
    if (!gdn_oracle_dims_ok(B, T, Hk, Hv, dk, dv))
        return -1;
    if (chains == NULL)
        n_chains = (int64_t)B * Hv;
    if (n_chains < 0)
        return -1;
    if (T > 0 && (q == NULL || k == NULL || v == NULL || beta == NULL ||
                  g == NULL || o == NULL))
        return -1;
    for (int64_t c = 0; chains != NULL && c < n_chains; ++c)
        if (chains[c] < 0 || chains[c] >= (int64_t)B * Hv)
            return -1;
    const int G = Hv / Hk;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : failed)
#endif
    for (int64_t c = 0; c < n_chains; ++c) {
        const int64_t id = chains ? chains[c] : c;
        const int b = (int)(id / Hv), hv = (int)(id % Hv), hq = hv / G;
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *e = (double *)malloc(sizeof(double) * (size_t)dv);
        double *f = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !e || !f) {
            free(S); free(e); free(f);
            failed = 1;
            continue;
        }
        const size_t ssz = (size_t)dk * dv;
        if (s0) {
            memcpy(S, s0 + ((size_t)b * Hv + hv) * ssz, sizeof(double) * ssz);
        } else {
            memset(S, 0, sizeof(double) * ssz);
        }
        double *qd = (double *)malloc(sizeof(double) * (size_t)(2 * dk + dv));
        if (!qd) {
            free(S); free(e); free(f);
            failed = 1;
            continue;
        }
        double *kd = qd + dk, *vd = kd + dk;
        for (int t = 0; t < T; ++t) {
            const size_t bt = (size_t)b * T + t;
            gdn_oracle_widen(q + (bt * Hk + hq) * dk, dk, qd);
            gdn_oracle_widen(k + (bt * Hk + hq) * dk, dk, kd);
            gdn_oracle_widen(v + (bt * Hv + hv) * dv, dv, vd);
            const double alpha = exp((double)g[bt * Hv + hv]);
            const double bet = (double)beta[bt * Hv + hv];
            double *ot = o + ((size_t)c * T + t) * dv;
            gdn_oracle_token(S, qd, kd, vd, alpha, bet, scale, dk, dv, e, f, ot);
        }
        if (sT)
            memcpy(sT + (size_t)c * ssz, S, sizeof(double) * ssz);
        free(S); free(e); free(f); free(qd);
    }
    return failed ? -2 : 0;
}

/*
 * Packed sequences with the input prologue.  Sequence i is token rows
 * cu[i] .. cu[i+1]-1 (cu: N+1 nondecreasing offsets from 0 to T) of
 *   q, k [T, Hk, dk]   v [T, Hv, dv]   beta, g [T, Hv]   o [T, Hv, dv]
 * and has its own state: s0, sT [N, Hv, dk, dv] (s0 NULL = zeros, sT NULL = not written).
 * `flags` selects the prologue applied to every token's stored inputs before Eq. (1):
 * 1 = L2-normalise q and k, 2 = beta from a logit, 4 = log alpha from a logit.
 * Returns 0, -1 on bad arguments, -2 on allocation failure.
 */
int gdn_oracle_run_packed(const float *q, const float *k, const float *v,
                          const float *beta, const float *g, const double *s0,
                          const int64_t *cu, int N, int T, int Hk, int Hv, int dk,
                          int dv, double scale, unsigned flags, double *o, double *sT,
                          int nthreads)
{
    if (!gdn_oracle_dims_ok(N, T, Hk, Hv, dk, dv) || cu == NULL)
        return -1;
    if (cu[0] != 0 || cu[N] != T)
        return -1;
    for (int i = 0; i < N; ++i)
        if (cu[i + 1] < cu[i])
            return -1;
    if (T > 0 && (q == NULL || k == NULL || v == NULL || beta == NULL ||
                  g == NULL || o == NULL))
        return -1;
    const int G = Hv / Hk;
    const int64_t n = (int64_t)N * Hv;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : failed)
#endif
    for (int64_t c = 0; c < n; ++c) {
        const int i = (int)(c / Hv), hv = (int)(c % Hv), hq = hv / G;
        const size_t ssz = (size_t)dk * dv;
        double *S = (double *)malloc(sizeof(double) * ssz);
        double *buf = (double *)malloc(sizeof(double) * (size_t)(2 * dk + 3 * dv));
        if (!S || !buf) {
            free(S); free(buf);
            failed = 1;
            continue;
        }
        double *qd = buf, *kd = qd + dk, *vd = kd + dk, *e = vd + dv, *f = e + dv;
        if (s0)
            memcpy(S, s0 + (size_t)c * ssz, sizeof(double) * ssz);
        else
            memset(S, 0, sizeof(double) * ssz);
        for (int64_t r = cu[i]; r < cu[i + 1]; ++r) {
            gdn_oracle_widen(q + ((size_t)r * Hk + hq) * dk, dk, qd);
            gdn_oracle_widen(k + ((size_t)r * Hk + hq) * dk, dk, kd);
            gdn_oracle_widen(v + ((size_t)r * Hv + hv) * dv, dv, vd);
            double gx = (double)g[(size_t)r * Hv + hv];
            double bx = (double)beta[(size_t)r * Hv + hv];
            if (flags & GDN_ORACLE_QK_L2NORM) {
                gdn_oracle_l2normalise(qd, dk);
                gdn_oracle_l2normalise(kd, dk);
            }
            if (flags & GDN_ORACLE_BETA_LOGIT)
                bx = gdn_oracle_sigmoid(bx);
            if (flags & GDN_ORACLE_G_LOGIT)
                gx = gdn_oracle_log_sigmoid(gx);
            gdn_oracle_token(S, qd, kd, vd, exp(gx), bx, scale, dk, dv, e, f,
                             o + ((size_t)r * Hv + hv) * dv);
        }
        if (sT)
            memcpy(sT + (size_t)c * ssz, S, sizeof(double) * ssz);
        free(S); free(buf);
    }
    return failed ? -2 : 0;
}

/*
 * One decode step: apply one token of Eq. (1) to every state in place.
 *   q, k [B, Hk, dk]   v [B, Hv, dv]   beta, g [B, Hv]
 *   state [B, Hv, dk, dv] (fp64, updated in place)   o [B, Hv, dv]
 */
int gdn_oracle_decode_step(const float *q, const float *k, const float *v,
                           const float *beta, const float *g, double *state,
                           double *o, int B, int Hk, int Hv, int dk, int dv,
                           double scale, int nthreads)
{
    if (!gdn_oracle_dims_ok(B, 1, Hk, Hv, dk, dv))
        return -1;
    if (B > 0 && (!q || !k || !v || !beta || !g || !state || !o))
        return -1;
    const int G = Hv / Hk;
    const int64_t n = (int64_t)B * Hv;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(| : failed)
#endif
    for (int64_t id = 0; id < n; ++id) {
        const int b = (int)(id / Hv), hv = (int)(id % Hv), hq = hv / G;
        double *e = (double *)malloc(sizeof(double) * (size_t)dv);
        double *f = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!e || !f) {
            free(e); free(f);
            failed = 1;
            continue;
        }
        double *qd = (double *)malloc(sizeof(double) * (size_t)(2 * dk + dv));
        if (!qd) {
            free(e); free(f);
            failed = 1;
            continue;
        }
        double *kd = qd + dk, *vd = kd + dk;
        gdn_oracle_widen(q + ((size_t)b * Hk + hq) * dk, dk, qd);
        gdn_oracle_widen(k + ((size_t)b * Hk + hq) * dk, dk, kd);
        gdn_oracle_widen(v + (size_t)id * dv, dv, vd);
        gdn_oracle_token(state + (size_t)id * dk * dv, qd, kd, vd,
                         exp((double)g[id]), (double)beta[id], scale, dk, dv,
                         e, f, o + (size_t)id * dv);
        free(e); free(f); free(qd);
    }
    return failed ? -2 : 0;
}

int gdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Backward of the recurrence (reverse-mode differentiation of Eq. (1), token by token).
 * Given the forward inputs and the gradients dO of the outputs o (and dST of the final
 * state, or NULL for zero), returns the gradients of every input:
 *   dq, dk [B, T, Hk, dk] (summed over the G value heads that share a q/k head)
 *   dv [B, T, Hv, dv]   dbeta, dg [B, T, Hv] (dg: gradient w.r.t. g = log alpha)
 *   dS0 [B, Hv, dk, dv]
 * All fp64.  With X = S_{t-1}, e = X^T k, u = dS_t^T k (dS_t: gradient w.r.t. S_t once the
 * read-out o_t = scale S_t^T q_t has added scale q dO_t^T):
 *   S_t = alpha (X - beta k e^T) + beta k v^T
 *   dq_t  = scale S_t dO_t
 *   dv_t  = beta u
 *   dbeta = u . (v - alpha e)
 *   dalpha = <dS_t, X> - beta u . e,   dg = alpha dalpha
 *   dk_t  = beta dS_t (v - alpha e) - alpha beta X u
 *   dS_{t-1} = alpha (dS_t - beta k u^T)
 * Returns 0, -1 on bad arguments, -2 on allocation failure.
 */
int gdn_oracle_backward(const float *q, const float *k, const float *v,
                        const float *beta, const float *g, const double *s0,
                        const double *dO, const double *dST, int B, int T, int Hk,
                        int Hv, int dk, int dv, double scale, double *dq, double *dk_out,
                        double *dv_out, double *dbeta, double *dg, double *dS0)
{
    if (!gdn_oracle_dims_ok(B, T, Hk, Hv, dk, dv))
        return -1;
    if (T > 0 && (!q || !k || !v || !beta || !g || !dO || !dq || !dk_out || !dv_out ||
                  !dbeta || !dg))
        return -1;
    if (!dS0)
        return -1;
    const int G = Hv / Hk;
    const size_t ssz = (size_t)dk * dv;
    /* dq and dk accumulate over the value heads of a group */
    if (T > 0) {
        memset(dq, 0, sizeof(double) * (size_t)B * T * Hk * dk);
        memset(dk_out, 0, sizeof(double) * (size_t)B * T * Hk * dk);
    }
    double *hist = (double *)malloc(sizeof(double) * ssz * (size_t)(T + 1));
    double *dS = (double *)malloc(sizeof(double) * ssz);
    double *buf = (double *)malloc(sizeof(double) * (size_t)(3 * dk + 6 * dv));
    if (!hist || !dS || !buf) {
        free(hist); free(dS); free(buf);
        return -2;
    }
    double *qd = buf, *kd = qd + dk, *vd = kd + dk, *e = vd + dv, *f = e + dv, *o = f + dv;
    double *u = o + dv, *w = u + dv, *ro = w + dv, *tmp = ro + dv;
    (void)tmp;
    for (int b = 0; b < B; ++b)
        for (int hv = 0; hv < Hv; ++hv) {
            const int hq = hv / G;
            const size_t chain = (size_t)b * Hv + hv;
            /* forward, keeping every state S_0 .. S_T */
            if (s0)
                memcpy(hist, s0 + chain * ssz, sizeof(double) * ssz);
            else
                memset(hist, 0, sizeof(double) * ssz);
            for (int t = 0; t < T; ++t) {
                const size_t bt = (size_t)b * T + t;
                memcpy(hist + (size_t)(t + 1) * ssz, hist + (size_t)t * ssz, sizeof(double) * ssz);
                gdn_oracle_widen(q + (bt * Hk + hq) * dk, dk, qd);
                gdn_oracle_widen(k + (bt * Hk + hq) * dk, dk, kd);
                gdn_oracle_widen(v + (bt * Hv + hv) * dv, dv, vd);
                gdn_oracle_token(hist + (size_t)(t + 1) * ssz, qd, kd, vd,
                                 exp((double)g[bt * Hv + hv]), (double)beta[bt * Hv + hv],
                                 scale, dk, dv, e, f, o);
            }
            /* reverse */
            if (dST)
                memcpy(dS, dST + chain * ssz, sizeof(double) * ssz);
            else
                memset(dS, 0, sizeof(double) * ssz);
            for (int t = T - 1; t >= 0; --t) {
                const size_t bt = (size_t)b * T + t;
                const double *X = hist + (size_t)t * ssz, *St = hist + (size_t)(t + 1) * ssz;
                const double alpha = exp((double)g[bt * Hv + hv]);
                const double bet = (double)beta[bt * Hv + hv];
                gdn_oracle_widen(q + (bt * Hk + hq) * dk, dk, qd);
                gdn_oracle_widen(k + (bt * Hk + hq) * dk, dk, kd);
                gdn_oracle_widen(v + (bt * Hv + hv) * dv, dv, vd);
                const double *dOt = dO + (bt * Hv + hv) * dv;
                /* read-out: o_t = scale S_t^T q  ->  dq_t and dS_t += scale q dO^T */
                double *dqt = dq + (bt * Hk + hq) * dk;
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j)
                        acc += St[(size_t)i * dv + j] * dOt[j];
                    dqt[i] += scale * acc;
                    for (int j = 0; j < dv; ++j)
                        dS[(size_t)i * dv + j] += scale * qd[i] * dOt[j];
                }
                /* e = X^T k, u = dS^T k */
                for (int j = 0; j < dv; ++j) {
                    double ae = 0.0, au = 0.0;
                    for (int i = 0; i < dk; ++i) {
                        ae += X[(size_t)i * dv + j] * kd[i];
                        au += dS[(size_t)i * dv + j] * kd[i];
                    }
                    e[j] = ae;
                    u[j] = au;
                }
                double db = 0.0, ue = 0.0, dsx = 0.0;
                for (int j = 0; j < dv; ++j) {
                    w[j] = vd[j] - alpha * e[j];
                    db += u[j] * w[j];
                    ue += u[j] * e[j];
                    dv_out[(bt * Hv + hv) * dv + j] = bet * u[j];
                }
                for (size_t n = 0; n < ssz; ++n)
                    dsx += dS[n] * X[n];
                dbeta[bt * Hv + hv] = db;
                dg[bt * Hv + hv] = alpha * (dsx - bet * ue);
                /* dk_t = beta dS w - alpha beta X u */
                double *dkt = dk_out + (bt * Hk + hq) * dk;
                for (int i = 0; i < dk; ++i) {
                    double a1 = 0.0, a2 = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        a1 += dS[(size_t)i * dv + j] * w[j];
                        a2 += X[(size_t)i * dv + j] * u[j];
                    }
                    dkt[i] += bet * a1 - alpha * bet * a2;
                }
                /* dS_{t-1} = alpha (dS - beta k u^T) */
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j)
                        dS[(size_t)i * dv + j] = alpha * (dS[(size_t)i * dv + j] - bet * kd[i] * u[j]);
            }
            memcpy(dS0 + chain * ssz, dS, sizeof(double) * ssz);
        }
    free(hist); free(dS); free(buf);
    return 0;
}
