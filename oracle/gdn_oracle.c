/*
 * CPU fp64 oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests, the package's smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code with the HIP kernels and must
 * never be on the product path.
 *
 * What it computes is the plain definition of the layer core, token by token:
 *
 *   S_t = S_{t-1} ( alpha_t (I - beta_t k_t k_t^T) ) + beta_t v_t k_t^T ,
 *   o_t = S_t q_t ,                      S in R^{dv x dk}, alpha_t = exp(log_alpha_t)
 *
 * (Gated Delta Networks paper, translated page, section 3.1 eq. (10); the
 * same rule in the paper-notes blog, section "Gated Delta Rule", and in the
 * Gated DeltaNet tutorial, section on why a forget gate is added.)
 *
 * The tutorial orders the step as: forget first (Sbar = alpha S), then
 * correct the error measured on the *decayed* state,
 * S = Sbar + beta (v - Sbar k) k^T.  Expanding gives eq. (10) exactly; the
 * recurrence below is written in that ordered form.  The output is read after
 * the update (o_t = S_t q_t: paper section 2.1, tutorial section on the
 * associative-memory view).  A missing initial state means zeros (paper
 * section 2.1 expands the recurrence from S_0 = 0).  Each sequence of a packed
 * batch starts from its own initial state: the tutorial requires a reset
 * between independent samples and none inside one request.
 *
 * A second, independent form -- oracle_gdn_naive_product -- multiplies the
 * explicit dk x dk transition matrices A_t = alpha_t (I - beta_t k_t k_t^T)
 * and adds B_t = beta_t v_t k_t^T (tutorial, decode-recursion section:
 * S_t = S_{t-1} A_t + B_t).  It costs O(dk^2 dv) per token and is meant for
 * brute force on tiny inputs.
 *
 * Layouts (row-major, contiguous):
 *   q, k       [T, H, dk]     tokens of all sequences concatenated
 *   v          [T, H, dv]
 *   log_alpha  [T, H]
 *   beta       [T, H]
 *   init/final [N, H, dv, dk] (NULL init means zeros)
 *   o          [T, H, dv]
 *   cu         int64 [N+1], cu[0] = 0, non-decreasing, cu[N] = T
 *
 * Return value: 0 on success, -1 on a malformed cu array, -2 on bad sizes,
 * -3 on allocation failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int check_args(int64_t n_seqs, const int64_t *cu, int64_t H, int64_t dk, int64_t dv)
{
    if (n_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0) return -2;
    if (n_seqs > 0 && cu[0] != 0) return -1;
    for (int64_t n = 0; n < n_seqs; ++n)
        if (cu[n + 1] < cu[n]) return -1;
    return 0;
}

/* One token of the recurrence for one head, in place on S (dv x dk). */
static void gated_delta_token(double *S, double *err, int64_t dk, int64_t dv,
                              const double *q, const double *k, const double *v,
                              double log_alpha, double beta, double *o)
{
    const double alpha = exp(log_alpha);
    /* forget: Sbar = alpha * S */
    for (int64_t i = 0; i < dv * dk; ++i) S[i] *= alpha;
    /* error of the decayed memory along k: beta * (v - Sbar k) */
    for (int64_t i = 0; i < dv; ++i) {
        double pred = 0.0;
        for (int64_t j = 0; j < dk; ++j) pred += S[i * dk + j] * k[j];
        err[i] = beta * (v[i] - pred);
    }
    /* write: S = Sbar + err k^T */
    for (int64_t i = 0; i < dv; ++i)
        for (int64_t j = 0; j < dk; ++j) S[i * dk + j] += err[i] * k[j];
    /* read after the write: o = S q */
    for (int64_t i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < dk; ++j) acc += S[i * dk + j] * q[j];
        o[i] = acc;
    }
}

int oracle_gdn_recurrent(int64_t n_seqs, const int64_t *cu, int64_t H, int64_t dk, int64_t dv,
                         const double *q, const double *k, const double *v,
                         const double *log_alpha, const double *beta,
                         const double *init_state, double *o, double *final_state,
                         int n_threads)
{
    int rc = check_args(n_seqs, cu, H, dk, dv);
    if (rc) return rc;
    const int64_t jobs = n_seqs * H;
    int failed = 0;
#ifdef _OPENMP
    if (n_threads <= 0) n_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads) reduction(| : failed)
#endif
    for (int64_t job = 0; job < jobs; ++job) {
        const int64_t n = job / H, h = job % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)(dv * dk));
        double *err = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !err) {
            free(S);
            free(err);
            failed = 1;
            continue;
        }
        if (init_state)
            memcpy(S, init_state + (n * H + h) * dv * dk, sizeof(double) * (size_t)(dv * dk));
        else
            memset(S, 0, sizeof(double) * (size_t)(dv * dk));
        for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
            const int64_t th = t * H + h;
            gated_delta_token(S, err, dk, dv, q + th * dk, k + th * dk, v + th * dv,
                              log_alpha[th], beta[th], o + th * dv);
        }
        if (final_state)
            memcpy(final_state + (n * H + h) * dv * dk, S, sizeof(double) * (size_t)(dv * dk));
        free(S);
        free(err);
    }
    return failed ? -3 : 0;
}

/* Brute-force form: explicit transition matrices, S <- S A_t + B_t. */
int oracle_gdn_naive_product(int64_t n_seqs, const int64_t *cu, int64_t H, int64_t dk, int64_t dv,
                             const double *q, const double *k, const double *v,
                             const double *log_alpha, const double *beta,
                             const double *init_state, double *o, double *final_state)
{
    int rc = check_args(n_seqs, cu, H, dk, dv);
    if (rc) return rc;
    double *S = (double *)malloc(sizeof(double) * (size_t)(dv * dk));
    double *Snew = (double *)malloc(sizeof(double) * (size_t)(dv * dk));
    double *A = (double *)malloc(sizeof(double) * (size_t)(dk * dk));
    if (!S || !Snew || !A) {
        free(S);
        free(Snew);
        free(A);
        return -3;
    }
    for (int64_t n = 0; n < n_seqs; ++n) {
        for (int64_t h = 0; h < H; ++h) {
            if (init_state)
                memcpy(S, init_state + (n * H + h) * dv * dk, sizeof(double) * (size_t)(dv * dk));
            else
                memset(S, 0, sizeof(double) * (size_t)(dv * dk));
            for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
                const int64_t th = t * H + h;
                const double *kt = k + th * dk, *vt = v + th * dv, *qt = q + th * dk;
                const double a = exp(log_alpha[th]), b = beta[th];
                /* A_t = alpha (I - beta k k^T) */
                for (int64_t r = 0; r < dk; ++r)
                    for (int64_t c = 0; c < dk; ++c)
                        A[r * dk + c] = a * ((r == c ? 1.0 : 0.0) - b * kt[r] * kt[c]);
                /* Snew = S A_t + beta v k^T */
                for (int64_t i = 0; i < dv; ++i)
                    for (int64_t c = 0; c < dk; ++c) {
                        double acc = 0.0;
                        for (int64_t r = 0; r < dk; ++r) acc += S[i * dk + r] * A[r * dk + c];
                        Snew[i * dk + c] = acc + b * vt[i] * kt[c];
                    }
                memcpy(S, Snew, sizeof(double) * (size_t)(dv * dk));
                for (int64_t i = 0; i < dv; ++i) {
                    double acc = 0.0;
                    for (int64_t c = 0; c < dk; ++c) acc += S[i * dk + c] * qt[c];
                    o[th * dv + i] = acc;
                }
            }
            if (final_state)
                memcpy(final_state + (n * H + h) * dv * dk, S, sizeof(double) * (size_t)(dv * dk));
        }
    }
    free(S);
    free(Snew);
    free(A);
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Reverse-mode gradient of oracle_gdn_recurrent.  The pages call the
 * chunked algorithm a training method but print no gradient formulas, so
 * this is the chain rule applied to the ordered step above, one token at a
 * time, newest token first:
 *
 *   forward   Sbar = alpha S_{t-1};  e = beta (v - Sbar k);  S_t = Sbar + e k^T;  o_t = S_t q
 *   reverse   G   += do_t q^T                       (G = dL/dS_t from here on)
 *             dq   = S_t^T do_t
 *             de   = G k,        dk  = G^T e        (through S_t = Sbar + e k^T)
 *             dbeta = de . (v - Sbar k),  dv = beta de,
 *             dSbar = G - beta de k^T,    dk -= beta Sbar^T de   (through e)
 *             dalpha = <dSbar, S_{t-1}>,  dlog_alpha = alpha dalpha
 *             G    = alpha dSbar                    (= dL/dS_{t-1})
 *
 * G starts from d_final (zeros when NULL); what is left after a sequence's
 * first token is d_init.  The states S_0 .. S_L of a sequence are kept (the
 * forward pass is replayed with gated_delta_token), so memory per chain is
 * (L + 1) dv dk doubles.
 *
 * d_o  [T, H, dv];  d_final, d_init [N, H, dv, dk] (NULL: zeros / not
 * returned);  dq, dk [T, H, dk];  dv [T, H, dv];  dlog_alpha, dbeta [T, H].
 */
int oracle_gdn_recurrent_bwd(int64_t n_seqs, const int64_t *cu, int64_t H, int64_t dk, int64_t dv,
                             const double *q, const double *k, const double *v,
                             const double *log_alpha, const double *beta,
                             const double *init_state, const double *d_o, const double *d_final,
                             double *dq, double *dkey, double *dval, double *dlog_alpha,
                             double *dbeta, double *d_init, int n_threads)
{
    int rc = check_args(n_seqs, cu, H, dk, dv);
    if (rc) return rc;
    const int64_t jobs = n_seqs * H;
    const int64_t sz = dv * dk;
    int failed = 0;
#ifdef _OPENMP
    if (n_threads <= 0) n_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads) reduction(| : failed)
#endif
    for (int64_t job = 0; job < jobs; ++job) {
        const int64_t n = job / H, h = job % H;
        const int64_t t0 = cu[n], L = cu[n + 1] - cu[n];
        double *states = (double *)malloc(sizeof(double) * (size_t)((L + 1) * sz));
        double *G = (double *)malloc(sizeof(double) * (size_t)sz);
        double *work = (double *)malloc(sizeof(double) * (size_t)(4 * dv));
        if (!states || !G || !work) {
            free(states);
            free(G);
            free(work);
            failed = 1;
            continue;
        }
        double *err = work, *pred = work + dv, *de = work + 2 * dv, *obuf = work + 3 * dv;
        if (init_state)
            memcpy(states, init_state + job * sz, sizeof(double) * (size_t)sz);
        else
            memset(states, 0, sizeof(double) * (size_t)sz);
        for (int64_t t = 0; t < L; ++t) {
            const int64_t th = (t0 + t) * H + h;
            memcpy(states + (t + 1) * sz, states + t * sz, sizeof(double) * (size_t)sz);
            gated_delta_token(states + (t + 1) * sz, err, dk, dv, q + th * dk, k + th * dk, v + th * dv,
                              log_alpha[th], beta[th], obuf);
        }
        if (d_final)
            memcpy(G, d_final + job * sz, sizeof(double) * (size_t)sz);
        else
            memset(G, 0, sizeof(double) * (size_t)sz);
        for (int64_t t = L - 1; t >= 0; --t) {
            const int64_t th = (t0 + t) * H + h;
            const double *Sp = states + t * sz, *Sc = states + (t + 1) * sz;
            const double *qt = q + th * dk, *kt = k + th * dk, *vt = v + th * dv, *dot = d_o + th * dv;
            const double alpha = exp(log_alpha[th]), b = beta[th];
            double *dqt = dq + th * dk, *dkt = dkey + th * dk, *dvt = dval + th * dv;
            /* o_t = S_t q */
            for (int64_t i = 0; i < dv; ++i)
                for (int64_t j = 0; j < dk; ++j) G[i * dk + j] += dot[i] * qt[j];
            for (int64_t j = 0; j < dk; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < dv; ++i) acc += Sc[i * dk + j] * dot[i];
                dqt[j] = acc;
            }
            /* e = beta (v - Sbar k), Sbar = alpha S_{t-1} */
            for (int64_t i = 0; i < dv; ++i) {
                double p = 0.0, g = 0.0;
                for (int64_t j = 0; j < dk; ++j) {
                    p += alpha * Sp[i * dk + j] * kt[j];
                    g += G[i * dk + j] * kt[j];
                }
                pred[i] = p;
                err[i] = b * (vt[i] - p);
                de[i] = g;
            }
            double db = 0.0;
            for (int64_t i = 0; i < dv; ++i) {
                db += de[i] * (vt[i] - pred[i]);
                dvt[i] = b * de[i];
            }
            dbeta[th] = db;
            for (int64_t j = 0; j < dk; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < dv; ++i)
                    acc += G[i * dk + j] * err[i] - b * alpha * Sp[i * dk + j] * de[i];
                dkt[j] = acc;
            }
            /* dSbar = G - beta de k^T; dalpha = <dSbar, S_{t-1}>; G = alpha dSbar */
            double da = 0.0;
            for (int64_t i = 0; i < dv; ++i)
                for (int64_t j = 0; j < dk; ++j) {
                    const double dsb = G[i * dk + j] - b * de[i] * kt[j];
                    da += dsb * Sp[i * dk + j];
                    G[i * dk + j] = alpha * dsb;
                }
            dlog_alpha[th] = alpha * da;
        }
        if (d_init) memcpy(d_init + job * sz, G, sizeof(double) * (size_t)sz);
        free(states);
        free(G);
        free(work);
    }
    return failed ? -3 : 0;
}
