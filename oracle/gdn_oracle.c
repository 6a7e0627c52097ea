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
