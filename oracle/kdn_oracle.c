/*
 * kdn_oracle.c -- plain fp64 CPU oracle for the Kalman Delta Network (KDN)
 * sequence mixer.  TEST INFRASTRUCTURE ONLY: nothing in the product path may
 * link, load or call this file; only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark use it.  It shares no code, header, table
 * or constant with the HIP library.
 *
 * What it computes is the token-by-token recurrence exactly as the KDN
 * reading notes ("Kalman Delta Networks: uncertainty-aware associative
 * memory", Chinese reading notes, Part 2) state it, with no chunking, no scan
 * and no reordering beyond the order of the additions inside a dot product:
 *
 *   Diagonal KDN (notes Part 2 sec. 4, Eq. (23)-(30); information scaling
 *   sec. 5, Eq. (60)-(65)):
 *     predict   p^_t   = alpha_t^2 (.) p_{t-1} + omega_t
 *     gain      kappa_t = p^_t (.) k_t / (r_t + sum_i p^_{t,i} k_{t,i}^2)
 *     mean      S^_t = D_t S_{t-1},  D_t = diag(alpha_t)           (Eq. 12)
 *     innovation delta_t = v_t - S^_t^T k_t                         (Eq. 13)
 *     write     S_t = S^_t + kappa_t delta_t^T                      (Eq. 14)
 *     readout   o_t = S_t^T q_t  (after this token's write)         (Eq. 17)
 *     variance  p_t = p^_t / (1 + u_t (.) p^_t),  u_t = (mu/r_t) k_t (.) k_t
 *               -- applied after the gain, so mu never changes the
 *               current write (sec. 5, "update order").
 *
 *   Isotropic KDN (notes Part 2 sec. 7, Eq. (40); Appendix C):
 *     a_t = mean_i alpha_{t,i}^2,  b^_t = a_t b_{t-1} + omega_t
 *     beta_t = b^_t / (r_t + b^_t |k_t|^2),  kappa_t = beta_t k_t
 *     memory lines identical to the diagonal variant (per-channel decay)
 *     b_t = b^_t / (1 + u_t b^_t),  u_t = mu |k_t|^2 / (d_k r_t)
 *
 *   Per-head options (notes Part 2 sec. 8, trained parameters): a learned
 *   information scale mu_h per head, and a learned initial covariance
 *   c_{0,h} I per head used when no initial variance is given.
 *   Diagnostic (notes Part 2 sec. 2): effective write strength
 *     beta_eff_t = k_t^T kappa_t = z_t / (r_t + z_t),
 *     z_t = sum_i p^_{t,i} k_{t,i}^2 (Diagonal), b^_t |k_t|^2 (Isotropic).
 *
 * Layouts (row-major): activations [B,T,H,D]; state S [B,H,dk,dv];
 * variances p [B,H,dk] (diagonal) or b [B,H] (isotropic); gates alpha
 * [B,T,H,dk], omega [B,T,H,dk] (diagonal) or [B,T,H] (isotropic), r [B,T,H].
 * Every (b,h) pair is an independent problem; OpenMP splits them.
 */
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static size_t act_index(int T, int H, int D, int b, int t, int h)
{
    return (((size_t)b * T + t) * H + h) * (size_t)D;
}

/* One (b,h) problem of Diagonal KDN.  S is dk x dv (row i = key channel),
 * p has dk entries; both are updated in place. */
static void diag_head(int B, int T, int H, int dk, int dv, int b, int h,
                      const double* q, const double* k, const double* v,
                      const double* alpha, const double* omega,
                      const double* r, double mu,
                      double* S, double* p, double* o,
                      double* kappa_out, double* phat_out, double* beff_out,
                      double* ph, double* kap, double* delta)
{
    (void)B;
    for (int t = 0; t < T; ++t) {
        const double* qt = q + act_index(T, H, dk, b, t, h);
        const double* kt = k + act_index(T, H, dk, b, t, h);
        const double* vt = v + act_index(T, H, dv, b, t, h);
        const double* at = alpha + act_index(T, H, dk, b, t, h);
        const double* wt = omega + act_index(T, H, dk, b, t, h);
        const double rt = r[((size_t)b * T + t) * H + h];
        double* ot = o + act_index(T, H, dv, b, t, h);

        /* predict the variance: p^ = alpha^2 p + omega */
        for (int i = 0; i < dk; ++i)
            ph[i] = at[i] * at[i] * p[i] + wt[i];

        /* Kalman gain from the predicted (pre-update) variance */
        double z = 0.0;
        for (int i = 0; i < dk; ++i)
            z += ph[i] * kt[i] * kt[i];
        for (int i = 0; i < dk; ++i)
            kap[i] = ph[i] * kt[i] / (rt + z);
        if (beff_out)
            beff_out[((size_t)b * T + t) * H + h] = z / (rt + z);

        /* predicted mean S^ = diag(alpha) S */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] *= at[i];

        /* innovation delta = v - S^^T k */
        for (int j = 0; j < dv; ++j)
            delta[j] = vt[j];
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                delta[j] -= S[(size_t)i * dv + j] * kt[i];

        /* write S = S^ + kappa delta^T */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] += kap[i] * delta[j];

        /* read after the write: o = S^T q */
        for (int j = 0; j < dv; ++j)
            ot[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                ot[j] += S[(size_t)i * dv + j] * qt[i];

        /* information-scaled reverse-KL variance update */
        for (int i = 0; i < dk; ++i) {
            const double u = (mu / rt) * kt[i] * kt[i];
            p[i] = ph[i] / (1.0 + u * ph[i]);
        }

        if (kappa_out)
            memcpy(kappa_out + act_index(T, H, dk, b, t, h), kap, sizeof(double) * dk);
        if (phat_out)
            memcpy(phat_out + act_index(T, H, dk, b, t, h), ph, sizeof(double) * dk);
    }
}

/* One (b,h) problem of Isotropic KDN; bvar is the head's scalar variance. */
static void iso_head(int B, int T, int H, int dk, int dv, int b, int h,
                     const double* q, const double* k, const double* v,
                     const double* alpha, const double* omega,
                     const double* r, double mu,
                     double* S, double* bvar, double* o,
                     double* beta_out, double* bhat_out, double* beff_out,
                     double* kap, double* delta)
{
    (void)B;
    for (int t = 0; t < T; ++t) {
        const double* qt = q + act_index(T, H, dk, b, t, h);
        const double* kt = k + act_index(T, H, dk, b, t, h);
        const double* vt = v + act_index(T, H, dv, b, t, h);
        const double* at = alpha + act_index(T, H, dk, b, t, h);
        const size_t bth = ((size_t)b * T + t) * H + h;
        const double wt = omega[bth];
        const double rt = r[bth];
        double* ot = o + act_index(T, H, dv, b, t, h);

        /* trace projection of the predicted covariance */
        double a = 0.0;
        for (int i = 0; i < dk; ++i)
            a += at[i] * at[i];
        a /= (double)dk;
        const double bh = a * (*bvar) + wt;

        /* scalar gain along k */
        double n = 0.0;
        for (int i = 0; i < dk; ++i)
            n += kt[i] * kt[i];
        const double beta = bh / (rt + bh * n);
        for (int i = 0; i < dk; ++i)
            kap[i] = beta * kt[i];

        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] *= at[i];
        for (int j = 0; j < dv; ++j)
            delta[j] = vt[j];
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                delta[j] -= S[(size_t)i * dv + j] * kt[i];
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] += kap[i] * delta[j];
        for (int j = 0; j < dv; ++j)
            ot[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                ot[j] += S[(size_t)i * dv + j] * qt[i];

        /* isotropic reverse-KL (harmonic-mean) update with scaling mu */
        const double u = mu * n / ((double)dk * rt);
        *bvar = bh / (1.0 + u * bh);

        if (beta_out)
            beta_out[bth] = beta;
        if (bhat_out)
            bhat_out[bth] = bh;
        if (beff_out)  /* z = k^T (b^ I) k */
            beff_out[bth] = bh * n / (rt + bh * n);
    }
}

/*
 * Diagonal KDN forward over [B,T,H] tokens.  S0 (nullable = zeros) and p0
 * (nullable = c0_h[h], or ones without c0_h) are the initial state; o, S_T,
 * p_T are written.  mu_h (nullable, [H]) overrides mu per head.
 * kappa_out / phat_out (nullable, [B,T,H,dk]) expose the gain and the
 * predicted variance for the tests, beff_out (nullable, [B,T,H]) the
 * effective write strength.  Returns 0, or -1 on bad sizes / memory.
 */
int kdn_oracle_diag_fwd(int B, int T, int H, int dk, int dv,
                        const double* q, const double* k, const double* v,
                        const double* alpha, const double* omega,
                        const double* r, const double* S0, const double* p0,
                        const double* c0_h, double mu, const double* mu_h,
                        double* o, double* S_T, double* p_T,
                        double* kappa_out, double* phat_out, double* beff_out,
                        int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0)
        return -1;
    const int BH = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(|| : failed)
#endif
    for (int bh = 0; bh < BH; ++bh) {
        const int b = bh / H, h = bh % H;
        double* S = S_T + (size_t)bh * dk * dv;
        double* p = p_T + (size_t)bh * dk;
        if (S0)
            memcpy(S, S0 + (size_t)bh * dk * dv, sizeof(double) * dk * dv);
        else
            memset(S, 0, sizeof(double) * dk * dv);
        for (int i = 0; i < dk; ++i)
            p[i] = p0 ? p0[(size_t)bh * dk + i] : (c0_h ? c0_h[h] : 1.0);
        double* scratch = (double*)malloc(sizeof(double) * (2 * (size_t)dk + dv));
        if (!scratch) {
            failed = 1;
            continue;
        }
        diag_head(B, T, H, dk, dv, b, h, q, k, v, alpha, omega, r, mu_h ? mu_h[h] : mu, S, p, o,
                  kappa_out, phat_out, beff_out, scratch, scratch + dk, scratch + 2 * dk);
        free(scratch);
    }
    return failed ? -1 : 0;
}

/*
 * Isotropic KDN forward.  omega is [B,T,H]; b0 (nullable = c0_h[h], or ones
 * without c0_h) and b_T are [B,H]; mu_h as in the Diagonal call.
 * beta_out / bhat_out / beff_out (nullable, [B,T,H]) expose the scalar gain,
 * the predicted variance and the effective write strength for the tests.
 */
int kdn_oracle_iso_fwd(int B, int T, int H, int dk, int dv,
                       const double* q, const double* k, const double* v,
                       const double* alpha, const double* omega,
                       const double* r, const double* S0, const double* b0,
                       const double* c0_h, double mu, const double* mu_h,
                       double* o, double* S_T, double* b_T,
                       double* beta_out, double* bhat_out, double* beff_out,
                       int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0)
        return -1;
    const int BH = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(|| : failed)
#endif
    for (int bh = 0; bh < BH; ++bh) {
        const int b = bh / H, h = bh % H;
        double* S = S_T + (size_t)bh * dk * dv;
        if (S0)
            memcpy(S, S0 + (size_t)bh * dk * dv, sizeof(double) * dk * dv);
        else
            memset(S, 0, sizeof(double) * dk * dv);
        b_T[bh] = b0 ? b0[bh] : (c0_h ? c0_h[h] : 1.0);
        double* scratch = (double*)malloc(sizeof(double) * ((size_t)dk + dv));
        if (!scratch) {
            failed = 1;
            continue;
        }
        iso_head(B, T, H, dk, dv, b, h, q, k, v, alpha, omega, r, mu_h ? mu_h[h] : mu, S, &b_T[bh], o,
                 beta_out, bhat_out, beff_out, scratch, scratch + dk);
        free(scratch);
    }
    return failed ? -1 : 0;
}

int kdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
