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

/*
 * ---------------------------------------------------------------------------
 * Backward pass (reverse-mode derivative of the two recurrences above).
 *
 * The notes train with the scanned recurrence (Part 2 sec. 8) but print no
 * gradient formulas, so these are derived here, one forward line at a time
 * in reverse order.  With adjoints G = dL/dS_t and pbar = dL/dp_t carried
 * backwards from dL/dS_T, dL/dp_T, and do_t = dL/do_t given per token:
 *
 *   readout   o = S^T q         G += q do^T,          dq = S do
 *   write     S = S^ + kap del^T  kapbar = G del,      delbar = G^T kap
 *   innovation del = v - S^^T k   dv = delbar,  S^bar = G - k delbar^T,
 *                                 dk += -S^ delbar
 *   decay     S^ = D S_{t-1}    dalpha_i += sum_j S^bar_ij S_{t-1,ij},
 *                               G <- D S^bar
 *   Diagonal variance  p = p^/(1+u p^), u = (mu/r) k^2:
 *       p^bar = pbar/(1+u p^)^2,  ubar = -pbar p^^2/(1+u p^)^2,
 *       dk += 2 ubar (mu/r) k,  dr -= sum ubar u / r,  dmu += sum ubar k^2/r
 *   Diagonal gain  kap = p^ k / d, d = r + sum p^ k^2:
 *       dbar = -sum kapbar kap / d,  dr += dbar,
 *       p^bar += kapbar k / d + dbar k^2,  dk += kapbar p^/d + 2 dbar p^ k
 *   predict   p^ = alpha^2 p_{t-1} + omega:
 *       dalpha += 2 p^bar alpha p_{t-1},  domega = p^bar,  pbar <- p^bar alpha^2
 *   Isotropic (a = mean alpha^2, n = |k|^2, e = r + b^ n, beta = b^/e,
 *   kap = beta k, b = b^/(1+u b^), u = mu n/(dk r)):
 *       b^bar = bbar/(1+u b^)^2, ubar = -bbar b^^2/(1+u b^)^2,
 *       nbar = ubar mu/(dk r), dr -= ubar u/r, dmu += ubar n/(dk r),
 *       betabar = kapbar . k, dk += beta kapbar,
 *       b^bar += betabar r/e^2, dr -= betabar b^/e^2, nbar -= betabar b^^2/e^2,
 *       dk += 2 nbar k, abar = b^bar b_{t-1}, domega = b^bar,
 *       bbar <- b^bar a, dalpha += 2 abar alpha / dk
 * ending with dS_0 = G and dp_0 = pbar (db_0 = bbar).  The forward states
 * S_{t-1} and p_{t-1} are kept for every token (this is a small-case
 * reference).  Pinned in the tests against central finite differences of
 * the forward functions above.
 * ---------------------------------------------------------------------------
 */

/* Inputs shared by the two backward calls, gathered to keep signatures short. */
typedef struct {
    int B, T, H, dk, dv;
    const double *q, *k, *v, *alpha, *omega, *r, *S0, *var0, *c0_h, *mu_h, *dO, *dST, *dvarT;
    double mu;
    double *dq, *dk_, *dv_, *dalpha, *domega, *dr, *dS0, *dvar0, *dmu;
} bwd_io;

static int bwd_head(const bwd_io* a, int iso, int b, int h)
{
    const int T = a->T, H = a->H, dk = a->dk, dv = a->dv;
    const size_t bh = (size_t)b * H + h, SZ = (size_t)dk * dv;
    const double mu = a->mu_h ? a->mu_h[h] : a->mu;
    const int nvar = iso ? 1 : dk;
    double* states = (double*)malloc(sizeof(double) * SZ * ((size_t)T + 1));
    double* vars = (double*)malloc(sizeof(double) * (size_t)nvar * ((size_t)T + 1));
    double* w = (double*)malloc(sizeof(double) * (SZ + 6 * (size_t)dk + 2 * (size_t)dv));
    if (!states || !vars || !w) {
        free(states); free(vars); free(w);
        return -1;
    }
    double* G = w;                 /* dk x dv */
    double* ph = G + SZ;           /* dk */
    double* kap = ph + dk;
    double* kapbar = kap + dk;
    double* kbar = kapbar + dk;
    double* abar = kbar + dk;
    double* pbar = abar + dk;      /* nvar */
    double* del = pbar + dk;       /* dv */
    double* delbar = del + dv;

    /* forward, keeping S_t and p_t (b_t) for t = 0..T */
    if (a->S0)
        memcpy(states, a->S0 + bh * SZ, sizeof(double) * SZ);
    else
        memset(states, 0, sizeof(double) * SZ);
    for (int i = 0; i < nvar; ++i)
        vars[i] = a->var0 ? a->var0[bh * nvar + i] : (a->c0_h ? a->c0_h[h] : 1.0);
    for (int t = 0; t < T; ++t) {
        const size_t tok = ((size_t)b * T + t) * H + h;
        const double* kt = a->k + tok * dk;
        const double* vt = a->v + tok * dv;
        const double* at = a->alpha + tok * dk;
        const double rt = a->r[tok];
        const double* Sp = states + (size_t)t * SZ;
        double* Sn = states + (size_t)(t + 1) * SZ;
        const double* pp = vars + (size_t)t * nvar;
        double* pn = vars + (size_t)(t + 1) * nvar;
        double n = 0.0;
        for (int i = 0; i < dk; ++i)
            n += kt[i] * kt[i];
        if (iso) {
            double aa = 0.0;
            for (int i = 0; i < dk; ++i)
                aa += at[i] * at[i];
            aa /= (double)dk;
            const double bhat = aa * pp[0] + a->omega[tok];
            const double beta = bhat / (rt + bhat * n);
            for (int i = 0; i < dk; ++i)
                kap[i] = beta * kt[i];
            pn[0] = bhat / (1.0 + mu * n / ((double)dk * rt) * bhat);
        } else {
            const double* wt = a->omega + tok * dk;
            double z = 0.0;
            for (int i = 0; i < dk; ++i) {
                ph[i] = at[i] * at[i] * pp[i] + wt[i];
                z += ph[i] * kt[i] * kt[i];
            }
            for (int i = 0; i < dk; ++i) {
                kap[i] = ph[i] * kt[i] / (rt + z);
                pn[i] = ph[i] / (1.0 + (mu / rt) * kt[i] * kt[i] * ph[i]);
            }
        }
        for (int j = 0; j < dv; ++j)
            del[j] = vt[j];
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                del[j] -= at[i] * Sp[(size_t)i * dv + j] * kt[i];
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                Sn[(size_t)i * dv + j] = at[i] * Sp[(size_t)i * dv + j] + kap[i] * del[j];
    }

    /* reverse */
    if (a->dST)
        memcpy(G, a->dST + bh * SZ, sizeof(double) * SZ);
    else
        memset(G, 0, sizeof(double) * SZ);
    for (int i = 0; i < nvar; ++i)
        pbar[i] = a->dvarT ? a->dvarT[bh * nvar + i] : 0.0;
    double mubar = 0.0;
    for (int t = T - 1; t >= 0; --t) {
        const size_t tok = ((size_t)b * T + t) * H + h;
        const double* qt = a->q + tok * dk;
        const double* kt = a->k + tok * dk;
        const double* vt = a->v + tok * dv;
        const double* at = a->alpha + tok * dk;
        const double* dot = a->dO + tok * dv;
        const double rt = a->r[tok];
        const double* Sp = states + (size_t)t * SZ;
        const double* Sn = states + (size_t)(t + 1) * SZ;
        const double* pp = vars + (size_t)t * nvar;

        /* recompute this token's gain quantities */
        double n = 0.0;
        for (int i = 0; i < dk; ++i)
            n += kt[i] * kt[i];
        double aa = 0.0, bhat = 0.0, beta = 0.0, e = 0.0, d = 0.0;
        if (iso) {
            for (int i = 0; i < dk; ++i)
                aa += at[i] * at[i];
            aa /= (double)dk;
            bhat = aa * pp[0] + a->omega[tok];
            e = rt + bhat * n;
            beta = bhat / e;
            for (int i = 0; i < dk; ++i)
                kap[i] = beta * kt[i];
        } else {
            const double* wt = a->omega + tok * dk;
            double z = 0.0;
            for (int i = 0; i < dk; ++i) {
                ph[i] = at[i] * at[i] * pp[i] + wt[i];
                z += ph[i] * kt[i] * kt[i];
            }
            d = rt + z;
            for (int i = 0; i < dk; ++i)
                kap[i] = ph[i] * kt[i] / d;
        }
        for (int j = 0; j < dv; ++j)
            del[j] = vt[j];
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                del[j] -= at[i] * Sp[(size_t)i * dv + j] * kt[i];

        /* readout o = S^T q */
        double* dqt = a->dq + tok * dk;
        for (int i = 0; i < dk; ++i) {
            double s = 0.0;
            for (int j = 0; j < dv; ++j) {
                G[(size_t)i * dv + j] += qt[i] * dot[j];
                s += Sn[(size_t)i * dv + j] * dot[j];
            }
            dqt[i] = s;
        }
        /* write S = S^ + kap del^T */
        for (int j = 0; j < dv; ++j)
            delbar[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            double s = 0.0;
            for (int j = 0; j < dv; ++j) {
                s += G[(size_t)i * dv + j] * del[j];
                delbar[j] += G[(size_t)i * dv + j] * kap[i];
            }
            kapbar[i] = s;
        }
        double* dvt = a->dv_ + tok * dv;
        for (int j = 0; j < dv; ++j)
            dvt[j] = delbar[j];
        /* innovation del = v - S^^T k and decay S^ = D S_{t-1} */
        for (int i = 0; i < dk; ++i) {
            double sk = 0.0, sa = 0.0;
            for (int j = 0; j < dv; ++j) {
                const double shb = G[(size_t)i * dv + j] - kt[i] * delbar[j];
                sk += at[i] * Sp[(size_t)i * dv + j] * delbar[j];
                sa += shb * Sp[(size_t)i * dv + j];
                G[(size_t)i * dv + j] = at[i] * shb;
            }
            kbar[i] = -sk;
            abar[i] = sa;
        }

        double rbar = 0.0;
        double* dwt = iso ? a->domega + tok : a->domega + tok * dk;
        if (iso) {
            const double u = mu * n / ((double)dk * rt);
            const double den = 1.0 + u * bhat;
            double bhbar = pbar[0] / (den * den);
            const double ubar = -pbar[0] * bhat * bhat / (den * den);
            double nbar = ubar * mu / ((double)dk * rt);
            rbar -= ubar * u / rt;
            mubar += ubar * n / ((double)dk * rt);
            double betabar = 0.0;
            for (int i = 0; i < dk; ++i) {
                betabar += kapbar[i] * kt[i];
                kbar[i] += beta * kapbar[i];
            }
            bhbar += betabar * rt / (e * e);
            rbar -= betabar * bhat / (e * e);
            nbar -= betabar * bhat * bhat / (e * e);
            for (int i = 0; i < dk; ++i)
                kbar[i] += 2.0 * nbar * kt[i];
            const double abar_s = bhbar * pp[0];
            dwt[0] = bhbar;
            pbar[0] = bhbar * aa;
            for (int i = 0; i < dk; ++i)
                abar[i] += 2.0 * abar_s * at[i] / (double)dk;
        } else {
            double dbar = 0.0;
            for (int i = 0; i < dk; ++i)
                dbar -= kapbar[i] * kap[i] / d;
            rbar += dbar;
            for (int i = 0; i < dk; ++i) {
                const double u = (mu / rt) * kt[i] * kt[i];
                const double den = 1.0 + u * ph[i];
                double phbar = pbar[i] / (den * den);
                const double ubar = -pbar[i] * ph[i] * ph[i] / (den * den);
                kbar[i] += 2.0 * ubar * (mu / rt) * kt[i];
                rbar -= ubar * u / rt;
                mubar += ubar * kt[i] * kt[i] / rt;
                phbar += kapbar[i] * kt[i] / d + dbar * kt[i] * kt[i];
                kbar[i] += kapbar[i] * ph[i] / d + 2.0 * dbar * ph[i] * kt[i];
                abar[i] += 2.0 * phbar * at[i] * pp[i];
                dwt[i] = phbar;
                pbar[i] = phbar * at[i] * at[i];
            }
        }
        a->dr[tok] = rbar;
        memcpy(a->dk_ + tok * dk, kbar, sizeof(double) * dk);
        memcpy(a->dalpha + tok * dk, abar, sizeof(double) * dk);
    }
    if (a->dS0)
        memcpy(a->dS0 + bh * SZ, G, sizeof(double) * SZ);
    if (a->dvar0)
        memcpy(a->dvar0 + bh * nvar, pbar, sizeof(double) * nvar);
    if (a->dmu)
        a->dmu[bh] = mubar;
    free(states); free(vars); free(w);
    return 0;
}

/*
 * Backward of kdn_oracle_diag_fwd (iso = 0) or kdn_oracle_iso_fwd (iso = 1)
 * for the loss L = sum(dO . o) + sum(dST . S_T) + sum(dvarT . var_T).
 * Forward arguments as in those calls (var0 = p0 or b0); dST, dvarT nullable
 * (zero).  Writes dq, dk, dv, dalpha, domega, dr (shapes of the inputs), and
 * when non-null dS0 [B,H,dk,dv], dvar0 (shape of var0) and dmu [B,H] (the
 * derivative by each (b,h)'s information scale).  Returns 0, -1 on bad sizes
 * or memory.
 */
int kdn_oracle_bwd(int iso, int B, int T, int H, int dk, int dv,
                   const double* q, const double* k, const double* v,
                   const double* alpha, const double* omega, const double* r,
                   const double* S0, const double* var0, const double* c0_h,
                   double mu, const double* mu_h,
                   const double* dO, const double* dST, const double* dvarT,
                   double* dq, double* dk_, double* dv_, double* dalpha,
                   double* domega, double* dr, double* dS0, double* dvar0,
                   double* dmu, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0)
        return -1;
    bwd_io a = {B, T, H, dk, dv, q, k, v, alpha, omega, r, S0, var0, c0_h, mu_h, dO, dST,
                dvarT, mu, dq, dk_, dv_, dalpha, domega, dr, dS0, dvar0, dmu};
    const int BH = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(|| : failed)
#endif
    for (int bh = 0; bh < BH; ++bh)
        if (bwd_head(&a, iso, bh / H, bh % H) != 0)
            failed = 1;
    return failed ? -1 : 0;
}
