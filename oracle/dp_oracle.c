/*
 * dp_oracle.c -- slow, plain fp64 CPU oracle for the DeltaProduct forward
 * recurrence, its gradient, and the OSDN phase-1 preconditioner scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP kernels.
 *
 * Sources (titles of the pages this follows):
 *   [DP]   "DeltaProduct: Improving State-Tracking in Linear RNNs via
 *          Householder Products" (study notes, arXiv 2502.10297v7).
 *   [OSDN] "OSDN: Improving Delta Rule with Provable Online Preconditioning
 *          in Linear Attention" (study notes, arXiv 2605.13473v1).
 *
 * What is computed is the plain sequential definition, one sub-step at a
 * time, in the order the pages state it:
 *   - per token, optional scalar forget gate applied once, before the first
 *     Householder sub-step ([DP] sec. 2.6, gated DeltaProduct; the
 *     conceptual per-token pseudocode there);
 *   - per sub-step j: unit key k = k_raw / max(|k_raw|_2, 1e-6)
 *     ([DP] sec. 2.2, key normalisation), beta clamped to [0, 2]
 *     ([DP] sec. 2.5, the range where every factor has spectral norm <= 1),
 *     prediction error e = v - H^T k, then H += beta * w e^T
 *     ([DP] sec. 2.1 Eq.(2) delta rule and sec. 2.2 Eq.(3)); the write key
 *     w is k itself, or a separately supplied write key for the asymmetric
 *     rule ([OSDN] sec. 2.2, Eqs.(2)/(5): residual with the read key, write
 *     with the scaled key);
 *   - readout o = H^T q after the token's last sub-step ([DP] sec. 2.6 and
 *     sec. 4.1 / Sec.5.1: only the last sub-step of each token is kept).
 * Phase 1 of OSDN ([OSDN] sec. 2.4, Alg.1): emit d_t * k_t first, then
 * d <- clamp(d + eta*beta*(1 - beta<d, k*k>)/max(|k|^2, eps) * (k*k)).
 Its gradient (oracle_precond_bwd) is the reverse-mode derivative of that
 * scan ([OSDN] sec. 2.5, closing paragraph: through kt_t = d_t * k_t into d_t
 * and k_t, then back through the recursion).
 *
 * All arithmetic is IEEE double, in the order written, no blocking, fusion or
 * reordering.  Heads (b, h) are independent, so they are spread over OpenMP
 * threads; each head runs strictly sequentially.
 *
 * Layouts (row-major, all double):
 *   q     [B, L, H, dk]
 *   k     [B, L, H, n_h, dk]   raw keys (normalised here)
 *   kt    [B, L, H, n_h, dk]   write keys, used as given (NULL: symmetric)
 *   v     [B, L, H, n_h, dv]
 *   beta  [B, L, H, n_h]
 *   g     [B, L, H]            (NULL: no gate)
 *   h0    [B, H, dk, dv]       initial state (NULL: zero)
 *   out   [B, L, H, dv]
 *   final_state [B, H, dk, dv] (NULL: not returned)
 * The state H of a head is dk x dv (key dimension by value dimension), the
 * orientation of [DP] sec. 2.1; [OSDN] uses its transpose S = H^T.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_KEY_EPS 1e-6

static double clampd(double x, double lo, double hi)
{
    if (x < lo) return lo;
    if (x > hi) return hi;
    return x;
}

/* unit read key: k / max(|k|_2, 1e-6)  ([DP] sec. 2.2) */
static void unit_key(const double* kr, int dk, double* kh)
{
    double n2 = 0.0;
    for (int r = 0; r < dk; ++r) n2 += kr[r] * kr[r];
    double nrm = sqrt(n2);
    double den = nrm > ORACLE_KEY_EPS ? nrm : ORACLE_KEY_EPS;
    for (int r = 0; r < dk; ++r) kh[r] = kr[r] / den;
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
 * One head (b, h) of the sequential DeltaProduct forward ([DP] sec. 2.2
 * Eq.(3), sec. 2.6), with an optional asymmetric write key ([OSDN] sec. 2.2)
 * and an optional per-key-channel gate ga [B, L, H, dk] (the KDA host of
 * [OSDN] sec. 2.7: H <- Diag(alpha_t) H before the token's sub-steps, so the
 * residual and the write see the decayed state).
 * out_h points at this head's first output row; consecutive tokens are
 * out_stride doubles apart.  S (dk*dv), kh (dk) and e (dv) are scratch.
 */
static void run_head(const double* q, const double* k, const double* kt, const double* v,
                     const double* beta, const double* g, const double* ga, int n_h, long b,
                     long h, int H, int L, int dk, int dv, const double* h0_h, double* out_h,
                     size_t out_stride, double* fs_h, double* S, double* kh, double* e)
{
    if (h0_h)
        memcpy(S, h0_h, sizeof(double) * (size_t)dk * dv);
    else
        memset(S, 0, sizeof(double) * (size_t)dk * dv);

    for (long t = 0; t < L; ++t) {
        const size_t tok = ((size_t)b * L + t) * H + h; /* (b, t, h) */
        if (ga) {
            /* Diag(alpha_t) H: row r of the state (key channel r) scales by alpha_t[r] */
            const double* al = ga + tok * dk;
            for (int r = 0; r < dk; ++r)
                for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] *= al[r];
        }
        if (g) {
            /* H_{i,0} = g_i H_{i-1}: once per token, before its sub-steps */
            const double gt = g[tok];
            for (size_t x = 0; x < (size_t)dk * dv; ++x) S[x] *= gt;
        }
        for (int j = 0; j < n_h; ++j) {
            const size_t sub = tok * n_h + j; /* (b, t, h, j) */
            unit_key(k + sub * dk, dk, kh);
            const double bt = clampd(beta[sub], 0.0, 2.0);
            const double* w = kt ? kt + sub * dk : kh;
            const double* vv = v + sub * dv;
            /* e = v - H^T k  (prediction error on the read key) */
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int r = 0; r < dk; ++r) acc += S[(size_t)r * dv + c] * kh[r];
                e[c] = vv[c] - acc;
            }
            /* H += beta * w e^T */
            for (int r = 0; r < dk; ++r) {
                const double bw = bt * w[r];
                for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] += bw * e[c];
            }
        }
        /* o = H^T q after the token's last sub-step */
        const double* qq = q + tok * dk;
        double* oo = out_h + (size_t)t * out_stride;
        for (int c = 0; c < dv; ++c) {
            double acc = 0.0;
            for (int r = 0; r < dk; ++r) acc += S[(size_t)r * dv + c] * qq[r];
            oo[c] = acc;
        }
    }
    if (fs_h) memcpy(fs_h, S, sizeof(double) * (size_t)dk * dv);
}

/*
 * Forward over the heads listed in heads[0..nsel) (flattened b * H + h), or
 * over all B*H heads when heads is NULL.  With heads == NULL, out is the full
 * [B, L, H, dv] tensor and final_state [B, H, dk, dv]; with a list, both are
 * compact: out [nsel, L, dv], final_state [nsel, dk, dv].  Returns 0, -1 on
 * bad arguments, -2 when scratch memory could not be allocated.
 */
static int fwd_impl(const double* q, const double* k, const double* kt, const double* v,
                    const double* beta, const double* g, const double* ga, int n_h, int B, int H, int L,
                    int dk, int dv, const double* h0, const long* heads, int nsel,
                    double* out, double* final_state, int nthreads)
{
    if (!q || !k || !v || !beta || !out) return -1;
    if (n_h < 1 || B < 0 || H < 0 || L < 0 || dk < 1 || dv < 1) return -1;
    const long nbh = (long)B * H;
    const long nrun = heads ? nsel : nbh;
    if (heads) {
        if (nsel < 0) return -1;
        for (long i = 0; i < nsel; ++i)
            if (heads[i] < 0 || heads[i] >= nbh) return -1;
    }
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    (void)nthreads;
#endif
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
    for (long i = 0; i < nrun; ++i) {
        const long bh = heads ? heads[i] : i;
        const long b = bh / H, h = bh % H;
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        double* kh = (double*)malloc(sizeof(double) * (size_t)dk);
        double* e = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!S || !kh || !e) {
            free(S); free(kh); free(e);
            bad |= 1;
            continue;
        }
        const double* h0_h = h0 ? h0 + (size_t)bh * dk * dv : NULL;
        double* out_h;
        size_t out_stride;
        double* fs_h;
        if (heads) {
            out_h = out + (size_t)i * L * dv;
            out_stride = (size_t)dv;
            fs_h = final_state ? final_state + (size_t)i * dk * dv : NULL;
        } else {
            out_h = out + ((size_t)b * L * H + h) * dv;
            out_stride = (size_t)H * dv;
            fs_h = final_state ? final_state + (size_t)bh * dk * dv : NULL;
        }
        run_head(q, k, kt, v, beta, g, ga, n_h, b, h, H, L, dk, dv, h0_h, out_h, out_stride,
                 fs_h, S, kh, e);
        free(S); free(kh); free(e);
    }
    return bad ? -2 : 0;
}

/* Full forward over all heads.  nthreads <= 0: OpenMP default. */
int oracle_fwd(const double* q, const double* k, const double* kt, const double* v,
               const double* beta, const double* g, const double* ga, int n_h, int B, int H,
               int L, int dk, int dv, const double* h0, double* out, double* final_state,
               int nthreads)
{
    return fwd_impl(q, k, kt, v, beta, g, ga, n_h, B, H, L, dk, dv, h0, NULL, 0, out,
                    final_state, nthreads);
}

/*
 * Forward for a subset of heads (sampled checks of large workloads): each
 * listed head is computed exactly as oracle_fwd computes it; outputs compact.
 */
int oracle_fwd_heads(const double* q, const double* k, const double* kt, const double* v,
                     const double* beta, const double* g, const double* ga, int n_h, int B,
                     int H, int L, int dk, int dv, const double* h0, const long* heads, int nsel,
                     double* out, double* final_state, int nthreads)
{
    if (!heads) return -1;
    return fwd_impl(q, k, kt, v, beta, g, ga, n_h, B, H, L, dk, dv, h0, heads, nsel, out,
                    final_state, nthreads);
}

/*
 * OSDN phase 1 ([OSDN] sec. 2.3-2.4, Alg.1), per head, sequential over
 * tokens.  Keys are [B, L, H, dk] raw keys, normalised here with the same
 * rule as the forward; beta [B, L, H] is clamped to [0, 2] as in the forward.
 * d_state [B, H, dk]: d_1 on entry, d_{L+1} on exit.  kt_out [B, L, H, dk]:
 * the write keys d_t * k_t, emitted BEFORE d is updated.
 *
 * Two variants the pages describe ride on the same scan:
 *   - ret [B, L, H] (NULL: none): the APF retention gate r_t of [OSDN]
 *     sec. 2.6 (Sec.4.4), which scales d_t inside the projection,
 *     d_{t+1} = P[r_t d_t + step]; the step itself still uses d_t;
 *   - beta_aware = 0: the beta-free phase-1 step of the 1.3B configuration
 *     ([OSDN] sec. 2.7, App.B/C), eta (1 - <d_t, s_t>) s_t, i.e. the
 *     beta-aware step with beta replaced by 1 (the division by
 *     max(|k|^2, eps) is 1 for unit keys and is kept).
 * The box [dmin, dmax] is the projection; dmin = -inf, dmax = +inf drop it.
 */
int oracle_precond_ex(const double* k, const double* beta, const double* ret, int beta_aware,
                      int B, int H, int L, int dk, double eta, double dmin, double dmax,
                      double eps, double* d_state, double* kt_out, int nthreads)
{
    if (!k || !beta || !d_state || !kt_out) return -1;
    if (B < 0 || H < 0 || L < 0 || dk < 1) return -1;
    long nbh = (long)B * H;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    (void)nthreads;
#endif
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
    for (long bh = 0; bh < nbh; ++bh) {
        const long b = bh / H, h = bh % H;
        double* d = d_state + (size_t)bh * dk;
        double* kh = (double*)malloc(sizeof(double) * (size_t)dk);
        if (!kh) {
            bad |= 1;
            continue;
        }
        for (long t = 0; t < L; ++t) {
            const size_t tok = ((size_t)b * L + t) * H + h;
            unit_key(k + tok * dk, dk, kh);
            const double bt = clampd(beta[tok], 0.0, 2.0);
            /* the beta of the phase-1 step: the clamped beta, or 1 (beta-free) */
            const double bu = beta_aware ? bt : 1.0;
            /* retention of d_t (APF); 1 without the gate */
            const double rt = ret ? ret[tok] : 1.0;
            /* emit the write key with the current d_t */
            double* ko = kt_out + tok * dk;
            for (int r = 0; r < dk; ++r) ko[r] = d[r] * kh[r];
            /* s = k*k, n = |k|^2, a = beta <d, s> */
            double n = 0.0, ds = 0.0;
            for (int r = 0; r < dk; ++r) {
                const double s = kh[r] * kh[r];
                n += s;
                ds += d[r] * s;
            }
            const double a = bu * ds;
            const double nb = n > eps ? n : eps;
            const double coef = eta * bu * (1.0 - a) / nb;
            /* retained d_t plus the step, projected onto the box [dmin, dmax]^dk */
            for (int r = 0; r < dk; ++r) d[r] = clampd(rt * d[r] + coef * (kh[r] * kh[r]), dmin, dmax);
        }
        free(kh);
    }
    return bad ? -2 : 0;
}

/* The phase-1 scan as [OSDN] Alg.1 states it: no retention, beta-aware step. */
int oracle_precond(const double* k, const double* beta, int B, int H, int L, int dk,
                   double eta, double dmin, double dmax, double eps, double* d_state,
                   double* kt_out, int nthreads)
{
    return oracle_precond_ex(k, beta, NULL, 1, B, H, L, dk, eta, dmin, dmax, eps, d_state,
                             kt_out, nthreads);
}

/*
 * Gradient of the phase-1 scan (reverse mode, last token first).  [OSDN]
 * sec. 2.5, closing paragraph (Sec.4.5): in training the write key
 * kt_t = d_t * kh_t passes its gradient to both d_t and k_t, and the gradient
 * of d then runs back through the preconditioner recursion of sec. 2.4 (with
 * the retention of sec. 2.6 and the beta-free step of sec. 2.7 as in
 * oracle_precond_ex).  Per token, with s = kh*kh, n = |kh|^2, nb = max(n, eps),
 * a = bu <d, s>, coef = eta bu (1 - a) / nb and x = r d + coef s (before the
 * projection onto the box):
 *   dx     = dd' where dmin <= x <= dmax, else 0     (dd' = gradient on d_{t+1})
 *   dd     = r dx - eta bu^2 / nb <dx, s> s + kh * dkt_t
 *   dr     = <dx, d>
 *   ds     = coef dx + <dx, s> (-eta bu^2 / nb d - [n > eps] coef / nb)
 *   dbu    = <dx, s> eta (1 - 2a) / nb
 *   dkh    = 2 kh * ds + d * dkt_t
 * then the unit-key normalisation and the beta clamp as in the forward's
 * gradient below (the derivative of a clamp at its end points is taken as 1).
 * The beta-free step has no beta gradient.
 *
 * Inputs as oracle_precond_ex (d0 [B, H, dk] the initial d, NULL: ones), plus
 * dkt [B, L, H, dk], the gradient on the emitted write keys, and dd_final
 * [B, H, dk] (NULL: zero), the gradient on the final d.  Outputs dk [B, L, H,
 * dk] (raw keys), dbeta [B, L, H], dret [B, L, H] (NULL: not returned; zero
 * without ret) and dd0 [B, H, dk] (NULL: not returned).  The forward is run
 * again first, keeping every d_t.  Returns 0, -1 on bad arguments, -2 when
 * scratch memory could not be allocated.
 */
int oracle_precond_bwd(const double* k, const double* beta, const double* ret, int beta_aware,
                       int B, int H, int L, int dk, double eta, double dmin, double dmax,
                       double eps, const double* d0, const double* dkt, const double* dd_final,
                       double* dk_out, double* dbeta, double* dret, double* dd0, int nthreads)
{
    if (!k || !beta || !dkt || !dk_out || !dbeta) return -1;
    if (B < 0 || H < 0 || L < 0 || dk < 1) return -1;
    long nbh = (long)B * H;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    (void)nthreads;
#endif
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
    for (long bh = 0; bh < nbh; ++bh) {
        const long b = bh / H, h = bh % H;
        /* D[t]: d_t, the preconditioner before token t's update (t = 0 .. L-1) */
        double* D = (double*)malloc(sizeof(double) * (size_t)dk * (size_t)(L > 0 ? L : 1));
        double* d = (double*)malloc(sizeof(double) * (size_t)dk);
        double* gd = (double*)malloc(sizeof(double) * (size_t)dk);
        double* kh = (double*)malloc(sizeof(double) * (size_t)dk);
        double* gx = (double*)malloc(sizeof(double) * (size_t)dk);
        double* gkh = (double*)malloc(sizeof(double) * (size_t)dk);
        if (!D || !d || !gd || !kh || !gx || !gkh) {
            free(D); free(d); free(gd); free(kh); free(gx); free(gkh);
            bad |= 1;
            continue;
        }
        /* forward again, keeping d_t */
        for (int r = 0; r < dk; ++r) d[r] = d0 ? d0[(size_t)bh * dk + r] : 1.0;
        for (long t = 0; t < L; ++t) {
            const size_t tok = ((size_t)b * L + t) * H + h;
            memcpy(D + (size_t)t * dk, d, sizeof(double) * (size_t)dk);
            unit_key(k + tok * dk, dk, kh);
            const double bu = beta_aware ? clampd(beta[tok], 0.0, 2.0) : 1.0;
            const double rt = ret ? ret[tok] : 1.0;
            double n = 0.0, ds = 0.0;
            for (int r = 0; r < dk; ++r) {
                const double s = kh[r] * kh[r];
                n += s;
                ds += d[r] * s;
            }
            const double nb = n > eps ? n : eps;
            const double coef = eta * bu * (1.0 - bu * ds) / nb;
            for (int r = 0; r < dk; ++r) d[r] = clampd(rt * d[r] + coef * (kh[r] * kh[r]), dmin, dmax);
        }
        /* reverse sweep */
        for (int r = 0; r < dk; ++r) gd[r] = dd_final ? dd_final[(size_t)bh * dk + r] : 0.0;
        for (long t = L - 1; t >= 0; --t) {
            const size_t tok = ((size_t)b * L + t) * H + h;
            const double* dt = D + (size_t)t * dk;
            const double* gk = dkt + tok * dk;
            unit_key(k + tok * dk, dk, kh);
            const double braw = beta[tok];
            const double bu = beta_aware ? clampd(braw, 0.0, 2.0) : 1.0;
            const double rt = ret ? ret[tok] : 1.0;
            double n = 0.0, ds = 0.0;
            for (int r = 0; r < dk; ++r) {
                const double s = kh[r] * kh[r];
                n += s;
                ds += dt[r] * s;
            }
            const double a = bu * ds;
            const double nb = n > eps ? n : eps;
            const double coef = eta * bu * (1.0 - a) / nb;
            /* through the projection */
            double gxs = 0.0, gr = 0.0;
            for (int r = 0; r < dk; ++r) {
                const double x = rt * dt[r] + coef * (kh[r] * kh[r]);
                gx[r] = (x >= dmin && x <= dmax) ? gd[r] : 0.0;
                gxs += gx[r] * (kh[r] * kh[r]);
                gr += gx[r] * dt[r];
            }
            if (dret) dret[tok] = ret ? gr : 0.0;
            /* beta: coef = eta (bu - bu^2 <d, s>) / nb */
            const double gbu = gxs * eta * (1.0 - 2.0 * a) / nb;
            dbeta[tok] = (beta_aware && braw >= 0.0 && braw <= 2.0) ? gbu : 0.0;
            /* s through x, a and n; kh through s and the emitted write key */
            const double cn = n > eps ? coef / nb : 0.0;
            double p = 0.0;
            for (int r = 0; r < dk; ++r) {
                const double gs = coef * gx[r] + gxs * (-eta * bu * bu / nb * dt[r] - cn);
                gkh[r] = 2.0 * kh[r] * gs + dt[r] * gk[r];
                p += kh[r] * gkh[r];
            }
            /* raw key through k / max(|k|, 1e-6) */
            const double* kr = k + tok * dk;
            double n2 = 0.0;
            for (int r = 0; r < dk; ++r) n2 += kr[r] * kr[r];
            const double nrm = sqrt(n2);
            double* dko = dk_out + tok * dk;
            for (int r = 0; r < dk; ++r)
                dko[r] = nrm > ORACLE_KEY_EPS ? (gkh[r] - kh[r] * p) / nrm : gkh[r] / ORACLE_KEY_EPS;
            /* d_t through x, a and the emitted write key */
            for (int r = 0; r < dk; ++r)
                gd[r] = rt * gx[r] - eta * bu * bu / nb * gxs * (kh[r] * kh[r]) + kh[r] * gk[r];
        }
        if (dd0) memcpy(dd0 + (size_t)bh * dk, gd, sizeof(double) * (size_t)dk);
        free(D); free(d); free(gd); free(kh); free(gx); free(gkh);
    }
    return bad ? -2 : 0;
}

/*
 * ------------------------------------------------------------------------
 * Gradient of the forward (reverse mode, one sub-step at a time).
 *
 * For a scalar loss with dout = dLoss/dout [B, L, H, dv] and dfinal =
 * dLoss/dfinal_state [B, H, dk, dv] (NULL: zero), this returns the gradients
 * w.r.t. every input of the forward above, by differentiating its
 * sequential definition step by step, last token first:
 *   readout o = H^T q:          dq = H dout,  dH += q dout^T
 *   sub-step H' = H + bt w e^T with e = v - H^T kh:
 *                               de = bt dH'^T w      (this is dv)
 *                               dbt = w^T dH' e,  dw = bt dH' e
 *                               dkh = -H de (+ dw when w = kh)
 *                               dH = dH' - kh de^T
 *   unit key kh = k / max(|k|, 1e-6):
 *                               dk = (dkh - kh <kh, dkh>) / |k|   (|k| > 1e-6)
 *                               dk = dkh / 1e-6                   (otherwise)
 *   beta clamp to [0, 2]:       dbeta = dbt where 0 <= beta <= 2, else 0
 *   gate H_0 = g H_prev:        dg = <dH_0, H_prev>,  dH_prev = g dH_0
 * and dh0 = dH after the first token.  The derivative of the clamp at its
 * end points is taken as 1 (the gradient passes at beta = 0 and beta = 2).
 * The per-channel gate of the forward is not differentiated here.
 *
 * heads == NULL: every head, gradients in the layouts of the inputs:
 *   dq [B,L,H,dk], dk [B,L,H,n_h,dk], dkt [B,L,H,n_h,dk] (when kt),
 *   dv [B,L,H,n_h,dv], dbeta [B,L,H,n_h], dg [B,L,H] (when g),
 *   dh0 [B,H,dk,dv].
 * heads != NULL: the listed heads only, compact: dq [n,L,dk], dk and dkt
 *   [n,L,n_h,dk], dv [n,L,n_h,dv], dbeta [n,L,n_h], dg [n,L], dh0 [n,dk,dv].
 * dkt, dg and dh0 may be NULL (not returned).  Returns 0, -1 on bad
 * arguments, -2 when scratch memory could not be allocated.
 */
static int bwd_impl(const double* q, const double* k, const double* kt, const double* v,
                    const double* beta, const double* g, int n_h, int B, int H, int L, int dk,
                    int dv, const double* h0, const double* dout, const double* dfinal,
                    const long* heads, int nsel, double* dq, double* dkr, double* dkt,
                    double* dvv, double* dbeta, double* dg, double* dh0, int nthreads)
{
    if (!q || !k || !v || !beta || !dout || !dq || !dkr || !dvv || !dbeta) return -1;
    if (n_h < 1 || B < 0 || H < 0 || L < 0 || dk < 1 || dv < 1) return -1;
    const long nbh = (long)B * H;
    const long nrun = heads ? nsel : nbh;
    if (heads) {
        if (nsel < 0) return -1;
        for (long i = 0; i < nsel; ++i)
            if (heads[i] < 0 || heads[i] >= nbh) return -1;
    }
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    (void)nthreads;
#endif
    const size_t DS = (size_t)dk * dv;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
    for (long i = 0; i < nrun; ++i) {
        const long bh = heads ? heads[i] : i;
        const long b = bh / H, h = bh % H;
        /* Hpre[t]: the state before token t's gate; Hs[j]: before sub-step j of one token */
        double* Hpre = (double*)malloc(sizeof(double) * DS * (size_t)(L > 0 ? L : 1));
        double* Hs = (double*)malloc(sizeof(double) * DS * (size_t)(n_h + 1));
        double* dH = (double*)malloc(sizeof(double) * DS);
        double* kh = (double*)malloc(sizeof(double) * (size_t)dk * n_h);
        double* e = (double*)malloc(sizeof(double) * (size_t)dv * n_h);
        double* de = (double*)malloc(sizeof(double) * (size_t)dv);
        double* dkh = (double*)malloc(sizeof(double) * (size_t)dk);
        if (!Hpre || !Hs || !dH || !kh || !e || !de || !dkh) {
            free(Hpre); free(Hs); free(dH); free(kh); free(e); free(de); free(dkh);
            bad |= 1;
            continue;
        }
        /* output addressing: element (t, [j,] x) of this head */
        size_t oq, sq, ok, sk, ov, sv, ob, sb, og, sg;
        if (heads) {
            oq = (size_t)i * L * dk;          sq = (size_t)dk;
            ok = (size_t)i * L * n_h * dk;    sk = (size_t)n_h * dk;
            ov = (size_t)i * L * n_h * dv;    sv = (size_t)n_h * dv;
            ob = (size_t)i * L * n_h;         sb = (size_t)n_h;
            og = (size_t)i * L;               sg = 1;
        } else {
            const size_t tok0 = (size_t)b * L * H + h;
            oq = tok0 * dk;                   sq = (size_t)H * dk;
            ok = tok0 * n_h * dk;             sk = (size_t)H * n_h * dk;
            ov = tok0 * n_h * dv;             sv = (size_t)H * n_h * dv;
            ob = tok0 * n_h;                  sb = (size_t)H * n_h;
            og = tok0;                        sg = (size_t)H;
        }
        const size_t odh = (size_t)(heads ? i : bh) * DS;

        /* forward, keeping the state before each token's gate */
        double* S = Hs; /* running state */
        if (h0)
            memcpy(S, h0 + (size_t)bh * DS, sizeof(double) * DS);
        else
            memset(S, 0, sizeof(double) * DS);
        for (long t = 0; t < L; ++t) {
            const size_t tok = ((size_t)b * L + t) * H + h;
            memcpy(Hpre + (size_t)t * DS, S, sizeof(double) * DS);
            if (g)
                for (size_t x = 0; x < DS; ++x) S[x] *= g[tok];
            for (int j = 0; j < n_h; ++j) {
                const size_t sub = tok * n_h + j;
                unit_key(k + sub * dk, dk, kh);
                const double bt = clampd(beta[sub], 0.0, 2.0);
                const double* w = kt ? kt + sub * dk : kh;
                for (int c = 0; c < dv; ++c) {
                    double acc = 0.0;
                    for (int r = 0; r < dk; ++r) acc += S[(size_t)r * dv + c] * kh[r];
                    e[c] = v[sub * dv + c] - acc;
                }
                for (int r = 0; r < dk; ++r)
                    for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] += bt * w[r] * e[c];
            }
        }

        /* reverse sweep */
        if (dfinal)
            memcpy(dH, dfinal + (size_t)bh * DS, sizeof(double) * DS);
        else
            memset(dH, 0, sizeof(double) * DS);
        for (long t = L - 1; t >= 0; --t) {
            const size_t tok = ((size_t)b * L + t) * H + h;
            /* recompute this token: Hs[j] is the state before sub-step j, Hs[n_h] after the last */
            memcpy(Hs, Hpre + (size_t)t * DS, sizeof(double) * DS);
            if (g)
                for (size_t x = 0; x < DS; ++x) Hs[x] *= g[tok];
            for (int j = 0; j < n_h; ++j) {
                const size_t sub = tok * n_h + j;
                const double* Sj = Hs + (size_t)j * DS;
                double* Sn = Hs + (size_t)(j + 1) * DS;
                double* khj = kh + (size_t)j * dk;
                double* ej = e + (size_t)j * dv;
                unit_key(k + sub * dk, dk, khj);
                const double bt = clampd(beta[sub], 0.0, 2.0);
                const double* w = kt ? kt + sub * dk : khj;
                for (int c = 0; c < dv; ++c) {
                    double acc = 0.0;
                    for (int r = 0; r < dk; ++r) acc += Sj[(size_t)r * dv + c] * khj[r];
                    ej[c] = v[sub * dv + c] - acc;
                }
                for (int r = 0; r < dk; ++r)
                    for (int c = 0; c < dv; ++c)
                        Sn[(size_t)r * dv + c] = Sj[(size_t)r * dv + c] + bt * w[r] * ej[c];
            }
            /* readout o = H^T q after the last sub-step */
            const double* qq = q + tok * dk;
            const double* Hl = Hs + (size_t)n_h * DS;
            const double* dO = dout + tok * dv;
            double* dqt = dq + oq + (size_t)t * sq;
            for (int r = 0; r < dk; ++r) {
                double acc = 0.0;
                for (int c = 0; c < dv; ++c) acc += Hl[(size_t)r * dv + c] * dO[c];
                dqt[r] = acc;
            }
            for (int r = 0; r < dk; ++r)
                for (int c = 0; c < dv; ++c) dH[(size_t)r * dv + c] += qq[r] * dO[c];
            /* sub-steps, last first */
            for (int j = n_h - 1; j >= 0; --j) {
                const size_t sub = tok * n_h + j;
                const double* Sj = Hs + (size_t)j * DS;
                const double* khj = kh + (size_t)j * dk;
                const double* ej = e + (size_t)j * dv;
                const double braw = beta[sub];
                const double bt = clampd(braw, 0.0, 2.0);
                const double* w = kt ? kt + sub * dk : khj;
                /* de = bt dH^T w */
                for (int c = 0; c < dv; ++c) {
                    double acc = 0.0;
                    for (int r = 0; r < dk; ++r) acc += w[r] * dH[(size_t)r * dv + c];
                    de[c] = bt * acc;
                }
                /* dbt = w^T dH e;  dw = bt dH e */
                double dbt = 0.0;
                double* dktj = dkt ? dkt + ok + (size_t)t * sk + (size_t)j * dk : NULL;
                for (int r = 0; r < dk; ++r) {
                    double acc = 0.0;
                    for (int c = 0; c < dv; ++c) acc += dH[(size_t)r * dv + c] * ej[c];
                    dbt += w[r] * acc;
                    /* dkh = -H de, plus dw when the write key is the read key */
                    double dr = 0.0;
                    for (int c = 0; c < dv; ++c) dr -= Sj[(size_t)r * dv + c] * de[c];
                    if (kt) {
                        if (dktj) dktj[r] = bt * acc;
                    } else {
                        dr += bt * acc;
                    }
                    dkh[r] = dr;
                }
                /* dv = de */
                double* dvj = dvv + ov + (size_t)t * sv + (size_t)j * dv;
                for (int c = 0; c < dv; ++c) dvj[c] = de[c];
                /* dbeta through the clamp */
                dbeta[ob + (size_t)t * sb + j] = (braw >= 0.0 && braw <= 2.0) ? dbt : 0.0;
                /* dk through the normalisation */
                const double* kr = k + sub * dk;
                double n2 = 0.0;
                for (int r = 0; r < dk; ++r) n2 += kr[r] * kr[r];
                const double nrm = sqrt(n2);
                double* dkj = dkr + ok + (size_t)t * sk + (size_t)j * dk;
                if (nrm > ORACLE_KEY_EPS) {
                    double p = 0.0;
                    for (int r = 0; r < dk; ++r) p += khj[r] * dkh[r];
                    for (int r = 0; r < dk; ++r) dkj[r] = (dkh[r] - khj[r] * p) / nrm;
                } else {
                    for (int r = 0; r < dk; ++r) dkj[r] = dkh[r] / ORACLE_KEY_EPS;
                }
                /* dH before the sub-step: dH - kh de^T */
                for (int r = 0; r < dk; ++r)
                    for (int c = 0; c < dv; ++c) dH[(size_t)r * dv + c] -= khj[r] * de[c];
            }
            /* gate: H_0 = g H_prev */
            if (g) {
                const double* Hp = Hpre + (size_t)t * DS;
                double acc = 0.0;
                for (size_t x = 0; x < DS; ++x) acc += dH[x] * Hp[x];
                if (dg) dg[og + (size_t)t * sg] = acc;
                for (size_t x = 0; x < DS; ++x) dH[x] *= g[tok];
            }
        }
        if (dh0) memcpy(dh0 + odh, dH, sizeof(double) * DS);
        free(Hpre); free(Hs); free(dH); free(kh); free(e); free(de); free(dkh);
    }
    return bad ? -2 : 0;
}

int oracle_bwd(const double* q, const double* k, const double* kt, const double* v,
               const double* beta, const double* g, int n_h, int B, int H, int L, int dk, int dv,
               const double* h0, const double* dout, const double* dfinal, double* dq,
               double* dk_out, double* dkt, double* dv_out, double* dbeta, double* dg,
               double* dh0, int nthreads)
{
    return bwd_impl(q, k, kt, v, beta, g, n_h, B, H, L, dk, dv, h0, dout, dfinal, NULL, 0, dq,
                    dk_out, dkt, dv_out, dbeta, dg, dh0, nthreads);
}

int oracle_bwd_heads(const double* q, const double* k, const double* kt, const double* v,
                     const double* beta, const double* g, int n_h, int B, int H, int L, int dk,
                     int dv, const double* h0, const double* dout, const double* dfinal,
                     const long* heads, int nsel, double* dq, double* dk_out, double* dkt,
                     double* dv_out, double* dbeta, double* dg, double* dh0, int nthreads)
{
    if (!heads) return -1;
    return bwd_impl(q, k, kt, v, beta, g, n_h, B, H, L, dk, dv, h0, dout, dfinal, heads, nsel,
                    dq, dk_out, dkt, dv_out, dbeta, dg, dh0, nthreads);
}
