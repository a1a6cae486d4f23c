/*
 * TEST INFRASTRUCTURE ONLY.  This is the fp64 CPU reference ("oracle") for the
 * complex-valued diagonal selective state-space scan.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never links, includes or calls anything in this directory,
 * and shares no source with it.
 *
 * What it computes is the literal sequential recurrence, one time step after
 * another, with no chunking, no blocking and no reordering:
 *
 *   s_t   = softplus(dt_t)                      real step, softplus on the real dt
 *   a_t   = exp(s_t * A)                        A is one complex scalar per head
 *         = exp(s_t Re A) (cos(s_t Im A) + i sin(s_t Im A))
 *   h_t   = a_t h_{t-1} + B_t (x) x_t           h_t is N x D complex, B_t in C^N, x_t in C^D
 *   y_t   = sum_n C_t[n] h_t[n,:] + Dskip x_t   C_t is NOT conjugated
 *
 * Sources (the pages this follows):
 *  - Mamba-3-Lite docs, "SSD Theory -- Complex States & the Chunkwise Algorithm",
 *    section 2 "Why it exists: the sequential scan is the bottleneck": the naive
 *    loop that multiplies the whole state by the per-head factor, adds the
 *    outer product of B_t and x_t, and reads out by summing C_t times the state
 *    over the state index.
 *  - Mamba-3-Lite docs, "Complex-Valued State Spaces", subsections "The
 *    recurrence", "Discretization" (softplus is applied to the real dt and the
 *    result then multiplies the complex A; the order is deliberate) and the
 *    walkthrough of the discretise helper and the naive scan (state layout
 *    (B,H,N,D), zero initial state).
 *  - burn-mamba docs, module "step_constant": the readout adds a skip term
 *    D x to C^T h.
 *
 * Readings where the pages leave a step open: y is returned as a complex value (both planes); softplus is the exact
 * log(1+e^dt), evaluated in the overflow-free form max(dt,0)+log1p(e^-|dt|);
 * a NULL Dskip means D = 0; a NULL initial state means h_{-1} = 0.
 *
 * Parallelism: OpenMP over the independent (batch, head) sequences only; the
 * loop over time inside one sequence is the plain serial recurrence.
 *
 * Later in this file, each with its own sources: the constant-input closed forms,
 * the reverse-mode gradients of the recurrence, the phase-state paper's
 * per-coordinate scan and its causal Born attention.
 */
#include <math.h>
#include <stddef.h>
#include <complex.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double softplus(double v)
{
    /* log(1 + e^v), written so that neither branch overflows */
    return fmax(v, 0.0) + log1p(exp(-fabs(v)));
}

/* a = exp(softplus(dt) * A), A = (are, aim): scale e^{s Re A}, rotation s Im A */
static void discretise(double dt, double are, double aim, double *ar, double *ai)
{
    double s = softplus(dt);
    double mag = exp(s * are);
    *ar = mag * cos(s * aim);
    *ai = mag * sin(s * aim);
}

/*
 * One time step for one (batch, head) state of N x D complex values:
 *   h <- a h + B (x) x ;  y = sum_n C[n] h[n,:] + d x
 */
static void one_step(int64_t D, int64_t N, double ar, double ai,
                     const double *xr, const double *xi,
                     const double *br, const double *bi,
                     const double *cr, const double *ci, double d,
                     double *hr, double *hi, double *yr, double *yi)
{
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t p = 0; p < D; ++p) {
            double orr = hr[n * D + p], oii = hi[n * D + p];
            /* a * h_old */
            double nr = ar * orr - ai * oii;
            double ni = ar * oii + ai * orr;
            /* + B[n] * x[p] */
            nr += br[n] * xr[p] - bi[n] * xi[p];
            ni += br[n] * xi[p] + bi[n] * xr[p];
            hr[n * D + p] = nr;
            hi[n * D + p] = ni;
        }
    }
    for (int64_t p = 0; p < D; ++p) {
        double sr = 0.0, si = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double vr = hr[n * D + p], vi = hi[n * D + p];
            sr += cr[n] * vr - ci[n] * vi;
            si += cr[n] * vi + ci[n] * vr;
        }
        yr[p] = sr + d * xr[p];
        yi[p] = si + d * xi[p];
    }
}

/*
 * Full forward over T steps.  Layouts (row-major, planar re/im):
 *   x  [B,T,H,D]   Bm, Cm [B,T,H,N]   dt [B,T,H]   A [H]   Dskip [H] or NULL
 *   h0 [B,H,N,D] or NULL (zero)       y [B,T,H,D]  hT [B,H,N,D] or NULL
 * nthreads <= 0 uses the OpenMP default.  Returns 0, or -1 on a bad argument
 * or allocation failure.
 */
int oracle_forward_f64(int64_t Bsz, int64_t T, int64_t H, int64_t D, int64_t N,
                       const double *x_re, const double *x_im,
                       const double *b_re, const double *b_im,
                       const double *c_re, const double *c_im,
                       const double *dt, const double *a_re, const double *a_im,
                       const double *dskip,
                       const double *h0_re, const double *h0_im,
                       double *y_re, double *y_im,
                       double *hT_re, double *hT_im, int nthreads)
{
    if (Bsz <= 0 || T < 0 || H <= 0 || D <= 0 || N <= 0)
        return -1;
    if (!x_re || !x_im || !b_re || !b_im || !c_re || !c_im || !dt || !a_re ||
        !a_im || !y_re || !y_im)
        return -1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t bh = 0; bh < Bsz * H; ++bh) {
        int64_t b = bh / H, h = bh % H;
        double *hr = (double *)calloc((size_t)(N * D), sizeof(double));
        double *hi = (double *)calloc((size_t)(N * D), sizeof(double));
        if (!hr || !hi) {
            free(hr);
            free(hi);
            failed |= 1;
            continue;
        }
        if (h0_re && h0_im) {
            memcpy(hr, h0_re + bh * N * D, sizeof(double) * (size_t)(N * D));
            memcpy(hi, h0_im + bh * N * D, sizeof(double) * (size_t)(N * D));
        }
        double d = dskip ? dskip[h] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            int64_t row = (b * T + t) * H + h; /* (b, t, h) */
            double ar, ai;
            discretise(dt[row], a_re[h], a_im[h], &ar, &ai);
            one_step(D, N, ar, ai, x_re + row * D, x_im + row * D,
                     b_re + row * N, b_im + row * N, c_re + row * N,
                     c_im + row * N, d, hr, hi, y_re + row * D, y_im + row * D);
        }
        if (hT_re && hT_im) {
            memcpy(hT_re + bh * N * D, hr, sizeof(double) * (size_t)(N * D));
            memcpy(hT_im + bh * N * D, hi, sizeof(double) * (size_t)(N * D));
        }
        free(hr);
        free(hi);
    }
    return failed ? -1 : 0;
}

/*
 * One decode step for every (batch, head): the same loop body as above applied
 * once to a persistent state, updated in place.
 *   x [B,H,D]  Bm, Cm [B,H,N]  dt [B,H]  A [H]  Dskip [H] or NULL
 *   h [B,H,N,D] in/out          y [B,H,D]
 */
int oracle_step_f64(int64_t Bsz, int64_t H, int64_t D, int64_t N,
                    const double *x_re, const double *x_im,
                    const double *b_re, const double *b_im,
                    const double *c_re, const double *c_im,
                    const double *dt, const double *a_re, const double *a_im,
                    const double *dskip, double *h_re, double *h_im,
                    double *y_re, double *y_im, int nthreads)
{
    if (Bsz <= 0 || H <= 0 || D <= 0 || N <= 0)
        return -1;
    if (!x_re || !x_im || !b_re || !b_im || !c_re || !c_im || !dt || !a_re ||
        !a_im || !h_re || !h_im || !y_re || !y_im)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (int64_t bh = 0; bh < Bsz * H; ++bh) {
        int64_t h = bh % H;
        double ar, ai;
        discretise(dt[bh], a_re[h], a_im[h], &ar, &ai);
        one_step(D, N, ar, ai, x_re + bh * D, x_im + bh * D, b_re + bh * N,
                 b_im + bh * N, c_re + bh * N, c_im + bh * N,
                 dskip ? dskip[h] : 0.0, h_re + bh * N * D, h_im + bh * N * D,
                 y_re + bh * D, y_im + bh * D);
    }
    return 0;
}

/*
 * A constant input held for n steps, in closed form (burn-mamba docs, module
 * step_constant: when the same token is fed again and again, the n unrolled
 * steps collapse to a geometric series in the per-step factor; here there is no
 * rotation operator between steps and the input enters with unit weight, so the
 * series is in the scalar decay a itself):
 *   a   = exp(softplus(dt) A),   a^n = exp(n softplus(dt) A)
 *   h_n = a^n h_0 + (1 - a^n) / (1 - a) * B (x) x      the ratio is n when a = 1
 *   y_n = sum_k C[k] h_n[k,:] + Dskip x                 the output of the n-th step
 * Same layouts as oracle_step_f64; h is replaced by h_n.  n >= 1.
 */
int oracle_step_n_f64(int64_t Bsz, int64_t H, int64_t D, int64_t N, int64_t n,
                      const double *x_re, const double *x_im,
                      const double *b_re, const double *b_im,
                      const double *c_re, const double *c_im,
                      const double *dt, const double *a_re, const double *a_im,
                      const double *dskip, double *h_re, double *h_im,
                      double *y_re, double *y_im, int nthreads)
{
    if (Bsz <= 0 || H <= 0 || D <= 0 || N <= 0 || n < 1)
        return -1;
    if (!x_re || !x_im || !b_re || !b_im || !c_re || !c_im || !dt || !a_re ||
        !a_im || !h_re || !h_im || !y_re || !y_im)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (int64_t bh = 0; bh < Bsz * H; ++bh) {
        int64_t h = bh % H;
        double s = softplus(dt[bh]);
        double complex z = s * (a_re[h] + a_im[h] * I);
        double complex a = cexp(z);
        double complex an = cexp((double)n * z);
        double complex ratio = (a == 1.0) ? (double complex)(double)n : (1.0 - an) / (1.0 - a);
        double d = dskip ? dskip[h] : 0.0;
        const double *xr = x_re + bh * D, *xi = x_im + bh * D;
        double *hr = h_re + bh * N * D, *hi = h_im + bh * N * D;
        for (int64_t k = 0; k < N; ++k) {
            double complex bk = b_re[bh * N + k] + b_im[bh * N + k] * I;
            for (int64_t p = 0; p < D; ++p) {
                double complex xp = xr[p] + xi[p] * I;
                double complex hv = hr[k * D + p] + hi[k * D + p] * I;
                double complex hn = an * hv + ratio * bk * xp;
                hr[k * D + p] = creal(hn);
                hi[k * D + p] = cimag(hn);
            }
        }
        for (int64_t p = 0; p < D; ++p) {
            double complex acc = 0.0;
            for (int64_t k = 0; k < N; ++k) {
                double complex ck = c_re[bh * N + k] + c_im[bh * N + k] * I;
                acc += ck * (hr[k * D + p] + hi[k * D + p] * I);
            }
            acc += d * (xr[p] + xi[p] * I);
            y_re[bh * D + p] = creal(acc);
            y_im[bh * D + p] = cimag(acc);
        }
    }
    return 0;
}

/*
 * The output of an endless constant input (same page: the stationary fixed
 * point, which no starting state influences).  For |a| < 1 the series of
 * decays sums to 1 / (1 - a), so
 *   y_inf = (sum_k C[k] B[k]) / (1 - a) * x + Dskip x
 * Layouts as oracle_step_f64, without a state.
 */
int oracle_step_infinite_f64(int64_t Bsz, int64_t H, int64_t D, int64_t N,
                             const double *x_re, const double *x_im,
                             const double *b_re, const double *b_im,
                             const double *c_re, const double *c_im,
                             const double *dt, const double *a_re, const double *a_im,
                             const double *dskip, double *y_re, double *y_im, int nthreads)
{
    if (Bsz <= 0 || H <= 0 || D <= 0 || N <= 0)
        return -1;
    if (!x_re || !x_im || !b_re || !b_im || !c_re || !c_im || !dt || !a_re ||
        !a_im || !y_re || !y_im)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (int64_t bh = 0; bh < Bsz * H; ++bh) {
        int64_t h = bh % H;
        double s = softplus(dt[bh]);
        double complex a = cexp(s * (a_re[h] + a_im[h] * I));
        double complex score = 0.0;
        for (int64_t k = 0; k < N; ++k)
            score += (c_re[bh * N + k] + c_im[bh * N + k] * I) *
                     (b_re[bh * N + k] + b_im[bh * N + k] * I);
        double complex gain = score / (1.0 - a);
        double d = dskip ? dskip[h] : 0.0;
        for (int64_t p = 0; p < D; ++p) {
            double complex xp = x_re[bh * D + p] + x_im[bh * D + p] * I;
            double complex yv = gain * xp + d * xp;
            y_re[bh * D + p] = creal(yv);
            y_im[bh * D + p] = cimag(yv);
        }
    }
    return 0;
}

/*
 * Gradients of the forward recurrence (reverse mode, one (batch, head) at a
 * time).  The pages train this scan with automatic differentiation of complex
 * tensors (Mamba-3-Lite docs, "SSD Theory", the autograd notes, and "The
 * Chunkwise Complex SSD Algorithm", the complex-dtype requirement); the
 * gradient of a real loss L with respect to a complex value u + i v is taken as
 * the pair (dL/du, dL/dv), written as the complex number dL/du + i dL/dv.
 * With that convention, for a product w = c z the gradient reaching z is
 * conj(c) times the gradient of w, and the one reaching c is the gradient of w
 * times conj(z).  Walking the recurrence backwards with G = dL/dh_t:
 *   G      += conj(C_t) (x) dy_t                      readout of step t
 *   dC_t[n] = sum_p dy_t[p] conj(h_t[n,p])
 *   dx_t[p] = sum_n conj(B_t[n]) G[n,p] + Dskip dy_t[p]
 *   dB_t[n] = sum_p G[n,p] conj(x_t[p])
 *   dz_t    = conj(a_t) sum_{n,p} G[n,p] conj(h_{t-1}[n,p])   z_t = s_t A, a_t = exp(z_t)
 *   ddt_t   = sigmoid(dt_t) Re(dz_t conj(A)),  dA += s_t dz_t,
 *   dDskip += Re(sum_p dy_t[p] conj(x_t[p]))
 *   G       = conj(a_t) G                              back to h_{t-1}
 * starting from G = dL/dh_T (dhT, or zero) and ending with dh0 = G.  With
 * T = 0 no step is walked: dh0 = dhT, and dA, dDskip are empty sums (zero).
 * Inputs as oracle_forward_f64 plus dy [B,T,H,D] and dhT [B,H,N,D] (or NULL);
 * outputs dx, dB, dC (input layouts), ddt [B,T,H], dA [H] and dDskip [H]
 * (summed over batch and time; dDskip may be NULL), dh0 [B,H,N,D] (or NULL).
 */
int oracle_backward_f64(int64_t Bsz, int64_t T, int64_t H, int64_t D, int64_t N,
                        const double *x_re, const double *x_im,
                        const double *b_re, const double *b_im,
                        const double *c_re, const double *c_im,
                        const double *dt, const double *a_re, const double *a_im,
                        const double *dskip,
                        const double *h0_re, const double *h0_im,
                        const double *dy_re, const double *dy_im,
                        const double *dhT_re, const double *dhT_im,
                        double *dx_re, double *dx_im, double *db_re, double *db_im,
                        double *dc_re, double *dc_im, double *ddt,
                        double *da_re, double *da_im, double *dd,
                        double *dh0_re, double *dh0_im, int nthreads)
{
    if (Bsz <= 0 || T < 0 || H <= 0 || D <= 0 || N <= 0)
        return -1;
    if (!x_re || !x_im || !b_re || !b_im || !c_re || !c_im || !dt || !a_re || !a_im ||
        !dy_re || !dy_im || !dx_re || !dx_im || !db_re || !db_im || !dc_re || !dc_im ||
        !ddt || !da_re || !da_im)
        return -1;
    const int64_t ND = N * D;
    /* per (b, h) partial sums of dA and dDskip, reduced in a fixed order below */
    double *pa = (double *)calloc((size_t)(Bsz * H * 3), sizeof(double));
    if (!pa)
        return -1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t bh = 0; bh < Bsz * H; ++bh) {
        int64_t b = bh / H, h = bh % H;
        /* states h_{-1} .. h_{T-1}, then the running gradient */
        double complex *hs = (double complex *)malloc(sizeof(double complex) * (size_t)((T + 1) * ND));
        double complex *G = (double complex *)malloc(sizeof(double complex) * (size_t)ND);
        if (!hs || !G) {
            free(hs);
            free(G);
            failed |= 1;
            continue;
        }
        double complex A = a_re[h] + a_im[h] * I;
        double d = dskip ? dskip[h] : 0.0;
        for (int64_t k = 0; k < ND; ++k)
            hs[k] = (h0_re && h0_im) ? h0_re[bh * ND + k] + h0_im[bh * ND + k] * I : 0.0;
        /* forward, keeping every state */
        for (int64_t t = 0; t < T; ++t) {
            int64_t row = (b * T + t) * H + h;
            double complex a = cexp(softplus(dt[row]) * A);
            const double complex *hp = hs + t * ND;
            double complex *hn = hs + (t + 1) * ND;
            for (int64_t n = 0; n < N; ++n) {
                double complex bn = b_re[row * N + n] + b_im[row * N + n] * I;
                for (int64_t p = 0; p < D; ++p)
                    hn[n * D + p] = a * hp[n * D + p] +
                                    bn * (x_re[row * D + p] + x_im[row * D + p] * I);
            }
        }
        /* backward */
        for (int64_t k = 0; k < ND; ++k)
            G[k] = (dhT_re && dhT_im) ? dhT_re[bh * ND + k] + dhT_im[bh * ND + k] * I : 0.0;
        double complex dA = 0.0;
        double dD = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            int64_t row = (b * T + t) * H + h;
            double s = softplus(dt[row]);
            double complex a = cexp(s * A);
            const double complex *ht = hs + (t + 1) * ND, *hp = hs + t * ND;
            for (int64_t n = 0; n < N; ++n) {
                double complex cn = c_re[row * N + n] + c_im[row * N + n] * I;
                for (int64_t p = 0; p < D; ++p)
                    G[n * D + p] += conj(cn) * (dy_re[row * D + p] + dy_im[row * D + p] * I);
            }
            for (int64_t n = 0; n < N; ++n) {
                double complex acc = 0.0;
                for (int64_t p = 0; p < D; ++p)
                    acc += (dy_re[row * D + p] + dy_im[row * D + p] * I) * conj(ht[n * D + p]);
                dc_re[row * N + n] = creal(acc);
                dc_im[row * N + n] = cimag(acc);
            }
            for (int64_t p = 0; p < D; ++p) {
                double complex dyp = dy_re[row * D + p] + dy_im[row * D + p] * I;
                double complex xp = x_re[row * D + p] + x_im[row * D + p] * I;
                double complex acc = d * dyp;
                for (int64_t n = 0; n < N; ++n)
                    acc += conj(b_re[row * N + n] + b_im[row * N + n] * I) * G[n * D + p];
                dx_re[row * D + p] = creal(acc);
                dx_im[row * D + p] = cimag(acc);
                dD += creal(dyp * conj(xp));
            }
            for (int64_t n = 0; n < N; ++n) {
                double complex acc = 0.0;
                for (int64_t p = 0; p < D; ++p)
                    acc += G[n * D + p] * conj(x_re[row * D + p] + x_im[row * D + p] * I);
                db_re[row * N + n] = creal(acc);
                db_im[row * N + n] = cimag(acc);
            }
            double complex ga = 0.0;
            for (int64_t k = 0; k < ND; ++k)
                ga += G[k] * conj(hp[k]);
            double complex dz = conj(a) * ga;
            ddt[row] = creal(dz * conj(A)) / (1.0 + exp(-dt[row]));
            dA += s * dz;
            for (int64_t k = 0; k < ND; ++k)
                G[k] = conj(a) * G[k];
        }
        if (dh0_re && dh0_im)
            for (int64_t k = 0; k < ND; ++k) {
                dh0_re[bh * ND + k] = creal(G[k]);
                dh0_im[bh * ND + k] = cimag(G[k]);
            }
        pa[3 * bh] = creal(dA);
        pa[3 * bh + 1] = cimag(dA);
        pa[3 * bh + 2] = dD;
        free(hs);
        free(G);
    }
    for (int64_t h = 0; h < H; ++h) {
        double sr = 0.0, si = 0.0, sd = 0.0;
        for (int64_t b = 0; b < Bsz; ++b) {
            sr += pa[3 * (b * H + h)];
            si += pa[3 * (b * H + h) + 1];
            sd += pa[3 * (b * H + h) + 2];
        }
        da_re[h] = sr;
        da_im[h] = si;
        if (dd)
            dd[h] = sd;
    }
    free(pa);
    return failed ? -1 : 0;
}

/*
 * The per-coordinate complex scan of the phase-state paper ("Complex Phase-State
 * Dynamics Reduce the Optimization Steps of Sequence Models", section 5.2,
 * eq. 2-3, and Algorithm 1):
 *   lambda_t = (1 + i phi_t) / (1 - i phi_t)    Cayley transform, |lambda| = 1
 *   alpha_t  = 1 / (1 + e^{-u_t})               selective gate in (0, 1)
 *   psi_t    = alpha_t lambda_t psi_{t-1} + b_t  every coordinate on its own
 * evaluated as the plain sequential recurrence (section 5.3's chunked scan is a
 * way of computing the same trajectory).  Layouts: phi, u [B,T,H,N] real,
 * b [B,T,H,N] complex (planar), psi0 [B,H,N] complex or NULL (zero); outputs
 * psi [B,T,H,N] (the state after each step) and psiT [B,H,N] (or NULL).
 */
int oracle_phase_scan_f64(int64_t Bsz, int64_t T, int64_t H, int64_t N,
                          const double *phi, const double *u,
                          const double *b_re, const double *b_im,
                          const double *psi0_re, const double *psi0_im,
                          double *psi_re, double *psi_im,
                          double *psiT_re, double *psiT_im, int nthreads)
{
    if (Bsz <= 0 || T < 0 || H <= 0 || N <= 0)
        return -1;
    if (!phi || !u || !b_re || !b_im || !psi_re || !psi_im)
        return -1;
    const int64_t HN = H * N;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (int64_t bk = 0; bk < Bsz * HN; ++bk) {
        int64_t b = bk / HN, k = bk % HN;
        double complex psi = (psi0_re && psi0_im) ? psi0_re[bk] + psi0_im[bk] * I : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            int64_t at = (b * T + t) * HN + k;
            double complex lambda = (1.0 + phi[at] * I) / (1.0 - phi[at] * I);
            double alpha = 1.0 / (1.0 + exp(-u[at]));
            psi = alpha * lambda * psi + (b_re[at] + b_im[at] * I);
            psi_re[at] = creal(psi);
            psi_im[at] = cimag(psi);
        }
        if (psiT_re && psiT_im) {
            psiT_re[bk] = creal(psi);
            psiT_im[bk] = cimag(psi);
        }
    }
    return 0;
}

/*
 * Causal Born attention of the phase-state paper ("Complex Phase-State Dynamics
 * Reduce the Optimization Steps of Sequence Models", section 5.5, eq. 5, and
 * Appendix A, Algorithm 3), per (batch, head):
 *   s_ij  = |<q_i|k_j>|^2 / (D tau_i)  for j <= i,   <q|k> = sum_d conj(q_d) k_d
 *   psi_i = (sum_{j<=i} s_ij v_j) / (sum_{j<=i} s_ij)
 * computed row by row exactly as written: every overlap, its squared modulus,
 * the weighted sum and the normalising sum, in fp64.  A row whose scores are
 * all zero (0/0) is returned as zero.  Layouts: q, k, v [B,T,H,D] complex
 * (planar); tau [B,T,H] or NULL (1); out [B,T,H,D].
 */
static void born_row(int64_t T, int64_t H, int64_t D, int64_t b, int64_t h, int64_t i,
                     const double *q_re, const double *q_im, const double *k_re,
                     const double *k_im, const double *v_re, const double *v_im,
                     const double *tau, double *o_re, double *o_im)
{
    const int64_t qi = ((b * T + i) * H + h) * D;
    const double t = tau ? tau[(b * T + i) * H + h] : 1.0;
    double complex *num = calloc((size_t)D, sizeof(double complex));
    double den = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
        const int64_t kj = ((b * T + j) * H + h) * D;
        double complex overlap = 0.0;
        for (int64_t d = 0; d < D; ++d)
            overlap += conj(q_re[qi + d] + q_im[qi + d] * I) * (k_re[kj + d] + k_im[kj + d] * I);
        const double mod = cabs(overlap);
        const double sij = mod * mod / ((double)D * t);
        for (int64_t d = 0; d < D; ++d)
            num[d] += sij * (v_re[kj + d] + v_im[kj + d] * I);
        den += sij;
    }
    for (int64_t d = 0; d < D; ++d) {
        const double complex o = den != 0.0 ? num[d] / den : 0.0;
        o_re[d] = creal(o);
        o_im[d] = cimag(o);
    }
    free(num);
}

int oracle_born_attention_f64(int64_t Bsz, int64_t T, int64_t H, int64_t D,
                              const double *q_re, const double *q_im,
                              const double *k_re, const double *k_im,
                              const double *v_re, const double *v_im,
                              const double *tau, double *out_re, double *out_im, int nthreads)
{
    if (Bsz <= 0 || T < 0 || H <= 0 || D <= 0)
        return -1;
    if (!q_re || !q_im || !k_re || !k_im || !v_re || !v_im || !out_re || !out_im)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < Bsz * T * H; ++r) {
        const int64_t b = r / (T * H), i = (r / H) % T, h = r % H;
        const int64_t at = r * D;  /* (b, i, h) row of [B,T,H,D] */
        born_row(T, H, D, b, h, i, q_re, q_im, k_re, k_im, v_re, v_im, tau, out_re + at, out_im + at);
    }
    return 0;
}

/*
 * The same output for a list of rows only: rows[3m..3m+2] = (b, i, h); the row's
 * D outputs go to out_re/out_im[m * D ...].  For checking sampled rows of large
 * problems.
 */
int oracle_born_attention_rows_f64(int64_t Bsz, int64_t T, int64_t H, int64_t D,
                                   const double *q_re, const double *q_im,
                                   const double *k_re, const double *k_im,
                                   const double *v_re, const double *v_im,
                                   const double *tau, int64_t nrows, const int64_t *rows,
                                   double *out_re, double *out_im, int nthreads)
{
    if (Bsz <= 0 || T <= 0 || H <= 0 || D <= 0 || nrows < 0 || !rows)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|| : failed)
    for (int64_t m = 0; m < nrows; ++m) {
        const int64_t b = rows[3 * m], i = rows[3 * m + 1], h = rows[3 * m + 2];
        if (b < 0 || b >= Bsz || i < 0 || i >= T || h < 0 || h >= H) {
            failed = 1;
            continue;
        }
        born_row(T, H, D, b, h, i, q_re, q_im, k_re, k_im, v_re, v_im, tau, out_re + m * D,
                 out_im + m * D);
    }
    return failed ? -1 : 0;
}

/* Threads OpenMP would use for a parallel region (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
