/*
 * oracle.c -- plain, slow, fp64 CPU reference for the gated N-D linear
 * convolution of HyenaND.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the GPU library, and it imports nothing from it.
 *
 * Sources (the reader has the pages, cited by title and section):
 *   [EXPL]  "Native multi-dimensional subquadratic operators via input-dependent
 *           long convolutions", explainer on autognosis.neco-logic.com,
 *           section "HyenaND: native-space implicit global kernel",
 *           sub-sections "Input dependence" (the output equation for y[i])
 *           and "Implementation" (FFT -> pointwise product -> inverse FFT).
 *   [SUMM]  "Native Multi-Dimensional Subquadratic Operators via Input
 *           Dependent Long Convolutions", gist.science summary (fr/pt),
 *           section "Methodology", item "Boundary handling": non-circular
 *           convolution by zero-padding every axis to twice the grid.
 *
 * What is computed, for every batch entry b and channel c:
 *
 *     y[b,c,i] = sum_{j in G} phi_c(x[b,c,j]) * x[b,c,j] * K_c[i - j],  i in G,
 *
 * G = [0,n_0) x ... x [0,n_{d-1}), phi_c(v) = 1 / (1 + exp(-(alpha_c v + beta_c)))
 * (the content gate of [EXPL], read as a per-channel logistic of an affine map),
 * K_c stored on the offsets [-(n_a-1), n_a-1] of every axis, offset 0 at index
 * n_a-1, depthwise (one kernel per channel, shared over b).  Outside G the
 * signal is zero (non-circular boundary of [SUMM]).
 *
 * Two independent routes:
 *   O1  oracle_direct / oracle_direct_points: the sum above, written out.
 *   O2  oracle_fftconv_pairs: explicit zero padding to N_a = 2 n_a, textbook
 *       radix-2 complex FFT (bit reversal + butterflies, fp64 twiddles from
 *       cos/sin), row-column over the axes, product, inverse, crop.
 * The circular mode of [SUMM] (periodic grids, no padding) has the same two
 * routes: oracle_direct_circ and oracle_fftconv_circ_pairs.
 * And the same two routes for the backward (the gradients of the input, the
 * gate parameters and the kernel; see the backward section below):
 *   O1  oracle_bwd_direct / oracle_bwd_direct_points,  O2  oracle_bwd_fft.
 *
 * Layouts: x  [B][C][n_0..n_{d-1}] fp32 (bf16 inputs are widened exactly by the
 * caller), K [C][2n_0-1 .. 2n_{d-1}-1] fp32, alpha/beta [C] fp32, outputs fp64.
 * Innermost axis last.  Every function returns 0 on success, 1 on a bad
 * argument, 2 when memory runs out.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_ENOMEM 2

/* Problem geometry, with leading axes of size 1 when d < 3. */
typedef struct {
    int d;
    int64_t n[3];    /* grid extent per axis                      */
    int64_t ke[3];   /* kernel extent 2n-1 per axis                */
    int64_t N[3];    /* padded FFT length: 2n (1 for absent axes)  */
    int64_t L;       /* voxels per (b,c)                           */
    int64_t KL;      /* kernel values per channel                  */
    int64_t NL;      /* padded voxels                              */
} geom_t;

static int geom_init(geom_t *g, int d, const int64_t *dims)
{
    if (d < 1 || d > 3 || !dims) return ORC_EINVAL;
    g->d = d;
    for (int a = 0; a < 3; ++a) { g->n[a] = 1; g->ke[a] = 1; g->N[a] = 1; }
    for (int a = 0; a < d; ++a) {
        int64_t n = dims[a];
        if (n < 1) return ORC_EINVAL;
        int ax = 3 - d + a;
        g->n[ax] = n;
        g->ke[ax] = 2 * n - 1;
        g->N[ax] = 2 * n;
    }
    g->L = g->n[0] * g->n[1] * g->n[2];
    g->KL = g->ke[0] * g->ke[1] * g->ke[2];
    g->NL = g->N[0] * g->N[1] * g->N[2];
    return ORC_OK;
}

/* The content gate of [EXPL]: u = phi(x) * x with phi the logistic of alpha*x+beta. */
static inline double gate(double x, double alpha, double beta)
{
    return x / (1.0 + exp(-(alpha * x + beta)));
}

int oracle_gate(const float *x, int64_t count, double alpha, double beta, double *u)
{
    if (!x || !u || count < 0) return ORC_EINVAL;
    for (int64_t i = 0; i < count; ++i) u[i] = gate((double)x[i], alpha, beta);
    return ORC_OK;
}

/* K_c[delta] with delta_a in [-(n_a-1), n_a-1]; stored with offset 0 at n_a-1. */
static inline double kval(const float *Kc, const geom_t *g, int64_t d0, int64_t d1, int64_t d2)
{
    int64_t i0 = d0 + g->n[0] - 1, i1 = d1 + g->n[1] - 1, i2 = d2 + g->n[2] - 1;
    return (double)Kc[(i0 * g->ke[1] + i1) * g->ke[2] + i2];
}

/* O1 for one output voxel i of one (b,c): the sum of [EXPL] written out. */
static double direct_one(const double *u, const float *Kc, const geom_t *g,
                         int64_t i0, int64_t i1, int64_t i2)
{
    double acc = 0.0;
    for (int64_t j0 = 0; j0 < g->n[0]; ++j0)
        for (int64_t j1 = 0; j1 < g->n[1]; ++j1) {
            const double *urow = u + (j0 * g->n[1] + j1) * g->n[2];
            for (int64_t j2 = 0; j2 < g->n[2]; ++j2)
                acc += urow[j2] * kval(Kc, g, i0 - j0, i1 - j1, i2 - j2);
        }
    return acc;
}

/* O1 over every output of every (b,c).  y is [B][C][L] fp64. */
int oracle_direct(const float *x, const float *alpha, const float *beta, const float *K,
                  double *y, int B, int C, int d, const int64_t *dims)
{
    geom_t g;
    if (!x || !alpha || !beta || !K || !y || B < 0 || C < 0) return ORC_EINVAL;
    if (geom_init(&g, d, dims)) return ORC_EINVAL;
    double *u = (double *)malloc(sizeof(double) * (size_t)(g.L ? g.L : 1));
    if (!u) return ORC_ENOMEM;
    for (int b = 0; b < B; ++b)
        for (int c = 0; c < C; ++c) {
            const int64_t p = (int64_t)b * C + c;
            const float *xs = x + p * g.L;
            for (int64_t j = 0; j < g.L; ++j) u[j] = gate((double)xs[j], alpha[c], beta[c]);
            const float *Kc = K + (int64_t)c * g.KL;
            double *ys = y + p * g.L;
#pragma omp parallel for schedule(static)
            for (int64_t i = 0; i < g.L; ++i) {
                int64_t i2 = i % g.n[2], i1 = (i / g.n[2]) % g.n[1], i0 = i / (g.n[1] * g.n[2]);
                ys[i] = direct_one(u, Kc, &g, i0, i1, i2);
            }
        }
    free(u);
    return ORC_OK;
}

/*
 * O1 at selected outputs.  pts is [npts][2+d] int64: (b, c, i_0 .. i_{d-1}).
 * Points that share (b,c) consecutively share one gate evaluation.
 */
int oracle_direct_points(const float *x, const float *alpha, const float *beta, const float *K,
                         int B, int C, int d, const int64_t *dims,
                         int64_t npts, const int64_t *pts, double *out)
{
    geom_t g;
    if (!x || !alpha || !beta || !K || !pts || !out || npts < 0) return ORC_EINVAL;
    if (geom_init(&g, d, dims)) return ORC_EINVAL;
    const int w = 2 + d;
    for (int64_t q = 0; q < npts; ++q) {
        const int64_t *pt = pts + q * w;
        if (pt[0] < 0 || pt[0] >= B || pt[1] < 0 || pt[1] >= C) return ORC_EINVAL;
        for (int a = 0; a < d; ++a)
            if (pt[2 + a] < 0 || pt[2 + a] >= dims[a]) return ORC_EINVAL;
    }
    double *u = (double *)malloc(sizeof(double) * (size_t)(g.L ? g.L : 1));
    if (!u) return ORC_ENOMEM;
    int64_t cur = -1;
    for (int64_t q = 0; q < npts; ++q) {
        const int64_t *pt = pts + q * w;
        const int64_t b = pt[0], c = pt[1], p = b * C + c;
        if (p != cur) {
            const float *xs = x + p * g.L;
            const double al = alpha[c], be = beta[c];
#pragma omp parallel for schedule(static)
            for (int64_t j = 0; j < g.L; ++j) u[j] = gate((double)xs[j], al, be);
            cur = p;
        }
        int64_t ii[3] = {0, 0, 0};
        for (int a = 0; a < d; ++a) ii[3 - d + a] = pt[2 + a];
        const float *Kc = K + c * g.KL;
        double acc = 0.0;
#pragma omp parallel for reduction(+ : acc) schedule(static)
        for (int64_t j0 = 0; j0 < g.n[0]; ++j0)
            for (int64_t j1 = 0; j1 < g.n[1]; ++j1) {
                const double *urow = u + (j0 * g.n[1] + j1) * g.n[2];
                for (int64_t j2 = 0; j2 < g.n[2]; ++j2)
                    acc += urow[j2] * kval(Kc, &g, ii[0] - j0, ii[1] - j1, ii[2] - j2);
            }
        out[q] = acc;
    }
    free(u);
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* O2: textbook radix-2 FFT, fp64.                                            */
/* ------------------------------------------------------------------------- */

static int is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

/*
 * In-place iterative radix-2 Cooley-Tukey transform of one line of length N:
 *   X[k] = sum_t x[t] exp(sign * 2 pi i t k / N),   sign = -1 forward, +1 inverse.
 * The inverse is unnormalised.  ct[t] = cos(2 pi t / N), st[t] = sin(2 pi t / N)
 * for t in [0, N/2).
 */
static void fft_line(double *re, double *im, int64_t N, int sign, const double *ct, const double *st)
{
    for (int64_t i = 1, j = 0; i < N; ++i) {
        int64_t bit = N >> 1;
        for (; j & bit; bit >>= 1) j ^= bit;
        j ^= bit;
        if (i < j) {
            double t = re[i]; re[i] = re[j]; re[j] = t;
            t = im[i]; im[i] = im[j]; im[j] = t;
        }
    }
    for (int64_t len = 2; len <= N; len <<= 1) {
        const int64_t half = len >> 1, step = N / len;
        for (int64_t s = 0; s < N; s += len)
            for (int64_t k = 0; k < half; ++k) {
                const double wr = ct[k * step], wi = sign * st[k * step];
                const int64_t a = s + k, b = a + half;
                const double tr = re[b] * wr - im[b] * wi;
                const double ti = re[b] * wi + im[b] * wr;
                re[b] = re[a] - tr; im[b] = im[a] - ti;
                re[a] += tr;        im[a] += ti;
            }
    }
}

/* N-D transform of an array of shape N[0] x N[1] x N[2] (row-major), axis by axis. */
static int fft_nd(double *re, double *im, const int64_t *N, int sign)
{
    for (int ax = 0; ax < 3; ++ax) {
        const int64_t n = N[ax];
        if (n == 1) continue;
        if (!is_pow2(n)) return ORC_EINVAL;
        double *ct = (double *)malloc(sizeof(double) * (size_t)(n / 2));
        double *st = (double *)malloc(sizeof(double) * (size_t)(n / 2));
        if (!ct || !st) { free(ct); free(st); return ORC_ENOMEM; }
        for (int64_t t = 0; t < n / 2; ++t) {
            ct[t] = cos(2.0 * M_PI * (double)t / (double)n);
            st[t] = sin(2.0 * M_PI * (double)t / (double)n);
        }
        int64_t inner = 1, outer = 1;
        for (int a = ax + 1; a < 3; ++a) inner *= N[a];
        for (int a = 0; a < ax; ++a) outer *= N[a];
        const int64_t lines = outer * inner;
        int fail = 0;
#pragma omp parallel
        {
            double *lr = (double *)malloc(sizeof(double) * (size_t)n);
            double *li = (double *)malloc(sizeof(double) * (size_t)n);
            if (!lr || !li) {
#pragma omp atomic write
                fail = 1;
            } else {
#pragma omp for schedule(static)
                for (int64_t l = 0; l < lines; ++l) {
                    const int64_t o = l / inner, in = l % inner;
                    const int64_t base = o * n * inner + in;
                    for (int64_t t = 0; t < n; ++t) { lr[t] = re[base + t * inner]; li[t] = im[base + t * inner]; }
                    fft_line(lr, li, n, sign, ct, st);
                    for (int64_t t = 0; t < n; ++t) { re[base + t * inner] = lr[t]; im[base + t * inner] = li[t]; }
                }
            }
            free(lr); free(li);
        }
        free(ct); free(st);
        if (fail) return ORC_ENOMEM;
    }
    return ORC_OK;
}

/*
 * Wrap placement of K_c into the padded grid: offset delta goes to index
 * delta mod N_a on every axis (the non-circular padding of [SUMM] makes the
 * slot N_a/2 = n_a stay zero).  re/im are zeroed by the caller.
 */
static void wrap_place(const float *Kc, const geom_t *g, double *re)
{
    for (int64_t a0 = 0; a0 < g->ke[0]; ++a0)
        for (int64_t a1 = 0; a1 < g->ke[1]; ++a1)
            for (int64_t a2 = 0; a2 < g->ke[2]; ++a2) {
                int64_t d0 = a0 - (g->n[0] - 1), d1 = a1 - (g->n[1] - 1), d2 = a2 - (g->n[2] - 1);
                int64_t m0 = (d0 % g->N[0] + g->N[0]) % g->N[0];
                int64_t m1 = (d1 % g->N[1] + g->N[1]) % g->N[1];
                int64_t m2 = (d2 % g->N[2] + g->N[2]) % g->N[2];
                re[(m0 * g->N[1] + m1) * g->N[2] + m2] = (double)Kc[(a0 * g->ke[1] + a1) * g->ke[2] + a2];
            }
}

/*
 * The full (true, unscaled) DFT of the wrap-placed kernel of every channel:
 *   Khat_c[k] = sum_m Ktilde_c[m] exp(-2 pi i sum_a k_a m_a / N_a)
 * re/im are [C][N_0 .. N_{d-1}] fp64.
 */
int oracle_kernel_spectrum(const float *K, int C, int d, const int64_t *dims, double *re, double *im)
{
    geom_t g;
    if (!K || !re || !im || C < 0) return ORC_EINVAL;
    if (geom_init(&g, d, dims)) return ORC_EINVAL;
    for (int c = 0; c < C; ++c) {
        double *r = re + (int64_t)c * g.NL, *i = im + (int64_t)c * g.NL;
        memset(r, 0, sizeof(double) * (size_t)g.NL);
        memset(i, 0, sizeof(double) * (size_t)g.NL);
        wrap_place(K + (int64_t)c * g.KL, &g, r);
        int rc = fft_nd(r, i, g.N, -1);
        if (rc) return rc;
    }
    return ORC_OK;
}

/*
 * O2 for a list of (b,c) pairs (pair index p = b*C + c).  y_out is [npairs][L].
 * Steps ([EXPL] "Implementation", [SUMM] "Boundary handling"): gate, zero pad
 * to N_a = 2 n_a, forward FFT of the padded signal and of the wrap-placed
 * kernel, pointwise product, inverse FFT, divide by prod N_a, keep [0, n_a).
 */
int oracle_fftconv_pairs(const float *x, const float *alpha, const float *beta, const float *K,
                         int B, int C, int d, const int64_t *dims,
                         int64_t npairs, const int64_t *pairs, double *y_out)
{
    geom_t g;
    if (!x || !alpha || !beta || !K || !pairs || !y_out || npairs < 0) return ORC_EINVAL;
    if (geom_init(&g, d, dims)) return ORC_EINVAL;
    for (int a = 0; a < 3; ++a)
        if (!is_pow2(g.N[a])) return ORC_EINVAL;
    for (int64_t q = 0; q < npairs; ++q)
        if (pairs[q] < 0 || pairs[q] >= (int64_t)B * C) return ORC_EINVAL;

    const size_t bytes = sizeof(double) * (size_t)g.NL;
    double *ur = (double *)malloc(bytes), *ui = (double *)malloc(bytes);
    double *kr = (double *)malloc(bytes), *ki = (double *)malloc(bytes);
    if (!ur || !ui || !kr || !ki) { free(ur); free(ui); free(kr); free(ki); return ORC_ENOMEM; }
    int64_t kc_cur = -1;
    int rc = ORC_OK;
    for (int64_t q = 0; q < npairs && rc == ORC_OK; ++q) {
        const int64_t p = pairs[q], c = p % C;
        if (c != kc_cur) {
            memset(kr, 0, bytes);
            memset(ki, 0, bytes);
            wrap_place(K + c * g.KL, &g, kr);
            rc = fft_nd(kr, ki, g.N, -1);
            if (rc) break;
            kc_cur = c;
        }
        memset(ur, 0, bytes);
        memset(ui, 0, bytes);
        const float *xs = x + p * g.L;
        for (int64_t j0 = 0; j0 < g.n[0]; ++j0)
            for (int64_t j1 = 0; j1 < g.n[1]; ++j1)
                for (int64_t j2 = 0; j2 < g.n[2]; ++j2)
                    ur[(j0 * g.N[1] + j1) * g.N[2] + j2] =
                        gate((double)xs[(j0 * g.n[1] + j1) * g.n[2] + j2], alpha[c], beta[c]);
        rc = fft_nd(ur, ui, g.N, -1);
        if (rc) break;
        for (int64_t m = 0; m < g.NL; ++m) {
            const double a = ur[m], b = ui[m];
            ur[m] = a * kr[m] - b * ki[m];
            ui[m] = a * ki[m] + b * kr[m];
        }
        rc = fft_nd(ur, ui, g.N, +1);
        if (rc) break;
        const double scale = 1.0 / (double)g.NL;
        double *ys = y_out + q * g.L;
        for (int64_t j0 = 0; j0 < g.n[0]; ++j0)
            for (int64_t j1 = 0; j1 < g.n[1]; ++j1)
                for (int64_t j2 = 0; j2 < g.n[2]; ++j2)
                    ys[(j0 * g.n[1] + j1) * g.n[2] + j2] = ur[(j0 * g.N[1] + j1) * g.N[2] + j2] * scale;
    }
    free(ur); free(ui); free(kr); free(ki);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* Circular mode ([SUMM] "Boundary handling": circular convolutions for       */
/* periodic physical systems, next to the zero-padded non-circular ones).     */
/* ------------------------------------------------------------------------- */
/*
 * On a periodic grid the kernel lives on the offsets modulo n_a: K_c is stored
 * [C][n_0]..[n_{d-1}] with index m_a = delta_a mod n_a (offset 0 at index 0),
 * and
 *     y[b,c,i] = sum_{j in G} u[b,c,j] K_c[(i - j) mod n],   u = phi(x) x.
 * The FFT route needs no padding: N_a = n_a, y = IFFT(FFT(u) FFT(K)) / prod n.
 */

/* O1, circular: every output of every (b,c). */
int oracle_direct_circ(const float *x, const float *alpha, const float *beta, const float *K,
                       double *y, int B, int C, int d, const int64_t *dims)
{
    geom_t g;
    if (!x || !alpha || !beta || !K || !y || B < 0 || C < 0) return ORC_EINVAL;
    if (geom_init(&g, d, dims)) return ORC_EINVAL;
    double *u = (double *)malloc(sizeof(double) * (size_t)(g.L ? g.L : 1));
    if (!u) return ORC_ENOMEM;
    for (int b = 0; b < B; ++b)
        for (int c = 0; c < C; ++c) {
            const int64_t p = (int64_t)b * C + c;
            const float *xs = x + p * g.L;
            for (int64_t j = 0; j < g.L; ++j) u[j] = gate((double)xs[j], alpha[c], beta[c]);
            const float *Kc = K + (int64_t)c * g.L;
            double *ys = y + p * g.L;
#pragma omp parallel for schedule(static)
            for (int64_t i = 0; i < g.L; ++i) {
                const int64_t i2 = i % g.n[2], i1 = (i / g.n[2]) % g.n[1], i0 = i / (g.n[1] * g.n[2]);
                double acc = 0.0;
                for (int64_t j0 = 0; j0 < g.n[0]; ++j0)
                    for (int64_t j1 = 0; j1 < g.n[1]; ++j1)
                        for (int64_t j2 = 0; j2 < g.n[2]; ++j2) {
                            const int64_t m0 = ((i0 - j0) % g.n[0] + g.n[0]) % g.n[0];
                            const int64_t m1 = ((i1 - j1) % g.n[1] + g.n[1]) % g.n[1];
                            const int64_t m2 = ((i2 - j2) % g.n[2] + g.n[2]) % g.n[2];
                            acc += u[(j0 * g.n[1] + j1) * g.n[2] + j2] * (double)Kc[(m0 * g.n[1] + m1) * g.n[2] + m2];
                        }
                ys[i] = acc;
            }
        }
    free(u);
    return ORC_OK;
}

/* O2, circular, for the listed pairs: FFT of size n on every axis, product, inverse, / prod n. */
int oracle_fftconv_circ_pairs(const float *x, const float *alpha, const float *beta, const float *K,
                              int B, int C, int d, const int64_t *dims,
                              int64_t npairs, const int64_t *pairs, double *y_out)
{
    geom_t g;
    if (!x || !alpha || !beta || !K || !pairs || !y_out || npairs < 0) return ORC_EINVAL;
    if (geom_init(&g, d, dims)) return ORC_EINVAL;
    for (int a = 0; a < 3; ++a)
        if (!is_pow2(g.n[a])) return ORC_EINVAL;
    for (int64_t q = 0; q < npairs; ++q)
        if (pairs[q] < 0 || pairs[q] >= (int64_t)B * C) return ORC_EINVAL;
    const size_t bytes = sizeof(double) * (size_t)g.L;
    double *ur = (double *)malloc(bytes), *ui = (double *)malloc(bytes);
    double *kr = (double *)malloc(bytes), *ki = (double *)malloc(bytes);
    if (!ur || !ui || !kr || !ki) { free(ur); free(ui); free(kr); free(ki); return ORC_ENOMEM; }
    int64_t kc_cur = -1;
    int rc = ORC_OK;
    for (int64_t q = 0; q < npairs && rc == ORC_OK; ++q) {
        const int64_t p = pairs[q], c = p % C;
        if (c != kc_cur) {
            for (int64_t m = 0; m < g.L; ++m) { kr[m] = (double)K[c * g.L + m]; ki[m] = 0.0; }
            if ((rc = fft_nd(kr, ki, g.n, -1))) break;
            kc_cur = c;
        }
        const float *xs = x + p * g.L;
        for (int64_t j = 0; j < g.L; ++j) { ur[j] = gate((double)xs[j], alpha[c], beta[c]); ui[j] = 0.0; }
        if ((rc = fft_nd(ur, ui, g.n, -1))) break;
        for (int64_t m = 0; m < g.L; ++m) {
            const double a = ur[m], b = ui[m];
            ur[m] = a * kr[m] - b * ki[m];
            ui[m] = a * ki[m] + b * kr[m];
        }
        if ((rc = fft_nd(ur, ui, g.n, +1))) break;
        for (int64_t j = 0; j < g.L; ++j) y_out[q * g.L + j] = ur[j] / (double)g.L;
    }
    free(ur); free(ui); free(kr); free(ki);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* Backward: the vector-Jacobian product of the output equation.             */
/* ------------------------------------------------------------------------- */
/*
 * [EXPL] section "Implementation and operation patterns", item "Concrete
 * implementation pattern (PyTorch)": the layer is an autograd function whose
 * backward recomputes the forward FFTs from the saved input and kernel
 * parameters (gradient checkpointing) and returns the gradients of the input
 * and of the kernel parameters.  With dy = dLoss/dy, the chain rule through
 * y[i] = sum_j u[j] K[i-j] and u = x s, s = sigma(alpha x + beta), gives
 *
 *   du[j]     = sum_{i in G} dy[i] K[i-j]                  (correlation with K)
 *   dx[j]     = du[j] (s + alpha x s (1-s))
 *   dalpha_c  = sum_{b,j} du[j] x^2 s (1-s)
 *   dbeta_c   = sum_{b,j} du[j] x s (1-s)
 *   dK_c[dl]  = sum_b sum_{j in G, j+dl in G} dy[j+dl] u[j]   (dl on K's offsets)
 *
 * Layouts as above; dy like x; dx fp64 [B][C][L]; dalpha, dbeta fp64 [C];
 * dK fp64 [C][KL].
 */

static inline double sigm(double v) { return 1.0 / (1.0 + exp(-v)); }

/* dx, and this pair's terms of dalpha and dbeta, from du. */
static void gate_vjp(const float *xs, const double *du, int64_t L, double alpha, double beta,
                     double *dx, double *da, double *db)
{
    double sa = 0.0, sb = 0.0;
    for (int64_t j = 0; j < L; ++j) {
        const double x = (double)xs[j], s = sigm(alpha * x + beta), ds = s * (1.0 - s);
        dx[j] = du[j] * (s + alpha * x * ds);
        sa += du[j] * x * x * ds;
        sb += du[j] * x * ds;
    }
    *da += sa;
    *db += sb;
}

/* The gate's vector-Jacobian product on its own, for an output gradient du of
 * u = phi(x) x over `count` elements: dx, and the sums of the dalpha and dbeta
 * terms (sums[0], sums[1]). */
int oracle_gate_vjp(const float *x, const double *du, int64_t count, double alpha, double beta, double *dx,
                    double *sums)
{
    if (!x || !du || !dx || !sums || count < 0) return ORC_EINVAL;
    sums[0] = sums[1] = 0.0;
    gate_vjp(x, du, count, alpha, beta, dx, &sums[0], &sums[1]);
    return ORC_OK;
}

/* O1 of the backward: every sum above written out. */
int oracle_bwd_direct(const float *x, const float *alpha, const float *beta, const float *K, const float *dy,
                      int B, int C, int d, const int64_t *dims,
                      double *dx, double *dalpha, double *dbeta, double *dK)
{
    geom_t g;
    if (!x || !alpha || !beta || !K || !dy || !dx || !dalpha || !dbeta || !dK || B < 0 || C < 0) return ORC_EINVAL;
    if (geom_init(&g, d, dims)) return ORC_EINVAL;
    const size_t n = (size_t)(g.L ? g.L : 1);
    double *u = (double *)malloc(sizeof(double) * n), *du = (double *)malloc(sizeof(double) * n);
    if (!u || !du) { free(u); free(du); return ORC_ENOMEM; }
    for (int c = 0; c < C; ++c) {
        const float *Kc = K + (int64_t)c * g.KL;
        double *dKc = dK + (int64_t)c * g.KL;
        for (int64_t m = 0; m < g.KL; ++m) dKc[m] = 0.0;
        dalpha[c] = 0.0;
        dbeta[c] = 0.0;
        for (int b = 0; b < B; ++b) {
            const int64_t p = (int64_t)b * C + c;
            const float *xs = x + p * g.L, *dys = dy + p * g.L;
            for (int64_t j = 0; j < g.L; ++j) u[j] = gate((double)xs[j], alpha[c], beta[c]);
#pragma omp parallel for schedule(static)
            for (int64_t j = 0; j < g.L; ++j) {
                const int64_t j2 = j % g.n[2], j1 = (j / g.n[2]) % g.n[1], j0 = j / (g.n[1] * g.n[2]);
                double acc = 0.0;
                for (int64_t i = 0; i < g.L; ++i) {
                    const int64_t i2 = i % g.n[2], i1 = (i / g.n[2]) % g.n[1], i0 = i / (g.n[1] * g.n[2]);
                    acc += (double)dys[i] * kval(Kc, &g, i0 - j0, i1 - j1, i2 - j2);
                }
                du[j] = acc;
            }
            gate_vjp(xs, du, g.L, alpha[c], beta[c], dx + p * g.L, &dalpha[c], &dbeta[c]);
#pragma omp parallel for schedule(static)
            for (int64_t m = 0; m < g.KL; ++m) {
                const int64_t e2 = m % g.ke[2], e1 = (m / g.ke[2]) % g.ke[1], e0 = m / (g.ke[1] * g.ke[2]);
                const int64_t l0 = e0 - (g.n[0] - 1), l1 = e1 - (g.n[1] - 1), l2 = e2 - (g.n[2] - 1);
                double acc = 0.0;
                for (int64_t j0 = 0; j0 < g.n[0]; ++j0) {
                    const int64_t i0 = j0 + l0;
                    if (i0 < 0 || i0 >= g.n[0]) continue;
                    for (int64_t j1 = 0; j1 < g.n[1]; ++j1) {
                        const int64_t i1 = j1 + l1;
                        if (i1 < 0 || i1 >= g.n[1]) continue;
                        for (int64_t j2 = 0; j2 < g.n[2]; ++j2) {
                            const int64_t i2 = j2 + l2;
                            if (i2 < 0 || i2 >= g.n[2]) continue;
                            acc += (double)dys[(i0 * g.n[1] + i1) * g.n[2] + i2] * u[(j0 * g.n[1] + j1) * g.n[2] + j2];
                        }
                    }
                }
                dKc[m] += acc;
            }
        }
    }
    free(u);
    free(du);
    return ORC_OK;
}

/*
 * O1 of the backward at chosen points.  xpts [nx][2+d] (b, c, j..) -> dx_out;
 * kpts [nk][1+d] (c, e..) with e the index into K's extents -> dK_out.
 */
int oracle_bwd_direct_points(const float *x, const float *alpha, const float *beta, const float *K,
                             const float *dy, int B, int C, int d, const int64_t *dims,
                             int64_t nx, const int64_t *xpts, double *dx_out,
                             int64_t nk, const int64_t *kpts, double *dK_out)
{
    geom_t g;
    if (!x || !alpha || !beta || !K || !dy || nx < 0 || nk < 0) return ORC_EINVAL;
    if ((nx && (!xpts || !dx_out)) || (nk && (!kpts || !dK_out))) return ORC_EINVAL;
    if (geom_init(&g, d, dims)) return ORC_EINVAL;
    for (int64_t q = 0; q < nx; ++q) {
        const int64_t *pt = xpts + q * (2 + d);
        if (pt[0] < 0 || pt[0] >= B || pt[1] < 0 || pt[1] >= C) return ORC_EINVAL;
        for (int a = 0; a < d; ++a)
            if (pt[2 + a] < 0 || pt[2 + a] >= dims[a]) return ORC_EINVAL;
    }
    for (int64_t q = 0; q < nk; ++q) {
        const int64_t *pt = kpts + q * (1 + d);
        if (pt[0] < 0 || pt[0] >= C) return ORC_EINVAL;
        for (int a = 0; a < d; ++a)
            if (pt[1 + a] < 0 || pt[1 + a] >= 2 * dims[a] - 1) return ORC_EINVAL;
    }
    for (int64_t q = 0; q < nx; ++q) {
        const int64_t *pt = xpts + q * (2 + d);
        const int64_t c = pt[1], p = pt[0] * C + c;
        int64_t jj[3] = {0, 0, 0};
        for (int a = 0; a < d; ++a) jj[3 - d + a] = pt[2 + a];
        const float *dys = dy + p * g.L, *Kc = K + c * g.KL;
        double du = 0.0;
#pragma omp parallel for reduction(+ : du) schedule(static)
        for (int64_t i0 = 0; i0 < g.n[0]; ++i0)
            for (int64_t i1 = 0; i1 < g.n[1]; ++i1)
                for (int64_t i2 = 0; i2 < g.n[2]; ++i2)
                    du += (double)dys[(i0 * g.n[1] + i1) * g.n[2] + i2] * kval(Kc, &g, i0 - jj[0], i1 - jj[1], i2 - jj[2]);
        const double xv = (double)x[p * g.L + (jj[0] * g.n[1] + jj[1]) * g.n[2] + jj[2]];
        const double s = sigm(alpha[c] * xv + beta[c]);
        dx_out[q] = du * (s + alpha[c] * xv * s * (1.0 - s));
    }
    for (int64_t q = 0; q < nk; ++q) {
        const int64_t *pt = kpts + q * (1 + d);
        const int64_t c = pt[0];
        int64_t l[3] = {0, 0, 0};
        for (int a = 0; a < d; ++a) l[3 - d + a] = pt[1 + a] - (dims[a] - 1);
        double acc = 0.0;
        for (int64_t b = 0; b < B; ++b) {
            const int64_t p = b * C + c;
            const float *xs = x + p * g.L, *dys = dy + p * g.L;
#pragma omp parallel for reduction(+ : acc) schedule(static)
            for (int64_t j0 = 0; j0 < g.n[0]; ++j0) {
                const int64_t i0 = j0 + l[0];
                if (i0 < 0 || i0 >= g.n[0]) continue;
                for (int64_t j1 = 0; j1 < g.n[1]; ++j1) {
                    const int64_t i1 = j1 + l[1];
                    if (i1 < 0 || i1 >= g.n[1]) continue;
                    for (int64_t j2 = 0; j2 < g.n[2]; ++j2) {
                        const int64_t i2 = j2 + l[2];
                        if (i2 < 0 || i2 >= g.n[2]) continue;
                        acc += (double)dys[(i0 * g.n[1] + i1) * g.n[2] + i2] *
                               gate((double)xs[(j0 * g.n[1] + j1) * g.n[2] + j2], alpha[c], beta[c]);
                    }
                }
            }
        }
        dK_out[q] = acc;
    }
    return ORC_OK;
}

/* Zero-padded copy of one (b,c) signal into the N-grid (re only; im zeroed). */
static void pad_into(const double *v, const geom_t *g, double *re, double *im)
{
    memset(re, 0, sizeof(double) * (size_t)g->NL);
    memset(im, 0, sizeof(double) * (size_t)g->NL);
    for (int64_t j0 = 0; j0 < g->n[0]; ++j0)
        for (int64_t j1 = 0; j1 < g->n[1]; ++j1)
            for (int64_t j2 = 0; j2 < g->n[2]; ++j2)
                re[(j0 * g->N[1] + j1) * g->N[2] + j2] = v[(j0 * g->n[1] + j1) * g->n[2] + j2];
}

/*
 * O2 of the backward for the listed channels (every batch entry of each):
 * zero padding to N = 2n, the textbook FFT of fft_nd, and
 *   du = crop(IFFT(FFT(pad dy) conj(FFT(wrap K)))) / prod N
 *   dK[dl] = IFFT(sum_b FFT(pad dy_b) conj(FFT(pad u_b)))[dl mod N] / prod N
 * (a correlation is a product with the conjugate spectrum; with N = 2n the
 * lags used never wrap).  Outputs: dx [nch][B][L], dalpha/dbeta [nch],
 * dK [nch][KL], in the order of `chans`.
 */
int oracle_bwd_fft(const float *x, const float *alpha, const float *beta, const float *K, const float *dy,
                   int B, int C, int d, const int64_t *dims, int64_t nch, const int64_t *chans,
                   double *dx, double *dalpha, double *dbeta, double *dK)
{
    geom_t g;
    if (!x || !alpha || !beta || !K || !dy || !chans || !dx || !dalpha || !dbeta || !dK || nch < 0) return ORC_EINVAL;
    if (geom_init(&g, d, dims)) return ORC_EINVAL;
    for (int a = 0; a < 3; ++a)
        if (!is_pow2(g.N[a])) return ORC_EINVAL;
    for (int64_t q = 0; q < nch; ++q)
        if (chans[q] < 0 || chans[q] >= C) return ORC_EINVAL;
    const size_t bytes = sizeof(double) * (size_t)g.NL;
    double *buf[10];
    int fail = 0;
    for (int k = 0; k < 10; ++k) {
        buf[k] = (double *)malloc(bytes);
        if (!buf[k]) fail = 1;
    }
    double *v = (double *)malloc(sizeof(double) * (size_t)g.L);
    if (fail || !v) {
        for (int k = 0; k < 10; ++k) free(buf[k]);
        free(v);
        return ORC_ENOMEM;
    }
    double *kr = buf[0], *ki = buf[1], *pr = buf[2], *pi = buf[3], *yr = buf[4], *yi = buf[5];
    double *ur = buf[6], *ui = buf[7], *tr = buf[8], *ti = buf[9];
    const double scale = 1.0 / (double)g.NL;
    int rc = ORC_OK;
    for (int64_t q = 0; q < nch && rc == ORC_OK; ++q) {
        const int64_t c = chans[q];
        memset(kr, 0, bytes);
        memset(ki, 0, bytes);
        wrap_place(K + c * g.KL, &g, kr);
        if ((rc = fft_nd(kr, ki, g.N, -1))) break;
        memset(pr, 0, bytes);
        memset(pi, 0, bytes);
        dalpha[q] = 0.0;
        dbeta[q] = 0.0;
        for (int64_t b = 0; b < B && rc == ORC_OK; ++b) {
            const int64_t p = b * C + c;
            const float *xs = x + p * g.L, *dys = dy + p * g.L;
            for (int64_t j = 0; j < g.L; ++j) v[j] = (double)dys[j];
            pad_into(v, &g, yr, yi);
            if ((rc = fft_nd(yr, yi, g.N, -1))) break;
            for (int64_t j = 0; j < g.L; ++j) v[j] = gate((double)xs[j], alpha[c], beta[c]);
            pad_into(v, &g, ur, ui);
            if ((rc = fft_nd(ur, ui, g.N, -1))) break;
            for (int64_t m = 0; m < g.NL; ++m) {
                /* P += DY conj(U);  T = DY conj(Khat) */
                pr[m] += yr[m] * ur[m] + yi[m] * ui[m];
                pi[m] += yi[m] * ur[m] - yr[m] * ui[m];
                tr[m] = yr[m] * kr[m] + yi[m] * ki[m];
                ti[m] = yi[m] * kr[m] - yr[m] * ki[m];
            }
            if ((rc = fft_nd(tr, ti, g.N, +1))) break;
            for (int64_t j0 = 0; j0 < g.n[0]; ++j0)
                for (int64_t j1 = 0; j1 < g.n[1]; ++j1)
                    for (int64_t j2 = 0; j2 < g.n[2]; ++j2)
                        v[(j0 * g.n[1] + j1) * g.n[2] + j2] = tr[(j0 * g.N[1] + j1) * g.N[2] + j2] * scale;
            gate_vjp(xs, v, g.L, alpha[c], beta[c], dx + (q * B + b) * g.L, &dalpha[q], &dbeta[q]);
        }
        if (rc) break;
        if ((rc = fft_nd(pr, pi, g.N, +1))) break;
        double *dKc = dK + q * g.KL;
        for (int64_t a0 = 0; a0 < g.ke[0]; ++a0)
            for (int64_t a1 = 0; a1 < g.ke[1]; ++a1)
                for (int64_t a2 = 0; a2 < g.ke[2]; ++a2) {
                    const int64_t d0 = a0 - (g.n[0] - 1), d1 = a1 - (g.n[1] - 1), d2 = a2 - (g.n[2] - 1);
                    const int64_t m0 = (d0 % g.N[0] + g.N[0]) % g.N[0];
                    const int64_t m1 = (d1 % g.N[1] + g.N[1]) % g.N[1];
                    const int64_t m2 = (d2 % g.N[2] + g.N[2]) % g.N[2];
                    dKc[(a0 * g.ke[1] + a1) * g.ke[2] + a2] = pr[(m0 * g.N[1] + m1) * g.N[2] + m2] * scale;
                }
    }
    for (int k = 0; k < 10; ++k) free(buf[k]);
    free(v);
    return rc;
}

/*
 * Backward of the circular mode: the same chain rule with every offset taken
 * modulo n (K stored by offset mod n, as for the circular forward):
 *   du[j]    = sum_{i in G} dy[i] K[(i - j) mod n]
 *   dK_c[m]  = sum_b sum_{j in G} dy[(j + m) mod n] u[j]
 * dx, dalpha, dbeta from du as in the non-circular backward.  O1 writes the
 * sums out; O2 takes them as products with conjugate spectra of size n.
 */
int oracle_bwd_direct_circ(const float *x, const float *alpha, const float *beta, const float *K, const float *dy,
                           int B, int C, int d, const int64_t *dims,
                           double *dx, double *dalpha, double *dbeta, double *dK)
{
    geom_t g;
    if (!x || !alpha || !beta || !K || !dy || !dx || !dalpha || !dbeta || !dK || B < 0 || C < 0) return ORC_EINVAL;
    if (geom_init(&g, d, dims)) return ORC_EINVAL;
    const size_t n = (size_t)(g.L ? g.L : 1);
    double *u = (double *)malloc(sizeof(double) * n), *du = (double *)malloc(sizeof(double) * n);
    if (!u || !du) { free(u); free(du); return ORC_ENOMEM; }
    for (int c = 0; c < C; ++c) {
        const float *Kc = K + (int64_t)c * g.L;
        double *dKc = dK + (int64_t)c * g.L;
        for (int64_t m = 0; m < g.L; ++m) dKc[m] = 0.0;
        dalpha[c] = 0.0;
        dbeta[c] = 0.0;
        for (int b = 0; b < B; ++b) {
            const int64_t p = (int64_t)b * C + c;
            const float *xs = x + p * g.L, *dys = dy + p * g.L;
            for (int64_t j = 0; j < g.L; ++j) u[j] = gate((double)xs[j], alpha[c], beta[c]);
#pragma omp parallel for schedule(static)
            for (int64_t j = 0; j < g.L; ++j) {
                const int64_t j2 = j % g.n[2], j1 = (j / g.n[2]) % g.n[1], j0 = j / (g.n[1] * g.n[2]);
                double acc = 0.0;
                for (int64_t i = 0; i < g.L; ++i) {
                    const int64_t i2 = i % g.n[2], i1 = (i / g.n[2]) % g.n[1], i0 = i / (g.n[1] * g.n[2]);
                    const int64_t m0 = ((i0 - j0) % g.n[0] + g.n[0]) % g.n[0];
                    const int64_t m1 = ((i1 - j1) % g.n[1] + g.n[1]) % g.n[1];
                    const int64_t m2 = ((i2 - j2) % g.n[2] + g.n[2]) % g.n[2];
                    acc += (double)dys[i] * (double)Kc[(m0 * g.n[1] + m1) * g.n[2] + m2];
                }
                du[j] = acc;
            }
            gate_vjp(xs, du, g.L, alpha[c], beta[c], dx + p * g.L, &dalpha[c], &dbeta[c]);
#pragma omp parallel for schedule(static)
            for (int64_t m = 0; m < g.L; ++m) {
                const int64_t m2 = m % g.n[2], m1 = (m / g.n[2]) % g.n[1], m0 = m / (g.n[1] * g.n[2]);
                double acc = 0.0;
                for (int64_t j = 0; j < g.L; ++j) {
                    const int64_t j2 = j % g.n[2], j1 = (j / g.n[2]) % g.n[1], j0 = j / (g.n[1] * g.n[2]);
                    const int64_t i0 = (j0 + m0) % g.n[0], i1 = (j1 + m1) % g.n[1], i2 = (j2 + m2) % g.n[2];
                    acc += (double)dys[(i0 * g.n[1] + i1) * g.n[2] + i2] * u[j];
                }
                dKc[m] += acc;
            }
        }
    }
    free(u);
    free(du);
    return ORC_OK;
}

int oracle_bwd_fft_circ(const float *x, const float *alpha, const float *beta, const float *K, const float *dy,
                        int B, int C, int d, const int64_t *dims, int64_t nch, const int64_t *chans,
                        double *dx, double *dalpha, double *dbeta, double *dK)
{
    geom_t g;
    if (!x || !alpha || !beta || !K || !dy || !chans || !dx || !dalpha || !dbeta || !dK || nch < 0) return ORC_EINVAL;
    if (geom_init(&g, d, dims)) return ORC_EINVAL;
    for (int a = 0; a < 3; ++a)
        if (!is_pow2(g.n[a])) return ORC_EINVAL;
    for (int64_t q = 0; q < nch; ++q)
        if (chans[q] < 0 || chans[q] >= C) return ORC_EINVAL;
    const size_t bytes = sizeof(double) * (size_t)g.L;
    double *buf[10];
    int fail = 0;
    for (int k = 0; k < 10; ++k) {
        buf[k] = (double *)malloc(bytes);
        if (!buf[k]) fail = 1;
    }
    double *v = (double *)malloc(bytes);
    if (fail || !v) {
        for (int k = 0; k < 10; ++k) free(buf[k]);
        free(v);
        return ORC_ENOMEM;
    }
    double *kr = buf[0], *ki = buf[1], *pr = buf[2], *pi = buf[3], *yr = buf[4], *yi = buf[5];
    double *ur = buf[6], *ui = buf[7], *tr = buf[8], *ti = buf[9];
    const double scale = 1.0 / (double)g.L;
    int rc = ORC_OK;
    for (int64_t q = 0; q < nch && rc == ORC_OK; ++q) {
        const int64_t c = chans[q];
        for (int64_t m = 0; m < g.L; ++m) { kr[m] = (double)K[c * g.L + m]; ki[m] = 0.0; pr[m] = 0.0; pi[m] = 0.0; }
        if ((rc = fft_nd(kr, ki, g.n, -1))) break;
        dalpha[q] = 0.0;
        dbeta[q] = 0.0;
        for (int64_t b = 0; b < B && rc == ORC_OK; ++b) {
            const int64_t p = b * C + c;
            const float *xs = x + p * g.L, *dys = dy + p * g.L;
            for (int64_t j = 0; j < g.L; ++j) {
                yr[j] = (double)dys[j]; yi[j] = 0.0;
                ur[j] = gate((double)xs[j], alpha[c], beta[c]); ui[j] = 0.0;
            }
            if ((rc = fft_nd(yr, yi, g.n, -1))) break;
            if ((rc = fft_nd(ur, ui, g.n, -1))) break;
            for (int64_t m = 0; m < g.L; ++m) {
                pr[m] += yr[m] * ur[m] + yi[m] * ui[m];
                pi[m] += yi[m] * ur[m] - yr[m] * ui[m];
                tr[m] = yr[m] * kr[m] + yi[m] * ki[m];
                ti[m] = yi[m] * kr[m] - yr[m] * ki[m];
            }
            if ((rc = fft_nd(tr, ti, g.n, +1))) break;
            for (int64_t j = 0; j < g.L; ++j) v[j] = tr[j] * scale;
            gate_vjp(xs, v, g.L, alpha[c], beta[c], dx + (q * B + b) * g.L, &dalpha[q], &dbeta[q]);
        }
        if (rc) break;
        if ((rc = fft_nd(pr, pi, g.n, +1))) break;
        for (int64_t m = 0; m < g.L; ++m) dK[q * g.L + m] = pr[m] * scale;
    }
    for (int k = 0; k < 10; ++k) free(buf[k]);
    free(v);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* Input-dependent kernel generator ([SUMM] "Methodology", "Input dependent   */
/* kernels via registers and FiLM", "Kernel synthesis").                       */
/* ------------------------------------------------------------------------- */
/*
 * For each sample b (the steps in the summary's order; the registers'
 * processing by the network is stood in for by one layer on the sample's
 * per-channel means):
 *   m_b[c]      = mean over the grid of x[b,c]
 *   a_{b,r,j}   = tanh(sum_c Wreg[r][j][c] m_b[c] + breg[r][j])     R registers, width D
 *   pi_{b,r}    = softmax_r( sum_j q[j] a_{b,r,j} )
 *   z_{b,j}     = sum_r pi_{b,r} a_{b,r,j}                          control variable z(x)
 *   gam_{b,k}   = 1 + sum_j Wgam[k][j] z_{b,j},  bet_{b,k} = sum_j Wbet[k][j] z_{b,j}   FiLM
 * and for each channel c and offset delta (delta_a in [-(n_a-1), n_a-1]):
 *   h_k(delta)  = sin(omega0 (sum_a W1[k][a] chat_a + b1[k])),  chat_a = delta_a / (n_a - 1)
 *   f(delta)    = sum_k W2[c][k] (gam_{b,k} h_k(delta) + bet_{b,k}) + b2[c]     (SIREN, FiLM-modulated)
 *   w_c(delta)  = exp(-|delta|^2 / (2 sigma_c^2))                              (Gaussian window)
 *   K_{b,c}     = w_c f                                              K(x) = w(c) (.) f(c; z(x))
 * with 16 hidden units.  K: fp64 [B][C][(2n_0-1)..].
 */
#define ORC_GEN_H 16

int oracle_generate_kernels(const float *x, int B, int C, int d, const int64_t *dims, int R, int D,
                            const float *Wreg, const float *breg, const float *q, const float *Wgam,
                            const float *Wbet, const float *W1, const float *b1, const float *W2,
                            const float *b2, const float *sigma, double omega0, double *K)
{
    geom_t g;
    if (!x || !K || !Wreg || !breg || !q || !Wgam || !Wbet || !W1 || !b1 || !W2 || !b2 || !sigma) return ORC_EINVAL;
    if (B < 0 || C < 0 || R < 1 || D < 1 || geom_init(&g, d, dims)) return ORC_EINVAL;
    double *m = (double *)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1));
    double *a = (double *)malloc(sizeof(double) * (size_t)R * D);
    double *z = (double *)malloc(sizeof(double) * (size_t)D);
    double *sc = (double *)malloc(sizeof(double) * (size_t)R);
    if (!m || !a || !z || !sc) { free(m); free(a); free(z); free(sc); return ORC_ENOMEM; }
    const int off = 3 - d;   /* geom axes are right-aligned: axis a of the grid is geom axis off + a */
    for (int b = 0; b < B; ++b) {
        for (int c = 0; c < C; ++c) {
            const float *xs = x + ((int64_t)b * C + c) * g.L;
            double acc = 0.0;
            for (int64_t j = 0; j < g.L; ++j) acc += (double)xs[j];
            m[c] = acc / (double)g.L;
        }
        for (int r = 0; r < R; ++r)
            for (int j = 0; j < D; ++j) {
                double v = breg[r * D + j];
                for (int c = 0; c < C; ++c) v += (double)Wreg[((int64_t)r * D + j) * C + c] * m[c];
                a[r * D + j] = tanh(v);
            }
        double smax = -1e300;
        for (int r = 0; r < R; ++r) {
            double v = 0.0;
            for (int j = 0; j < D; ++j) v += (double)q[j] * a[r * D + j];
            sc[r] = v;
            if (v > smax) smax = v;
        }
        double ssum = 0.0;
        for (int r = 0; r < R; ++r) { sc[r] = exp(sc[r] - smax); ssum += sc[r]; }
        for (int j = 0; j < D; ++j) {
            double v = 0.0;
            for (int r = 0; r < R; ++r) v += sc[r] / ssum * a[r * D + j];
            z[j] = v;
        }
        double gam[ORC_GEN_H], bet[ORC_GEN_H];
        for (int k = 0; k < ORC_GEN_H; ++k) {
            double vg = 1.0, vb = 0.0;
            for (int j = 0; j < D; ++j) { vg += (double)Wgam[k * D + j] * z[j]; vb += (double)Wbet[k * D + j] * z[j]; }
            gam[k] = vg;
            bet[k] = vb;
        }
        for (int c = 0; c < C; ++c) {
            double *Kc = K + ((int64_t)b * C + c) * g.KL;
            const double s2 = 2.0 * (double)sigma[c] * (double)sigma[c];
#pragma omp parallel for schedule(static)
            for (int64_t e0 = 0; e0 < g.ke[0]; ++e0)
                for (int64_t e1 = 0; e1 < g.ke[1]; ++e1)
                    for (int64_t e2 = 0; e2 < g.ke[2]; ++e2) {
                        const int64_t e[3] = {e0, e1, e2};
                        double chat[3] = {0.0, 0.0, 0.0}, r2 = 0.0;
                        for (int ax = 0; ax < 3; ++ax) {
                            const double dl = (double)(e[ax] - (g.n[ax] - 1));
                            if (g.n[ax] > 1) chat[ax] = dl / (double)(g.n[ax] - 1);
                            r2 += dl * dl;
                        }
                        double f = (double)b2[c];
                        for (int k = 0; k < ORC_GEN_H; ++k) {
                            double arg = (double)b1[k];
                            for (int ax = 0; ax < d; ++ax) arg += (double)W1[k * d + ax] * chat[off + ax];
                            f += (double)W2[c * ORC_GEN_H + k] * (gam[k] * sin(omega0 * arg) + bet[k]);
                        }
                        Kc[(e0 * g.ke[1] + e1) * g.ke[2] + e2] = exp(-r2 / s2) * f;
                    }
        }
    }
    free(m); free(a); free(z); free(sc);
    return ORC_OK;
}

/* Threads OpenMP will use (reported by the CPU-baseline leg). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
