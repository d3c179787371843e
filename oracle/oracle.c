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

/* Threads OpenMP will use (reported by the CPU-baseline leg). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
