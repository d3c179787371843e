/*
 * Runs every entry point of oracle/oracle.c on small seeded inputs held in
 * buffers of exactly the documented sizes, in a build under AddressSanitizer
 * and UndefinedBehaviorSanitizer, and checks that the oracle's two routes
 * agree (the written-out sums against the FFT routes, forward and backward,
 * zero-padded and circular; point evaluations against whole-grid ones).
 * Prints one line per failed expectation and exits non-zero if there was any.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gate(const float *x, int64_t count, double alpha, double beta, double *u);
int oracle_gate_vjp(const float *x, const double *du, int64_t count, double alpha, double beta, double *dx,
                    double *sums);
int oracle_direct(const float *x, const float *alpha, const float *beta, const float *K, double *y, int B, int C,
                  int d, const int64_t *dims);
int oracle_direct_points(const float *x, const float *alpha, const float *beta, const float *K, int B, int C, int d,
                         const int64_t *dims, int64_t npts, const int64_t *pts, double *out);
int oracle_kernel_spectrum(const float *K, int C, int d, const int64_t *dims, double *re, double *im);
int oracle_fftconv_pairs(const float *x, const float *alpha, const float *beta, const float *K, int B, int C, int d,
                         const int64_t *dims, int64_t npairs, const int64_t *pairs, double *y_out);
int oracle_direct_circ(const float *x, const float *alpha, const float *beta, const float *K, double *y, int B,
                       int C, int d, const int64_t *dims);
int oracle_fftconv_circ_pairs(const float *x, const float *alpha, const float *beta, const float *K, int B, int C,
                              int d, const int64_t *dims, int64_t npairs, const int64_t *pairs, double *y_out);
int oracle_bwd_direct(const float *x, const float *alpha, const float *beta, const float *K, const float *dy, int B,
                      int C, int d, const int64_t *dims, double *dx, double *dalpha, double *dbeta, double *dK);
int oracle_bwd_direct_points(const float *x, const float *alpha, const float *beta, const float *K, const float *dy,
                             int B, int C, int d, const int64_t *dims, int64_t nx, const int64_t *xpts,
                             double *dx_out, int64_t nk, const int64_t *kpts, double *dK_out);
int oracle_bwd_fft(const float *x, const float *alpha, const float *beta, const float *K, const float *dy, int B,
                   int C, int d, const int64_t *dims, int64_t nch, const int64_t *chans, double *dx, double *dalpha,
                   double *dbeta, double *dK);
int oracle_bwd_direct_circ(const float *x, const float *alpha, const float *beta, const float *K, const float *dy,
                           int B, int C, int d, const int64_t *dims, double *dx, double *dalpha, double *dbeta,
                           double *dK);
int oracle_bwd_fft_circ(const float *x, const float *alpha, const float *beta, const float *K, const float *dy, int B,
                        int C, int d, const int64_t *dims, int64_t nch, const int64_t *chans, double *dx,
                        double *dalpha, double *dbeta, double *dK);
int oracle_generate_kernels(const float *x, int B, int C, int d, const int64_t *dims, int R, int D,
                            const float *Wreg, const float *breg, const float *q, const float *Wgam,
                            const float *Wbet, const float *W1, const float *b1, const float *W2, const float *b2,
                            const float *sigma, double omega0, double *K);

static int g_bad = 0;

#define EXPECT(call, want)                                                                           \
    do {                                                                                             \
        const int got_ = (call);                                                                     \
        if (got_ != (want)) {                                                                        \
            printf("line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, (int)(want));  \
            ++g_bad;                                                                                 \
        }                                                                                            \
    } while (0)

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static float urand(void) /* xorshift64*, uniform in [-1, 1) */
{
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (float)((double)((g_state * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

static void* buf(size_t n)
{
    void* p = malloc(n ? n : 1);
    if (!p) {
        printf("out of host memory\n");
        exit(2);
    }
    return p;
}

static float* frand(size_t n)
{
    float* p = buf(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) p[i] = urand();
    return p;
}

static void close_to(const char* what, const double* a, const double* b, int64_t n, double tol)
{
    double worst = 0.0, scale = 1e-30;
    for (int64_t i = 0; i < n; ++i) {
        worst = fmax(worst, fabs(a[i] - b[i]));
        scale = fmax(scale, fabs(b[i]));
    }
    if (!(worst <= tol * scale)) {
        printf("%s: max difference %.3e against scale %.3e\n", what, worst, scale);
        ++g_bad;
    }
}

/* dx of the FFT routes is [C][B][L]; the written-out routes' is [B][C][L]. */
static void to_bcl(double* dst, const double* cbl, int B, int C, int64_t L)
{
    for (int b = 0; b < B; ++b)
        for (int c = 0; c < C; ++c)
            memcpy(dst + ((int64_t)b * C + c) * L, cbl + ((int64_t)c * B + b) * L, sizeof(double) * (size_t)L);
}

static void run(int d, const int64_t* dims, int B, int C, int pow2)
{
    int64_t L = 1, KL = 1;
    for (int a = 0; a < d; ++a) {
        L *= dims[a];
        KL *= 2 * dims[a] - 1;
    }
    const int64_t n_all = (int64_t)B * C * L;
    float *x = frand(n_all), *dy = frand(n_all), *al = frand(C), *be = frand(C), *K = frand(C * KL);
    double *y1 = buf(sizeof(double) * n_all), *y2 = buf(sizeof(double) * n_all);
    EXPECT(oracle_direct(x, al, be, K, y1, B, C, d, dims), 0);

    /* Point evaluations: the first and last voxel of every pair. */
    const int w = 2 + d;
    int64_t* pts = buf(sizeof(int64_t) * 2 * B * C * w);
    double* pv = buf(sizeof(double) * 2 * B * C);
    double* pw = buf(sizeof(double) * 2 * B * C);
    for (int p = 0; p < B * C; ++p)
        for (int e = 0; e < 2; ++e) {
            int64_t* r = pts + (2 * p + e) * w;
            r[0] = p / C;
            r[1] = p % C;
            for (int a = 0; a < d; ++a) r[2 + a] = e ? dims[a] - 1 : 0;
            pw[2 * p + e] = y1[(int64_t)p * L + (e ? L - 1 : 0)];
        }
    EXPECT(oracle_direct_points(x, al, be, K, B, C, d, dims, 2 * B * C, pts, pv), 0);
    close_to("direct_points", pv, pw, 2 * B * C, 1e-12);

    int64_t* chans = buf(sizeof(int64_t) * C);
    for (int c = 0; c < C; ++c) chans[c] = c;
    double *dx1 = buf(sizeof(double) * n_all), *da1 = buf(sizeof(double) * C), *db1 = buf(sizeof(double) * C);
    double* dK1 = buf(sizeof(double) * C * KL);
    EXPECT(oracle_bwd_direct(x, al, be, K, dy, B, C, d, dims, dx1, da1, db1, dK1), 0);
    {
        int64_t xp[1 * 5], kp[1 * 4];
        xp[0] = B - 1;
        xp[1] = C - 1;
        kp[0] = C - 1;
        for (int a = 0; a < d; ++a) {
            xp[2 + a] = dims[a] - 1;
            kp[1 + a] = 0;
        }
        double ox, ok, wx = dx1[n_all - 1], wk = dK1[(int64_t)(C - 1) * KL];
        EXPECT(oracle_bwd_direct_points(x, al, be, K, dy, B, C, d, dims, 1, xp, &ox, 1, kp, &ok), 0);
        close_to("bwd_points dx", &ox, &wx, 1, 1e-12);
        close_to("bwd_points dK", &ok, &wk, 1, 1e-12);
    }

    if (pow2) {
        int64_t* pairs = buf(sizeof(int64_t) * B * C);
        for (int p = 0; p < B * C; ++p) pairs[p] = p;
        EXPECT(oracle_fftconv_pairs(x, al, be, K, B, C, d, dims, B * C, pairs, y2), 0);
        close_to("fftconv vs direct", y2, y1, n_all, 1e-10);

        int64_t NL = 1;
        for (int a = 0; a < d; ++a) NL *= 2 * dims[a];
        double *re = buf(sizeof(double) * C * NL), *im = buf(sizeof(double) * C * NL);
        EXPECT(oracle_kernel_spectrum(K, C, d, dims, re, im), 0);
        /* Bin 0 is the sum of the kernel's values. */
        double s0 = 0.0;
        for (int64_t i = 0; i < KL; ++i) s0 += K[i];
        close_to("spectrum bin 0", re, &s0, 1, 1e-12);

        double *dx2 = buf(sizeof(double) * n_all), *da2 = buf(sizeof(double) * C), *db2 = buf(sizeof(double) * C);
        double* dK2 = buf(sizeof(double) * C * KL);
        EXPECT(oracle_bwd_fft(x, al, be, K, dy, B, C, d, dims, C, chans, dx2, da2, db2, dK2), 0);
        to_bcl(y2, dx2, B, C, L);
        close_to("bwd dx", y2, dx1, n_all, 1e-10);
        close_to("bwd dalpha", da2, da1, C, 1e-10);
        close_to("bwd dbeta", db2, db1, C, 1e-10);
        close_to("bwd dK", dK2, dK1, C * KL, 1e-10);

        /* Circular mode: kernels of the grid's own extent. */
        float* Kc = frand(C * L);
        EXPECT(oracle_direct_circ(x, al, be, Kc, y1, B, C, d, dims), 0);
        EXPECT(oracle_fftconv_circ_pairs(x, al, be, Kc, B, C, d, dims, B * C, pairs, y2), 0);
        close_to("circ fftconv vs direct", y2, y1, n_all, 1e-10);
        double* dKc1 = buf(sizeof(double) * C * L);
        double* dKc2 = buf(sizeof(double) * C * L);
        EXPECT(oracle_bwd_direct_circ(x, al, be, Kc, dy, B, C, d, dims, dx1, da1, db1, dKc1), 0);
        EXPECT(oracle_bwd_fft_circ(x, al, be, Kc, dy, B, C, d, dims, C, chans, dx2, da2, db2, dKc2), 0);
        to_bcl(y2, dx2, B, C, L);
        close_to("circ bwd dx", y2, dx1, n_all, 1e-10);
        close_to("circ bwd dalpha", da2, da1, C, 1e-10);
        close_to("circ bwd dK", dKc2, dKc1, C * L, 1e-10);
        free(pairs); free(re); free(im); free(dx2); free(da2); free(db2); free(dK2); free(Kc); free(dKc1);
        free(dKc2);
    }

    /* The kernel generator: R = 3 registers, control width D = 5. */
    {
        const int R = 3, D = 5, H = 16;
        float *Wreg = frand(R * D * C), *breg = frand(R * D), *q = frand(D), *Wgam = frand(H * D),
              *Wbet = frand(H * D), *W1 = frand(H * d), *b1 = frand(H), *W2 = frand(C * H), *b2 = frand(C),
              *sig = frand(C);
        for (int c = 0; c < C; ++c) sig[c] = 1.0f + fabsf(sig[c]);
        double* Kg = buf(sizeof(double) * B * C * KL);
        EXPECT(oracle_generate_kernels(x, B, C, d, dims, R, D, Wreg, breg, q, Wgam, Wbet, W1, b1, W2, b2, sig, 10.0,
                                       Kg),
               0);
        int finite = 1;
        for (int64_t i = 0; i < (int64_t)B * C * KL; ++i) finite &= isfinite(Kg[i]) != 0;
        if (!finite) {
            printf("generated kernels not finite\n");
            ++g_bad;
        }
        EXPECT(oracle_generate_kernels(x, B, C, d, dims, 0, D, Wreg, breg, q, Wgam, Wbet, W1, b1, W2, b2, sig, 10.0,
                                       Kg),
               1);
        free(Wreg); free(breg); free(q); free(Wgam); free(Wbet); free(W1); free(b1); free(W2); free(b2); free(sig);
        free(Kg);
    }

    /* The gate and its vector-Jacobian product on one pair. */
    {
        double *u = buf(sizeof(double) * L), *gdx = buf(sizeof(double) * L), sums[2];
        EXPECT(oracle_gate(x, L, 0.5, -0.25, u), 0);
        EXPECT(oracle_gate_vjp(x, u, L, 0.5, -0.25, gdx, sums), 0);
        EXPECT(oracle_gate(NULL, L, 0.5, -0.25, u), 1);
        free(u);
        free(gdx);
    }
    EXPECT(oracle_direct(NULL, al, be, K, y1, B, C, d, dims), 1);
    EXPECT(oracle_direct(x, al, be, K, y1, B, C, 4, dims), 1);

    free(x); free(dy); free(al); free(be); free(K); free(y1); free(y2); free(pts); free(pv); free(pw); free(chans);
    free(dx1); free(da1); free(db1); free(dK1);
}

int main(void)
{
    const int64_t d1[1] = {16}, d2[2] = {4, 8}, d3[3] = {2, 4, 4}, r2[2] = {5, 3}, r3[3] = {3, 2, 5};
    run(1, d1, 2, 3, 1);
    run(2, d2, 2, 2, 1);
    run(3, d3, 1, 2, 1);
    run(2, r2, 2, 2, 0);
    run(3, r3, 1, 2, 0);
    printf("%s: %d failed expectation(s)\n", g_bad ? "FAIL" : "ok", g_bad);
    return g_bad ? 1 : 0;
}
