/*
 * Drives every entry point of include/hyenand.h through its argument checks
 * and its planning, chunking and workspace layout, in a build whose kernel
 * launchers are host stand-ins (stub_launch.cpp) and whose host code runs
 * under AddressSanitizer and UndefinedBehaviorSanitizer.  "Device" buffers are
 * host allocations of exactly the documented sizes, so a chunk or offset that
 * leaves its buffer is reported by the sanitizer.  Prints one line per failed
 * expectation and exits non-zero if there was any.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "hyenand.h"

void stub_set_launch_status(int s);
long stub_launch_calls(void);
long stub_failures(void);

static int g_bad = 0;

#define EXPECT(call, want)                                                                          \
    do {                                                                                            \
        const int got_ = (call);                                                                    \
        if (got_ != (want)) {                                                                       \
            printf("line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, (int)(want)); \
            ++g_bad;                                                                                \
        }                                                                                           \
    } while (0)

#define CHECK(cond)                                         \
    do {                                                    \
        if (!(cond)) {                                      \
            printf("line %d: %s is false\n", __LINE__, #cond); \
            ++g_bad;                                        \
        }                                                   \
    } while (0)

/* Exactly n bytes (at least one, so that an empty region still has an address). */
static void* buf(size_t n)
{
    void* p = malloc(n ? n : 1);
    if (!p) {
        printf("out of host memory (%zu bytes)\n", n);
        exit(2);
    }
    memset(p, 0, n ? n : 1);
    return p;
}

static int64_t prod(int d, const int64_t* dims)
{
    int64_t v = 1;
    for (int i = 0; i < d; ++i) v *= dims[i];
    return v;
}

typedef struct {
    int d;
    int64_t dims[3];
    int B, C, dtype, circ;
} shape_t;

/* Forward, backward (with and without dK) and spectrum of one shape, with the
 * recommended and the minimum workspaces; then every launch failing. */
static void run_shape(const shape_t* s)
{
    const int d = s->d, B = s->B, C = s->C, dt = s->dtype, circ = s->circ;
    const int64_t* dims = s->dims;
    const size_t es = dt == HYENAND_BF16 ? 2 : 4;
    const int64_t vox = prod(d, dims);
    int64_t kl = 1;
    for (int i = 0; i < d; ++i) kl *= circ ? dims[i] : 2 * dims[i] - 1;
    const size_t kb = circ ? hyenand_kernel_spectrum_circ_bytes(C, d, dims) : hyenand_kernel_spectrum_bytes(C, d, dims);
    CHECK(kb > 0);
    CHECK((circ ? hyenand_kernel_spectrum_circ_tile(d, dims) : hyenand_kernel_spectrum_tile(d, dims)) > 0);
    float* K = buf(4 * (size_t)C * kl);
    void* Kh = buf(kb);
    void* x = buf(es * B * C * vox);
    void* y = buf(es * B * C * vox);
    void* dy = buf(es * B * C * vox);
    float* al = buf(4 * (size_t)C);
    float* be = buf(4 * (size_t)C);
    float* da = buf(4 * (size_t)C);
    float* db = buf(4 * (size_t)C);
    float* dK = buf(4 * (size_t)C * kl);

    EXPECT(circ ? hyenand_kernel_spectrum_circ(K, Kh, C, d, dims, NULL) : hyenand_kernel_spectrum(K, Kh, C, d, dims, NULL),
           HYENAND_OK);

    const size_t wr = circ ? hyenand_fftconv_circ_workspace_bytes(B, C, d, dims, dt)
                           : hyenand_fftconv_workspace_bytes(B, C, d, dims, dt);
    const size_t wm = circ ? hyenand_fftconv_circ_workspace_min_bytes(B, C, d, dims, dt)
                           : hyenand_fftconv_workspace_min_bytes(B, C, d, dims, dt);
    CHECK(wm <= wr);
    for (int pass = 0; pass < 2; ++pass) {
        const size_t wb = pass ? wm : wr;
        void* w = wb ? buf(wb) : NULL;
        EXPECT(circ ? hyenand_fftconv_fwd_circ(x, al, be, Kh, y, B, C, d, dims, dt, w, wb, NULL)
                    : hyenand_fftconv_fwd(x, al, be, Kh, y, B, C, d, dims, dt, w, wb, NULL),
               HYENAND_OK);
        if (!circ) {
            int nl = -1, per = -1;
            EXPECT(hyenand_fftconv_launch_plan(B, C, d, dims, dt, wb, &nl, &per), HYENAND_OK);
            CHECK(nl >= 1 && per >= 1 && per <= C);
            const long before = stub_launch_calls();
            int traced = -1;
            EXPECT(hyenand_fftconv_fwd_traced(x, al, be, Kh, y, B, C, d, dims, dt, w, wb, NULL, NULL, 0, &traced),
                   HYENAND_OK);
            /* The stand-in counts one call per chunk; the plan counts kernels. */
            const long chunks = stub_launch_calls() - before;
            CHECK(chunks >= 1 && chunks == (C + per - 1) / per);
        }
        if (wb > 0) {
            EXPECT(circ ? hyenand_fftconv_fwd_circ(x, al, be, Kh, y, B, C, d, dims, dt, w, wm - 8, NULL)
                        : hyenand_fftconv_fwd(x, al, be, Kh, y, B, C, d, dims, dt, w, wm - 8, NULL),
                   HYENAND_ERR_WORKSPACE);
            EXPECT(circ ? hyenand_fftconv_fwd_circ(x, al, be, Kh, y, B, C, d, dims, dt, NULL, wb, NULL)
                        : hyenand_fftconv_fwd(x, al, be, Kh, y, B, C, d, dims, dt, NULL, wb, NULL),
                   HYENAND_ERR_WORKSPACE);
        }
        free(w);
    }

    for (int with_dk = 0; with_dk < 2; ++with_dk)
        for (int pass = 0; pass < 2; ++pass) {
            const size_t wb = circ ? (pass ? hyenand_fftconv_bwd_circ_workspace_min_bytes(B, C, d, dims, dt, with_dk)
                                           : hyenand_fftconv_bwd_circ_workspace_bytes(B, C, d, dims, dt, with_dk))
                                   : (pass ? hyenand_fftconv_bwd_workspace_min_bytes(B, C, d, dims, dt, with_dk)
                                           : hyenand_fftconv_bwd_workspace_bytes(B, C, d, dims, dt, with_dk));
            CHECK(wb > 0);
            void* w = buf(wb);
            float* dk = with_dk ? dK : NULL;
            EXPECT(circ ? hyenand_fftconv_bwd_circ(x, al, be, Kh, dy, y, da, db, dk, B, C, d, dims, dt, w, wb, NULL)
                        : hyenand_fftconv_bwd(x, al, be, Kh, dy, y, da, db, dk, B, C, d, dims, dt, w, wb, NULL),
                   HYENAND_OK);
            const size_t small = (circ ? hyenand_fftconv_bwd_circ_workspace_min_bytes(B, C, d, dims, dt, with_dk)
                                       : hyenand_fftconv_bwd_workspace_min_bytes(B, C, d, dims, dt, with_dk)) - 8;
            EXPECT(circ ? hyenand_fftconv_bwd_circ(x, al, be, Kh, dy, y, da, db, dk, B, C, d, dims, dt, w, small, NULL)
                        : hyenand_fftconv_bwd(x, al, be, Kh, dy, y, da, db, dk, B, C, d, dims, dt, w, small, NULL),
                   HYENAND_ERR_WORKSPACE);
            free(w);
        }
    /* B = 0: the sums over an empty batch are zero-filled. */
    {
        const size_t wb = 8;
        void* w = buf(wb);
        EXPECT(circ ? hyenand_fftconv_bwd_circ(NULL, al, be, NULL, NULL, NULL, da, db, dK, 0, C, d, dims, dt, w, wb, NULL)
                    : hyenand_fftconv_bwd(NULL, al, be, NULL, NULL, NULL, da, db, dK, 0, C, d, dims, dt, w, wb, NULL),
               HYENAND_OK);
        free(w);
    }

    /* Every launch failing maps to HYENAND_ERR_HIP. */
    stub_set_launch_status(1);
    EXPECT(circ ? hyenand_kernel_spectrum_circ(K, Kh, C, d, dims, NULL) : hyenand_kernel_spectrum(K, Kh, C, d, dims, NULL),
           HYENAND_ERR_HIP);
    {
        void* w = wr ? buf(wr) : NULL;
        EXPECT(circ ? hyenand_fftconv_fwd_circ(x, al, be, Kh, y, B, C, d, dims, dt, w, wr, NULL)
                    : hyenand_fftconv_fwd(x, al, be, Kh, y, B, C, d, dims, dt, w, wr, NULL),
               HYENAND_ERR_HIP);
        free(w);
        const size_t wb = circ ? hyenand_fftconv_bwd_circ_workspace_bytes(B, C, d, dims, dt, 1)
                               : hyenand_fftconv_bwd_workspace_bytes(B, C, d, dims, dt, 1);
        w = buf(wb);
        EXPECT(circ ? hyenand_fftconv_bwd_circ(x, al, be, Kh, dy, y, da, db, dK, B, C, d, dims, dt, w, wb, NULL)
                    : hyenand_fftconv_bwd(x, al, be, Kh, dy, y, da, db, dK, B, C, d, dims, dt, w, wb, NULL),
               HYENAND_ERR_HIP);
        free(w);
    }
    stub_set_launch_status(0);

    free(K); free(Kh); free(x); free(y); free(dy); free(al); free(be); free(da); free(db); free(dK);
}

/* Per-sample spectra ([B][C]) with the forward and the backward. */
static void run_per_sample(const shape_t* s)
{
    const int d = s->d, B = s->B, C = s->C, dt = s->dtype;
    const int64_t* dims = s->dims;
    const size_t es = dt == HYENAND_BF16 ? 2 : 4;
    const int64_t vox = prod(d, dims);
    int64_t kl = 1;
    for (int i = 0; i < d; ++i) kl *= 2 * dims[i] - 1;
    const size_t kb = hyenand_kernel_spectrum_bytes(B * C, d, dims);
    float* K = buf(4 * (size_t)B * C * kl);
    void* Kh = buf(kb);
    void* x = buf(es * B * C * vox);
    void* y = buf(es * B * C * vox);
    void* dy = buf(es * B * C * vox);
    float* al = buf(4 * (size_t)C);
    float* be = buf(4 * (size_t)C);
    float* da = buf(4 * (size_t)C);
    float* db = buf(4 * (size_t)C);
    float* dK = buf(4 * (size_t)B * C * kl);
    EXPECT(hyenand_kernel_spectrum(K, Kh, B * C, d, dims, NULL), HYENAND_OK);
    const size_t wm = hyenand_fftconv_workspace_min_bytes(B, C, d, dims, dt);
    void* w = wm ? buf(wm) : NULL;
    EXPECT(hyenand_fftconv_fwd_per_sample(x, al, be, Kh, y, B, C, d, dims, dt, w, wm, NULL), HYENAND_OK);
    free(w);
    /* The per-sample backward runs the batch entries one at a time (a batch of one). */
    const size_t wb = hyenand_fftconv_bwd_workspace_min_bytes(1, C, d, dims, dt, 1);
    w = buf(wb);
    EXPECT(hyenand_fftconv_bwd_per_sample(x, al, be, Kh, dy, y, da, db, dK, B, C, d, dims, dt, w, wb, NULL),
           HYENAND_OK);
    free(w);
    free(K); free(Kh); free(x); free(y); free(dy); free(al); free(be); free(da); free(db); free(dK);
}

/* The kernel generator with exact parameter and workspace sizes. */
static void run_generator(const shape_t* s, int R, int D)
{
    const int d = s->d, B = s->B, C = s->C, dt = s->dtype;
    const int64_t* dims = s->dims;
    const size_t es = dt == HYENAND_BF16 ? 2 : 4;
    const int64_t vox = prod(d, dims);
    const int H = HYENAND_GEN_HIDDEN;
    hyenand_generator g;
    g.R = R;
    g.D = D;
    g.Wreg = buf(4 * (size_t)R * D * C);
    g.breg = buf(4 * (size_t)R * D);
    g.q = buf(4 * (size_t)D);
    g.Wgam = buf(4 * (size_t)H * D);
    g.Wbet = buf(4 * (size_t)H * D);
    g.W1 = buf(4 * (size_t)H * d);
    g.b1 = buf(4 * (size_t)H);
    g.W2 = buf(4 * (size_t)C * H);
    g.b2 = buf(4 * (size_t)C);
    g.sigma = buf(4 * (size_t)C);
    g.omega0 = 10.f;
    void* x = buf(es * B * C * vox);
    void* Kh = buf(hyenand_kernel_spectrum_bytes(B * C, d, dims));
    const size_t wb = hyenand_generate_workspace_bytes(B, C, d, dims);
    CHECK(wb > 0);
    /* 256-byte aligned, as the entry point requires. */
    unsigned char* raw = buf(wb + 512);
    unsigned char* w = raw + (256 - (uintptr_t)raw % 256);
    EXPECT(hyenand_generate_kernel_spectrum(x, &g, Kh, B, C, d, dims, dt, w, wb, NULL), HYENAND_OK);
    EXPECT(hyenand_generate_kernel_spectrum(x, &g, Kh, B, C, d, dims, dt, w, wb - 1, NULL), HYENAND_ERR_WORKSPACE);
    EXPECT(hyenand_generate_kernel_spectrum(x, &g, Kh, B, C, d, dims, dt, w + 8, wb, NULL), HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_generate_kernel_spectrum(x, NULL, Kh, B, C, d, dims, dt, w, wb, NULL), HYENAND_ERR_INVALID_ARG);
    hyenand_generator bad = g;
    bad.R = 0;
    EXPECT(hyenand_generate_kernel_spectrum(x, &bad, Kh, B, C, d, dims, dt, w, wb, NULL), HYENAND_ERR_INVALID_ARG);
    bad.R = 65;
    EXPECT(hyenand_generate_kernel_spectrum(x, &bad, Kh, B, C, d, dims, dt, w, wb, NULL), HYENAND_ERR_INVALID_ARG);
    bad = g;
    bad.sigma = NULL;
    EXPECT(hyenand_generate_kernel_spectrum(x, &bad, Kh, B, C, d, dims, dt, w, wb, NULL), HYENAND_ERR_INVALID_ARG);
    stub_set_launch_status(1);
    EXPECT(hyenand_generate_kernel_spectrum(x, &g, Kh, B, C, d, dims, dt, w, wb, NULL), HYENAND_ERR_HIP);
    stub_set_launch_status(0);

    /* The generated forward with the recommended and the minimum workspace
     * (one channel per chunk), its argument checks, and a failing launch. */
    {
        const size_t gr = hyenand_fftconv_fwd_generated_workspace_bytes(B, C, d, dims, dt);
        const size_t gm = hyenand_fftconv_fwd_generated_workspace_min_bytes(B, C, d, dims, dt);
        CHECK(gm >= wb && gr >= gm);
        unsigned char* graw = buf(gr + 512);
        unsigned char* gws = graw + (256 - (uintptr_t)graw % 256);
        void* y = buf(es * B * C * vox);
        float* al = buf(4 * (size_t)C);
        EXPECT(hyenand_fftconv_fwd_generated(x, al, al, &g, Kh, y, B, C, d, dims, dt, gws, gr, NULL), HYENAND_OK);
        EXPECT(hyenand_fftconv_fwd_generated(x, al, al, &g, Kh, y, B, C, d, dims, dt, gws, gm, NULL), HYENAND_OK);
        stub_set_launch_status(1);
        EXPECT(hyenand_fftconv_fwd_generated(x, al, al, &g, Kh, y, B, C, d, dims, dt, gws, gm, NULL), HYENAND_ERR_HIP);
        stub_set_launch_status(0);
        const long before = stub_launch_calls();
        EXPECT(hyenand_fftconv_fwd_generated(x, al, al, &g, Kh, y, B, C, d, dims, dt, gws, wb - 8, NULL),
               HYENAND_ERR_WORKSPACE);
        if (gm > wb)
            EXPECT(hyenand_fftconv_fwd_generated(x, al, al, &g, Kh, y, B, C, d, dims, dt, gws, gm - 8, NULL),
                   HYENAND_ERR_WORKSPACE);
        EXPECT(hyenand_fftconv_fwd_generated(x, NULL, al, &g, Kh, y, B, C, d, dims, dt, gws, gm, NULL),
               HYENAND_ERR_INVALID_ARG);
        EXPECT(hyenand_fftconv_fwd_generated(x, al, al, &g, Kh, NULL, B, C, d, dims, dt, gws, gm, NULL),
               HYENAND_ERR_INVALID_ARG);
        EXPECT(hyenand_fftconv_fwd_generated(x, al, al, NULL, Kh, y, B, C, d, dims, dt, gws, gm, NULL),
               HYENAND_ERR_INVALID_ARG);
        EXPECT(hyenand_fftconv_fwd_generated(x, al, al, &g, Kh, y, B, C, d, dims, dt, gws + 64, gm, NULL),
               HYENAND_ERR_INVALID_ARG);
        EXPECT(hyenand_fftconv_fwd_generated(NULL, NULL, NULL, &g, NULL, NULL, 0, C, d, dims, dt, NULL, 0, NULL),
               HYENAND_OK);
        CHECK(stub_launch_calls() == before);
        free(graw);
        free(y);
        free(al);
    }
    free((void*)g.Wreg); free((void*)g.breg); free((void*)g.q); free((void*)g.Wgam); free((void*)g.Wbet);
    free((void*)g.W1); free((void*)g.b1); free((void*)g.W2); free((void*)g.b2); free((void*)g.sigma);
    free(x); free(Kh); free(raw);
}

/* Argument checks that return before any launch. */
static void run_rejections(void)
{
    const int64_t d2[2] = {256, 8}, big1[1] = {(int64_t)1 << 25}, zero2[2] = {0, 8}, wide2[2] = {2048, 8},
                  odd2[2] = {30, 16};
    float al[4] = {0}, be[4] = {0};
    static float xbuf[256 * 8 + 4];
    static double khbuf[1 << 16];
    static double wbuf[1 << 16];
    void* x = xbuf;
    void* y = xbuf;
    const long before = stub_launch_calls();
    EXPECT(hyenand_fftconv_fwd(NULL, al, be, khbuf, y, 1, 1, 2, d2, HYENAND_F32, wbuf, sizeof wbuf, NULL),
           HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_fftconv_fwd(x, NULL, be, khbuf, y, 1, 1, 2, d2, HYENAND_F32, wbuf, sizeof wbuf, NULL),
           HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_fftconv_fwd(x, al, be, NULL, y, 1, 1, 2, d2, HYENAND_F32, wbuf, sizeof wbuf, NULL),
           HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_fftconv_fwd(x, al, be, khbuf, y, 1, 1, 2, d2, 7, wbuf, sizeof wbuf, NULL), HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_fftconv_fwd(x, al, be, khbuf, y, -1, 1, 2, d2, HYENAND_F32, wbuf, sizeof wbuf, NULL),
           HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_fftconv_fwd(x, al, be, khbuf, y, 1, -1, 2, d2, HYENAND_F32, wbuf, sizeof wbuf, NULL),
           HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_fftconv_fwd(x, al, be, khbuf, y, 1, 1, 0, d2, HYENAND_F32, wbuf, sizeof wbuf, NULL),
           HYENAND_ERR_UNSUPPORTED);
    EXPECT(hyenand_fftconv_fwd(x, al, be, khbuf, y, 1, 1, 4, d2, HYENAND_F32, wbuf, sizeof wbuf, NULL),
           HYENAND_ERR_UNSUPPORTED);
    EXPECT(hyenand_fftconv_fwd(x, al, be, khbuf, y, 1, 1, 2, NULL, HYENAND_F32, wbuf, sizeof wbuf, NULL),
           HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_fftconv_fwd(x, al, be, khbuf, y, 1, 1, 2, zero2, HYENAND_F32, wbuf, sizeof wbuf, NULL),
           HYENAND_ERR_UNSUPPORTED);
    EXPECT(hyenand_fftconv_fwd(x, al, be, khbuf, y, 1, 1, 2, wide2, HYENAND_F32, wbuf, sizeof wbuf, NULL),
           HYENAND_ERR_UNSUPPORTED);
    EXPECT(hyenand_fftconv_fwd(x, al, be, khbuf, y, 1, 1, 2, odd2, HYENAND_F32, wbuf, sizeof wbuf, NULL),
           HYENAND_ERR_UNSUPPORTED);
    EXPECT(hyenand_fftconv_fwd(x, al, be, khbuf, y, 1, 1, 1, big1, HYENAND_F32, wbuf, sizeof wbuf, NULL),
           HYENAND_ERR_UNSUPPORTED);
    EXPECT(hyenand_fftconv_fwd((char*)x + 2, al, be, khbuf, y, 1, 1, 2, d2, HYENAND_F32, wbuf, sizeof wbuf, NULL),
           HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_fftconv_fwd(x, al, be, (char*)khbuf + 4, y, 1, 1, 2, d2, HYENAND_F32, wbuf, sizeof wbuf, NULL),
           HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_fftconv_fwd(x, al, be, khbuf, y, 1, 1, 2, d2, HYENAND_F32, (char*)wbuf + 4, sizeof wbuf, NULL),
           HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_fftconv_fwd(NULL, NULL, NULL, NULL, NULL, 0, 3, 2, d2, HYENAND_F32, NULL, 0, NULL), HYENAND_OK);
    EXPECT(hyenand_fftconv_fwd(NULL, NULL, NULL, NULL, NULL, 3, 0, 2, d2, HYENAND_F32, NULL, 0, NULL), HYENAND_OK);
    EXPECT(hyenand_fftconv_fwd_traced(x, al, be, khbuf, y, 1, 1, 2, d2, HYENAND_F32, wbuf, sizeof wbuf, NULL, NULL,
                                      -1, NULL),
           HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_fftconv_fwd_traced(x, al, be, khbuf, y, 1, 1, 2, d2, HYENAND_F32, wbuf, sizeof wbuf, NULL, NULL,
                                      2, NULL),
           HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_fftconv_bwd(x, al, be, khbuf, x, y, NULL, be, NULL, 1, 1, 2, d2, HYENAND_F32, wbuf, sizeof wbuf,
                               NULL),
           HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_fftconv_bwd(x, al, be, khbuf, NULL, y, al, be, NULL, 1, 1, 2, d2, HYENAND_F32, wbuf, sizeof wbuf,
                               NULL),
           HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_kernel_spectrum(NULL, khbuf, 1, 2, d2, NULL), HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_kernel_spectrum(xbuf, khbuf, -1, 2, d2, NULL), HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_kernel_spectrum(xbuf, khbuf, 1, 5, d2, NULL), HYENAND_ERR_UNSUPPORTED);
    EXPECT(hyenand_kernel_spectrum(xbuf, khbuf, 1, 2, NULL, NULL), HYENAND_ERR_INVALID_ARG);
    EXPECT(hyenand_kernel_spectrum(xbuf, khbuf, 1, 2, wide2, NULL), HYENAND_ERR_UNSUPPORTED);
    CHECK(stub_launch_calls() == before);
    /* Without a GPU the allocation-free forward cannot find its static array. */
    CHECK(hyenand_fftconv_fwd_noalloc_max_workspace() > 0);
    EXPECT(hyenand_fftconv_fwd_noalloc(x, al, be, khbuf, y, 1, 1, 2, d2, HYENAND_F32, NULL), HYENAND_ERR_HIP);
    CHECK(stub_launch_calls() == before);
    CHECK(hyenand_kernel_spectrum_bytes(1, 2, wide2) == 0);
    CHECK(hyenand_fftconv_workspace_bytes(1, 1, 2, d2, 7) == 0);
    CHECK(hyenand_fftconv_workspace_bytes(0, 1, 2, d2, HYENAND_F32) == 0);
    CHECK(hyenand_generate_workspace_bytes(1, 1, 1, big1) == 0);
    for (int s = -1; s <= 5; ++s) CHECK(hyenand_status_string(s) != NULL);
    CHECK(hyenand_version() > 0);
}

int main(void)
{
    const shape_t shapes[] = {
        {1, {128}, 2, 3, HYENAND_F32, 0},          /* short 1-D: one launch, no workspace */
        {1, {1024}, 1, 2, HYENAND_BF16, 0},        /* the longest short 1-D line */
        {1, {4096}, 1, 2, HYENAND_F32, 0},         /* long 1-D (four-step) */
        {1, {1 << 16}, 2, 3, HYENAND_BF16, 0},     /* long 1-D, two batch entries */
        {2, {8, 8}, 2, 3, HYENAND_F32, 0},         /* on-chip 2-D */
        {2, {32, 16}, 2, 5, HYENAND_BF16, 0},      /* on-chip 2-D, unequal extents */
        {2, {256, 8}, 1, 2, HYENAND_F32, 0},       /* 512-point out-axis lines */
        {2, {4, 1024}, 3, 2, HYENAND_F32, 0},      /* 2048-point rows */
        {3, {8, 4, 16}, 2, 3, HYENAND_F32, 0},     /* 3-D, unequal extents */
        {3, {2, 2, 2}, 1, 1, HYENAND_BF16, 0},     /* smallest 3-D */
        {1, {64}, 2, 2, HYENAND_F32, 1},           /* circular 1-D */
        {2, {16, 8}, 2, 3, HYENAND_BF16, 1},       /* circular 2-D */
        {3, {4, 8, 4}, 1, 2, HYENAND_F32, 1},      /* circular 3-D */
    };
    const int n = (int)(sizeof shapes / sizeof shapes[0]);
    for (int i = 0; i < n; ++i) run_shape(&shapes[i]);
    for (int i = 0; i < n; ++i)
        if (!shapes[i].circ && !(shapes[i].d == 1 && shapes[i].dims[0] > 1024)) {
            run_per_sample(&shapes[i]);
            run_generator(&shapes[i], 4, 8);
        }
    run_generator(&shapes[8], 64, 64);
    run_rejections();
    if (stub_failures() > 0) {
        printf("%ld stand-in check(s) failed\n", stub_failures());
        ++g_bad;
    }
    printf("%s: %d failed expectation(s), %ld launches\n", g_bad ? "FAIL" : "ok", g_bad, stub_launch_calls());
    return g_bad ? 1 : 0;
}
