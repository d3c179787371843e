/*
 * hyenand.h -- C ABI of the gated N-D FFT convolution (HyenaND hot path) for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (explainer "Native multi-dimensional subquadratic operators via
 * input-dependent long convolutions", section "HyenaND: native-space implicit
 * global kernel", output equation for y[i]):
 *
 *     y[b,c,i] = sum_{j in G} phi_c(x[b,c,j]) * x[b,c,j] * K_c[i - j],   i in G,
 *     phi_c(v) = 1 / (1 + exp(-(alpha_c * v + beta_c))),
 *
 * over a native d-dimensional grid G = [0,n_0) x ... x [0,n_{d-1}), with the
 * non-circular boundary of the gist.science summary of the same paper
 * ("Methodology", "Boundary handling": every axis zero-padded to 2 n before the
 * FFT, the output cropped back to G).  The kernel is depthwise (one K_c per
 * channel, shared by the batch).  The evaluation route is the FFT convolution
 * path of the explainer's "Implementation" item: forward FFT, pointwise product
 * with the kernel spectrum, inverse FFT.
 *
 * Conventions shared by every entry point:
 *   - All array arguments are device pointers owned by the caller (e.g. torch
 *     tensors).  The library allocates nothing and keeps no state between calls
 *     (the one exception, hyenand_fftconv_fwd_noalloc at the end, holds a
 *     static device scratch array).
 *   - Layouts are row-major with the last grid axis contiguous:
 *       x, y   [B][C][dims[0]]..[dims[d-1]]     dtype HYENAND_F32 or HYENAND_BF16
 *       alpha, beta [C]                          fp32
 *       K      [C][2*dims[0]-1]..[2*dims[d-1]-1] fp32, offset 0 of each axis at
 *              index dims[a]-1 (K holds K_c[delta] for delta_a in [-(n_a-1), n_a-1])
 *       K_hat  library-defined complex64 layout, size from
 *              hyenand_kernel_spectrum_bytes (see below)
 *   - Supported shapes: d in {1, 2, 3}; every dims[a] a power of two in
 *     [2, 1024]; for d = 1 also n a power of two up to 2^24 (long signals, the
 *     summary's 1-D genomics context: see "Long 1-D signals" below).  Other
 *     shapes return HYENAND_ERR_UNSUPPORTED.
 *   - Pointers must be aligned to their element size (x, y: 4 bytes for fp32,
 *     2 for bf16; alpha, beta, K: 4; K_hat, workspace: 8).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default
 *     stream) and return once the kernels are enqueued.  Concurrent calls need
 *     distinct workspaces and outputs.  y must not alias x, K_hat or workspace.
 *   - Argument errors are detected before anything is enqueued.  A failed
 *     launch returns HYENAND_ERR_HIP.  No exception or abort crosses the ABI.
 *   - B == 0 or C == 0 is a valid empty call: HYENAND_OK, nothing enqueued.
 */
#ifndef HYENAND_H
#define HYENAND_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes of every entry point. */
#define HYENAND_OK 0
#define HYENAND_ERR_INVALID_ARG 1 /* null pointer, negative count, bad dtype, misaligned pointer */
#define HYENAND_ERR_UNSUPPORTED 2 /* shape outside the supported set                            */
#define HYENAND_ERR_WORKSPACE 3   /* workspace smaller than the minimum for the call             */
#define HYENAND_ERR_HIP 4         /* a kernel launch failed                                      */

/* I/O element types of x and y (the FFT arithmetic is always fp32). */
#define HYENAND_F32 0
#define HYENAND_BF16 1

/* Static description of a return code. */
const char* hyenand_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int hyenand_version(void);

/*
 * Bytes of the kernel spectrum K_hat for C channels of a grid `dims`.  0 for an
 * unsupported shape.  Layout, per channel (complex64 = two fp32, real first),
 * with N_a = 2 n_a and (out, mid, in) = the grid axes (3-D), (axis 0, -, axis 1)
 * (2-D) or (-, -, axis 0) (1-D), absent axes of length 1, S = N_in / 2, and
 * T = hyenand_kernel_spectrum_tile(d, dims) (a power of two dividing S):
 *   main, N_out * N_mid * S values, slot-tile-major: the value for
 *     (k_out, k_mid, k_in) sits at ((k_in / T) * N_out * N_mid
 *                                   + k_out * N_mid + k_mid) * T + k_in % T,
 *     holding  g * Khat(k)                           for k_in >= 1,
 *              g * (Khat(k,0) + Khat(k,S)) / 2       for k_in = 0;
 *   then dblk[k_out][k_mid]:  g * (Khat(k,0) - Khat(k,S)) / 2,
 * where Khat is the DFT over the padded grid of the kernel placed at offset
 * delta -> index delta mod N_a, and g = 1 / (2 * prod_a N_a).  (For d = 1 the
 * main block is simply [k_in].)  The slot tiles make each out-axis workgroup's
 * block of the spectrum contiguous.
 *
 * Long 1-D signals (d = 1, n > 1024): the padded length N = 2n is transformed
 * as an N1 x N2 array, N2 = min(N/4, 2048) for N <= 2^22, 4096 up to 2^24
 * and 8192 for N = 2^25, N1 = N / N2 (sample m = N2 n1 + n2;
 * column transforms of N1 points, twiddle W_N^(n2 k1), row transforms of N2
 * points).  K_hat holds N complex values per channel, the value of frequency
 * k = k1 + N1 k2 at [k1][k2], equal to Khat(k) / N (no Nyquist packing).  The
 * workspace minimum is B * N * 8 bytes (one channel).  The backward takes
 * long signals (the same decomposition, run backwards for du and the kernel
 * gradient); the circular mode does not (UNSUPPORTED).
 */
size_t hyenand_kernel_spectrum_bytes(int C, int d, const int64_t* dims);

/*
 * Slot tile T of the K_hat layout above for a grid `dims` (0 for an
 * unsupported shape).
 */
int hyenand_kernel_spectrum_tile(int d, const int64_t* dims);

/*
 * Kernel spectrum precompute (once per parameter set; not part of the timed
 * forward): wrap-place each K_c into the zero-padded grid, real N-D FFT, fold
 * the normalisation.  K: device fp32 [C][2n-1 ...]; K_hat: device, at least
 * hyenand_kernel_spectrum_bytes(C, d, dims) bytes, fully overwritten.
 * Errors: INVALID_ARG (null pointer with C > 0, C < 0, misalignment),
 * UNSUPPORTED (shape), HIP (launch).
 */
int hyenand_kernel_spectrum(const float* K, void* K_hat, int C, int d, const int64_t* dims, void* stream);

/*
 * Workspace bytes recommended for hyenand_fftconv_fwd: whole channels (all B
 * batch entries of a channel are processed together) up to about 256 MiB.  The
 * minimum accepted is one channel, B * n_0 * (prod of the middle padded axes) *
 * S * 8 bytes (0 for d = 1); a larger workspace processes more channels per
 * kernel chain.  0 for d = 1, for an empty call, or for an unsupported shape.
 */
size_t hyenand_fftconv_workspace_bytes(int B, int C, int d, const int64_t* dims, int dtype);

/* Minimum workspace bytes (one channel); 0 when none is needed. */
size_t hyenand_fftconv_workspace_min_bytes(int B, int C, int d, const int64_t* dims, int dtype);

/*
 * Forward gated convolution:  y = crop(IFFT(FFT(pad(phi(x) * x)) * Khat)).
 * x, y: device [B][C][dims], dtype `dtype` (bf16 is widened exactly to fp32 on
 * load and rounded to nearest even on store).  phi_alpha, phi_beta: device fp32
 * [C].  K_hat: from hyenand_kernel_spectrum for the same C, d, dims.
 * workspace: device scratch of workspace_bytes >= the minimum (unused and may be
 * NULL for d = 1); its contents on entry and exit are unspecified.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE (too small), HIP.
 */
int hyenand_fftconv_fwd(const void* x, const float* phi_alpha, const float* phi_beta, const void* K_hat, void* y,
                        int B, int C, int d, const int64_t* dims, int dtype, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * How hyenand_fftconv_fwd would run with this workspace size: *n_launches
 * kernel launches and *chunk_channels channels per chunk (chunks are balanced).
 * Either output pointer may be NULL.  Errors as hyenand_fftconv_fwd's argument
 * checks (no data pointers are examined).
 */
int hyenand_fftconv_launch_plan(int B, int C, int d, const int64_t* dims, int dtype, size_t workspace_bytes,
                                int* n_launches, int* chunk_channels);

/*
 * hyenand_fftconv_fwd with a launch trace, for measurement.  Arguments and
 * errors as hyenand_fftconv_fwd, plus: events[k] (caller-created hipEvent_t,
 * cast to void*) is recorded on `stream` before the k-th kernel launch of the
 * call and once more after the last launch, for k < n_events (extra launches
 * are not recorded).  The kernels of one channel chunk run in this order:
 * d = 1: conv1d;  d = 2: row_fwd, col_out, row_inv;  d = 3: row_fwd,
 * col_mid_fwd, col_out, col_mid_inv, row_inv.  *n_launches (may be NULL)
 * receives the number of launches.  n_events < 0, or events NULL with
 * n_events > 0, is INVALID_ARG.
 */
int hyenand_fftconv_fwd_traced(const void* x, const float* phi_alpha, const float* phi_beta, const void* K_hat,
                               void* y, int B, int C, int d, const int64_t* dims, int dtype, void* workspace,
                               size_t workspace_bytes, void* stream, void* const* events, int n_events,
                               int* n_launches);

/*
 * Backward (vector-Jacobian product) of hyenand_fftconv_fwd.  The explainer's
 * autograd pattern ("Implementation and operation patterns", item "Concrete
 * implementation pattern (PyTorch)") saves only the input and the kernel
 * parameters and recomputes the forward transforms in the backward; this call
 * does exactly that.  With dy = dLoss/dy and u = s x, s = sigmoid(alpha x + beta):
 *
 *     du[j]    = sum_{i in G} dy[i] K[i - j]              (correlation with K)
 *     dx[j]    = du[j] (s + alpha x s (1 - s))
 *     dalpha_c = sum_{b,j} du x^2 s (1 - s),    dbeta_c = sum_{b,j} du x s (1 - s)
 *     dK_c[l]  = sum_b sum_{j in G, j+l in G} dy[j+l] u[j]   for every offset l of K
 *
 * evaluated as conj(K_hat) products and Sum_b FFT(dy) conj(FFT(u)) on the same
 * zero-padded grid.  x, dy, dx: device [B][C][dims] of `dtype`; dx is written.
 * phi_alpha, phi_beta, K_hat: as for the forward.  dalpha, dbeta: device fp32
 * [C], overwritten.  dK: device fp32 [C][2n-1 ...] (the layout of K),
 * overwritten; NULL skips the kernel gradient (and its workspace).  dx must
 * not alias x, dy, K_hat or the workspace.  The sums over the batch are taken
 * in a fixed order (bit-identical results from call to call).  B == 0 with
 * C > 0 writes zeros to dalpha, dbeta and dK.  workspace: device scratch of at
 * least hyenand_fftconv_bwd_workspace_min_bytes (with_dK = dK != NULL);
 * contents unspecified on entry and exit.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE (too small or NULL), HIP.
 */
int hyenand_fftconv_bwd(const void* x, const float* phi_alpha, const float* phi_beta, const void* K_hat,
                        const void* dy, void* dx, float* dalpha, float* dbeta, float* dK, int B, int C, int d,
                        const int64_t* dims, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward workspace bytes: recommended (whole channels up to about 512 MiB)
 * and minimum (one channel).  Per channel: B * n_0 * (prod of the middle padded
 * axes) * S complex for the output-gradient planes, the same again plus the
 * kernel-gradient spectrum (N_out N_mid S complex, or B S for d = 1) when
 * with_dK, and 8 bytes per line pair for the partial sums.  0 for an empty
 * call or an unsupported shape.
 */
size_t hyenand_fftconv_bwd_workspace_bytes(int B, int C, int d, const int64_t* dims, int dtype, int with_dK);
size_t hyenand_fftconv_bwd_workspace_min_bytes(int B, int C, int d, const int64_t* dims, int dtype, int with_dK);

/*
 * hyenand_fftconv_bwd with a launch trace (events as for
 * hyenand_fftconv_fwd_traced).  Kernels of one channel chunk, in order:
 * d = 1: conv1d_bwd, gate_reduce[, corr1d, dk_row];  d = 2: row_fwd(dy)
 * [, row_fwd(u)], col_out_bwd, row_inv_bwd, gate_reduce[, dk_row];  d = 3:
 * row_fwd(dy)[, row_fwd(u)], col_mid_fwd(dy)[, col_mid_fwd(u)], col_out_bwd,
 * col_mid_inv, row_inv_bwd, gate_reduce[, mid_inv(dK), dk_row]  (bracketed:
 * only with dK).
 */
int hyenand_fftconv_bwd_traced(const void* x, const float* phi_alpha, const float* phi_beta, const void* K_hat,
                               const void* dy, void* dx, float* dalpha, float* dbeta, float* dK, int B, int C,
                               int d, const int64_t* dims, int dtype, void* workspace, size_t workspace_bytes,
                               void* stream, void* const* events, int n_events, int* n_launches);

/*
 * Circular mode.  The gist.science summary of the paper ("Methodology",
 * "Boundary handling") gives the method circular convolutions for periodic
 * physical systems next to the zero-padded non-circular ones.  On a periodic
 * grid the offset i - j is taken modulo n:
 *
 *     y[b,c,i] = sum_{j in G} phi_c(x[b,c,j]) x[b,c,j] K_c[(i - j) mod n],
 *
 * with the kernel stored by offset modulo n: K  [C][dims[0]]..[dims[d-1]] fp32,
 * index m_a = delta_a mod n_a (offset 0 at index 0).  The transforms have
 * length N_a = n_a (no padding, no crop).  Supported: d in {1, 2, 3}, every
 * dims[a] a power of two in [4, 1024].  The entry points mirror the
 * non-circular ones (same conventions, errors and K_hat layout, with N_a = n_a
 * and S = n_in / 2); a circular K_hat must only be used with
 * hyenand_fftconv_fwd_circ and hyenand_fftconv_bwd_circ.  The minimum workspace is one channel,
 * B * n_0 * (n_1 for 3-D) * S * 8 bytes (0 for d = 1).
 */
size_t hyenand_kernel_spectrum_circ_bytes(int C, int d, const int64_t* dims);
int hyenand_kernel_spectrum_circ_tile(int d, const int64_t* dims);
int hyenand_kernel_spectrum_circ(const float* K, void* K_hat, int C, int d, const int64_t* dims, void* stream);
size_t hyenand_fftconv_circ_workspace_bytes(int B, int C, int d, const int64_t* dims, int dtype);
size_t hyenand_fftconv_circ_workspace_min_bytes(int B, int C, int d, const int64_t* dims, int dtype);
int hyenand_fftconv_fwd_circ(const void* x, const float* phi_alpha, const float* phi_beta, const void* K_hat, void* y,
                             int B, int C, int d, const int64_t* dims, int dtype, void* workspace,
                             size_t workspace_bytes, void* stream);
/*
 * Backward of the circular mode: hyenand_fftconv_bwd with offsets modulo n,
 *   du[j] = sum_i dy[i] K[(i - j) mod n],  dK_c[m] = sum_b sum_j dy[(j + m) mod n] u[j],
 * dK laid out like the circular K ([C][dims], index = offset mod n); K_hat from
 * hyenand_kernel_spectrum_circ.  Arguments, workspace rules and errors as for
 * hyenand_fftconv_bwd, with the workspace sized by the _circ_ queries below.
 */
int hyenand_fftconv_bwd_circ(const void* x, const float* phi_alpha, const float* phi_beta, const void* K_hat,
                             const void* dy, void* dx, float* dalpha, float* dbeta, float* dK, int B, int C, int d,
                             const int64_t* dims, int dtype, void* workspace, size_t workspace_bytes, void* stream);
size_t hyenand_fftconv_bwd_circ_workspace_bytes(int B, int C, int d, const int64_t* dims, int dtype, int with_dK);
size_t hyenand_fftconv_bwd_circ_workspace_min_bytes(int B, int C, int d, const int64_t* dims, int dtype,
                                                    int with_dK);
/* hyenand_fftconv_bwd_circ with the launch trace of hyenand_fftconv_fwd_traced. */
int hyenand_fftconv_bwd_circ_traced(const void* x, const float* phi_alpha, const float* phi_beta,
                                    const void* K_hat, const void* dy, void* dx, float* dalpha, float* dbeta,
                                    float* dK, int B, int C, int d, const int64_t* dims, int dtype, void* workspace,
                                    size_t workspace_bytes, void* stream, void* const* events, int n_events,
                                    int* n_launches);
/* hyenand_fftconv_fwd_circ with the launch trace of hyenand_fftconv_fwd_traced. */
int hyenand_fftconv_fwd_circ_traced(const void* x, const float* phi_alpha, const float* phi_beta,
                                    const void* K_hat, void* y, int B, int C, int d, const int64_t* dims, int dtype,
                                    void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                                    int n_events, int* n_launches);

/*
 * Input-dependent kernels.  The gist.science summary ("Methodology", "Input
 * dependent kernels via registers and FiLM", "Kernel synthesis") conditions
 * the kernel on the whole input sample, K(x) = w(c) * f(c; z(x)), so every
 * batch entry has its own kernel while the FFT path stays the same:
 *
 *     y[b,c,i] = sum_{j in G} phi_c(x[b,c,j]) x[b,c,j] K_{b,c}[i - j].
 *
 * K_hat here holds B * C spectra in the order [B][C]: it is the output of
 * hyenand_kernel_spectrum called on the kernels [B * C][2n-1 ...] (batch entry
 * major), hyenand_kernel_spectrum_bytes(B * C, d, dims) bytes.  Everything
 * else (arguments, workspace, errors) is as for hyenand_fftconv_fwd; the
 * zero-padded boundary only.
 */
int hyenand_fftconv_fwd_per_sample(const void* x, const float* phi_alpha, const float* phi_beta, const void* K_hat,
                                   void* y, int B, int C, int d, const int64_t* dims, int dtype, void* workspace,
                                   size_t workspace_bytes, void* stream);
/* hyenand_fftconv_fwd_per_sample with the launch trace of hyenand_fftconv_fwd_traced. */
int hyenand_fftconv_fwd_per_sample_traced(const void* x, const float* phi_alpha, const float* phi_beta,
                                          const void* K_hat, void* y, int B, int C, int d, const int64_t* dims,
                                          int dtype, void* workspace, size_t workspace_bytes, void* stream,
                                          void* const* events, int n_events, int* n_launches);

/*
 * Backward with input-dependent kernels: the gradients of
 * y[b,c,i] = sum_j phi_c(x[b,c,j]) x[b,c,j] K_{b,c}[i - j] for the output
 * gradient dy, by the chain rule as for hyenand_fftconv_bwd but with each
 * batch entry's own kernel:
 *   du[b,c,j] = sum_i dy[b,c,i] K_{b,c}[i - j],  dK_{b,c}[l] = sum_j dy[b,c,j+l] u[b,c,j],
 * dalpha_c and dbeta_c summed over the batch.  K_hat: the [B][C] spectra of
 * hyenand_fftconv_fwd_per_sample.  dK (nullable): fp32 [B][C][2n_0-1]..[2n_{d-1}-1],
 * one kernel gradient per (b, c), every element written.  The batch entries
 * run one after the other, each as a batch of one, so the workspace is sized
 * by hyenand_fftconv_bwd_workspace_bytes(1, C, ...) (any size from the
 * _min_bytes of B = 1 upward works).  Other arguments, errors and limits as for
 * hyenand_fftconv_bwd (zero-padded boundary).
 */
int hyenand_fftconv_bwd_per_sample(const void* x, const float* phi_alpha, const float* phi_beta, const void* K_hat,
                                   const void* dy, void* dx, float* dalpha, float* dbeta, float* dK, int B, int C,
                                   int d, const int64_t* dims, int dtype, void* workspace, size_t workspace_bytes,
                                   void* stream);
/* hyenand_fftconv_bwd_per_sample with the launch trace of hyenand_fftconv_fwd_traced. */
int hyenand_fftconv_bwd_per_sample_traced(const void* x, const float* phi_alpha, const float* phi_beta,
                                          const void* K_hat, const void* dy, void* dx, float* dalpha, float* dbeta,
                                          float* dK, int B, int C, int d, const int64_t* dims, int dtype,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          void* const* events, int n_events, int* n_launches);

/*
 * Input-dependent kernels generated on the GPU, straight into their spectra
 * (gist.science summary, "Methodology": R register tokens that take in the
 * whole sample, a control variable z(x) as their softmax-weighted mean, a
 * coordinate SIREN modulated by FiLM, and K(x) = w(c) (.) f(c; z(x)) with a
 * Gaussian window w).  For every sample b and channel c:
 *   m[c]   = mean of x[b,c] over the grid
 *   a[r]   = tanh(Wreg[r] m + breg[r])            r < R, width D   (Wreg [R][D][C])
 *   z      = sum_r softmax_r(q . a[r]) a[r]
 *   gam    = 1 + Wgam z,  bet = Wbet z            (16 each; Wgam, Wbet [16][D])
 *   K[b,c](delta) = exp(-|delta|^2 / (2 sigma_c^2))
 *                   (sum_u W2[c][u] (gam_u sin(omega0 (W1[u] . chat + b1[u])) + bet_u) + b2[c])
 * for offsets delta_a in [-(n_a-1), n_a-1], chat_a = delta_a / (n_a - 1),
 * 16 hidden units (W1 [16][d], b1 [16], W2 [C][16], b2 [C], sigma [C]).
 * The kernels are never formed in space: K_hat receives their spectra, B * C
 * of them in the layout of hyenand_kernel_spectrum on [B*C] kernels, ready for
 * hyenand_fftconv_fwd_per_sample / _bwd_per_sample.  All parameter arrays are
 * fp32 device pointers.  Zero-padded mode, d in {1, 2, 3}, every n in
 * [2, 1024] (not the long 1-D path: UNSUPPORTED); 1 <= R, D <= 64, C <= 8192; B C
 * (N_out N_mid / 128) below 2^31 (else UNSUPPORTED).  Workspace:
 * hyenand_generate_workspace_bytes (partial sums of the means, per-pair
 * coefficients and the channels' 1-D axis spectra).  Errors as
 * hyenand_fftconv_fwd.
 */
#define HYENAND_GEN_HIDDEN 16
typedef struct hyenand_generator {
    int R, D;           /* registers, control width                                  */
    const float* Wreg;  /* [R][D][C]                                                 */
    const float* breg;  /* [R][D]                                                    */
    const float* q;     /* [D]     softmax scores q . a[r]                           */
    const float* Wgam;  /* [16][D] FiLM scale 1 + Wgam z                             */
    const float* Wbet;  /* [16][D] FiLM shift Wbet z                                 */
    const float* W1;    /* [16][d] SIREN first layer on the normalised offsets       */
    const float* b1;    /* [16]                                                      */
    const float* W2;    /* [C][16] per-channel read-out                              */
    const float* b2;    /* [C]                                                       */
    const float* sigma; /* [C]     Gaussian window width (voxels)                    */
    float omega0;       /* SIREN frequency                                           */
} hyenand_generator;
size_t hyenand_generate_workspace_bytes(int B, int C, int d, const int64_t* dims);
int hyenand_generate_kernel_spectrum(const void* x, const hyenand_generator* gen, void* K_hat, int B, int C, int d,
                                     const int64_t* dims, int dtype, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * Forward with the input-dependent kernels generated in the same call (the
 * explainer has the input-dependent parameters computed on the fly, nSubQ
 * implementation, item on the input-dependent parameterisation overhead): the
 * generator of hyenand_generate_kernel_spectrum writes every (b, c) spectrum
 * into K_hat, then the forward chains read them, all on `stream`.  Results
 * equal hyenand_generate_kernel_spectrum followed by
 * hyenand_fftconv_fwd_per_sample, bit for bit.
 * x, y, phi_alpha, phi_beta, dtype: as hyenand_fftconv_fwd.  gen: as
 * hyenand_generate_kernel_spectrum (same shapes).  K_hat: device
 * [B][C] spectra of hyenand_kernel_spectrum_bytes(B * C, d, dims) bytes,
 * written (the per-sample backward takes it).  workspace: 256-byte aligned,
 * at least hyenand_fftconv_fwd_generated_workspace_min_bytes (the generator's
 * region, then the forward's); hyenand_fftconv_fwd_generated_workspace_bytes
 * is the recommended size.  Contents unspecified on entry and exit.
 * Errors as hyenand_generate_kernel_spectrum and hyenand_fftconv_fwd.
 */
size_t hyenand_fftconv_fwd_generated_workspace_bytes(int B, int C, int d, const int64_t* dims, int dtype);
size_t hyenand_fftconv_fwd_generated_workspace_min_bytes(int B, int C, int d, const int64_t* dims, int dtype);
int hyenand_fftconv_fwd_generated(const void* x, const float* phi_alpha, const float* phi_beta,
                                  const hyenand_generator* gen, void* K_hat, void* y, int B, int C, int d,
                                  const int64_t* dims, int dtype, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): hyenand_fftconv_fwd with its workspace in a static device array
 * of hyenand_fftconv_fwd_noalloc_max_workspace() bytes (64 MiB) that the
 * library holds on every GPU it runs on until the process ends; the call
 * itself allocates and frees nothing.  The caller passes inputs and outputs as
 * for hyenand_fftconv_fwd (same layouts, errors and results).  Channels run
 * in chunks that fit the array; a shape whose single channel (all B batch
 * entries) needs more than the array (hyenand_fftconv_workspace_min_bytes
 * above the maximum, e.g. the 512^3 grid) returns HYENAND_ERR_WORKSPACE before
 * anything is enqueued.  Every call on a GPU shares that GPU's array (which
 * keeps the last call's contents; the forward writes every workspace value
 * before reading it), so calls that overlap in time on one GPU (other streams,
 * other host threads) race: serialise them.  The first call on a device looks
 * up the array's device address (HYENAND_ERR_HIP if that fails).
 */
size_t hyenand_fftconv_fwd_noalloc_max_workspace(void);
int hyenand_fftconv_fwd_noalloc(const void* x, const float* phi_alpha, const float* phi_beta, const void* K_hat,
                                void* y, int B, int C, int d, const int64_t* dims, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HYENAND_H */
