// api.cpp -- the C ABI declared in include/hyenand.h: argument validation,
// workspace sizing, chunking over channels, launch and error mapping.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/hyenand.h"
#include "gen.h"
#include "launch.h"
#include "plan.h"

using namespace hyenand;

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// How a forward call is split into channel chunks (the kernel chain runs once
// per chunk).  Chunks are balanced so that the last one is not a sliver.
struct CallPlan {
    int per;        // channels per chunk
    int chunks;
    int launches;
};

CallPlan plan_call(const Geom& g, int B, int C, size_t ws_bytes)
{
    CallPlan cp{C, 1, 1};
    if ((g.d == 1 && !g.lng) || fused2d_fits(g)) return cp;  // one launch for every pair, no workspace
    int per = chunk_channels(g, B, C, ws_bytes);
    if (per > C) per = C;
    if (per < 1) per = 1;
    const int chunks = (C + per - 1) / per;
    cp.per = (C + chunks - 1) / chunks;
    cp.chunks = (C + cp.per - 1) / cp.per;
    cp.launches = cp.chunks * (g.d == 3 ? 5 : 3);  // long 1-D: column, row, column
    return cp;
}

}  // namespace

extern "C" {

const char* hyenand_status_string(int s)
{
    switch (s) {
    case HYENAND_OK: return "ok";
    case HYENAND_ERR_INVALID_ARG: return "invalid argument";
    case HYENAND_ERR_UNSUPPORTED: return "unsupported shape";
    case HYENAND_ERR_WORKSPACE: return "workspace too small";
    case HYENAND_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
    }
}

int hyenand_version(void) { return 100; }

static size_t spectrum_bytes(int C, int d, const int64_t* dims, bool circ)
{
    Geom g;
    if (C < 0 || !make_geom(d, dims, &g, circ)) return 0;
    return (size_t)C * (size_t)g.ksz * 8u;
}

static int spectrum_tile(int d, const int64_t* dims, bool circ)
{
    Geom g;
    if (!make_geom(d, dims, &g, circ)) return 0;
    return g.lt;
}

size_t hyenand_kernel_spectrum_bytes(int C, int d, const int64_t* dims) { return spectrum_bytes(C, d, dims, false); }
int hyenand_kernel_spectrum_tile(int d, const int64_t* dims) { return spectrum_tile(d, dims, false); }
size_t hyenand_kernel_spectrum_circ_bytes(int C, int d, const int64_t* dims) { return spectrum_bytes(C, d, dims, true); }
int hyenand_kernel_spectrum_circ_tile(int d, const int64_t* dims) { return spectrum_tile(d, dims, true); }

static int kernel_spectrum_impl(const float* K, void* K_hat, int C, int d, const int64_t* dims, void* stream,
                                bool circ)
{
    if (C < 0) return HYENAND_ERR_INVALID_ARG;
    if (d < 1 || d > 3 || !dims) return d < 1 || d > 3 ? HYENAND_ERR_UNSUPPORTED : HYENAND_ERR_INVALID_ARG;
    Geom g;
    if (!make_geom(d, dims, &g, circ)) return HYENAND_ERR_UNSUPPORTED;
    if (C == 0) return HYENAND_OK;
    if (!K || !K_hat) return HYENAND_ERR_INVALID_ARG;
    if (!aligned(K, 4) || !aligned(K_hat, 8)) return HYENAND_ERR_INVALID_ARG;
    ConvArgs a{};
    a.K = K;
    a.khat = static_cast<const float2*>(K_hat);
    a.g = g;
    a.B = 1;
    a.C = C;
    a.c0 = 0;
    a.nch = C;
    hipError_t e = launch_spectrum(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HYENAND_OK : HYENAND_ERR_HIP;
}

int hyenand_kernel_spectrum(const float* K, void* K_hat, int C, int d, const int64_t* dims, void* stream)
{
    return kernel_spectrum_impl(K, K_hat, C, d, dims, stream, false);
}

int hyenand_kernel_spectrum_circ(const float* K, void* K_hat, int C, int d, const int64_t* dims, void* stream)
{
    return kernel_spectrum_impl(K, K_hat, C, d, dims, stream, true);
}

static size_t workspace_bytes(int B, int C, int d, const int64_t* dims, int dtype, bool circ, bool minimum)
{
    Geom g;
    if (B <= 0 || C <= 0 || (dtype != HYENAND_F32 && dtype != HYENAND_BF16) || !make_geom(d, dims, &g, circ)) return 0;
    if (fused2d_fits(g)) return 0;  // the on-chip 2-D forward needs none
    return minimum ? (size_t)B * (size_t)g.wsp * 8u : recommended_workspace(g, B, C);
}

size_t hyenand_fftconv_workspace_bytes(int B, int C, int d, const int64_t* dims, int dtype)
{
    return workspace_bytes(B, C, d, dims, dtype, false, false);
}

size_t hyenand_fftconv_workspace_min_bytes(int B, int C, int d, const int64_t* dims, int dtype)
{
    return workspace_bytes(B, C, d, dims, dtype, false, true);
}

size_t hyenand_fftconv_circ_workspace_bytes(int B, int C, int d, const int64_t* dims, int dtype)
{
    return workspace_bytes(B, C, d, dims, dtype, true, false);
}

size_t hyenand_fftconv_circ_workspace_min_bytes(int B, int C, int d, const int64_t* dims, int dtype)
{
    return workspace_bytes(B, C, d, dims, dtype, true, true);
}

// resolve_ws (optional): supplies the workspace once the arguments are valid
// (the allocation-free entry point's static scratch).
static int fftconv_fwd_impl(const void* x, const float* alpha, const float* beta, const void* K_hat, void* y, int B,
                            int C, int d, const int64_t* dims, int dtype, void* workspace, size_t workspace_bytes,
                            void* stream, LaunchTrace* trace, bool circ, bool per_sample = false,
                            int (*resolve_ws)(void**, size_t*) = nullptr)
{
    if (B < 0 || C < 0) return HYENAND_ERR_INVALID_ARG;
    if (dtype != HYENAND_F32 && dtype != HYENAND_BF16) return HYENAND_ERR_INVALID_ARG;
    if (d < 1 || d > 3) return HYENAND_ERR_UNSUPPORTED;
    if (!dims) return HYENAND_ERR_INVALID_ARG;
    Geom g;
    if (!make_geom(d, dims, &g, circ)) return HYENAND_ERR_UNSUPPORTED;
    if (B == 0 || C == 0) return HYENAND_OK;
    const size_t es = dtype == HYENAND_BF16 ? 2 : 4;
    if (!x || !y || !alpha || !beta || !K_hat) return HYENAND_ERR_INVALID_ARG;
    if (!aligned(x, es) || !aligned(y, es) || !aligned(alpha, 4) || !aligned(beta, 4) || !aligned(K_hat, 8))
        return HYENAND_ERR_INVALID_ARG;
    if (resolve_ws) {
        const int rc = resolve_ws(&workspace, &workspace_bytes);
        if (rc != HYENAND_OK) return rc;
    }
    if (g.wsp > 0 && !fused2d_fits(g)) {
        if (!workspace) return HYENAND_ERR_WORKSPACE;
        if (!aligned(workspace, 8)) return HYENAND_ERR_INVALID_ARG;
        if (chunk_channels(g, B, C, workspace_bytes) < 1) return HYENAND_ERR_WORKSPACE;
    }
    const CallPlan cp = plan_call(g, B, C, workspace_bytes);
    ConvArgs a{};
    a.x = x;
    a.y = y;
    a.alpha = alpha;
    a.beta = beta;
    a.khat = static_cast<const float2*>(K_hat);
    a.khat_bstride = per_sample ? (long long)C * g.ksz : 0;
    a.ws = static_cast<float2*>(workspace);
    a.g = g;
    a.B = B;
    a.C = C;
    a.bf16 = dtype == HYENAND_BF16;
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (int c0 = 0; c0 < C; c0 += cp.per) {
        a.c0 = c0;
        a.nch = (C - c0) < cp.per ? (C - c0) : cp.per;
        if (launch_forward_chunk(a, st, trace) != hipSuccess) return HYENAND_ERR_HIP;
    }
    if (trace) trace->mark(st);
    return HYENAND_OK;
}

int hyenand_fftconv_fwd(const void* x, const float* alpha, const float* beta, const void* K_hat, void* y, int B,
                        int C, int d, const int64_t* dims, int dtype, void* workspace, size_t workspace_bytes,
                        void* stream)
{
    return fftconv_fwd_impl(x, alpha, beta, K_hat, y, B, C, d, dims, dtype, workspace, workspace_bytes, stream,
                            nullptr, false);
}

int hyenand_fftconv_fwd_circ(const void* x, const float* alpha, const float* beta, const void* K_hat, void* y, int B,
                             int C, int d, const int64_t* dims, int dtype, void* workspace, size_t workspace_bytes,
                             void* stream)
{
    return fftconv_fwd_impl(x, alpha, beta, K_hat, y, B, C, d, dims, dtype, workspace, workspace_bytes, stream,
                            nullptr, true);
}

int hyenand_fftconv_launch_plan(int B, int C, int d, const int64_t* dims, int dtype, size_t workspace_bytes,
                                int* n_launches, int* chunk_channels_out)
{
    if (B < 0 || C < 0 || (dtype != HYENAND_F32 && dtype != HYENAND_BF16)) return HYENAND_ERR_INVALID_ARG;
    if (!dims) return d < 1 || d > 3 ? HYENAND_ERR_UNSUPPORTED : HYENAND_ERR_INVALID_ARG;
    Geom g;
    if (!make_geom(d, dims, &g)) return HYENAND_ERR_UNSUPPORTED;
    CallPlan cp{0, 0, 0};
    if (B > 0 && C > 0) {
        if (g.wsp > 0 && !fused2d_fits(g) && chunk_channels(g, B, C, workspace_bytes) < 1)
            return HYENAND_ERR_WORKSPACE;
        cp = plan_call(g, B, C, workspace_bytes);
    }
    if (n_launches) *n_launches = cp.launches;
    if (chunk_channels_out) *chunk_channels_out = cp.per;
    return HYENAND_OK;
}

int hyenand_fftconv_fwd_traced(const void* x, const float* alpha, const float* beta, const void* K_hat, void* y,
                               int B, int C, int d, const int64_t* dims, int dtype, void* workspace,
                               size_t workspace_bytes, void* stream, void* const* events, int n_events,
                               int* n_launches)
{
    if (n_events < 0 || (n_events > 0 && !events)) return HYENAND_ERR_INVALID_ARG;
    LaunchTrace tr{reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)), n_events, 0};
    const int rc = fftconv_fwd_impl(x, alpha, beta, K_hat, y, B, C, d, dims, dtype, workspace, workspace_bytes,
                                    stream, &tr, false);
    if (n_launches) *n_launches = tr.count > 0 ? tr.count - 1 : 0;
    return rc;
}

int hyenand_fftconv_fwd_circ_traced(const void* x, const float* alpha, const float* beta, const void* K_hat, void* y,
                                    int B, int C, int d, const int64_t* dims, int dtype, void* workspace,
                                    size_t workspace_bytes, void* stream, void* const* events, int n_events,
                                    int* n_launches)
{
    if (n_events < 0 || (n_events > 0 && !events)) return HYENAND_ERR_INVALID_ARG;
    LaunchTrace tr{reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)), n_events, 0};
    const int rc = fftconv_fwd_impl(x, alpha, beta, K_hat, y, B, C, d, dims, dtype, workspace, workspace_bytes,
                                    stream, &tr, true);
    if (n_launches) *n_launches = tr.count > 0 ? tr.count - 1 : 0;
    return rc;
}

// ------------------------------------------------------------------ backward
static size_t bwd_workspace(int B, int C, int d, const int64_t* dims, int dtype, int with_dK, bool circ, bool minimum)
{
    Geom g;
    if (B <= 0 || C <= 0 || (dtype != HYENAND_F32 && dtype != HYENAND_BF16) || !make_geom(d, dims, &g, circ))
        return 0;
    return minimum ? bwd_channel_bytes(g, B, with_dK != 0) : recommended_bwd_workspace(g, B, C, with_dK != 0);
}

size_t hyenand_fftconv_bwd_workspace_bytes(int B, int C, int d, const int64_t* dims, int dtype, int with_dK)
{
    return bwd_workspace(B, C, d, dims, dtype, with_dK, false, false);
}

size_t hyenand_fftconv_bwd_workspace_min_bytes(int B, int C, int d, const int64_t* dims, int dtype, int with_dK)
{
    return bwd_workspace(B, C, d, dims, dtype, with_dK, false, true);
}

size_t hyenand_fftconv_bwd_circ_workspace_bytes(int B, int C, int d, const int64_t* dims, int dtype, int with_dK)
{
    return bwd_workspace(B, C, d, dims, dtype, with_dK, true, false);
}

size_t hyenand_fftconv_bwd_circ_workspace_min_bytes(int B, int C, int d, const int64_t* dims, int dtype, int with_dK)
{
    return bwd_workspace(B, C, d, dims, dtype, with_dK, true, true);
}

static int fftconv_bwd_impl(const void* x, const float* alpha, const float* beta, const void* K_hat, const void* dy,
                            void* dx, float* dalpha, float* dbeta, float* dK, int B, int C, int d,
                            const int64_t* dims, int dtype, void* workspace, size_t workspace_bytes, void* stream,
                            LaunchTrace* trace, bool circ, bool per_sample = false)
{
    if (B < 0 || C < 0) return HYENAND_ERR_INVALID_ARG;
    if (dtype != HYENAND_F32 && dtype != HYENAND_BF16) return HYENAND_ERR_INVALID_ARG;
    if (d < 1 || d > 3) return HYENAND_ERR_UNSUPPORTED;
    if (!dims) return HYENAND_ERR_INVALID_ARG;
    Geom g;
    if (!make_geom(d, dims, &g, circ)) return HYENAND_ERR_UNSUPPORTED;
    if (C == 0) return HYENAND_OK;
    if (!dalpha || !dbeta || !aligned(dalpha, 4) || !aligned(dbeta, 4) || (dK && !aligned(dK, 4)))
        return HYENAND_ERR_INVALID_ARG;
    const bool dk = dK != nullptr;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const long long kl = (long long)g.ke_out * g.ke_mid * g.ke_in;
    if (B == 0) {
        // Sums over an empty batch (the per-sample dK has no entries).
        if (launch_zero(dalpha, C, st) != hipSuccess || launch_zero(dbeta, C, st) != hipSuccess ||
            (dk && !per_sample && launch_zero(dK, (long long)C * kl, st) != hipSuccess))
            return HYENAND_ERR_HIP;
        if (trace) trace->mark(st);
        return HYENAND_OK;
    }
    const size_t es = dtype == HYENAND_BF16 ? 2 : 4;
    if (!x || !alpha || !beta || !K_hat || !dy || !dx) return HYENAND_ERR_INVALID_ARG;
    if (!aligned(x, es) || !aligned(dy, es) || !aligned(dx, es) || !aligned(alpha, 4) || !aligned(beta, 4) ||
        !aligned(K_hat, 8))
        return HYENAND_ERR_INVALID_ARG;
    if (!workspace) return HYENAND_ERR_WORKSPACE;
    if (!aligned(workspace, 8)) return HYENAND_ERR_INVALID_ARG;
    // Per-sample kernels: the batch entries run one after the other, each as a
    // batch of one with its own spectra and dK, dalpha / dbeta accumulated.
    const int Bk = per_sample ? 1 : B;
    int per = bwd_chunk_channels(g, Bk, C, dk, workspace_bytes);
    if (per < 1) return HYENAND_ERR_WORKSPACE;
    const int chunks = (C + per - 1) / per;
    per = (C + chunks - 1) / chunks;  // balanced chunks
    ConvArgs a{};
    a.x = x;
    a.y = dx;
    a.dy = dy;
    a.alpha = alpha;
    a.beta = beta;
    a.khat = static_cast<const float2*>(K_hat);
    a.dalpha = dalpha;
    a.dbeta = dbeta;
    a.dK = dK;
    a.g = g;
    a.B = Bk;
    a.C = C;
    a.bf16 = dtype == HYENAND_BF16;
    float2* w = static_cast<float2*>(workspace);
    const long long plane = (long long)per * Bk * g.wsp;
    a.ws = w;
    a.ws_u = dk ? w + plane : nullptr;
    a.dkw = dk ? w + plane * 2 : nullptr;
    a.part = w + plane * (dk ? 2 : 1) +
             (dk ? ((g.d == 1 && !g.lng) ? (long long)per * Bk * g.S : (long long)per * g.kmain) : 0);
    const int nb = per_sample ? B : 1;
    for (int b = 0; b < nb; ++b) {
        if (per_sample) {
            const long long eo = (long long)b * C * g.vox * (long long)es;  // byte offset of sample b
            a.x = static_cast<const char*>(x) + eo;
            a.dy = static_cast<const char*>(dy) + eo;
            a.y = static_cast<char*>(dx) + eo;
            a.khat = static_cast<const float2*>(K_hat) + (long long)b * C * g.ksz;
            a.dK = dk ? dK + (long long)b * C * kl : nullptr;
            a.accum = b > 0;
        }
        for (int c0 = 0; c0 < C; c0 += per) {
            a.c0 = c0;
            a.nch = (C - c0) < per ? (C - c0) : per;
            if (launch_backward_chunk(a, dk, st, trace) != hipSuccess) return HYENAND_ERR_HIP;
        }
    }
    if (trace) trace->mark(st);
    return HYENAND_OK;
}

int hyenand_fftconv_bwd(const void* x, const float* phi_alpha, const float* phi_beta, const void* K_hat,
                        const void* dy, void* dx, float* dalpha, float* dbeta, float* dK, int B, int C, int d,
                        const int64_t* dims, int dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    return fftconv_bwd_impl(x, phi_alpha, phi_beta, K_hat, dy, dx, dalpha, dbeta, dK, B, C, d, dims, dtype,
                            workspace, workspace_bytes, stream, nullptr, false);
}

int hyenand_fftconv_bwd_circ(const void* x, const float* phi_alpha, const float* phi_beta, const void* K_hat,
                             const void* dy, void* dx, float* dalpha, float* dbeta, float* dK, int B, int C, int d,
                             const int64_t* dims, int dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    return fftconv_bwd_impl(x, phi_alpha, phi_beta, K_hat, dy, dx, dalpha, dbeta, dK, B, C, d, dims, dtype,
                            workspace, workspace_bytes, stream, nullptr, true);
}

int hyenand_fftconv_bwd_traced(const void* x, const float* phi_alpha, const float* phi_beta, const void* K_hat,
                               const void* dy, void* dx, float* dalpha, float* dbeta, float* dK, int B, int C,
                               int d, const int64_t* dims, int dtype, void* workspace, size_t workspace_bytes,
                               void* stream, void* const* events, int n_events, int* n_launches)
{
    if (n_events < 0 || (n_events > 0 && !events)) return HYENAND_ERR_INVALID_ARG;
    LaunchTrace tr{reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)), n_events, 0};
    const int rc = fftconv_bwd_impl(x, phi_alpha, phi_beta, K_hat, dy, dx, dalpha, dbeta, dK, B, C, d, dims, dtype,
                                    workspace, workspace_bytes, stream, &tr, false);
    if (n_launches) *n_launches = tr.count > 0 ? tr.count - 1 : 0;
    return rc;
}

int hyenand_fftconv_bwd_circ_traced(const void* x, const float* phi_alpha, const float* phi_beta,
                                    const void* K_hat, const void* dy, void* dx, float* dalpha, float* dbeta,
                                    float* dK, int B, int C, int d, const int64_t* dims, int dtype, void* workspace,
                                    size_t workspace_bytes, void* stream, void* const* events, int n_events,
                                    int* n_launches)
{
    if (n_events < 0 || (n_events > 0 && !events)) return HYENAND_ERR_INVALID_ARG;
    LaunchTrace tr{reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)), n_events, 0};
    const int rc = fftconv_bwd_impl(x, phi_alpha, phi_beta, K_hat, dy, dx, dalpha, dbeta, dK, B, C, d, dims, dtype,
                                    workspace, workspace_bytes, stream, &tr, true);
    if (n_launches) *n_launches = tr.count > 0 ? tr.count - 1 : 0;
    return rc;
}

// ------------------------------------------------------- per-sample kernels
int hyenand_fftconv_bwd_per_sample(const void* x, const float* phi_alpha, const float* phi_beta, const void* K_hat,
                                   const void* dy, void* dx, float* dalpha, float* dbeta, float* dK, int B, int C,
                                   int d, const int64_t* dims, int dtype, void* workspace, size_t workspace_bytes,
                                   void* stream)
{
    return fftconv_bwd_impl(x, phi_alpha, phi_beta, K_hat, dy, dx, dalpha, dbeta, dK, B, C, d, dims, dtype,
                            workspace, workspace_bytes, stream, nullptr, false, true);
}

int hyenand_fftconv_bwd_per_sample_traced(const void* x, const float* phi_alpha, const float* phi_beta,
                                          const void* K_hat, const void* dy, void* dx, float* dalpha, float* dbeta,
                                          float* dK, int B, int C, int d, const int64_t* dims, int dtype,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          void* const* events, int n_events, int* n_launches)
{
    if (n_events < 0 || (n_events > 0 && !events)) return HYENAND_ERR_INVALID_ARG;
    LaunchTrace tr{reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)), n_events, 0};
    const int rc = fftconv_bwd_impl(x, phi_alpha, phi_beta, K_hat, dy, dx, dalpha, dbeta, dK, B, C, d, dims, dtype,
                                    workspace, workspace_bytes, stream, &tr, false, true);
    if (n_launches) *n_launches = tr.count > 0 ? tr.count - 1 : 0;
    return rc;
}

int hyenand_fftconv_fwd_per_sample(const void* x, const float* alpha, const float* beta, const void* K_hat, void* y,
                                   int B, int C, int d, const int64_t* dims, int dtype, void* workspace,
                                   size_t workspace_bytes, void* stream)
{
    return fftconv_fwd_impl(x, alpha, beta, K_hat, y, B, C, d, dims, dtype, workspace, workspace_bytes, stream,
                            nullptr, false, true);
}

int hyenand_fftconv_fwd_per_sample_traced(const void* x, const float* alpha, const float* beta, const void* K_hat,
                                          void* y, int B, int C, int d, const int64_t* dims, int dtype,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          void* const* events, int n_events, int* n_launches)
{
    if (n_events < 0 || (n_events > 0 && !events)) return HYENAND_ERR_INVALID_ARG;
    LaunchTrace tr{reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)), n_events, 0};
    const int rc = fftconv_fwd_impl(x, alpha, beta, K_hat, y, B, C, d, dims, dtype, workspace, workspace_bytes,
                                    stream, &tr, false, true);
    if (n_launches) *n_launches = tr.count > 0 ? tr.count - 1 : 0;
    return rc;
}

// ------------------------------------------------- generated (per-sample) kernels
}  // extern "C"

namespace {

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct GenLayout {
    size_t partial, coef, basis[3], btab, total;
};

GenLayout gen_layout(const Geom& g, int B, int C)
{
    GenLayout l{};
    size_t o = 0;
    l.partial = o;
    o += align256((size_t)B * C * gen_splits(g.vox) * sizeof(double));
    l.coef = o;
    o += align256((size_t)B * C * kGenCoef * sizeof(float));
    const int Ns[3] = {g.N_out, g.N_mid, g.N_in};
    for (int ax = 0; ax < 3; ++ax) {
        l.basis[ax] = o;
        if (Ns[ax] > 1) o += align256((size_t)C * kGenLines * Ns[ax] * 8u);
    }
    l.btab = o;
    if (g.S >= 16) o += align256((size_t)C * (g.S / 16) * kGenKS * 64 * sizeof(float));
    l.total = o;
    return l;
}

}  // namespace

extern "C" {

size_t hyenand_generate_workspace_bytes(int B, int C, int d, const int64_t* dims)
{
    Geom g;
    if (B <= 0 || C <= 0 || !make_geom(d, dims, &g) || g.lng) return 0;
    return gen_layout(g, B, C).total;
}

}  // extern "C"

namespace {

// Argument checks of the generator and its GenArgs (every pair's spectrum);
// *empty is set when B or C is 0 (nothing to do).
int gen_setup(const void* x, const hyenand_generator* gen, void* K_hat, int B, int C, int d, const int64_t* dims,
              int dtype, void* workspace, size_t workspace_bytes, GenArgs* out, bool* empty)
{
    *empty = false;
    if (B < 0 || C < 0 || !gen) return HYENAND_ERR_INVALID_ARG;
    if (dtype != HYENAND_F32 && dtype != HYENAND_BF16) return HYENAND_ERR_INVALID_ARG;
    if (d < 1 || d > 3) return HYENAND_ERR_UNSUPPORTED;
    if (!dims) return HYENAND_ERR_INVALID_ARG;
    Geom g;
    if (!make_geom(d, dims, &g) || g.lng) return HYENAND_ERR_UNSUPPORTED;
    if (gen->R < 1 || gen->R > 64 || gen->D < 1 || gen->D > 64 || C > 8192) return HYENAND_ERR_INVALID_ARG;
    // One-dimensional grids of the passes (the means pass: pairs x segments;
    // the spectrum pass: pairs x blocks of rows) stay below 2^31 workgroups.
    const long long pairs = (long long)B * C, rows = (long long)g.N_out * g.N_mid;
    if (pairs * gen_splits(g.vox) >= (1LL << 31) || pairs * ((rows + kGenRows - 1) / kGenRows) >= (1LL << 31))
        return HYENAND_ERR_UNSUPPORTED;
    if (B == 0 || C == 0) {
        *empty = true;
        return HYENAND_OK;
    }
    const size_t es = dtype == HYENAND_BF16 ? 2 : 4;
    const float* ps[10] = {gen->Wreg, gen->breg, gen->q, gen->Wgam, gen->Wbet, gen->W1, gen->b1, gen->W2, gen->b2,
                           gen->sigma};
    for (const float* p : ps)
        if (!p || !aligned(p, 4)) return HYENAND_ERR_INVALID_ARG;
    if (!x || !K_hat || !aligned(x, es) || !aligned(K_hat, 8)) return HYENAND_ERR_INVALID_ARG;
    const GenLayout lay = gen_layout(g, B, C);
    if (!workspace || workspace_bytes < lay.total) return HYENAND_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return HYENAND_ERR_INVALID_ARG;
    GenArgs a{};
    a.x = x;
    a.bf16 = dtype == HYENAND_BF16;
    a.B = B;
    a.C = C;
    a.R = gen->R;
    a.D = gen->D;
    a.g = g;
    a.Wreg = gen->Wreg; a.breg = gen->breg; a.q = gen->q; a.Wgam = gen->Wgam; a.Wbet = gen->Wbet;
    a.W1 = gen->W1; a.b1 = gen->b1; a.W2 = gen->W2; a.b2 = gen->b2; a.sigma = gen->sigma;
    a.omega0 = gen->omega0;
    char* w = static_cast<char*>(workspace);
    a.partial = reinterpret_cast<double*>(w + lay.partial);
    a.splits = gen_splits(g.vox);
    a.coef = reinterpret_cast<float*>(w + lay.coef);
    const int Ns[3] = {g.N_out, g.N_mid, g.N_in};
    for (int ax = 0; ax < 3; ++ax) a.basis[ax] = Ns[ax] > 1 ? reinterpret_cast<float2*>(w + lay.basis[ax]) : nullptr;
    a.btab = g.S >= 16 ? reinterpret_cast<float*>(w + lay.btab) : nullptr;
    a.khat = static_cast<float2*>(K_hat);
    a.c0 = 0;
    a.nch = C;
    *out = a;
    return HYENAND_OK;
}

}  // namespace

extern "C" {

int hyenand_generate_kernel_spectrum(const void* x, const hyenand_generator* gen, void* K_hat, int B, int C, int d,
                                     const int64_t* dims, int dtype, void* workspace, size_t workspace_bytes,
                                     void* stream)
{
    GenArgs a{};
    bool empty = false;
    const int rc = gen_setup(x, gen, K_hat, B, C, d, dims, dtype, workspace, workspace_bytes, &a, &empty);
    if (rc != HYENAND_OK || empty) return rc;
    return launch_generate_spectrum(a, static_cast<hipStream_t>(stream)) == hipSuccess ? HYENAND_OK : HYENAND_ERR_HIP;
}

// The generated forward's workspace: the generator's region, then the
// forward's (recommended or minimum), each 256-byte aligned.
static size_t generated_workspace(int B, int C, int d, const int64_t* dims, int dtype, bool minimum)
{
    const size_t gw = hyenand_generate_workspace_bytes(B, C, d, dims);
    if (gw == 0 || (dtype != HYENAND_F32 && dtype != HYENAND_BF16)) return 0;
    return align256(gw) + workspace_bytes(B, C, d, dims, dtype, false, minimum);
}

size_t hyenand_fftconv_fwd_generated_workspace_bytes(int B, int C, int d, const int64_t* dims, int dtype)
{
    return generated_workspace(B, C, d, dims, dtype, false);
}

size_t hyenand_fftconv_fwd_generated_workspace_min_bytes(int B, int C, int d, const int64_t* dims, int dtype)
{
    return generated_workspace(B, C, d, dims, dtype, true);
}

int hyenand_fftconv_fwd_generated(const void* x, const float* alpha, const float* beta, const hyenand_generator* gen,
                                  void* K_hat, void* y, int B, int C, int d, const int64_t* dims, int dtype,
                                  void* workspace, size_t workspace_bytes, void* stream)
{
    // The generator's checks (and its region at the start of the workspace).
    GenArgs ga{};
    bool empty = false;
    int rc = gen_setup(x, gen, K_hat, B, C, d, dims, dtype, workspace, workspace_bytes, &ga, &empty);
    if (rc != HYENAND_OK || empty) return rc;
    const size_t gw = align256(hyenand_generate_workspace_bytes(B, C, d, dims));
    Geom g;
    make_geom(d, dims, &g);
    const size_t fw = workspace_bytes - gw;
    void* fws = static_cast<char*>(workspace) + gw;
    // The forward's checks, as hyenand_fftconv_fwd_per_sample.
    const size_t es = dtype == HYENAND_BF16 ? 2 : 4;
    if (!y || !alpha || !beta || !aligned(y, es) || !aligned(alpha, 4) || !aligned(beta, 4))
        return HYENAND_ERR_INVALID_ARG;
    if (g.wsp > 0 && !fused2d_fits(g) && chunk_channels(g, B, C, fw) < 1) return HYENAND_ERR_WORKSPACE;
    const CallPlan cp = plan_call(g, B, C, fw);
    hipStream_t st = static_cast<hipStream_t>(stream);
    // Every pair's spectra in one pass (one launch per chunk measured slower:
    // 128^3, C = 32: 3.17 against 3.08 ms per call), then the chunks' chains.
    if (launch_generate_spectrum(ga, st) != hipSuccess) return HYENAND_ERR_HIP;
    ConvArgs a{};
    a.x = x;
    a.y = y;
    a.alpha = alpha;
    a.beta = beta;
    a.khat = static_cast<const float2*>(K_hat);
    a.khat_bstride = (long long)C * g.ksz;
    a.ws = static_cast<float2*>(fws);
    a.g = g;
    a.B = B;
    a.C = C;
    a.bf16 = dtype == HYENAND_BF16;
    for (int c0 = 0; c0 < C; c0 += cp.per) {
        a.c0 = c0;
        a.nch = (C - c0) < cp.per ? (C - c0) : cp.per;
        if (launch_forward_chunk(a, st) != hipSuccess) return HYENAND_ERR_HIP;
    }
    return HYENAND_OK;
}

// ------------------------------------------------------ allocation-free forward
// For callers that cannot allocate (code under HIP graph capture, tight serving
// loops): the forward with its workspace in a static device array instead of a
// caller buffer.  Each GPU the library runs on holds its own copy of the array
// (kFwdScratchBytes) until the process ends.  In host code `scratch` names a
// host-side stand-in: its device address on the current device comes from
// hipGetSymbolAddress, taken once per device and kept in scratch_dev.
}  // extern "C"

namespace {

constexpr size_t kFwdScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) float2 scratch[kFwdScratchBytes / sizeof(float2)];

std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];

int resolve_scratch(void** ws, size_t* bytes)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HYENAND_ERR_HIP;
    std::lock_guard<std::mutex> lk(scratch_mu);
    if (!scratch_dev[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HYENAND_ERR_HIP;
        scratch_dev[dev] = p;
    }
    *ws = scratch_dev[dev];
    *bytes = kFwdScratchBytes;
    return HYENAND_OK;
}

}  // namespace

extern "C" {

size_t hyenand_fftconv_fwd_noalloc_max_workspace(void) { return kFwdScratchBytes; }

int hyenand_fftconv_fwd_noalloc(const void* x, const float* alpha, const float* beta, const void* K_hat, void* y,
                                int B, int C, int d, const int64_t* dims, int dtype, void* stream)
{
    return fftconv_fwd_impl(x, alpha, beta, K_hat, y, B, C, d, dims, dtype, nullptr, 0, stream, nullptr, false,
                            false, resolve_scratch);
}

}  // extern "C"
