// Host-only stand-ins for the kernel launchers, linked with the C ABI's host
// code (api.cpp) into a sanitizer build that runs without a GPU.  The driver
// passes host buffers of exactly the documented sizes as "device" pointers;
// every stand-in touches the first and last element of each region its
// kernels would read or write for the chunk it is given (and checks that the
// workspace regions of one launch do not overlap), so AddressSanitizer reports
// any chunk, offset or size that the planner gets wrong.  Each stand-in then
// returns the status set with stub_set_launch_status (hipSuccess by default).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "../../dimensional_fft_long_amd/csrc/gen.h"
#include "../../dimensional_fft_long_amd/csrc/launch.h"

namespace {

hipError_t g_status = hipSuccess;
long g_calls = 0;
long g_failures = 0;
volatile unsigned char g_sink = 0;

void touch(const void* p, long long bytes)
{
    if (bytes <= 0) return;
    if (!p) {
        std::fprintf(stderr, "stub: null region of %lld bytes\n", bytes);
        ++g_failures;
        return;
    }
    const unsigned char* c = static_cast<const unsigned char*>(p);
    g_sink = g_sink ^ c[0] ^ c[bytes - 1];
}

void touch_rw(void* p, long long bytes)
{
    touch(p, bytes);
    if (p && bytes > 0) {
        unsigned char* c = static_cast<unsigned char*>(p);
        c[0] = g_sink;
        c[bytes - 1] = g_sink;
    }
}

struct Region {
    const char* p;
    long long n;
};

void disjoint(const Region* r, int k)
{
    for (int i = 0; i < k; ++i)
        for (int j = i + 1; j < k; ++j) {
            if (!r[i].p || !r[j].p || r[i].n <= 0 || r[j].n <= 0) continue;
            if (r[i].p < r[j].p + r[j].n && r[j].p < r[i].p + r[i].n) {
                std::fprintf(stderr, "stub: workspace regions %d and %d overlap\n", i, j);
                ++g_failures;
            }
        }
}

using hyenand::ConvArgs;
using hyenand::Geom;

// The channels [c0, c0 + nch) of every batch entry of a [B][C][vox] tensor.
void touch_pairs(const void* base, const ConvArgs& a, long long es, bool write)
{
    const char* p = static_cast<const char*>(base);
    for (int b = 0; b < a.B; ++b) {
        const long long lo = ((long long)b * a.C + a.c0) * a.g.vox * es;
        const long long n = (long long)a.nch * a.g.vox * es;
        if (write) touch_rw(const_cast<char*>(p) + lo, n);
        else touch(p + lo, n);
    }
}

void touch_conv(const ConvArgs& a, bool bwd)
{
    const Geom& g = a.g;
    const long long es = a.bf16 ? 2 : 4;
    touch_pairs(a.x, a, es, false);
    touch_pairs(a.y, a, es, true);
    if (bwd) touch_pairs(a.dy, a, es, false);
    touch(a.alpha + a.c0, 4LL * a.nch);
    touch(a.beta + a.c0, 4LL * a.nch);
    const long long last = (long long)(a.B - 1) * a.khat_bstride + (long long)(a.c0 + a.nch) * g.ksz;
    touch(a.khat + (long long)a.c0 * g.ksz, 8LL * (last - (long long)a.c0 * g.ksz));
    const bool uses_ws = (g.d >= 2 || g.lng) && !hyenand::fused2d_fits(g);
    const long long pairs = (long long)a.nch * a.B;
    if (!bwd) {
        if (uses_ws) touch_rw(a.ws, 8LL * pairs * g.wsp);
        return;
    }
    const long long plane = pairs * g.wsp;
    const long long dkw = (g.d == 1 && !g.lng) ? pairs * g.S : (long long)a.nch * g.kmain;
    const long long part = pairs * hyenand::pair_lines(g);
    touch_rw(a.ws, 8LL * plane);
    if (a.ws_u) touch_rw(a.ws_u, 8LL * plane);
    if (a.dkw) touch_rw(a.dkw, 8LL * dkw);
    touch_rw(a.part, 8LL * part);
    const Region r[4] = {{(const char*)a.ws, 8LL * plane},
                         {(const char*)a.ws_u, a.ws_u ? 8LL * plane : 0},
                         {(const char*)a.dkw, a.dkw ? 8LL * dkw : 0},
                         {(const char*)a.part, 8LL * part}};
    disjoint(r, 4);
    touch_rw(a.dalpha + a.c0, 4LL * a.nch);
    touch_rw(a.dbeta + a.c0, 4LL * a.nch);
    if (a.dK) {
        const long long kl = (long long)g.ke_out * g.ke_mid * g.ke_in;
        touch_rw(a.dK + (long long)a.c0 * kl, 4LL * a.nch * kl);
    }
}

}  // namespace

extern "C" void stub_set_launch_status(int s) { g_status = static_cast<hipError_t>(s); }
extern "C" long stub_launch_calls(void) { return g_calls; }
extern "C" long stub_failures(void) { return g_failures; }

namespace hyenand {

hipError_t launch_forward_chunk(const ConvArgs& a, hipStream_t, LaunchTrace*)
{
    ++g_calls;
    touch_conv(a, false);
    return g_status;
}

hipError_t launch_backward_chunk(const ConvArgs& a, bool dk, hipStream_t, LaunchTrace*)
{
    ++g_calls;
    if (dk != (a.dK != nullptr)) {
        std::fprintf(stderr, "stub: dk flag disagrees with the dK pointer\n");
        ++g_failures;
    }
    touch_conv(a, true);
    return g_status;
}

hipError_t launch_zero(float* p, long long n, hipStream_t)
{
    ++g_calls;
    touch_rw(p, 4LL * n);
    return g_status;
}

hipError_t launch_spectrum(const ConvArgs& a, hipStream_t)
{
    ++g_calls;
    const Geom& g = a.g;
    touch(a.K, 4LL * a.C * g.ke_out * g.ke_mid * g.ke_in);
    touch_rw(const_cast<float2*>(a.khat), 8LL * a.C * g.ksz);
    return g_status;
}

namespace {

hipError_t generate_prep(const GenArgs& a)
{
    ++g_calls;
    const Geom& g = a.g;
    const long long pairs = (long long)a.B * a.C;
    touch(a.x, pairs * g.vox * (a.bf16 ? 2 : 4));
    touch(a.Wreg, 4LL * a.R * a.D * a.C);
    touch(a.breg, 4LL * a.R * a.D);
    touch(a.q, 4LL * a.D);
    touch(a.Wgam, 4LL * kGenHidden * a.D);
    touch(a.Wbet, 4LL * kGenHidden * a.D);
    touch(a.W1, 4LL * kGenHidden * g.d);
    touch(a.b1, 4LL * kGenHidden);
    touch(a.W2, 4LL * a.C * kGenHidden);
    touch(a.b2, 4LL * a.C);
    touch(a.sigma, 4LL * a.C);
    if (a.splits < 1 || a.splits != gen_splits(g.vox)) {
        std::fprintf(stderr, "stub: splits %d\n", a.splits);
        ++g_failures;
    }
    touch_rw(a.partial, 8LL * pairs * a.splits);
    touch_rw(a.coef, 4LL * pairs * kGenCoef);
    const int Ns[3] = {g.N_out, g.N_mid, g.N_in};
    const long long nbt = g.S >= 16 ? 4LL * a.C * (g.S / 16) * kGenKS * 64 : 0;
    if ((nbt > 0) != (a.btab != nullptr)) {
        std::fprintf(stderr, "stub: operand table present %d for S = %d\n", a.btab != nullptr, g.S);
        ++g_failures;
    }
    if (a.btab) touch_rw(a.btab, nbt);
    Region r[6] = {{(const char*)a.partial, 8LL * pairs * a.splits}, {(const char*)a.coef, 4LL * pairs * kGenCoef}};
    r[5] = {(const char*)a.btab, nbt};
    for (int ax = 0; ax < 3; ++ax) {
        const long long n = Ns[ax] > 1 ? 8LL * a.C * kGenLines * Ns[ax] : 0;
        if ((Ns[ax] > 1) != (a.basis[ax] != nullptr)) {
            std::fprintf(stderr, "stub: basis %d present %d for length %d\n", ax, a.basis[ax] != nullptr, Ns[ax]);
            ++g_failures;
        }
        if (a.basis[ax]) touch_rw(a.basis[ax], n);
        r[2 + ax] = {(const char*)a.basis[ax], n};
    }
    disjoint(r, 6);
    return g_status;
}

hipError_t generate_pairs(const GenArgs& a)
{
    if (a.c0 < 0 || a.nch < 0 || a.c0 + a.nch > a.C) {
        std::fprintf(stderr, "stub: channel range [%d, %d) of %d\n", a.c0, a.c0 + a.nch, a.C);
        ++g_failures;
        return g_status;
    }
    for (int b = 0; b < a.B; ++b)
        touch_rw(a.khat + ((long long)b * a.C + a.c0) * a.g.ksz, 8LL * a.nch * a.g.ksz);
    return g_status;
}

}  // namespace

hipError_t launch_generate_spectrum(const GenArgs& a, hipStream_t)
{
    const hipError_t e = generate_prep(a);
    if (e != hipSuccess) return e;
    if (a.c0 != 0 || a.nch != a.C) {
        std::fprintf(stderr, "stub: spectra of channels [%d, %d) of %d\n", a.c0, a.c0 + a.nch, a.C);
        ++g_failures;
    }
    return generate_pairs(a);
}

}  // namespace hyenand
