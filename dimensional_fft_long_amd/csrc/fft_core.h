// fft_core.h -- workgroup FFT building blocks for the gated N-D convolution.
//
// The FFT convolution path (explainer "Native multi-dimensional subquadratic
// operators via input-dependent long convolutions", section "HyenaND:
// native-space implicit global kernel", item "Implementation") needs forward
// and inverse complex FFTs of power-of-two length L <= 2048 along every axis.
// Lines live in LDS as a tile T[pos * LP + line] (line index fastest), and all
// threads of a workgroup run a Stockham autosort FFT over the tile, one radix
// pass at a time (radix 8 / 4 / 2 butterflies in registers, one LDS read and
// one LDS write per point per pass, two workgroup barriers per pass).
//
// Zero padding to twice the grid (gist.science summary, "Methodology",
// "Boundary handling") means the input of every forward transform has only its
// first L/2 points non-zero and every inverse transform only needs its first
// L/2 outputs: the first pass reads half its inputs and the last pass writes
// half its outputs (PIN / POUT below).
//
// The code is written against a small execution context `Ctx` that provides
// the thread index, the workgroup barrier and the twiddle table; the device
// context is in hyenand_kernels.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hyenand {

// ----------------------------------------------------------------- complex
__host__ __device__ inline float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__host__ __device__ inline float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__host__ __device__ inline float2 cmul(float2 a, float2 b)
{
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
// a * conj(w)
__host__ __device__ inline float2 cmulc(float2 a, float2 w)
{
    return make_float2(a.x * w.x + a.y * w.y, a.y * w.x - a.x * w.y);
}
__host__ __device__ inline float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
__host__ __device__ inline float2 cscale(float2 a, float s) { return make_float2(a.x * s, a.y * s); }
// a * (-i) when !INV (forward sign), a * (+i) when INV
template <bool INV>
__host__ __device__ inline float2 mul_mi(float2 a)
{
    return INV ? make_float2(-a.y, a.x) : make_float2(a.y, -a.x);
}

// ----------------------------------------------------------- twiddle table
// W_2048^t = exp(-2 pi i t / 2048), t in [0, 2048), evaluated at compile time
// in double precision (Taylor series of sin on the first quadrant, extended by
// the quadrant symmetries) and rounded once to float.  Any power-of-two length
// L <= 2048 uses W_L^s = W_2048^(s * 2048 / L).
constexpr int TW_N = 2048;

struct TwTable {
    float2 w[TW_N];
};

// sin(pi * m / 1024) for m in [0, 512], by its Taylor series (|x| <= pi/2).
constexpr double quarter_sin(int m)
{
    const double x = 3.14159265358979323846264338327950288 * (double)m / 1024.0;
    const double x2 = x * x;
    double term = x, sum = x;
    for (int k = 1; k < 16; ++k) {
        term *= -x2 / (double)((2 * k) * (2 * k + 1));
        sum += term;
    }
    return sum;
}

constexpr TwTable make_twiddles()
{
    TwTable t{};
    for (int i = 0; i < TW_N; ++i) {
        const int q = i / 512, r = i % 512;
        const double s = quarter_sin(r), c = quarter_sin(512 - r);
        double cs = 0.0, sn = 0.0;
        if (q == 0) { cs = c; sn = s; }
        else if (q == 1) { cs = -s; sn = c; }
        else if (q == 2) { cs = -c; sn = -s; }
        else { cs = s; sn = -c; }
        t.w[i].x = (float)cs;
        t.w[i].y = (float)(-sn);
    }
    return t;
}

// ------------------------------------------------------------- radix DFTs
// In-place DFT of R points held in registers, natural order in and out:
//   X[s] = sum_r v[r] exp(-+ 2 pi i r s / R)   (- forward, + inverse).
// PIN: v[r] = 0 for r >= R/2 (those registers are not read).
// POUT: only X[0 .. R/2) are produced (the rest is left undefined).
template <int R, bool INV, bool PIN, bool POUT>
struct Dft;

template <bool INV, bool PIN, bool POUT>
struct Dft<2, INV, PIN, POUT> {
    __host__ __device__ static inline void run(float2* v)
    {
        if constexpr (PIN) {
            v[1] = v[0];
        } else {
            const float2 a = v[0], b = v[1];
            v[0] = cadd(a, b);
            if constexpr (!POUT) v[1] = csub(a, b);
        }
    }
};

template <bool INV, bool PIN, bool POUT>
struct Dft<4, INV, PIN, POUT> {
    __host__ __device__ static inline void run(float2* v)
    {
        float2 a0, a1, b0, b1;
        if constexpr (PIN) {
            a0 = v[0]; a1 = v[1]; b0 = v[0]; b1 = mul_mi<INV>(v[1]);
        } else {
            a0 = cadd(v[0], v[2]); a1 = cadd(v[1], v[3]);
            b0 = csub(v[0], v[2]); b1 = mul_mi<INV>(csub(v[1], v[3]));
        }
        v[0] = cadd(a0, a1);
        v[1] = cadd(b0, b1);
        if constexpr (!POUT) {
            v[2] = csub(a0, a1);
            v[3] = csub(b0, b1);
        }
    }
};

// Decimation in frequency: a_r = v_r + v_{r+4}, b_r = (v_r - v_{r+4}) W8^r,
// X[2s] = DFT4(a)[s], X[2s+1] = DFT4(b)[s].
template <bool INV, bool PIN, bool POUT>
struct Dft<8, INV, PIN, POUT> {
    __host__ __device__ static inline float2 w8_1(float2 a)
    {
        constexpr float h = 0.70710678118654752440f;
        return INV ? make_float2((a.x - a.y) * h, (a.x + a.y) * h) : make_float2((a.x + a.y) * h, (a.y - a.x) * h);
    }
    __host__ __device__ static inline float2 w8_3(float2 a)
    {
        constexpr float h = 0.70710678118654752440f;
        return INV ? make_float2((-a.x - a.y) * h, (a.x - a.y) * h) : make_float2((a.y - a.x) * h, (-a.x - a.y) * h);
    }
    __host__ __device__ static inline void run(float2* v)
    {
        float2 a[4], b[4];
        if constexpr (PIN) {
            a[0] = v[0]; a[1] = v[1]; a[2] = v[2]; a[3] = v[3];
            b[0] = v[0]; b[1] = w8_1(v[1]); b[2] = mul_mi<INV>(v[2]); b[3] = w8_3(v[3]);
        } else {
            a[0] = cadd(v[0], v[4]); a[1] = cadd(v[1], v[5]); a[2] = cadd(v[2], v[6]); a[3] = cadd(v[3], v[7]);
            b[0] = csub(v[0], v[4]);
            b[1] = w8_1(csub(v[1], v[5]));
            b[2] = mul_mi<INV>(csub(v[2], v[6]));
            b[3] = w8_3(csub(v[3], v[7]));
        }
        Dft<4, INV, false, POUT>::run(a);
        Dft<4, INV, false, POUT>::run(b);
        v[0] = a[0]; v[1] = b[0]; v[2] = a[1]; v[3] = b[1];
        if constexpr (!POUT) {
            v[4] = a[2]; v[5] = b[2]; v[6] = a[3]; v[7] = b[3];
        }
    }
};

// ------------------------------------------------------------ radix plans
// Radix of pass p for a length L = 2^k transform (pass 0 first), 0 past the end.
__host__ __device__ constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v >> 1); }

__host__ __device__ constexpr int plan_radix(int L, int p)
{
    const int k = ilog2(L);
    // k: passes
    // 1: 2 | 2: 4 | 3: 8 | 4: 4 4 | 5: 8 4 | 6: 8 8 | 7: 8 4 4 | 8: 8 8 4
    // 9: 8 8 8 | 10: 8 8 4 4 | 11: 8 8 8 4
    const int r8 = (k % 3 == 1 && k >= 4) ? (k - 4) / 3 : k / 3;
    const int r4 = (k % 3 == 1 && k >= 4) ? 2 : (k % 3 == 2 ? 1 : 0);
    const int r2 = (k == 1) ? 1 : 0;
    if (p < r8) return 8;
    if (p < r8 + r4) return 4;
    if (p < r8 + r4 + r2) return 2;
    return 0;
}

__host__ __device__ constexpr int plan_passes(int L)
{
    int p = 0;
    while (plan_radix(L, p) != 0) ++p;
    return p;
}

// ------------------------------------------------------- one Stockham pass
// Butterfly g in [0, NL * L / R): line l = g % NL, j = g / NL.  Inputs at
// positions j + r L/R; twiddle W_{NS R}^{(j mod NS) r}; outputs at
// (j / NS) NS R + (j mod NS) + r NS, where NS is the product of the radices of
// the passes already done.  Two barriers: all reads of the pass complete
// before any write, and all writes before the next pass reads.
template <int L, int R, int NS, int NL, int LP, int NT, bool INV, bool PIN, bool POUT, class Ctx>
__host__ __device__ inline void stockham_pass(const Ctx& ctx, float2* T)
{
    constexpr int NB = NL * (L / R);
    constexpr int PER = (NB + NT - 1) / NT;
    constexpr int RIN = PIN ? R / 2 : R;
    constexpr int ROUT = POUT ? R / 2 : R;
    constexpr int TWS = TW_N / (NS * R);
    const int tid = ctx.tid();
    float2 v[PER][R];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int g = tid + i * NT;
        if ((NB % NT) == 0 || g < NB) {
            const int l = g % NL, j = g / NL;
#pragma unroll
            for (int r = 0; r < RIN; ++r) v[i][r] = T[(j + r * (L / R)) * LP + l];
        }
    }
    ctx.sync();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int g = tid + i * NT;
        if ((NB % NT) == 0 || g < NB) {
            const int l = g % NL, j = g / NL;
            if constexpr (NS > 1) {
                const int k = j % NS;
#pragma unroll
                for (int r = 1; r < RIN; ++r) {
                    const float2 w = ctx.tw(k * r * TWS);
                    v[i][r] = INV ? cmulc(v[i][r], w) : cmul(v[i][r], w);
                }
            }
            Dft<R, INV, PIN, POUT>::run(v[i]);
            const int base = (j / NS) * NS * R + (j % NS);
#pragma unroll
            for (int r = 0; r < ROUT; ++r) T[(base + r * NS) * LP + l] = v[i][r];
        }
    }
    ctx.sync();
}

template <int L, int P, int NPASS, int NS, int NL, int LP, int NT, bool INV, bool PIN, bool POUT>
struct PassChain {
    template <class Ctx>
    __host__ __device__ static inline void run(const Ctx& ctx, float2* T)
    {
        constexpr int R = plan_radix(L, P);
        stockham_pass<L, R, NS, NL, LP, NT, INV, PIN && P == 0, POUT && P == NPASS - 1>(ctx, T);
        PassChain<L, P + 1, NPASS, NS * R, NL, LP, NT, INV, PIN, POUT>::run(ctx, T);
    }
};

template <int L, int NPASS, int NS, int NL, int LP, int NT, bool INV, bool PIN, bool POUT>
struct PassChain<L, NPASS, NPASS, NS, NL, LP, NT, INV, PIN, POUT> {
    template <class Ctx>
    __host__ __device__ static inline void run(const Ctx&, float2*) {}
};

// Length-L FFT of the NL lines of tile T (element (pos, line) at pos*LP + line),
// in place, natural order.  Unnormalised in both directions.  With PIN only
// positions < L/2 are read on entry; with POUT only positions < L/2 are valid
// on exit.  Ends with a barrier.
template <int L, int NL, int LP, int NT, bool INV, bool PIN, bool POUT, class Ctx>
__host__ __device__ inline void tile_fft(const Ctx& ctx, float2* T)
{
    static_assert(L >= 2 && L <= TW_N && (L & (L - 1)) == 0, "power-of-two length up to 2048");
    PassChain<L, 0, plan_passes(L), 1, NL, LP, NT, INV, PIN, POUT>::run(ctx, T);
}

}  // namespace hyenand
