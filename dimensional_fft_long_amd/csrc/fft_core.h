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
// the thread index (tid()), the workgroup barrier (sync()), the LDS twiddle
// tables (twl, reversed-plan tables at kRevBase; stage() fills them and must
// precede a barrier that precedes the first transform pass with twiddles) and
// the gate (gate()); the device context is in kernels_dev.h.  A context
// wrapped in TwCachedCtx also carries register copies of some passes'
// twiddles (TwCache below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hyenand {

// ----------------------------------------------------------------- complex
__host__ __device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__host__ __device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__host__ __device__ __forceinline__ float2 cmul(float2 a, float2 b)
{
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
// a * conj(w)
__host__ __device__ __forceinline__ float2 cmulc(float2 a, float2 w)
{
    return make_float2(a.x * w.x + a.y * w.y, a.y * w.x - a.x * w.y);
}
__host__ __device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
__host__ __device__ __forceinline__ float2 cscale(float2 a, float s) { return make_float2(a.x * s, a.y * s); }
// a * (-i) when !INV (forward sign), a * (+i) when INV
template <bool INV>
__host__ __device__ __forceinline__ float2 mul_mi(float2 a)
{
    return INV ? make_float2(-a.y, a.x) : make_float2(a.y, -a.x);
}

// ----------------------------------------------------------- twiddle table
// W_8192^t = exp(-2 pi i t / 8192), t in [0, 8192), evaluated at compile time
// in double precision (Taylor series of sin on the first quadrant, extended by
// the quadrant symmetries) and rounded once to float.  Any power-of-two length
// L <= 8192 uses W_L^s = W_8192^(s * 8192 / L).  (4096- and 8192-point
// transforms serve the long 1-D path only.)
constexpr int TW_N = 8192;

struct TwTable {
    float2 w[TW_N];
};

// sin(pi * m / (TW_N / 2)) for m in [0, TW_N / 4], by its Taylor series (|x| <= pi/2).
constexpr double quarter_sin(int m)
{
    const double x = 3.14159265358979323846264338327950288 * (double)m / (double)(TW_N / 2);
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
    constexpr int Q = TW_N / 4;
    for (int i = 0; i < TW_N; ++i) {
        const int q = i / Q, r = i % Q;
        const double s = quarter_sin(r), c = quarter_sin(Q - r);
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

// Evaluated once per translation unit (the per-plan tables below index it).
inline constexpr TwTable kTwBase = make_twiddles();

// ------------------------------------------------------------- radix DFTs
// In-place DFT of R points held in registers, natural order in and out:
//   X[s] = sum_r v[r] exp(-+ 2 pi i r s / R)   (- forward, + inverse).
// PIN: v[r] = 0 for r >= R/2 (those registers are not read).
// POUT: only X[0 .. R/2) are produced (the rest is left undefined).
template <int R, bool INV, bool PIN, bool POUT>
struct Dft;

template <bool INV, bool PIN, bool POUT>
struct Dft<2, INV, PIN, POUT> {
    __host__ __device__ static __forceinline__ void run(float2* v)
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
    __host__ __device__ static __forceinline__ void run(float2* v)
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
    __host__ __device__ static __forceinline__ float2 w8_1(float2 a)
    {
        constexpr float h = 0.70710678118654752440f;
        return INV ? make_float2((a.x - a.y) * h, (a.x + a.y) * h) : make_float2((a.x + a.y) * h, (a.y - a.x) * h);
    }
    __host__ __device__ static __forceinline__ float2 w8_3(float2 a)
    {
        constexpr float h = 0.70710678118654752440f;
        return INV ? make_float2((-a.x - a.y) * h, (a.x - a.y) * h) : make_float2((a.y - a.x) * h, (-a.x - a.y) * h);
    }
    __host__ __device__ static __forceinline__ void run(float2* v)
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
    // 9: 8 8 8 | 10: 8 8 4 4 | 11: 8 8 8 4 | 12: 8 8 8 8 | 13: 8 4 8 4 8
    // The 8192-point plan (long 1-D rows only) is a palindrome, so that the
    // forward and reversed plans share one 64 KiB set of twiddle tables.
    if (k == 13) return p < 5 ? (p % 2 == 0 ? 8 : 4) : 0;
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

// ------------------------------------------------------------ pass pieces
// Radix and stride of pass p of the forward plan (REV = false) or of the
// reversed plan (REV = true, used by inverse transforms so that the positions
// held after a forward transform are those read by the inverse's first pass).
template <int L, bool REV>
__host__ __device__ constexpr int pass_radix(int p)
{
    return REV ? plan_radix(L, plan_passes(L) - 1 - p) : plan_radix(L, p);
}

template <int L, bool REV>
__host__ __device__ constexpr int pass_ns(int p)
{
    int ns = 1;
    for (int q = 0; q < p; ++q) ns *= pass_radix<L, REV>(q);
    return ns;
}

// Twiddle tables staged in LDS, one per pass with NS > 1, laid out [k][r-1]
// (k in [0, NS), r in [1, R)) so that the lanes of a wave, which differ in k,
// read addresses R-1 apart (no bank conflicts) and a butterfly reads R-1
// consecutive entries.  Entry (k, r) = W_{NS R}^{k r} = W_2048^{k r 2048/(NS R)}.
// The forward-plan tables (F) come first, then the reversed-plan tables (R).
template <int L, bool REV>
__host__ __device__ constexpr int tw_local_off(int p)
{
    int off = 0;
    for (int q = 1; q < p; ++q) off += pass_ns<L, REV>(q) * (pass_radix<L, REV>(q) - 1);
    return off;
}

template <int L, bool REV>
__host__ __device__ constexpr int tw_plan_size()
{
    return tw_local_off<L, REV>(plan_passes(L));
}

constexpr int kPlanF = 1, kPlanR = 2;

// A symmetric radix sequence (512 = 8 x 8 x 8) gives the reversed plan the
// forward plan's passes and tables: one copy in LDS serves both (a 512-point
// out-axis workgroup then needs 36.8 instead of 40.8 KiB: four per CU instead
// of three; measured on the 256^2 forward, the out-axis kernel's time did not
// change, 147-150 us).
template <int L>
__host__ __device__ constexpr bool plans_share_tables()
{
    for (int p = 0; p < plan_passes(L); ++p)
        if (pass_radix<L, false>(p) != pass_radix<L, true>(p)) return false;
    return true;
}

template <int L, int PLANS>
__host__ __device__ constexpr bool shared_rev_tables()
{
    return (PLANS & kPlanF) && (PLANS & kPlanR) && plans_share_tables<L>();
}

template <int L, int PLANS>
__host__ __device__ constexpr int tw_table_size()
{
    return ((PLANS & kPlanF) ? tw_plan_size<L, false>() : 0) +
           ((PLANS & kPlanR) && !shared_rev_tables<L, PLANS>() ? tw_plan_size<L, true>() : 0);
}

template <int L, int PLANS>
__host__ __device__ constexpr int tw_rev_base()
{
    return (PLANS & kPlanF) && !shared_rev_tables<L, PLANS>() ? tw_plan_size<L, false>() : 0;
}

// The tables of the plans in PLANS as one array (compile time).
template <int L, int PLANS>
__host__ __device__ constexpr int tw_table_alloc()
{
    return tw_table_size<L, PLANS>() > 0 ? tw_table_size<L, PLANS>() : 1;
}

template <int L, int PLANS>
struct PlanTwiddles {
    float2 w[tw_table_alloc<L, PLANS>()];
};

template <int L, int PLANS>
constexpr PlanTwiddles<L, PLANS> make_plan_twiddles()
{
    const TwTable& base = kTwBase;
    PlanTwiddles<L, PLANS> t{};
    int off = 0;
    for (int rev = 0; rev < 2; ++rev) {
        if (!(PLANS & (rev ? kPlanR : kPlanF))) continue;
        if (rev && shared_rev_tables<L, PLANS>()) continue;
        for (int p = 1; p < plan_passes(L); ++p) {
            const int NS = rev ? pass_ns<L, true>(p) : pass_ns<L, false>(p);
            const int R = rev ? pass_radix<L, true>(p) : pass_radix<L, false>(p);
            for (int k = 0; k < NS; ++k)
                for (int r = 1; r < R; ++r) t.w[off++] = base.w[k * r * (TW_N / (NS * R))];
        }
    }
    return t;
}

// Element (pos, line) of a tile of layout code LP (plan.h row_lay): pos * P +
// line + D * (pos >> SH); with D = 0 the plain stride LP.  The split form
// takes pos = a + c, c a constant of the unrolled loop (so that it folds into
// the instruction's offset), and is exact when a or c is a multiple of 2^SH:
// for the passes of the padded row layouts (512, 1024 and 2048 points, SH <= 3)
// c = r L/R on loads, c = r NS on stores, and a = R j with R = 8 when NS = 1
// (tests/host/row_layout.cpp checks every access against the plain form).
template <int LP>
__host__ __device__ __forceinline__ int tile_idx(int pos, int line)
{
    constexpr int P = LP & 255, D = (LP >> 8) & 15, SH = (LP >> 12) & 15;
    return pos * P + line + (D ? D * (pos >> SH) : 0);
}
template <int LP>
__host__ __device__ __forceinline__ int tile_idx_split(int a, int c, int line)
{
    constexpr int P = LP & 255, D = (LP >> 8) & 15, SH = (LP >> 12) & 15;
    if constexpr (D == 0) return (a + c) * P + line;
    else return a * P + D * (a >> SH) + line + (c * P + D * (c >> SH));
}

// Registers of one Stockham pass over NL lines: butterfly g in [0, NL*L/R),
// line l = g % NL, j = g / NL; thread t owns g = t + i*NT.
//   inputs:  positions j + r*L/R
//   outputs: positions (j/NS)*NS*R + (j%NS) + r*NS  (= j + r*L/R on the last pass)
template <int L, int R, int NL, int NT>
struct PassRegs {
    static constexpr int NB = NL * (L / R);
    static constexpr int PER = (NB + NT - 1) / NT;
    float2 v[PER][R];
};

template <int NB, int NT>
__host__ __device__ __forceinline__ bool bf_valid(int g)
{
    return (NB % NT) == 0 || g < NB;
}

// Inputs from the LDS tile T[pos*LP + line]; with PIN only r < R/2.
template <int L, int R, int NL, int LP, int NT, bool PIN, class Ctx>
__host__ __device__ __forceinline__ void pass_load_lds(const Ctx& ctx, const float2* T, PassRegs<L, R, NL, NT>& s)
{
    using PR = PassRegs<L, R, NL, NT>;
    const int tid = ctx.tid();
#pragma unroll
    for (int i = 0; i < PR::PER; ++i) {
        const int g = tid + i * NT;
        if (bf_valid<PR::NB, NT>(g)) {
            const int l = g % NL, j = g / NL;
#pragma unroll
            for (int r = 0; r < (PIN ? R / 2 : R); ++r) s.v[i][r] = T[tile_idx_split<LP>(j, r * (L / R), l)];
        }
    }
}

// Global-memory accessors come in two forms: f(pos, line), or f(j, q, line)
// with pos = j + q, where q = r*L/R is the same for every lane (a constant of
// the unrolled loop) and j is the lane's own part.  The second form lets an
// accessor fold q into a wave-uniform base address and keep one 32-bit lane
// offset per butterfly instead of a 64-bit address per element.
template <class F>
__host__ __device__ constexpr bool split_accessor()
{
    return requires(const F& f) { f(0, 0, 0); };
}

template <class F>
__host__ __device__ constexpr bool split_visitor()
{
    return requires(const F& f, float2& v) { f(0, 0, 0, v); };
}

// Inputs through an accessor (global memory); with PIN only r < R/2.
template <int L, int R, int NL, int NT, bool PIN, class Ctx, class F>
__host__ __device__ __forceinline__ void pass_load_fn(const Ctx& ctx, const F& f, PassRegs<L, R, NL, NT>& s)
{
    using PR = PassRegs<L, R, NL, NT>;
    const int tid = ctx.tid();
#pragma unroll
    for (int i = 0; i < PR::PER; ++i) {
        const int g = tid + i * NT;
        if (bf_valid<PR::NB, NT>(g)) {
            const int l = g % NL, j = g / NL;
#pragma unroll
            for (int r = 0; r < (PIN ? R / 2 : R); ++r) {
                if constexpr (split_accessor<F>()) s.v[i][r] = f(j, r * (L / R), l);
                else s.v[i][r] = f(j + r * (L / R), l);
            }
        }
    }
}

// Twiddles of one pass for the butterflies a thread owns:
// W_{NS R}^{(j mod NS) r}, r in [1, R).  When NT/NL is a multiple of NS the
// butterflies g = t + i*NT of a thread share j mod NS and one set serves all
// of them (U = 1); passes without twiddles (NS = 1) hold none.
template <int L, int R, int NS, int NL, int NT>
struct PassTw {
    static constexpr int PER = PassRegs<L, R, NL, NT>::PER;
    static constexpr bool kShared = NT % NL == 0 && (NT / NL) % NS == 0;
    static constexpr int U = NS == 1 ? 0 : (kShared ? 1 : PER);
    float2 w[U > 0 ? U : 1][R - 1];
};

// Register copies of the twiddles of passes [1, PEND) of the forward plan of
// length L for NL lines on NT threads.  A kernel that runs several transforms
// of one shape loads them once (TwCache::load) and hands them to the passes
// through its context (TwCachedCtx); a pass takes the copy whose radix,
// stride and shape match its own (a twiddle's value depends on nothing else:
// the reversed plan of a symmetric radix sequence reuses every copy, an
// inverse conjugates it), else it reads the LDS table.  Each copy costs
// 2 (R-1) U registers per thread.
template <int L, int NL, int NT, int PEND, int P = 1, bool END = (P >= PEND || P >= plan_passes(L))>
struct TwCache {
    static constexpr int R = pass_radix<L, false>(P), NS = pass_ns<L, false>(P);
    PassTw<L, R, NS, NL, NT> here;
    TwCache<L, NL, NT, PEND, P + 1> rest;
    template <int R2, int NS2, int NL2, int NT2>
    __host__ __device__ static constexpr bool has()
    {
        return (R2 == R && NS2 == NS && NL2 == NL && NT2 == NT) ||
               TwCache<L, NL, NT, PEND, P + 1>::template has<R2, NS2, NL2, NT2>();
    }
    template <int R2, int NS2>
    __host__ __device__ __forceinline__ const PassTw<L, R2, NS2, NL, NT>& get() const
    {
        if constexpr (R2 == R && NS2 == NS) return here;
        else return rest.template get<R2, NS2>();
    }
    // rd(e): entry e of the context's tables, whose forward-plan tables come
    // first (the LDS copy, once it is staged and a barrier has passed).
    template <class Ctx, class Rd>
    __host__ __device__ __forceinline__ void load(const Ctx& ctx, const Rd& rd)
    {
        const int tid = ctx.tid();
#pragma unroll
        for (int u = 0; u < PassTw<L, R, NS, NL, NT>::U; ++u) {
            const int e = tw_local_off<L, false>(P) + ((tid + u * NT) / NL % NS) * (R - 1);
#pragma unroll
            for (int r = 1; r < R; ++r) here.w[u][r - 1] = rd(e + r - 1);
        }
        rest.load(ctx, rd);
    }
};

template <int L, int NL, int NT, int PEND, int P>
struct TwCache<L, NL, NT, PEND, P, true> {
    template <int, int, int, int>
    __host__ __device__ static constexpr bool has() { return false; }
    template <class Ctx, class Rd>
    __host__ __device__ __forceinline__ void load(const Ctx&, const Rd&) {}
};

// A context whose passes take their twiddles from a TwCache where it has them.
template <class Base, class Cache>
struct TwCachedCtx : Base {
    const Cache* twc;
};

// Whether the context Ctx holds the factors of a pass (radix R, stride NS,
// NL lines, NT threads) in registers.
template <class Ctx>
struct TwCacheOf {
    template <int, int, int, int>
    __host__ __device__ static constexpr bool has() { return false; }
};

template <class Base, class Cache>
struct TwCacheOf<TwCachedCtx<Base, Cache>> : Cache {};

// Twiddle W_{NS R}^{(j mod NS) r} and radix-R DFT on every owned butterfly.
// The factors come from the context's TwCache when it holds this pass, else
// from its LDS tables (TOFF: offset of this pass's table there).
template <int L, int R, int NS, int NL, int NT, bool INV, bool PIN, bool POUT, int TOFF, class Ctx>
__host__ __device__ __forceinline__ void pass_compute(const Ctx& ctx, PassRegs<L, R, NL, NT>& s)
{
    using PR = PassRegs<L, R, NL, NT>;
    constexpr bool kCached = TwCacheOf<Ctx>::template has<R, NS, NL, NT>();
    const int tid = ctx.tid();
#pragma unroll
    for (int i = 0; i < PR::PER; ++i) {
        const int g = tid + i * NT;
        if (bf_valid<PR::NB, NT>(g)) {
            const int j = g / NL;
            if constexpr (NS > 1 && kCached) {
                const auto& tw = ctx.twc->template get<R, NS>();
                const int u = tw.kShared ? 0 : i;
#pragma unroll
                for (int r = 1; r < (PIN ? R / 2 : R); ++r) {
                    const float2 w = tw.w[u][r - 1];
                    s.v[i][r] = INV ? cmulc(s.v[i][r], w) : cmul(s.v[i][r], w);
                }
            } else if constexpr (NS > 1) {
                const float2* tw = ctx.twl + TOFF + (j % NS) * (R - 1) - 1;
#pragma unroll
                for (int r = 1; r < (PIN ? R / 2 : R); ++r) {
                    const float2 w = tw[r];
                    s.v[i][r] = INV ? cmulc(s.v[i][r], w) : cmul(s.v[i][r], w);
                }
            }
            Dft<R, INV, PIN, POUT>::run(s.v[i]);
        }
    }
}

// Outputs to the LDS tile; with POUT only r < R/2.
template <int L, int R, int NS, int NL, int LP, int NT, bool POUT, class Ctx>
__host__ __device__ __forceinline__ void pass_store_lds(const Ctx& ctx, float2* T, const PassRegs<L, R, NL, NT>& s)
{
    using PR = PassRegs<L, R, NL, NT>;
    const int tid = ctx.tid();
#pragma unroll
    for (int i = 0; i < PR::PER; ++i) {
        const int g = tid + i * NT;
        if (bf_valid<PR::NB, NT>(g)) {
            const int l = g % NL, j = g / NL;
            const int base = (j / NS) * NS * R + (j % NS);
#pragma unroll
            for (int r = 0; r < (POUT ? R / 2 : R); ++r) T[tile_idx_split<LP>(base, r * NS, l)] = s.v[i][r];
        }
    }
}

// Visit every output of a last pass (positions j + r*L/R, natural order):
// f(pos, line, value&) or the split form f(j, q, line, value&); with POUT
// only r < R/2.
template <int L, int R, int NL, int NT, bool POUT, class Ctx, class F>
__host__ __device__ __forceinline__ void pass_visit(const Ctx& ctx, PassRegs<L, R, NL, NT>& s, const F& f)
{
    using PR = PassRegs<L, R, NL, NT>;
    const int tid = ctx.tid();
#pragma unroll
    for (int i = 0; i < PR::PER; ++i) {
        const int g = tid + i * NT;
        if (bf_valid<PR::NB, NT>(g)) {
            const int l = g % NL, j = g / NL;
#pragma unroll
            for (int r = 0; r < (POUT ? R / 2 : R); ++r) {
                if constexpr (split_visitor<F>()) f(j, r * (L / R), l, s.v[i][r]);
                else f(j + r * (L / R), l, s.v[i][r]);
            }
        }
    }
}

// In-place LDS passes [P, PEND) of the (reversed) plan, two barriers each.
template <int L, bool REV, int P, int PEND, int NL, int LP, int NT, bool INV>
struct LdsPasses {
    template <class Ctx>
    __host__ __device__ static __forceinline__ void run(const Ctx& ctx, float2* T)
    {
        if constexpr (P < PEND) {
            constexpr int R = pass_radix<L, REV>(P), NS = pass_ns<L, REV>(P);
            constexpr int TOFF = (REV ? Ctx::kRevBase : 0) + tw_local_off<L, REV>(P);
            PassRegs<L, R, NL, NT> s;
            pass_load_lds<L, R, NL, LP, NT, false>(ctx, T, s);
            ctx.sync();
            pass_compute<L, R, NS, NL, NT, INV, false, false, TOFF>(ctx, s);
            pass_store_lds<L, R, NS, NL, LP, NT, false>(ctx, T, s);
            ctx.sync();
            LdsPasses<L, REV, P + 1, PEND, NL, LP, NT, INV>::run(ctx, T);
        }
    }
};

// Length-L FFT of the NL lines of tile T (element (pos, line) at pos*LP +
// line), in place, natural order, unnormalised.  With PIN only positions < L/2
// are read on entry; with POUT only positions < L/2 are valid on exit.  The
// caller has synchronised the tile; ends with a barrier.
template <int L, int NL, int LP, int NT, bool INV, bool PIN, bool POUT, class Ctx>
__host__ __device__ __forceinline__ void tile_fft(const Ctx& ctx, float2* T)
{
    static_assert(L >= 2 && L <= TW_N && (L & (L - 1)) == 0, "power-of-two length up to 8192");
    constexpr int NP = plan_passes(L);
    constexpr int R0 = pass_radix<L, false>(0);
    PassRegs<L, R0, NL, NT> s;
    pass_load_lds<L, R0, NL, LP, NT, PIN>(ctx, T, s);
    ctx.sync();
    pass_compute<L, R0, 1, NL, NT, INV, PIN, POUT && NP == 1, 0>(ctx, s);
    pass_store_lds<L, R0, 1, NL, LP, NT, POUT && NP == 1>(ctx, T, s);
    ctx.sync();
    if constexpr (NP > 1) {
        LdsPasses<L, false, 1, NP - 1, NL, LP, NT, INV>::run(ctx, T);
        constexpr int RL = pass_radix<L, false>(NP - 1), NSL = pass_ns<L, false>(NP - 1);
        PassRegs<L, RL, NL, NT> t;
        pass_load_lds<L, RL, NL, LP, NT, false>(ctx, T, t);
        ctx.sync();
        pass_compute<L, RL, NSL, NL, NT, INV, false, POUT, tw_local_off<L, false>(NP - 1)>(ctx, t);
        pass_store_lds<L, RL, NSL, NL, LP, NT, POUT>(ctx, T, t);
        ctx.sync();
    }
}

// Forward transform of NL lines whose first-pass inputs are the registers `s`
// (positions j + r*L/R0, as left by pass_load_fn; PIN: only positions < L/2
// are non-zero) and whose last pass is left in registers (positions
// j + r*L/R_last).  The tile T is scratch; the caller must not touch it
// before a barrier.
template <int L, int NL, int NT, bool PIN, int LP = NL, class Ctx>
__host__ __device__ __forceinline__ auto fwd_from_regs(const Ctx& ctx, float2* T,
                                                       PassRegs<L, pass_radix<L, false>(0), NL, NT>& s)
{
    constexpr int NP = plan_passes(L);
    constexpr int R0 = pass_radix<L, false>(0);
    pass_compute<L, R0, 1, NL, NT, false, PIN, false, 0>(ctx, s);
    if constexpr (NP == 1) {
        return s;
    } else {
        pass_store_lds<L, R0, 1, NL, LP, NT, false>(ctx, T, s);
        ctx.sync();
        LdsPasses<L, false, 1, NP - 1, NL, LP, NT, false>::run(ctx, T);
        constexpr int RL = pass_radix<L, false>(NP - 1), NSL = pass_ns<L, false>(NP - 1);
        PassRegs<L, RL, NL, NT> t;
        pass_load_lds<L, RL, NL, LP, NT, false>(ctx, T, t);
        pass_compute<L, RL, NSL, NL, NT, false, false, false, tw_local_off<L, false>(NP - 1)>(ctx, t);
        return t;
    }
}

// Forward transform whose first pass reads through the accessor f (see
// pass_load_fn).  `after_load()` runs once the first pass's loads are issued
// and before they are used (a place to issue more independent loads).
template <int L, int NL, int NT, bool PIN, int LP = NL, class Ctx, class F, class H>
__host__ __device__ __forceinline__ auto fwd_from_fn(const Ctx& ctx, float2* T, const F& f, const H& after_load)
{
    PassRegs<L, pass_radix<L, false>(0), NL, NT> s;
    pass_load_fn<L, pass_radix<L, false>(0), NL, NT, PIN>(ctx, f, s);
    after_load();
    return fwd_from_regs<L, NL, NT, PIN, LP>(ctx, T, s);
}

// Inverse transform (reversed plan) whose first-pass inputs are the registers
// `s` (positions j + r*L/R, as left by fwd_from_fn or by a load); returns the
// last pass's registers (positions j + r*L/R0 in natural order, R0 the
// forward plan's first radix; POUT: only positions < L/2 are valid).  The
// tile T must be free for writing (a barrier after its last read).
template <int L, int NL, int NT, bool POUT, int LP = NL, class Ctx, class S>
__host__ __device__ __forceinline__ auto inv_to_regs(const Ctx& ctx, float2* T, S& s)
{
    constexpr int NP = plan_passes(L);
    constexpr int R0 = pass_radix<L, true>(0);
    pass_compute<L, R0, 1, NL, NT, true, false, POUT && NP == 1, 0>(ctx, s);
    if constexpr (NP == 1) {
        return s;
    } else {
        pass_store_lds<L, R0, 1, NL, LP, NT, false>(ctx, T, s);
        ctx.sync();
        LdsPasses<L, true, 1, NP - 1, NL, LP, NT, true>::run(ctx, T);
        constexpr int RL = pass_radix<L, true>(NP - 1), NSL = pass_ns<L, true>(NP - 1);
        PassRegs<L, RL, NL, NT> t;
        pass_load_lds<L, RL, NL, LP, NT, false>(ctx, T, t);
        pass_compute<L, RL, NSL, NL, NT, true, false, POUT, Ctx::kRevBase + tw_local_off<L, true>(NP - 1)>(ctx, t);
        return t;
    }
}

// Inverse transform whose last pass writes through gfn (see pass_visit).
template <int L, int NL, int NT, bool POUT, int LP = NL, class Ctx, class S, class G>
__host__ __device__ __forceinline__ void inv_to_fn(const Ctx& ctx, float2* T, S& s, const G& gfn)
{
    auto t = inv_to_regs<L, NL, NT, POUT, LP>(ctx, T, s);
    pass_visit<L, pass_radix<L, false>(0), NL, NT, POUT>(ctx, t, gfn);
}

// Forward transform from f (first pass) to g (last pass), full output.
template <int L, int NL, int NT, bool PIN, class Ctx, class F, class G, class H>
__host__ __device__ __forceinline__ void fwd_fn_to_fn(const Ctx& ctx, float2* T, const F& f, const G& gfn,
                                                      const H& after_load)
{
    constexpr int NP = plan_passes(L);
    auto s = fwd_from_fn<L, NL, NT, PIN>(ctx, T, f, after_load);
    constexpr int RL = pass_radix<L, false>(NP - 1);
    pass_visit<L, RL, NL, NT, false>(ctx, s, gfn);
}

// Inverse transform from f (first pass, all L positions) to g (last pass).
template <int L, int NL, int NT, bool POUT, class Ctx, class F, class G, class H>
__host__ __device__ __forceinline__ void inv_fn_to_fn(const Ctx& ctx, float2* T, const F& f, const G& gfn,
                                                      const H& after_load)
{
    constexpr int R0 = pass_radix<L, true>(0);
    PassRegs<L, R0, NL, NT> s;
    pass_load_fn<L, R0, NL, NT, false>(ctx, f, s);
    after_load();
    inv_to_fn<L, NL, NT, POUT>(ctx, T, s, gfn);
}

}  // namespace hyenand
