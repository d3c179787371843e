// mfma_dft.h -- a radix-8 pass of the FFT engine as dense matrix products on
// the gfx950 matrix cores (MFMA), for the 512-point out-axis transforms.
//
// The explainer ("Native multi-dimensional subquadratic operators via
// input-dependent long convolutions", section "HyenaND: native-space implicit
// global kernel", complexity analysis) puts the cost of the path in the forward
// and inverse FFTs.  A radix-8 Stockham pass with its twiddles is, for each
// butterfly, an 8 x 8 complex matrix times the butterfly's 8 inputs:
//   out[s] = sum_r W_64^{(8 s + k) r} in[r]     (k = the butterfly's twiddle
//                                                 class, j mod 8; conjugated
//                                                 for the inverse)
// so the 16 butterflies of one twiddle class form a 16 x 16 real product
// D = A B (A the real form of the complex matrix, rows and columns interleaved
// re / im; B sixteen butterflies, one per column), one MFMA 16x16x16.
//
// fp32 accuracy from bf16 operands: x = hi + lo with hi = bf16(x),
// lo = bf16(x - hi) (16 significant bits), and D = Ahi Bhi + Ahi Blo + Alo Bhi
// accumulated in fp32 (the dropped Alo Blo term and the split leave a relative
// error near 2^-17 per pass).  bf16 keeps fp32's exponent range, so no scaling
// is needed.
//
// Lane layout of v_mfma_f32_16x16x16_bf16 (64 lanes, g = lane / 16,
// n = lane % 16): A row n, columns 4g..4g+3; B rows 4g..4g+3 of column n;
// D rows 4g..4g+3 of column n.  Rows of B / D here are (re, im) of inputs /
// outputs r = 2g, 2g + 1.
#pragma once

#include "fft_core.h"

namespace hyenand {

typedef short mf_s4 __attribute__((ext_vector_type(4)));
typedef float mf_f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ short mf_bits(float v) { return __builtin_bit_cast(short, (__bf16)v); }
__device__ __forceinline__ float mf_value(short b) { return __builtin_bit_cast(float, (unsigned)(unsigned short)b << 16); }

// hi / lo bf16 parts of four floats.
__device__ __forceinline__ void mf_split(float v0, float v1, float v2, float v3, mf_s4& hi, mf_s4& lo)
{
    hi[0] = mf_bits(v0); hi[1] = mf_bits(v1); hi[2] = mf_bits(v2); hi[3] = mf_bits(v3);
    lo[0] = mf_bits(v0 - mf_value(hi[0]));
    lo[1] = mf_bits(v1 - mf_value(hi[1]));
    lo[2] = mf_bits(v2 - mf_value(hi[2]));
    lo[3] = mf_bits(v3 - mf_value(hi[3]));
}

// bf16 bits of a float, rounded to nearest even (compile time).
constexpr unsigned short mf_bf16_rne(float f)
{
    const unsigned u = __builtin_bit_cast(unsigned, f);
    return (unsigned short)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
constexpr float mf_bf16_float(unsigned short b) { return __builtin_bit_cast(float, (unsigned)b << 16); }

// The A operands of every lane, both directions and all 8 twiddle classes:
// lane's row m = lane % 16 (output s = m / 2, part re / im), columns 4g + i
// (input r = 2g + i / 2, part re / im) of the real form [[re, -im], [im, re]]
// of W_64^{+-(8 s + k) r}, split into bf16 hi and lo parts.  W_64^e comes from
// the engine's compile-time twiddle table (W_4096^{64 e}).
struct MfTable {
    unsigned short hi[2][8][64][4], lo[2][8][64][4];
};

constexpr MfTable make_mf_table()
{
    MfTable t{};
    for (int inv = 0; inv < 2; ++inv)
        for (int k = 0; k < 8; ++k)
            for (int lane = 0; lane < 64; ++lane) {
                const int m = lane % 16, g = lane / 16, s = m / 2, p = m % 2;
                for (int i = 0; i < 4; ++i) {
                    const int r = 2 * g + i / 2, q = i % 2;
                    const int e = ((8 * s + k) * r) & 63;
                    const float re = kTwBase.w[e * 64].x, im0 = kTwBase.w[e * 64].y;
                    const float im = inv ? -im0 : im0;
                    const float v = p == 0 ? (q == 0 ? re : -im) : (q == 0 ? im : re);
                    const unsigned short h = mf_bf16_rne(v);
                    t.hi[inv][k][lane][i] = h;
                    t.lo[inv][k][lane][i] = mf_bf16_rne(v - mf_bf16_float(h));
                }
            }
    return t;
}

template <int U>
__constant__ const MfTable g_mf_table = make_mf_table();

// Operands of the two twiddle classes a wave handles (2w, 2w + 1).
struct MfOperands {
    mf_s4 hi[2], lo[2];
};

template <bool INV>
__device__ __forceinline__ MfOperands mf_operands(int tid)
{
    MfOperands o;
    const int w = tid / 64, lane = tid % 64;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const unsigned short* h = g_mf_table<0>.hi[INV][2 * w + c][lane];
        const unsigned short* l = g_mf_table<0>.lo[INV][2 * w + c][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o.hi[c][i] = (short)h[i];
            o.lo[c][i] = (short)l[i];
        }
    }
    return o;
}

// The middle pass of a 512-point transform (radix 8, NS = 8) over the 8 lines
// of tile T (element (pos, line) at pos * 8 + line), in place, four waves:
// wave w takes the twiddle classes 2w and 2w + 1, four groups of 16
// butterflies each (two j's of the class x 8 lines).  Loads, a barrier, the
// products, stores and a barrier, like an LDS pass of the engine.
template <class Ctx>
__device__ __forceinline__ void mf_pass512_mid(const Ctx& ctx, float2* T, const MfOperands& A)
{
    const int tid = ctx.tid(), w = tid / 64, lane = tid % 64, g = lane / 16, n = lane % 16, l = n % 8;
    float2 in[8][2];
#pragma unroll
    for (int grp = 0; grp < 8; ++grp) {
        const int k = 2 * w + grp / 4, jj = (grp % 4) * 2 + n / 8, j = jj * 8 + k;
        in[grp][0] = T[(j + (2 * g) * 64) * 8 + l];
        in[grp][1] = T[(j + (2 * g + 1) * 64) * 8 + l];
    }
    ctx.sync();
#pragma unroll
    for (int grp = 0; grp < 8; ++grp) {
        const int c = grp / 4, k = 2 * w + c, jj = (grp % 4) * 2 + n / 8;
        mf_s4 bhi, blo;
        mf_split(in[grp][0].x, in[grp][0].y, in[grp][1].x, in[grp][1].y, bhi, blo);
        mf_f4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A.hi[c], bhi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A.hi[c], blo, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A.lo[c], bhi, acc, 0, 0, 0);
        T[(jj * 64 + k + (2 * g) * 8) * 8 + l] = make_float2(acc[0], acc[1]);
        T[(jj * 64 + k + (2 * g + 1) * 8) * 8 + l] = make_float2(acc[2], acc[3]);
    }
    ctx.sync();
}

// fwd_from_regs / inv_to_regs of fft_core.h for L = 512, 8 lines, 256
// threads, with the middle pass on the matrix cores.
template <int NT, bool PIN, class Ctx>
__device__ __forceinline__ PassRegs<512, 8, 8, NT> mf_fwd_from_regs(const Ctx& ctx, float2* T,
                                                                    PassRegs<512, 8, 8, NT>& s,
                                                                    const MfOperands& A)
{
    static_assert(NT == 256, "four waves");
    pass_compute<512, 8, 1, 8, NT, false, PIN, false, 0>(ctx, s);
    pass_store_lds<512, 8, 1, 8, 8, NT, false>(ctx, T, s);
    ctx.sync();
    mf_pass512_mid(ctx, T, A);
    PassRegs<512, 8, 8, NT> t;
    pass_load_lds<512, 8, 8, 8, NT, false>(ctx, T, t);
    pass_compute<512, 8, 64, 8, NT, false, false, false, tw_local_off<512, false>(2)>(ctx, t);
    return t;
}

template <int NT, bool POUT, class Ctx>
__device__ __forceinline__ PassRegs<512, 8, 8, NT> mf_inv_to_regs(const Ctx& ctx, float2* T,
                                                                  PassRegs<512, 8, 8, NT>& s,
                                                                  const MfOperands& A)
{
    static_assert(NT == 256, "four waves");
    pass_compute<512, 8, 1, 8, NT, true, false, false, 0>(ctx, s);
    pass_store_lds<512, 8, 1, 8, 8, NT, false>(ctx, T, s);
    ctx.sync();
    mf_pass512_mid(ctx, T, A);
    PassRegs<512, 8, 8, NT> t;
    pass_load_lds<512, 8, 8, 8, NT, false>(ctx, T, t);
    pass_compute<512, 8, 64, 8, NT, true, false, POUT, Ctx::kRevBase + tw_local_off<512, true>(2)>(ctx, t);
    return t;
}

}  // namespace hyenand
