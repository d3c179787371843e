// fused2d.h -- the whole 2-D forward of one (b, c) pair in one workgroup, its
// half spectrum held in LDS (no workspace, one launch for every pair).
//
// The FFT convolution path (explainer "Native multi-dimensional subquadratic
// operators via input-dependent long convolutions", section "HyenaND:
// native-space implicit global kernel", item "Implementation": FFT, product
// with the kernel spectrum, inverse FFT) with the zero-padded boundary of the
// gist.science summary ("Methodology", "Boundary handling") and the fusion the
// summary's "Implementation: nSubQ" describes (fused kernels, the intermediates
// kept in on-chip memory instead of HBM), for grids whose half spectrum fits in
// a workgroup's LDS with room for several workgroups per CU: n_out x n_in up to
// 64 x 64 (32 KiB of fp32 complex; see fused2d_fits in plan.h).
//
//   phase 1  rows:    gate, pruned real FFT of two rows per complex line,
//                     separation into two half spectra -> P[row][slot]
//   phase 2  columns: per tile of TWC slots, pruned forward FFT of length LO
//                     from P, product with the kernel spectrum (mirror product
//                     for slot 0), pruned inverse FFT back into P (n_out rows)
//   phase 3  rows:    Hermitian rebuild, pruned inverse real FFT, crop, cast,
//                     store y
//
// P holds n_out rows of S = LI/2 slots (slot 0 packs the real bins 0 and LI/2
// as in the multi-pass path); the transforms use the same FFT engine, the same
// kernel spectrum layout and the same factor-2 folding as the multi-pass
// kernels.
#pragma once

#include "conv_bodies.h"

namespace hyenand {

// Line pairs per row batch, slots per column tile and threads of the fused
// kernel for padded lengths LO (out axis) x LI (inner axis).
constexpr int f2_npb(int LO, int LI)
{
    const int lines = LO / 4;                     // n_out / 2 line pairs
    const int cap = 2048 / LI < 1 ? 1 : 2048 / LI;  // tile of up to 2048 complex
    return lines < cap ? lines : cap;
}
constexpr int f2_twc(int LO, int LI)
{
    const int S = LI / 2;
    const int cap = 2048 / LO < 1 ? 1 : 2048 / LO;
    return S < cap ? S : cap;
}
constexpr int f2_nt(int LO, int LI)
{
    const int a = LI * f2_npb(LO, LI) / 8, b = LO * f2_twc(LO, LI) / 8;
    const int m = a > b ? a : b;
    return m < 64 ? 64 : (m > 256 ? 256 : m);
}
constexpr int f2_lp(int LO, int LI) { return f2_npb(LO, LI) + 1; }
constexpr int f2_tile(int LO, int LI)
{
    const int r = LI * f2_lp(LO, LI), c = LO * f2_twc(LO, LI);
    return r > c ? r : c;
}
// LDS bytes of the fused kernel: P and the transform tile (the twiddle tables
// come on top: about 6 KiB for 256-point lines).
constexpr int f2_lds_bytes(int LO, int LI) { return 8 * ((LO / 2) * (LI / 2) + f2_tile(LO, LI)); }

// Pair order: pairs p = c * B + b (channel-major) are spread so that XCD x (the
// workgroups with id = x mod 8) runs a contiguous range of pairs: the B batch
// entries of a channel, which read the same kernel spectrum, meet in one L2.
__host__ __device__ __forceinline__ int f2_pair(int bid, int P)
{
    const int P8 = P & ~7;
    return bid < P8 ? (bid % 8) * (P8 / 8) + bid / 8 : bid;
}

template <int LO, int LI, bool BF16, class CtxR, class CtxC>
__host__ __device__ __forceinline__ void fused2d_body(const CtxR& cr, const CtxC& cc, int bid, const ConvArgs& a,
                                                      float2* P, float2* T)
{
    constexpr int n_out = LO / 2, n_in = LI / 2, S = LI / 2;
    constexpr int NPB = f2_npb(LO, LI), LP = f2_lp(LO, LI), TWC = f2_twc(LO, LI), NT = f2_nt(LO, LI);
    constexpr int R0 = pass_radix<LO, false>(0);
    constexpr int RL = pass_radix<LO, false>(plan_passes(LO) - 1);
    const Geom& g = a.g;
    const int tid = cr.tid();
    const int p = f2_pair(bid, a.B * a.C);
    const int c = p / a.B, b = p % a.B;
    const long long xo = ((long long)b * a.C + c) * g.vox;
    const float al = a.alpha[c], be = a.beta[c];
    const float2* kc = a.khat + (long long)c * g.ksz + (long long)b * a.khat_bstride;
    cr.stage();
    cc.stage();

    // ---- phase 1: rows -> P
    for (int lp0 = 0; lp0 < n_out / 2; lp0 += NPB) {
        cr.sync();  // T free (previous batch's separation reads done); twiddles staged
        for (int idx = tid; idx < NPB * n_in; idx += NT) {
            const int lp = idx / n_in, m = idx % n_in;
            const long long o = xo + (long long)(2 * (lp0 + lp)) * n_in + m;
            T[m * LP + lp] = make_float2(cr.gate(load_x<BF16>(a, o), al, be), cr.gate(load_x<BF16>(a, o + n_in), al, be));
        }
        cr.sync();
        tile_fft<LI, NPB, LP, NT, false, true, false>(cr, T);
        // 2 U_a[k] = Z[k] + conj Z[LI-k], 2 U_b[k] = -i (Z[k] - conj Z[LI-k]); slot 0 packs (bin 0, bin S).
        for (int idx = tid; idx < NPB * S; idx += NT) {
            const int lp = idx / S, k = idx % S;
            const float2 Z = T[k * LP + lp];
            const float2 Zm = T[(k == 0 ? S : LI - k) * LP + lp];
            float2 oa, ob;
            if (k == 0) {
                oa = make_float2(2.f * Z.x, 2.f * Zm.x);
                ob = make_float2(2.f * Z.y, 2.f * Zm.y);
            } else {
                oa = make_float2(Z.x + Zm.x, Z.y - Zm.y);
                ob = make_float2(Z.y + Zm.y, Zm.x - Z.x);
            }
            const int r = 2 * (lp0 + lp);
            P[r * S + k] = oa;
            P[(r + 1) * S + k] = ob;
        }
    }
    cr.sync();

    // ---- phase 2: columns of P (forward, product, inverse), TWC slots at a time
    using P0 = PassRegs<LO, R0, TWC, NT>;
    using PL = PassRegs<LO, RL, TWC, NT>;
    OutTile o;
    o.c_local = 0; o.t = 0; o.b = b; o.rows[0] = 0; o.rows[1] = 0; o.self_mirror = true;
    for (int k0 = 0; k0 < S; k0 += TWC) {
        P0 s;
        pass_load_fn<LO, R0, TWC, NT, true>(cc, [&](int pos, int l) -> float2 { return P[pos * S + k0 + l]; }, s);
        // Kernel spectrum values for the positions this thread multiplies (slot 0: mirror product below).
        float2 kv[PL::PER][RL];
#pragma unroll
        for (int i = 0; i < PL::PER; ++i) {
            const int gi = tid + i * NT, l = gi % TWC, j = gi / TWC;
            const bool ok = bf_valid<PL::NB, NT>(gi);
#pragma unroll
            for (int r = 0; r < RL; ++r) {
                const int pos = ok ? j + r * (LO / RL) : 0;
                kv[i][r] = kc[tm_index(g, LO, pos, k0 + l)];
            }
        }
        PL t = fwd_from_regs<LO, TWC, NT, true>(cc, T, s);
        cc.sync();  // every LDS read of the forward transform is done: T is free
        if (k0 == 0) {
            // Slot 0 (k_in = 0: line 0 of the first tile) takes the mirror
            // product, through T: the whole tile goes to T and comes back
            // (unconditional loops, so the registers stay registers).
#pragma unroll
            for (int i = 0; i < PL::PER; ++i) {
                const int gi = tid + i * NT, l = gi % TWC, j = gi / TWC;
                if (bf_valid<PL::NB, NT>(gi)) {
#pragma unroll
                    for (int r = 0; r < RL; ++r) T[(j + r * (LO / RL)) * TWC + l] = t.v[i][r];
                }
            }
            cc.sync();
            out_slot0_product<LO, 1, TWC, NT>(cc, g, o, kc, T);
            cc.sync();
#pragma unroll
            for (int i = 0; i < PL::PER; ++i) {
                const int gi = tid + i * NT, l = gi % TWC, j = gi / TWC;
                if (bf_valid<PL::NB, NT>(gi)) {
#pragma unroll
                    for (int r = 0; r < RL; ++r) t.v[i][r] = T[(j + r * (LO / RL)) * TWC + l];
                }
            }
            cc.sync();
        }
#pragma unroll
        for (int i = 0; i < PL::PER; ++i) {
            const int gi = tid + i * NT, l = gi % TWC;
            const bool mult = k0 + l != 0;
#pragma unroll
            for (int r = 0; r < RL; ++r) {
                const float2 m = cmul(t.v[i][r], kv[i][r]);
                t.v[i][r] = mult ? m : t.v[i][r];
            }
        }
        inv_to_fn<LO, TWC, NT, true>(cc, T, t, [&](int pos, int l, const float2& x) { P[pos * S + k0 + l] = x; });
        cc.sync();  // the inverse's LDS reads are done before the next tile writes T
    }

    // ---- phase 3: rows of P -> y
    for (int lp0 = 0; lp0 < n_out / 2; lp0 += NPB) {
        for (int idx = tid; idx < NPB * S; idx += NT) {
            const int lp = idx / S, k = idx % S;
            const int r = 2 * (lp0 + lp);
            const float2 ya = P[r * S + k], yb = P[(r + 1) * S + k];
            if (k == 0) {
                T[lp] = make_float2(ya.x, yb.x);
                T[S * LP + lp] = make_float2(ya.y, yb.y);
            } else {
                T[k * LP + lp] = make_float2(ya.x - yb.y, ya.y + yb.x);
                T[(LI - k) * LP + lp] = make_float2(ya.x + yb.y, yb.x - ya.y);
            }
        }
        cr.sync();
        tile_fft<LI, NPB, LP, NT, true, false, true>(cr, T);
        for (int idx = tid; idx < NPB * n_in; idx += NT) {
            const int lp = idx / n_in, m = idx % n_in;
            const float2 z = T[m * LP + lp];
            const long long oo = xo + (long long)(2 * (lp0 + lp)) * n_in + m;
            store_y<BF16>(a, oo, z.x);
            store_y<BF16>(a, oo + n_in, z.y);
        }
        cr.sync();  // T free for the next batch
    }
}

}  // namespace hyenand
