// gen.h -- input-dependent kernels generated on the GPU, straight into their
// spectra (one spectrum per (b, c) pair, the per-sample layout).
//
// The generator (gist.science summary of the paper, "Methodology", items on
// registers, FiLM conditioning and kernel synthesis): per sample b,
//   m[c]   = mean of x[b,c] over the grid                  (the registers' view
//   a[r]   = tanh(Wreg[r] m + breg[r])                      of the whole sample)
//   z      = sum_r softmax_r(q . a[r]) a[r]                 control z(x)
//   gam    = 1 + Wgam z,  bet = Wbet z                      FiLM of the SIREN
// and per channel c and offset delta:
//   K[b,c](delta) = w_c(delta) (sum_u W2[c,u] (gam_u sin(theta_u(delta)) + bet_u) + b2[c])
//   theta_u(delta) = omega0 (sum_a W1[u,a] delta_a / (n_a - 1) + b1[u]),
//   w_c(delta)     = exp(-|delta|^2 / (2 sigma_c^2))        Gaussian window.
//
// No spatial kernel is ever formed.  With v_u = W2[c,u] gam_u and
// e = sum_u W2[c,u] bet_u + b2[c], K = sum_u v_u w sin(theta_u) + e w, and both
// the window and exp(i theta_u) factor over the axes (theta_u is a sum of one
// term per axis; b1 rides on the innermost axis), so with
//   A_{c,u,a} = FFT_{N_a}(wrap_a(G_{c,a} exp(i phi_{u,a}))),   G_{c,a}(t) = exp(-t^2 / (2 sigma_c^2)),
//   W_{c,a}   = FFT_{N_a}(wrap_a(G_{c,a}))
// (1-D transforms of the zero-padded, wrap-placed axis sequences: the padded
// N-D grid's wrap placement is the product of the axes'), the N-D spectrum of
// each pair is
//   Khat(k) = sum_u (v_u / 2i) [prod_a A_{c,u,a}(k_a) - prod_a conj A_{c,u,a}(-k_a)] + e prod_a W_{c,a}(k_a)
// (sin = (exp(i theta) - exp(-i theta)) / 2i, and the spectrum of the
// conjugate of a sequence is the conjugate of its spectrum at -k).  That is 33
// complex multiply-adds per spectrum value instead of an N-D transform of a
// materialised kernel.  The result is stored in the library's spectrum layout
// (plan.h: 1 / (2 prod N) folded in, the Nyquist bin packed into slot 0).
//
// Passes: gen_stats (means), gen_film (registers, control, FiLM -> v, e per
// pair), gen_basis (the 1-D axis spectra, per channel), gen_spectrum.
#pragma once

#include "conv_bodies.h"

namespace hyenand {

constexpr int kGenHidden = 16;
constexpr int kGenLines = kGenHidden + 1;       // the 16 units' axis sequences and the window's
constexpr int kGenCoef = kGenHidden + 1;        // v_u (16) and e per pair
constexpr int kGenRows = 128;                   // spectrum rows per gen_spectrum workgroup
constexpr int kGenNT = 256;
// Workgroups per pair of the means pass: up to 256, one per 16 elements per thread.
inline int gen_splits(long long vox)
{
    const long long s = (vox + 16LL * kGenNT - 1) / (16LL * kGenNT);
    return (int)(s < 1 ? 1 : (s > 256 ? 256 : s));
}

struct GenArgs {
    const void* x;          // [B][C][vox], fp32 or bf16
    int bf16;
    int B, C, R, D;
    Geom g;
    const float *Wreg, *breg, *q, *Wgam, *Wbet, *W1, *b1, *W2, *b2, *sigma;
    float omega0;
    double* partial;        // [B][C][splits]: sums over the splits of each pair's grid
    int splits;
    float* coef;            // [B][C][17]: v_0..v_15, e
    float2* basis[3];       // per geometry axis (out, mid, in): [C][17][N_a] (NULL for absent axes)
    float* btab;            // S >= 16: the matrix-core engine's B operands, [C][S / 16][17][64]
    float2* khat;           // [B][C][ksz]
    int c0, nch;            // spectrum pass: the channels [c0, c0 + nch) of every batch entry
};

// ------------------------------------------------------------- gen_stats
// Workgroup (pair, split): the fp64 sum of one contiguous segment of x[b,c]
// (an LDS tree in a fixed order); gen_film adds a pair's splits in order.
template <bool BF16, class Ctx>
__device__ __forceinline__ void gen_stats_body(const Ctx& ctx, int bid, const GenArgs& a, double* R)
{
    const int tid = ctx.tid();
    const int pair = bid / a.splits, sp = bid % a.splits;
    const long long n = a.g.vox, seg = (n + a.splits - 1) / a.splits;
    const long long lo = (long long)sp * seg, hi = lo + seg < n ? lo + seg : n;
    const long long base = (long long)pair * n;
    double s = 0.0;
    if (((base + lo) & 3) == 0 && ((hi - lo) & 3) == 0) {
        // Four elements per load (segments of four-aligned elements).
        for (long long i = lo + 4 * tid; i < hi; i += 4 * kGenNT) {
            if constexpr (BF16) {
                const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.x) + base + i);
                s += (double)__builtin_bit_cast(float, v.x << 16) + (double)__builtin_bit_cast(float, v.x & 0xffff0000u) +
                     (double)__builtin_bit_cast(float, v.y << 16) + (double)__builtin_bit_cast(float, v.y & 0xffff0000u);
            } else {
                const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + base + i);
                s += (double)v.x + (double)v.y + (double)v.z + (double)v.w;
            }
        }
    } else {
        for (long long i = lo + tid; i < hi; i += kGenNT) {
            if constexpr (BF16) s += (double)bf16_to_f32(static_cast<const uint16_t*>(a.x)[base + i]);
            else s += (double)static_cast<const float*>(a.x)[base + i];
        }
    }
    R[tid] = s;
    ctx.sync();
    for (int h = kGenNT / 2; h >= 1; h /= 2) {
        if (tid < h) R[tid] += R[tid + h];
        ctx.sync();
    }
    if (tid == 0) a.partial[bid] = R[0];
}

// -------------------------------------------------------------- gen_film
// One sample per workgroup: register activations, softmax-weighted control,
// FiLM parameters, then the per-pair coefficients v_u = W2[c,u] gam_u and
// e = sum_u W2[c,u] bet_u + b2[c].  S: LDS scratch of C + R*D + R + D + 32
// floats.
template <class Ctx>
__device__ __forceinline__ void gen_film_body(const Ctx& ctx, int b, const GenArgs& a, float* S)
{
    const int tid = ctx.tid(), R = a.R, D = a.D, C = a.C;
    float* m = S;                   // [C] the sample's per-channel means
    float* act = m + C;             // [R][D]
    float* score = act + R * D;     // [R]
    float* z = score + R;           // [D]
    float* gam = z + D;             // [16]
    float* bet = gam + kGenHidden;  // [16]
    // A wave per channel: strided partial sums, then a butterfly over the
    // lanes (a fixed order; lane 0's total is used).
    const int lane = tid % 64, wave = tid / 64;
    for (int c = wave; c < C; c += kGenNT / 64) {
        const double* pp = a.partial + ((long long)b * C + c) * a.splits;
        double s = 0.0;
        for (int k = lane; k < a.splits; k += 64) s += pp[k];
        for (int o = 32; o >= 1; o /= 2) s += __shfl_xor(s, o);
        if (lane == 0) m[c] = (float)(s / (double)a.g.vox);
    }
    ctx.sync();
    for (int i = tid; i < R * D; i += kGenNT) {
        float v = a.breg[i];
        const float* w = a.Wreg + (long long)i * C;
        for (int c = 0; c < C; ++c) v += w[c] * m[c];
        act[i] = tanhf(v);
    }
    ctx.sync();
    for (int r = tid; r < R; r += kGenNT) {
        float v = 0.f;
        for (int j = 0; j < D; ++j) v += a.q[j] * act[r * D + j];
        score[r] = v;
    }
    ctx.sync();
    if (tid == 0) {
        float mx = score[0];
        for (int r = 1; r < R; ++r) mx = fmaxf(mx, score[r]);
        float sum = 0.f;
        for (int r = 0; r < R; ++r) {
            score[r] = expf(score[r] - mx);
            sum += score[r];
        }
        for (int r = 0; r < R; ++r) score[r] /= sum;
    }
    ctx.sync();
    for (int j = tid; j < D; j += kGenNT) {
        float v = 0.f;
        for (int r = 0; r < R; ++r) v += score[r] * act[r * D + j];
        z[j] = v;
    }
    ctx.sync();
    for (int u = tid; u < kGenHidden; u += kGenNT) {
        float vg = 1.f, vb = 0.f;
        for (int j = 0; j < D; ++j) {
            vg += a.Wgam[u * D + j] * z[j];
            vb += a.Wbet[u * D + j] * z[j];
        }
        gam[u] = vg;
        bet[u] = vb;
    }
    ctx.sync();
    for (int c = tid; c < C; c += kGenNT) {
        float* o = a.coef + ((long long)b * C + c) * kGenCoef;
        float e = a.b2[c];
        for (int u = 0; u < kGenHidden; ++u) {
            const float w = a.W2[c * kGenHidden + u];
            o[u] = w * gam[u];
            e += w * bet[u];
        }
        o[kGenHidden] = e;
    }
}

// ------------------------------------------------------------- gen_basis
// The axis spectra of geometry axis AX (length L = N_a): line (c, u), u < 16:
// G_{c,a} exp(i phi_{u,a}); u = 16: G_{c,a}; wrap-placed (offset t at index
// t mod L, index n_a empty), forward FFT, stored [c][u][L].
template <int L, int AX, class Ctx>
__device__ __forceinline__ void gen_basis_body(const Ctx& ctx, int bid, const GenArgs& a, float2* T)
{
    constexpr int NP = row_np(L), LP = row_lp(L), NT = row_nt(L);
    const Geom& g = a.g;
    const int n = AX == 0 ? g.n_out : (AX == 1 ? g.n_mid : g.n_in);
    // the grid axis of this geometry axis (W1's column): out is grid axis 0
    // (d >= 2), mid grid axis 1 (d = 3), in the last grid axis
    const int gax = AX == 2 ? g.d - 1 : AX;
    const int lines = a.C * kGenLines;
    const int tid = ctx.tid();
    ctx.stage();
    for (int idx = tid; idx < NP * L; idx += NT) {
        const int lp = idx / L, m = idx % L, h = bid * NP + lp;
        float2 v = make_float2(0.f, 0.f);
        if (h < lines) {
            const int c = h / kGenLines, u = h % kGenLines;
            const int t = unwrap(m, n, L);
            if (t != kEmpty) {
                const float s = a.sigma[c];
                const float gw = expf(-(float)t * (float)t / (2.f * s * s));
                if (u == kGenHidden) {
                    v = make_float2(gw, 0.f);
                } else {
                    float ph = a.omega0 * a.W1[u * g.d + gax] * ((float)t / (float)(n - 1));
                    if (AX == 2) ph += a.omega0 * a.b1[u];
                    float sn, cs;
                    sincosf(ph, &sn, &cs);
                    v = make_float2(gw * cs, gw * sn);
                }
            }
        }
        T[m * LP + lp] = v;
    }
    ctx.sync();
    tile_fft<L, NP, LP, NT, false, false, false>(ctx, T);
    float2* out = a.basis[AX];
    for (int idx = tid; idx < NP * L; idx += NT) {
        const int lp = idx / L, m = idx % L, h = bid * NP + lp;
        if (h < lines) out[(long long)h * L + m] = T[m * LP + lp];
    }
}

// ---------------------------------------------------------- gen_spectrum
// Workgroup (pair p = b C + c, block of kGenRows rows k_out N_mid + k_mid):
// the row factors of the 33 terms into LDS, then the terms summed for every
// k_in of the block's rows; slot 0 packs k_in = 0 and N_in / 2 (through LDS,
// after the main sums).  Two engines for the main sums: the VALU one below
// (any S), and for S >= 16 the matrix-core one, which reads the sums as the
// complex matrix product Khat[r, s] = sum_f RC[r, f] IN[f, s] (33 terms f:
// RC the row factors, IN the innermost axis' factors) and runs it as fp32
// MFMA products (v_mfma_f32_16x16x4_f32: full fp32 operands, fp32 sums).
__device__ __forceinline__ float2 gen_axis(const GenArgs& a, int ax, int c, int u, int k, int N)
{
    return N == 1 ? make_float2(1.f, 0.f) : a.basis[ax][((long long)c * kGenLines + u) * N + k];
}

// RC row stride: 34 complex (272 bytes, 16-byte aligned rows for float4
// reads); entry 33 is padding.
constexpr int kGenTerms = 2 * kGenHidden + 1, kGenRC = kGenTerms + 1;

struct GenBlock {
    int rows, r0, nr, c, p;
    long long kbase;
    float gsc;
};

__device__ __forceinline__ GenBlock gen_block(const GenArgs& a, int bid)
{
    const Geom& g = a.g;
    GenBlock k;
    k.rows = g.N_out * g.N_mid;
    const int nblk = (k.rows + kGenRows - 1) / kGenRows;
    const int q = bid / nblk;
    k.r0 = (bid % nblk) * kGenRows;
    k.nr = k.rows - k.r0 < kGenRows ? k.rows - k.r0 : kGenRows;
    k.c = a.c0 + q % a.nch;
    k.p = (q / a.nch) * a.C + k.c;
    k.kbase = (long long)k.p * g.ksz;
    k.gsc = 1.0f / (2.0f * (float)g.N_in * (float)g.N_out * (float)g.N_mid);
    return k;
}

// The innermost axis' factor of term f at k_in = s: A_u(s) (f = u < 16),
// -conj A_u(-s) (f = 16 + u), W(s) (f = 32), 0 (f = 33).
__device__ __forceinline__ float2 gen_in_factor(const GenArgs& a, int c, int f, int s)
{
    const int N = a.g.N_in;
    if (f < kGenHidden) return gen_axis(a, 2, c, f, s, N);
    if (f < 2 * kGenHidden) {
        const float2 v = gen_axis(a, 2, c, f - kGenHidden, (N - s) & (N - 1), N);
        return make_float2(-v.x, v.y);
    }
    return f == 2 * kGenHidden ? gen_axis(a, 2, c, kGenHidden, s, N) : make_float2(0.f, 0.f);
}

// Row factors: RC[r][u] = (v_u / 2i) A_out A_mid at (k_out, k_mid),
// RC[r][16 + u] = (v_u / 2i) conj(A_out A_mid at (-k_out, -k_mid)),
// RC[r][32] = e W_out W_mid; RC[r][33] = 0.
// Also the innermost axis' factors at the Nyquist bin k_in = S into XF[33]
// (the same for every row of the block).  TPR threads per row, each taking
// the terms f = q, q + TPR, ... (the row's indices computed once; every
// length is a power of two, so indices wrap by masks).
template <class Ctx>
__device__ __forceinline__ void gen_row_factors(const Ctx& ctx, const GenArgs& a, const GenBlock& k, float2* RC,
                                                float2* XF)
{
    constexpr int TPR = kGenNT / kGenRows;
    static_assert(TPR * kGenRows == kGenNT, "whole threads per row");
    const Geom& g = a.g;
    const int tid = ctx.tid();
    if (tid < kGenTerms) XF[tid] = gen_in_factor(a, k.c, tid, g.S);
    const int r = tid / TPR, q = tid % TPR;
    if (r >= k.nr) return;
    const int row = k.r0 + r, lm = 31 - __builtin_clz(g.N_mid);
    const int ko = row >> lm, km = row & (g.N_mid - 1);
    const int kom = (g.N_out - ko) & (g.N_out - 1), kmm = (g.N_mid - km) & (g.N_mid - 1);
    const float* cf = a.coef + (long long)k.p * kGenCoef;
    // Axis sequences of channel c: A_ax[u][k] at base_ax + u * N_ax + k (absent axes: 1).
    const float2* bo = g.N_out > 1 ? a.basis[0] + (long long)k.c * kGenLines * g.N_out : nullptr;
    const float2* bm = g.N_mid > 1 ? a.basis[1] + (long long)k.c * kGenLines * g.N_mid : nullptr;
    auto axis = [](const float2* b, int N, int u, int kk) {
        return b ? b[u * N + kk] : make_float2(1.f, 0.f);
    };
#pragma unroll
    for (int j = 0; j < (kGenRC + TPR - 1) / TPR; ++j) {
        const int f = q + TPR * j;
        if (f >= kGenRC) break;
        float2 v = make_float2(0.f, 0.f);
        if (f == 2 * kGenHidden) {
            v = cscale(cmul(axis(bo, g.N_out, kGenHidden, ko), axis(bm, g.N_mid, kGenHidden, km)), cf[kGenHidden]);
        } else if (f < 2 * kGenHidden) {
            const int u = f & (kGenHidden - 1);
            const bool mir = f >= kGenHidden;
            float2 pr = cmul(axis(bo, g.N_out, u, mir ? kom : ko), axis(bm, g.N_mid, u, mir ? kmm : km));
            if (mir) pr = cconj(pr);
            const float h = 0.5f * cf[u];  // v / 2i = -i v / 2
            v = make_float2(h * pr.y, -h * pr.x);
        }
        RC[r * kGenRC + f] = v;
    }
}

// The Nyquist bin k_in = S of every row (one row per thread), then slot 0 and
// the trailing block from X0 (k_in = 0) and XS.
template <class Ctx>
__device__ __forceinline__ void gen_pack_slot0(const Ctx& ctx, const GenArgs& a, const GenBlock& k, const float2* RC,
                                               const float2* XF, const float2* X0, float2* XS)
{
    const Geom& g = a.g;
    const int tid = ctx.tid();
    if (tid < k.nr) {
        const int r = tid;
        float2 acc = make_float2(0.f, 0.f);
#pragma unroll
        for (int f = 0; f < kGenTerms; ++f) acc = cadd(acc, cmul(RC[r * kGenRC + f], XF[f]));
        XS[r] = acc;
    }
    ctx.sync();
    for (int r = tid; r < k.nr; r += kGenNT) {
        const float2 z0 = X0[r], zs = XS[r];
        a.khat[k.kbase + tm_index(g, k.rows, k.r0 + r, 0)] = cscale(cadd(z0, zs), 0.5f * k.gsc);
        a.khat[k.kbase + g.kmain + k.r0 + r] = cscale(csub(z0, zs), 0.5f * k.gsc);
    }
}

// VALU engine: threads as (slot lane, row lane), slots k_in in [0, S) over SL
// lanes holding that slot's 33 factors in registers, rows over the
// kGenNT / SL row lanes (S is a power of two).
template <class Ctx>
__device__ __forceinline__ void gen_spectrum_body(const Ctx& ctx, int bid, const GenArgs& a, float2* RC, float2* XF,
                                                  float2* X0, float2* XS)
{
    const Geom& g = a.g;
    const GenBlock k = gen_block(a, bid);
    const int tid = ctx.tid();
    gen_row_factors(ctx, a, k, RC, XF);
    ctx.sync();
    const int S = g.S;
    const int SL = S < kGenNT ? S : kGenNT, RL = kGenNT / SL;
    const int sl = tid % SL, rl = tid / SL;
    for (int s = sl; s < S; s += SL) {
        float2 in[2 * kGenHidden];
#pragma unroll
        for (int f = 0; f < 2 * kGenHidden; ++f) in[f] = gen_in_factor(a, k.c, f, s);
        const float2 win = gen_in_factor(a, k.c, 2 * kGenHidden, s);
        for (int r = rl; r < k.nr; r += RL) {
            const float4* f4 = reinterpret_cast<const float4*>(RC + r * kGenRC);
            float2 acc = cmul(RC[r * kGenRC + 2 * kGenHidden], win);
#pragma unroll
            for (int f = 0; f < 2 * kGenHidden; f += 2) {
                const float4 pa = f4[f / 2];
                acc = cadd(acc, cmul(make_float2(pa.x, pa.y), in[f]));
                acc = cadd(acc, cmul(make_float2(pa.z, pa.w), in[f + 1]));
            }
            if (s == 0) X0[r] = acc;
            else a.khat[k.kbase + tm_index(g, k.rows, k.r0 + r, s)] = cscale(acc, k.gsc);
        }
    }
    gen_pack_slot0(ctx, a, k, RC, XF, X0, XS);
}

// Matrix-core engine (S >= 16; wave w owns the 16-row tiles w, w + 4, ... of
// the block, RT = kGenRows / 64 of them).  As real products over K = 68 (term
// f, part t at k = 2 f + t):
//   Re Khat[r, s] = sum_k Are[r, k] B[k, s],  Im Khat[r, s] = sum_k Aim[r, k] B[k, s],
//   B[2f, s] = Re IN[f, s],  B[2f + 1, s] = Im IN[f, s],
//   Are[r, 2f] = Re RC[r, f],  Are[r, 2f + 1] = -Im RC[r, f],
//   Aim[r, 2f] = Im RC[r, f],  Aim[r, 2f + 1] = Re RC[r, f],
// in 17 steps of v_mfma_f32_16x16x4_f32 per part.  Operand layout of that
// instruction: lane l holds A[l % 16][k0 + l / 16] and B[k0 + l / 16][l % 16];
// the result D[4 (l / 16) + i][l % 16] is in element i of lane l.  The row
// operands stay in registers; the B operands come from a per-channel table in
// exactly that lane order (gen_btab_body: 17 coalesced loads per tile), the
// next tile's loaded while the current tile's products run.
typedef float gen_f4 __attribute__((ext_vector_type(4)));
constexpr int kGenKS = (2 * kGenRC) / 4;  // 17 steps of 4

// The B operand table of one (channel, 16-slot tile): [17][64] floats,
// entry (j, l) = B[4 j + l / 16][16 tile + l % 16].
template <class Ctx>
__device__ __forceinline__ void gen_btab_body(const Ctx& ctx, int bid, const GenArgs& a)
{
    const int nst = a.g.S / 16, c = bid / nst, st = bid % nst;
    float* out = a.btab + (long long)bid * kGenKS * 64;
    for (int i = ctx.tid(); i < kGenKS * 64; i += kGenNT) {
        const int j = i / 64, l = i % 64, kk = 4 * j + l / 16;
        const float2 v = gen_in_factor(a, c, kk / 2, 16 * st + l % 16);
        out[i] = (kk & 1) ? v.y : v.x;
    }
}

template <class Ctx>
__device__ __forceinline__ void gen_spectrum_mfma_body(const Ctx& ctx, int bid, const GenArgs& a, float2* RC,
                                                       float2* XF, float2* X0, float2* XS)
{
    constexpr int RT = kGenRows / 64;
    static_assert(RT * 64 == kGenRows && kGenNT == 256, "four waves of 16-row tiles");
    const Geom& g = a.g;
    const GenBlock k = gen_block(a, bid);
    const int tid = ctx.tid(), lane = tid % 64, w = tid / 64;
    gen_row_factors(ctx, a, k, RC, XF);
    ctx.sync();
    constexpr int KS = kGenKS;
    const int kq = lane / 16;
    float are[RT][KS], aim[RT][KS];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int ra = 64 * t + 16 * w + lane % 16;
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const int kk = 4 * j + kq, f = kk / 2;
            const float2 v = ra < k.nr ? RC[ra * kGenRC + f] : make_float2(0.f, 0.f);
            are[t][j] = (kk & 1) ? -v.y : v.x;
            aim[t][j] = (kk & 1) ? v.x : v.y;
        }
    }
    const int S = g.S, nst = S / 16;
    const float* bt = a.btab + (long long)k.c * nst * KS * 64 + lane;
    float bn[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) bn[j] = bt[j * 64];
    for (int st = 0; st < nst; ++st) {
        float b[KS];
#pragma unroll
        for (int j = 0; j < KS; ++j) b[j] = bn[j];
        if (st + 1 < nst) {
#pragma unroll
            for (int j = 0; j < KS; ++j) bn[j] = bt[((st + 1) * KS + j) * 64];
        }
        const int s = 16 * st + lane % 16;
        gen_f4 dre[RT], dim[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) dre[t] = dim[t] = gen_f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KS; ++j) {
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                dre[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(are[t][j], b[j], dre[t], 0, 0, 0);
                dim[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(aim[t][j], b[j], dim[t], 0, 0, 0);
            }
        }
#pragma unroll
        for (int t = 0; t < RT; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 64 * t + 16 * w + 4 * kq + i;
                if (r >= k.nr) continue;
                const float2 v = make_float2(dre[t][i], dim[t][i]);
                if (s == 0) X0[r] = v;
                else a.khat[k.kbase + tm_index(g, k.rows, k.r0 + r, s)] = cscale(v, k.gsc);
            }
        }
    }
    gen_pack_slot0(ctx, a, k, RC, XF, X0, XS);
}

}  // namespace hyenand
