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
constexpr int kGenRows = 64;                    // spectrum rows per gen_spectrum workgroup
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
    float2* khat;           // [B][C][ksz]
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
    for (long long i = lo + tid; i < hi; i += kGenNT) {
        if constexpr (BF16) s += (double)bf16_to_f32(static_cast<const uint16_t*>(a.x)[base + i]);
        else s += (double)static_cast<const float*>(a.x)[base + i];
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
    for (int c = tid; c < C; c += kGenNT) {
        const double* pp = a.partial + ((long long)b * C + c) * a.splits;
        double s = 0.0;
        for (int k = 0; k < a.splits; ++k) s += pp[k];
        m[c] = (float)(s / (double)a.g.vox);
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
// the row factors of the 33 terms into LDS, then each thread runs over its
// k_in, holding that column's factors in registers, and sums the terms row by
// row.  Slot 0 packs k_in = 0 and N_in / 2 (through LDS, after the row loop).
__device__ __forceinline__ float2 gen_axis(const GenArgs& a, int ax, int c, int u, int k, int N)
{
    return N == 1 ? make_float2(1.f, 0.f) : a.basis[ax][((long long)c * kGenLines + u) * N + k];
}

template <class Ctx>
__device__ __forceinline__ void gen_spectrum_body(const Ctx& ctx, int bid, const GenArgs& a, float2* RC, float2* X0,
                                                  float2* XS)
{
    const Geom& g = a.g;
    const int rows = g.N_out * g.N_mid, nblk = (rows + kGenRows - 1) / kGenRows;
    const int p = bid / nblk, r0 = (bid % nblk) * kGenRows;
    const int c = p % a.C;
    const int tid = ctx.tid();
    const float* cf = a.coef + (long long)p * kGenCoef;
    const int nr = rows - r0 < kGenRows ? rows - r0 : kGenRows;
    // Row factors: RC[r][u] = (v_u / 2i) A_out A_mid at (k_out, k_mid),
    // RC[r][16 + u] = (v_u / 2i) conj(A_out A_mid at (-k_out, -k_mid)), RC[r][32] = e W_out W_mid.
    // Row stride NF = 34 complex (272 bytes, 16-byte aligned rows for float4
    // reads); entry 33 is padding.
    constexpr int NT3 = 2 * kGenHidden + 1, NF = NT3 + 1;
    for (int i = tid; i < nr * NT3; i += kGenNT) {
        const int r = i / NT3, f = i % NT3, row = r0 + r;
        const int ko = row / g.N_mid, km = row % g.N_mid;
        float2 v;
        if (f == 2 * kGenHidden) {
            v = cscale(cmul(gen_axis(a, 0, c, kGenHidden, ko, g.N_out), gen_axis(a, 1, c, kGenHidden, km, g.N_mid)),
                       cf[kGenHidden]);
        } else {
            const int u = f % kGenHidden;
            const bool mir = f >= kGenHidden;
            const int kom = mir ? (g.N_out - ko) % g.N_out : ko, kmm = mir ? (g.N_mid - km) % g.N_mid : km;
            float2 pr = cmul(gen_axis(a, 0, c, u, kom, g.N_out), gen_axis(a, 1, c, u, kmm, g.N_mid));
            if (mir) pr = cconj(pr);
            const float h = 0.5f * cf[u];  // v / 2i = -i v / 2
            v = make_float2(h * pr.y, -h * pr.x);
        }
        RC[r * NF + f] = v;
    }
    ctx.sync();
    const int S = g.S, N = g.N_in;
    const float gsc = 1.0f / (2.0f * (float)N * (float)g.N_out * (float)g.N_mid);
    const long long kbase = (long long)p * g.ksz;
    // Threads as (slot lane, row lane): slots k_in in [0, S) over SL lanes,
    // rows split over kGenNT / SL row lanes (S is a power of two).
    const int SL = S < kGenNT ? S : kGenNT, RL = kGenNT / SL;
    const int sl = tid % SL, rl = tid / SL;
    for (int s = sl; s < S; s += SL) {
        float2 in[kGenHidden], inm[kGenHidden];
#pragma unroll
        for (int u = 0; u < kGenHidden; ++u) {
            in[u] = gen_axis(a, 2, c, u, s, N);
            inm[u] = cconj(gen_axis(a, 2, c, u, (N - s) % N, N));
        }
        const float2 win = gen_axis(a, 2, c, kGenHidden, s, N);
        for (int r = rl; r < nr; r += RL) {
            const float4* f4 = reinterpret_cast<const float4*>(RC + r * NF);
            float2 acc = cmul(RC[r * NF + 2 * kGenHidden], win);
#pragma unroll
            for (int u = 0; u < kGenHidden; u += 2) {
                const float4 pa = f4[u / 2], pb = f4[(kGenHidden + u) / 2];
                acc = cadd(acc, cmul(make_float2(pa.x, pa.y), in[u]));
                acc = cadd(acc, cmul(make_float2(pa.z, pa.w), in[u + 1]));
                acc = csub(acc, cmul(make_float2(pb.x, pb.y), inm[u]));
                acc = csub(acc, cmul(make_float2(pb.z, pb.w), inm[u + 1]));
            }
            if (s == 0) X0[r] = acc;
            else a.khat[kbase + tm_index(g, rows, r0 + r, s)] = cscale(acc, gsc);
        }
    }
    // The Nyquist bin k_in = S of every row (one row per thread).
    if (tid < nr) {
        const int r = tid;
        float2 acc = cmul(RC[r * NF + 2 * kGenHidden], gen_axis(a, 2, c, kGenHidden, S, N));
        for (int u = 0; u < kGenHidden; ++u) {
            acc = cadd(acc, cmul(RC[r * NF + u], gen_axis(a, 2, c, u, S, N)));
            acc = csub(acc, cmul(RC[r * NF + kGenHidden + u], cconj(gen_axis(a, 2, c, u, (N - S) % N, N))));
        }
        XS[r] = acc;
    }
    ctx.sync();
    for (int r = tid; r < nr; r += kGenNT) {
        const float2 z0 = X0[r], zs = XS[r];
        a.khat[kbase + tm_index(g, rows, r0 + r, 0)] = cscale(cadd(z0, zs), 0.5f * gsc);
        a.khat[kbase + g.kmain + r0 + r] = cscale(csub(z0, zs), 0.5f * gsc);
    }
}

}  // namespace hyenand
