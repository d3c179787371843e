// conv_bodies.h -- workgroup bodies of the gated N-D FFT convolution kernels.
//
// What is computed (explainer "Native multi-dimensional subquadratic operators
// via input-dependent long convolutions", section "HyenaND: native-space
// implicit global kernel": y[i] = sum_j phi(x[j]) x[j] K[i-j], evaluated as
// FFT -> pointwise product with the kernel spectrum -> inverse FFT; gist.science
// summary of the same paper, "Methodology", "Boundary handling": zero padding
// to twice the grid, output cropped back):
//
//   u      = sigmoid(alpha_c x + beta_c) * x                          (gate)
//   U      = FFT_N(pad(u))            N = 2n on every axis             (forward)
//   Y      = U * Khat_c                                               (product)
//   y      = crop(IFFT_N(Y)) / prod N                                 (inverse)
//
// Pass structure (layouts in plan.h):
//   row_fwd   gate + real FFT of the innermost axis, two rows packed as one
//             complex line (u_a + i u_b); separated into two half spectra.
//   col_mid   forward / inverse FFT along the middle axis (3-D only).
//   col_out   forward FFT along the outermost axis, product with the kernel
//             spectrum, inverse FFT -- in one workgroup, per line tile, for
//             every batch entry of a channel.
//   row_inv   inverse real FFT of the innermost axis, crop, cast, store y.
//   conv1d    all of the above for d = 1 (one line per signal).
//   spec_*    the kernel spectrum (forward transforms only, full inputs).
//
// Every body is a function of (execution context, workgroup index, arguments,
// LDS tile); the device kernels in kernels_dev.h wrap them.
#pragma once

#include "fft_core.h"
#include "plan.h"

#include <type_traits>

namespace hyenand {

// ------------------------------------------------------------- element I/O
__host__ __device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __builtin_bit_cast(float, (uint32_t)h << 16); }

// Round to nearest even; NaN stays NaN.
__host__ __device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// I/O element type is a template parameter so that element loops carry no
// runtime branch (loads can then be issued back to back).  x is read once and
// y written once: non-temporal accesses keep them from evicting the
// workspace, which the next kernel reads back (256^2: 0.346 -> 0.329 ms).
template <bool BF16>
__host__ __device__ __forceinline__ float load_x(const ConvArgs& a, long long i)
{
    if constexpr (BF16) return bf16_to_f32(__builtin_nontemporal_load(static_cast<const uint16_t*>(a.x) + i));
    else return __builtin_nontemporal_load(static_cast<const float*>(a.x) + i);
}

// Same for another input of the I/O dtype (the output gradient of the backward).
template <bool BF16>
__host__ __device__ __forceinline__ float load_in(const void* p, long long i)
{
    if constexpr (BF16) return bf16_to_f32(__builtin_nontemporal_load(static_cast<const uint16_t*>(p) + i));
    else return __builtin_nontemporal_load(static_cast<const float*>(p) + i);
}

template <bool BF16>
__host__ __device__ __forceinline__ void store_y(const ConvArgs& a, long long i, float v)
{
    if constexpr (BF16) __builtin_nontemporal_store(f32_to_bf16(v), static_cast<uint16_t*>(a.y) + i);
    else __builtin_nontemporal_store(v, static_cast<float*>(a.y) + i);
}

// Workspace plane row of grid row r (r = j_out * n_mid + j_mid): the mid axis
// is padded to N_mid in the workspace.
__host__ __device__ __forceinline__ long long ws_row(const Geom& g, int r)
{
    return (long long)(r / g.n_mid) * g.N_mid + (r % g.n_mid);
}

// Rows of one pair's workspace plane and the stride between its slot tiles.
__host__ __device__ __forceinline__ long long ws_rows(const Geom& g) { return (long long)g.n_out * g.N_mid; }
__host__ __device__ __forceinline__ long long ws_tile_stride(const Geom& g) { return ws_rows(g) * g.lt; }

// Line pair h of a row workgroup (d >= 2): pair slot q = h / hp (channel-major
// in the chunk: c = c0 + q / B, b = q % B) and rows r = 2 (h % hp), r + 1.
template <int NP, int NT, class Ctx>
__host__ __device__ __forceinline__ void row_meta(const Ctx& ctx, int bid, const ConvArgs& a, RowMeta* M)
{
    const Geom& g = a.g;
    const int hp = g.n_out * g.n_mid / 2;
    const int H = a.nch * a.B * hp;
    for (int lp = ctx.tid(); lp < NP; lp += NT) {
        const int h = bid * NP + lp;
        RowMeta m{};
        m.valid = h < H;
        if (m.valid) {
            const int q = h / hp, r = (h % hp) * 2;
            const int c = a.c0 + q / a.B, b = q % a.B;
            m.o0 = ((long long)b * a.C + c) * g.vox + (long long)r * g.n_in;
            m.o1 = m.o0 + g.n_in;
            m.w0 = (long long)q * g.wsp + ws_row(g, r) * g.lt;
            m.w1 = (long long)q * g.wsp + ws_row(g, r + 1) * g.lt;
            m.al0 = m.al1 = a.alpha[c];
            m.be0 = m.be1 = a.beta[c];
            m.valid1 = 1;
        }
        M[lp] = m;
    }
}

// --------------------------------------------------------------- row_fwd
// NP line pairs per workgroup; gate, FFT of u_a + i u_b, separation.  Element
// loops run ITER = NP*n/NT iterations per thread; every load of a loop is
// issued before the first use (invalid tail lines read offset 0 and are zeroed).
// GATE = false transforms x as it is (the backward's output gradient).
// CIRC (circular mode): rows of n = L samples, nothing pruned.
template <int L, bool BF16, bool GATE, bool CIRC, class Ctx>
__host__ __device__ __forceinline__ void row_fwd_body(const Ctx& ctx, int bid, const ConvArgs& a, float2* T,
                                                      RowMeta* M)
{
    constexpr int NP = row_np(L), LP = row_lay(L), NT = row_nt(L), n = CIRC ? L : L / 2, S = L / 2;
    constexpr int ITER = NP * n / NT, ITS = NP * S / NT;  // element loops over samples / slots
    static_assert(NP * n % NT == 0 && NP * S % NT == 0, "whole element loops");
    const int tid = ctx.tid();
    ctx.stage();
    row_meta<NP, NT>(ctx, bid, a, M);
    ctx.sync();
    float xa[ITER], xb[ITER];
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
        const int idx = tid + i * NT, lp = idx / n, m = idx % n;
        xa[i] = load_x<BF16>(a, M[lp].o0 + m);
        xb[i] = load_x<BF16>(a, M[lp].o1 + m);
    }
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
        const int idx = tid + i * NT, lp = idx / n, m = idx % n;
        const RowMeta& md = M[lp];
        float2 z = GATE ? make_float2(ctx.gate(xa[i], md.al0, md.be0), ctx.gate(xb[i], md.al1, md.be1))
                        : make_float2(xa[i], xb[i]);
        if (!md.valid) z = make_float2(0.f, 0.f);
        T[tile_idx<LP>(m, lp)] = z;
    }
    ctx.sync();
    tile_fft<L, NP, LP, NT, false, !CIRC, false>(ctx, T);
    // Separate the two rows: with Z = FFT(u_a + i u_b),
    //   2 U_a[k] = Z[k] + conj Z[L-k],   2 U_b[k] = -i (Z[k] - conj Z[L-k]).
    // The factor 2 is folded into the kernel spectrum.
    // Lanes run over (slot in tile, line pair, slot tile) so that a wave's
    // stores cover whole runs of the tile-major workspace.
    const long long tstride = ws_tile_stride(a.g);
#pragma unroll
    for (int i = 0; i < ITS; ++i) {
        const int idx = tid + i * NT, u = idx & (a.g.lt - 1), rest = idx >> a.g.lt_log;
        const int lp = rest % NP, k = ((rest / NP) << a.g.lt_log) + u;
        const long long wo = (long long)(k >> a.g.lt_log) * tstride + u;
        const RowMeta& md = M[lp];
        const float2 Z = T[tile_idx<LP>(k, lp)];
        const float2 Zm = T[tile_idx<LP>(k == 0 ? S : L - k, lp)];
        float2 oa, ob;
        if (k == 0) {
            oa = make_float2(2.f * Z.x, 2.f * Zm.x);
            ob = make_float2(2.f * Z.y, 2.f * Zm.y);
        } else {
            oa = make_float2(Z.x + Zm.x, Z.y - Zm.y);
            ob = make_float2(Z.y + Zm.y, Zm.x - Z.x);
        }
        if (md.valid) {
            a.ws[md.w0 + wo] = oa;
            a.ws[md.w1 + wo] = ob;
        }
    }
}

// ------------------------------------------------------- backward epilogue
// Gradient of the gate u = x s, s = sigmoid(alpha x + beta), for one element:
// returns dx = du (s + alpha x s (1-s)) and sets the element's terms of
// dalpha and dbeta, du x s (1-s) * (x, 1).
template <class Ctx>
__host__ __device__ __forceinline__ float gate_vjp(const Ctx& ctx, float du, float x, float al, float be,
                                                   float2& terms)
{
    const float s = ctx.sigmoid(al * x + be);
    const float t = du * x * s * (1.0f - s);
    terms = make_float2(t * x, t);
    return du * s + al * t;
}

// Backward epilogue of a row workgroup whose inverse transform left du in T
// (line pair lp: du_a + i du_b at T[m*LP + lp], m < n): dx stored through
// store_y (y holds dx), and each line pair's sums of the dalpha and dbeta
// terms, taken in a fixed order (an LDS tree over the n elements of each
// line), written to part: one float2 per line pair for d >= 2 (both rows
// belong to one (b, c) pair), one per signal for d = 1 (part[2h], part[2h+1]).
// xa, xb: the x values of the thread's elements, loaded before the transform.
// n: samples per line (L / 2 zero-padded, L circular).
template <int L, int n, bool BF16, int ITER, int LP, int TSZ, class Ctx>
__host__ __device__ __forceinline__ void bwd_epilogue(const Ctx& ctx, int bid, const ConvArgs& a, float2* T,
                                                      const RowMeta* M, const float* xa, const float* xb)
{
    constexpr int NP = row_np(L), NT = row_nt(L);
    const int tid = ctx.tid();
    float2 ea[ITER], eb[ITER];
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
        const int idx = tid + i * NT, lp = idx / n, m = idx % n;
        const RowMeta& md = M[lp];
        const float2 z = T[tile_idx<LP>(m, lp)];
        ea[i] = make_float2(0.f, 0.f);
        eb[i] = make_float2(0.f, 0.f);
        if (md.valid) {
            store_y<BF16>(a, md.o0 + m, gate_vjp(ctx, z.x, xa[i], md.al0, md.be0, ea[i]));
            if (md.valid1) store_y<BF16>(a, md.o1 + m, gate_vjp(ctx, z.y, xb[i], md.al1, md.be1, eb[i]));
        }
    }
    ctx.sync();  // every read of du in T is done
    // The two rows' terms sit side by side in T when they fit (n = L/2);
    // circular lines (n = L) take them one row after the other.
    constexpr int NH = 2 * NP * n <= TSZ ? 2 : 1;
    for (int r0 = 0; r0 < 2; r0 += NH) {
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            const int idx = tid + i * NT;
            T[idx] = r0 ? eb[i] : ea[i];
            if (NH == 2) T[NP * n + idx] = eb[i];
        }
        ctx.sync();
        for (int h = n / 2; h >= 1; h /= 2) {
            for (int e = tid; e < NH * NP * h; e += NT) {
                const int half = e / (NP * h), r = e % (NP * h), lp = r / h, m = r % h;
                float2* E = T + half * NP * n;
                E[lp * n + m] = cadd(E[lp * n + m], E[lp * n + m + h]);
            }
            ctx.sync();
        }
        for (int lp = tid; lp < NP; lp += NT) {
            const RowMeta& md = M[lp];
            if (!md.valid) continue;
            const long long h = (long long)bid * NP + lp;
            const float2 s0 = T[lp * n];
            if (a.g.d == 1) {
                if (r0 == 0) a.part[2 * h] = s0;
                if (md.valid1 && (NH == 2 || r0 == 1)) a.part[2 * h + 1] = NH == 2 ? T[NP * n + lp * n] : s0;
            } else if (NH == 2) {
                a.part[h] = cadd(s0, T[NP * n + lp * n]);
            } else {
                a.part[h] = r0 == 0 ? s0 : cadd(a.part[h], s0);  // this thread wrote part[h] in the first pass
            }
        }
        if (NH == 1 && r0 == 0) ctx.sync();  // the second row's terms overwrite T
    }
}

// --------------------------------------------------------------- row_inv
// BWD: the inverse transforms carry du; the epilogue computes dx and the
// partial sums of dalpha and dbeta (x is read again: the forward saves no
// intermediate, the explainer's gradient-checkpointing pattern).
// CIRC (circular mode): every one of the L outputs is kept.
template <int L, bool BF16, bool BWD, bool CIRC, class Ctx>
__host__ __device__ __forceinline__ void row_inv_body(const Ctx& ctx, int bid, const ConvArgs& a, float2* T,
                                                      RowMeta* M)
{
    constexpr int NP = row_np(L), LP = row_lay(L), NT = row_nt(L), n = CIRC ? L : L / 2, S = L / 2;
    constexpr int ITER = NP * S / NT, ITO = NP * n / NT;
    static_assert(NP * S % NT == 0 && NP * n % NT == 0, "whole element loops");
    const int tid = ctx.tid();
    ctx.stage();
    row_meta<NP, NT>(ctx, bid, a, M);
    ctx.sync();
    // Rebuild Z = Y_a + i Y_b over the full length from the two half spectra
    // (Hermitian extension), slot 0 holding (bin 0, bin L/2).
    // Lanes run over (slot in tile, line pair, slot tile): whole runs of the
    // tile-major workspace per wave.
    const long long tstride = ws_tile_stride(a.g);
    auto slot = [&](int idx, int& lp) {
        const int u = idx & (a.g.lt - 1), rest = idx >> a.g.lt_log;
        lp = rest % NP;
        return ((rest / NP) << a.g.lt_log) + u;
    };
    float2 ya[ITER], yb[ITER];
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
        int lp;
        const int k = slot(tid + i * NT, lp);
        const long long wo = (long long)(k >> a.g.lt_log) * tstride + (k & (a.g.lt - 1));
        ya[i] = a.ws[M[lp].w0 + wo];
        yb[i] = a.ws[M[lp].w1 + wo];
    }
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
        int lp;
        const int k = slot(tid + i * NT, lp);
        if (k == 0) {
            T[tile_idx<LP>(0, lp)] = make_float2(ya[i].x, yb[i].x);
            T[tile_idx<LP>(S, lp)] = make_float2(ya[i].y, yb[i].y);
        } else {
            T[tile_idx<LP>(k, lp)] = make_float2(ya[i].x - yb[i].y, ya[i].y + yb[i].x);
            T[tile_idx<LP>(L - k, lp)] = make_float2(ya[i].x + yb[i].y, yb[i].x - ya[i].y);
        }
    }
    float xa[BWD ? ITO : 1], xb[BWD ? ITO : 1];
    if constexpr (BWD) {
#pragma unroll
        for (int i = 0; i < ITO; ++i) {
            const int idx = tid + i * NT, lp = idx / n, m = idx % n;
            xa[i] = load_x<BF16>(a, M[lp].o0 + m);
            xb[i] = load_x<BF16>(a, M[lp].o1 + m);
        }
    }
    ctx.sync();
    tile_fft<L, NP, LP, NT, true, false, !CIRC>(ctx, T);
    if constexpr (BWD) {
        bwd_epilogue<L, n, BF16, ITO, LP, lay_elems(L, NP, LP)>(ctx, bid, a, T, M, xa, xb);
    } else {
#pragma unroll
        for (int i = 0; i < ITO; ++i) {
            const int idx = tid + i * NT, lp = idx / n, m = idx % n;
            const RowMeta& md = M[lp];
            const float2 z = T[tile_idx<LP>(m, lp)];
            if (md.valid) {
                store_y<BF16>(a, md.o0 + m, z.x);
                store_y<BF16>(a, md.o1 + m, z.y);
            }
        }
    }
}

// --------------------------------------------------------------- col_mid
// FFT along the middle axis of a 3-D grid, TW adjacent lines per workgroup.
// Forward: n_mid non-zero inputs -> N_mid outputs.  Inverse: N_mid inputs ->
// the n_mid outputs that are kept.  The first pass reads the workspace and the
// last pass writes it back (in place; every read precedes a barrier that
// precedes every write).
template <int L, bool INV, bool CIRC, class Ctx>
__host__ __device__ __forceinline__ void col_mid_body(const Ctx& ctx, int bid, const ConvArgs& a, float2* T)
{
    constexpr int TW = col_tw(L), NT = col_nt(L);
    const Geom& g = a.g;
    const int lines = g.n_out * g.S;
    const int tpp = (lines + TW - 1) / TW;
    const int q = bid / tpp, lam0 = (bid % tpp) * TW;
    float2* base = a.ws + (long long)q * g.wsp;
    const int sl = ilog2(g.S);
    const long long rows = ws_rows(g);
    auto off = [&](int pos, int l) -> long long {
        const int lam = lam0 + l;
        return tm_index(g, rows, (long long)(lam >> sl) * g.N_mid + pos, lam & (g.S - 1));
    };
    auto ld = [&](int pos, int l) -> float2 {
        const bool ok = lam0 + l < lines;
        const float2 v = base[ok ? off(pos, l) : 0];
        return ok ? v : make_float2(0.f, 0.f);
    };
    auto st = [&](int pos, int l, const float2& v) {
        if (lam0 + l < lines) base[off(pos, l)] = v;
    };
    auto after_load = [&]() { ctx.stage(); };
    if constexpr (INV) inv_fn_to_fn<L, TW, NT, !CIRC>(ctx, T, ld, st, after_load);
    else fwd_fn_to_fn<L, TW, NT, !CIRC>(ctx, T, ld, st, after_load);
}

// Rows of the middle axis handled together by one out-axis workgroup: with
// NR = 2 the rows {rp, N_mid - rp} (and {0, N_mid/2} for rp = 0), so that the
// slot-0 line of k_mid and its mirror -k_mid are in the same tile.
//
// Workgroup order: consecutive workgroup ids are dispatched round-robin over
// the eight XCDs, each with its own L2.  Work item w = u*B + b (u the tile
// index, b the batch entry) goes to id (w mod W8/8)*8 + w / (W8/8) for the
// first W8 = W & ~7 items, so XCD x runs the contiguous items
// [x W8/8, (x+1) W8/8) in order: the B workgroups of a tile read the same
// kernel spectrum tile and neighbouring tiles share the cache lines at the
// edges of their row segments, both within one L2.
struct OutTile {
    int c_local, t, b, rows[2];
    bool self_mirror;
};

template <int NR, int TW>
__host__ __device__ __forceinline__ OutTile out_tile(const Geom& g, int B, int nch, int bid)
{
    OutTile o;
    const int ct = (g.S + TW - 1) / TW;
    const int nrp = NR == 1 ? 1 : g.N_mid / 2;
    const int tpc = nrp * ct;
    const int W = nch * tpc * B, W8 = W & ~7;
    const int w = bid < W8 ? (bid % 8) * (W8 / 8) + bid / 8 : bid;
    const int u = w / B;
    o.b = w % B;
    o.c_local = u / tpc;
    const int r2 = u % tpc;
    // Two-row tiles that fill their slot tile (TW >= lt: each row segment is
    // one whole run of the tile-major plane) take the row pairs fastest, so
    // that the workgroups one XCD runs together read adjacent runs (rows rp,
    // rp + 1, ... and their mirrors) at every out-axis position: 128^3
    // k_col_out 251.5 -> 225.6 us per launch.  Tiles of half a slot tile
    // (the backward's 8-slot tiles of 16-slot runs) keep the two halves of a
    // run together, then take the row pairs (128^3 k_col_out_bwd 194.7 ->
    // 187.0 us against the slot tiles fastest).  Narrower tiles share their
    // slot tile with more neighbours and keep the slot tiles fastest (512^3:
    // 2.77 ms, against 2.97 with the row pairs fastest).
    int rp;
    if (NR == 2 && TW >= g.lt) {
        rp = r2 % nrp;
        o.t = r2 / nrp;
    } else if (NR == 2 && 2 * TW == g.lt && ct % 2 == 0) {
        const int hi = r2 / (2 * nrp), rem = r2 % (2 * nrp);
        rp = rem / 2;
        o.t = 2 * hi + rem % 2;
    } else {
        rp = r2 / ct;
        o.t = r2 % ct;
    }
    if (NR == 1) {
        o.rows[0] = 0; o.rows[1] = 0; o.self_mirror = true;
    } else {
        o.rows[0] = rp;
        o.rows[1] = rp == 0 ? g.N_mid / 2 : g.N_mid - rp;
        o.self_mirror = rp == 0;
    }
    return o;
}

// Product for the lines with k_in = 0 (present in tile t = 0, column 0 of each
// row), in place in T (element (pos, row*TW) at pos*NL + row*TW).  Those lines
// carry Z = A + iB (packed bins 0 and N_in/2) and need the mirror element
// (-k_out, -k_mid):  W = Z Sv + conj(Z(-k)) Dv.  Each job owns an element and
// its mirror, so no two threads touch the same element.
// CONJ multiplies by the conjugate spectrum (the backward's correlation with
// K): Sv, Dv of a real kernel conjugate like the spectrum itself.
template <int L, int NR, int TW, int NT, bool CONJ = false, int LP = NR * TW, class Ctx>
__host__ __device__ __forceinline__ void out_slot0_product(const Ctx& ctx, const Geom& g, const OutTile& o,
                                                           const float2* kc, float2* T)
{
    constexpr int NL = NR * TW;
    const long long PS = (long long)g.N_mid * g.lt;  // slot 0 of (k_out, k_mid): (k_out N_mid + k_mid) lt
    const int njobs = o.self_mirror ? NR * (L / 2 + 1) : L;
    for (int job = ctx.tid(); job < njobs; job += NT) {
        int ra, rb, pa, pb;
        if (o.self_mirror) {
            ra = job / (L / 2 + 1); rb = ra;
            pa = job % (L / 2 + 1); pb = (L - pa) % L;
        } else {
            ra = 0; rb = 1; pa = job; pb = (L - job) % L;
        }
        const int ea = tile_idx<LP>(pa, ra * TW), eb = tile_idx<LP>(pb, rb * TW);
        const float2 Za = T[ea], Zb = T[eb];
        auto kv = [](float2 v) { return CONJ ? cconj(v) : v; };
        // row of the ra / rb block by selection, not by indexing o.rows with a
        // runtime value (which would put o in scratch memory)
        const long long rwa = ra == 0 ? o.rows[0] : o.rows[1], rwb = rb == 0 ? o.rows[0] : o.rows[1];
        const float2 Sa = kv(kc[pa * PS + rwa * g.lt]);
        const float2 Sb = kv(kc[pb * PS + rwb * g.lt]);
        const float2 Da = kv(kc[g.kmain + (long long)pa * g.N_mid + rwa]);
        const float2 Db = kv(kc[g.kmain + (long long)pb * g.N_mid + rwb]);
        const float2 Wa = cadd(cmul(Za, Sa), cmul(cconj(Zb), Da));
        const float2 Wb = cadd(cmul(Zb, Sb), cmul(cconj(Za), Db));
        T[ea] = Wa;
        if (eb != ea) T[eb] = Wb;
    }
}

// --------------------------------------------------------------- col_out
// p advanced by a 32-bit byte offset (a lane offset added to a wave-uniform
// base: the form global loads and stores take without 64-bit lane arithmetic).
template <class T>
__host__ __device__ __forceinline__ T* add_bytes(T* p, unsigned bytes)
{
    using Byte = std::conditional_t<std::is_const_v<T>, const char, char>;
    return reinterpret_cast<T*>(reinterpret_cast<Byte*>(p) + bytes);
}

// Work items of the out-axis kernel: (channel, tile, batch entry).
template <int NR, int TW>
__host__ __device__ __forceinline__ int out_items(const Geom& g, int B, int nch)
{
    const int ct = (g.S + TW - 1) / TW;
    const int nrp = NR == 1 ? 1 : g.N_mid / 2;
    return nch * nrp * ct * B;
}

// Addresses of one out-axis work item.  The tile's slots k0 + [0, TW) lie in
// one slot tile of the tile-major planes (the slot tile is a power of two, a
// multiple of TW or S < TW), whose rows are k_out * N_mid + k_mid; the tile
// starts at slot u0 = k0 % lt of its slot tile.
struct OutView {
    OutTile o;
    int k0, u0;
    const float2* kc;  // the channel's kernel spectrum
    const float2* kt;  // its slot tile
    float2* base;      // the pair's workspace slot tile
};

template <int NR, int TW>
__host__ __device__ __forceinline__ OutView out_view(const ConvArgs& a, int item)
{
    const Geom& g = a.g;
    OutView v;
    v.o = out_tile<NR, TW>(g, a.B, a.nch, item);
    v.k0 = v.o.t * TW;
    v.u0 = v.k0 & (g.lt - 1);
    v.kc = a.khat + (long long)(a.c0 + v.o.c_local) * g.ksz + (long long)v.o.b * a.khat_bstride;
    v.kt = v.kc + (long long)(v.k0 >> g.lt_log) * ((long long)g.N_out * g.N_mid * g.lt);
    v.base = a.ws + ((long long)v.o.c_local * a.B + v.o.b) * g.wsp + (long long)(v.k0 >> g.lt_log) * ws_tile_stride(g);
    return v;
}

// Out axis: forward FFT whose first pass reads the n_out rows of the
// workspace, product with the kernel spectrum in registers (the forward's last
// pass leaves each thread holding exactly the positions the inverse's first
// pass needs), inverse FFT whose last pass writes the n_out kept rows back.
// Looping kernels (out_looped) run the items bid, bid + nblk, ... (nblk = the
// grid, one workgroup per CU): no workgroup launch and tail per item, and the
// item ids keep the XCD-blocked order of out_tile when nblk is a multiple of 8.
// CIRC (circular mode): all L positions are read and written.
template <int L, int NR, bool CIRC, class Ctx>
__host__ __device__ __forceinline__ void col_out_body(const Ctx& ctx, int bid, int nblk, const ConvArgs& a,
                                                      float2* T)
{
    constexpr int TW = out_tw(L, NR);
    constexpr int NL = NR * TW, NT = out_nt(L, NR), LP = out_lay(L, NR);
    constexpr int R0 = pass_radix<L, false>(0);
    constexpr int RL = pass_radix<L, false>(plan_passes(L) - 1);
    constexpr bool kLoop = out_looped(L, NR);
    const Geom& g = a.g;
    const int W = out_items<NR, TW>(g, a.B, a.nch);
    if (bid >= W) return;
    const int tid = ctx.tid();
    // Position stride of the planes; element (pos = j + q, line l) is at q*PS
    // (wave-uniform, q a constant of the unrolled loops) plus the lane's byte
    // offset 8*(j*PS + row*lt + u0 + l%TW) inside one slot tile of a plane
    // (N_out N_mid lt complex with N <= 2048, lt <= 64: at most 2 GiB).
    const long long PS = (long long)g.N_mid * g.lt;
    auto lane_bytes = [&](const OutView& v, int j, int l) -> unsigned {
        return 8u * ((unsigned)j * (unsigned)PS + (unsigned)v.o.rows[l / TW] * (unsigned)g.lt + (unsigned)(v.u0 + l % TW));
    };
    auto at = [](auto* p, long long q_elems, unsigned bytes) { return add_bytes(p + q_elems, bytes); };
    using P0 = PassRegs<L, R0, NL, NT>;
    using PL = PassRegs<L, RL, NL, NT>;
    // FULL (wave-uniform): every line of the tile lies inside the grid (the
    // tile's slots k0 .. k0 + TW - 1 are all below S), so the loads, products
    // and stores need no per-lane guards; only edge tiles take the guarded code.
    auto load_cols = [&]<bool FULL>(const OutView& v, P0& s) {
        pass_load_fn<L, R0, NL, NT, !CIRC>(ctx, [&](int j, int q, int l) -> float2 {
            if constexpr (FULL) {
                return *at(v.base, q * PS, lane_bytes(v, j, l));
            } else {
                const bool ok = v.k0 + l % TW < g.S;
                const float2 x = *at(v.base, q * PS, ok ? lane_bytes(v, j, l) : 0u);
                return ok ? x : make_float2(0.f, 0.f);
            }
        }, s);
    };
    // Kernel spectrum values for the positions this thread multiplies (the
    // forward's last pass: positions j + r*L/RL); kok: a line inside the grid
    // whose k_in is not 0 (the k_in = 0 lines take the mirror product).
    float2 kv[PL::PER][RL];
    bool kok[PL::PER];
    auto load_kv = [&]<bool FULL>(const OutView& v) {
#pragma unroll
        for (int i = 0; i < PL::PER; ++i) {
            const int gi = tid + i * NT, l = gi % NL, j = gi / NL;
            kok[i] = bf_valid<PL::NB, NT>(gi) && (FULL || v.k0 + l % TW < g.S) && v.k0 + l % TW != 0;
            const unsigned lb = (FULL && bf_valid<PL::NB, NT>(gi)) || kok[i] ? lane_bytes(v, j, l) : 8u;
#pragma unroll
            for (int r = 0; r < RL; ++r) kv[i][r] = *at(v.kt, (long long)r * (L / RL) * PS, lb);
        }
    };
    auto full_tile = [&](const OutView& v) { return v.k0 + TW <= g.S; };
    auto load_item = [&](const OutView& v, P0& s) {
        if (full_tile(v)) {
            load_cols.template operator()<true>(v, s);
            load_kv.template operator()<true>(v);
        } else {
            load_cols.template operator()<false>(v, s);
            load_kv.template operator()<false>(v);
        }
    };
    // One item: forward from the loaded columns, product, inverse and store
    // (c: the context whose passes run the transforms).
    auto run_item = [&](const auto& c, const OutView& v, P0& s) {
        auto t = fwd_from_regs<L, NL, NT, !CIRC, LP>(c, T, s);
        ctx.sync();  // every LDS read of the forward transform is done: T is free
        if (v.o.t == 0) {
            pass_visit<L, RL, NL, NT, false>(ctx, t, [&](int pos, int l, float2& x) {
                if (l % TW == 0) T[tile_idx<LP>(pos, l)] = x;
            });
            ctx.sync();
            out_slot0_product<L, NR, TW, NT, false, LP>(ctx, g, v.o, v.kc, T);
            ctx.sync();
            pass_visit<L, RL, NL, NT, false>(ctx, t, [&](int pos, int l, float2& x) {
                if (l % TW == 0) x = T[tile_idx<LP>(pos, l)];
            });
            ctx.sync();
        }
        // Lines outside the grid and the k_in = 0 lines (final already) keep
        // their values; tiles with neither multiply every line.
        const bool full = full_tile(v);
        if (full && v.o.t != 0 && (PL::NB % NT) == 0) {
#pragma unroll
            for (int i = 0; i < PL::PER; ++i) {
#pragma unroll
                for (int r = 0; r < RL; ++r) t.v[i][r] = cmul(t.v[i][r], kv[i][r]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < PL::PER; ++i) {
#pragma unroll
                for (int r = 0; r < RL; ++r) {
                    const float2 m = cmul(t.v[i][r], kv[i][r]);
                    t.v[i][r] = kok[i] ? m : t.v[i][r];
                }
            }
        }
        if (full) {
            inv_to_fn<L, NL, NT, !CIRC, LP>(c, T, t, [&](int j, int q, int l, const float2& x) {
                *at(v.base, q * PS, lane_bytes(v, j, l)) = x;
            });
        } else {
            inv_to_fn<L, NL, NT, !CIRC, LP>(c, T, t, [&](int j, int q, int l, const float2& x) {
                if (v.k0 + l % TW < g.S) *at(v.base, q * PS, lane_bytes(v, j, l)) = x;
            });
        }
    };
    OutView v = out_view<NR, TW>(a, bid);
    const auto tw_staged = ctx.stage_load();  // oldest loads: waited for first
    P0 s;
    load_item(v, s);
    ctx.stage_store(tw_staged);
    if constexpr (out_tw_regs(L, NR) > 0 && !kLoop) {
        // The first twiddled pass's factors in registers for the forward and
        // the (same-plan) inverse transform: one barrier after staging, then
        // one LDS read per factor instead of one per factor and transform.
        using Cache = TwCache<L, NL, NT, 1 + out_tw_regs(L, NR)>;
        Cache twc;
        ctx.sync();
        twc.load(ctx, [&](int e) { return ctx.twl[e]; });
        run_item(TwCachedCtx<Ctx, Cache>{ctx, &twc}, v, s);
    } else if constexpr (!kLoop) {
        run_item(ctx, v, s);
    } else {
        for (int item = bid;;) {
            const int nxt = item + nblk;
            run_item(ctx, v, s);
            if (nxt >= W) break;
            item = nxt;
            v = out_view<NR, TW>(a, nxt);
            load_item(v, s);
            ctx.sync();  // the inverse's last LDS reads are done: T is free
        }
    }
}

// Kernel-gradient product for the k_in = 0 lines of tile 0: T holds, in
// column 0 of each row block, the forward out-axis transform Zd of the output
// gradient and, in column 1, Zu of the gated input (both packed: Z = A + iB,
// A and B the spectra of the bin-0 and bin-N_in/2 planes).  Writes to column
// 2 the packed product  P = A_d conj(A_u) + i B_d conj(B_u),  with
// A = (Z(k) + conj Z(-k))/2 and B = (Z(k) - conj Z(-k))/(2i); the mirror
// element takes P(-k) = conj(A_d) A_u + i conj(B_d) B_u (A and B Hermitian).
template <int L, int NR, int TW, int NT, class Ctx>
__host__ __device__ __forceinline__ void out_slot0_corr(const Ctx& ctx, const OutTile& o, float2* T)
{
    constexpr int NL = NR * TW;
    const int njobs = o.self_mirror ? NR * (L / 2 + 1) : L;
    for (int job = ctx.tid(); job < njobs; job += NT) {
        int ra, rb, pa, pb;
        if (o.self_mirror) {
            ra = job / (L / 2 + 1); rb = ra;
            pa = job % (L / 2 + 1); pb = (L - pa) % L;
        } else {
            ra = 0; rb = 1; pa = job; pb = (L - job) % L;
        }
        const int ea = pa * NL + ra * TW, eb = pb * NL + rb * TW;
        const float2 Da = T[ea], Db = T[eb], Ua = T[ea + 1], Ub = T[eb + 1];
        const float2 Ad = cscale(cadd(Da, cconj(Db)), 0.5f), Au = cscale(cadd(Ua, cconj(Ub)), 0.5f);
        const float2 vd = csub(Da, cconj(Db)), vu = csub(Ua, cconj(Ub));
        const float2 Bd = make_float2(0.5f * vd.y, -0.5f * vd.x), Bu = make_float2(0.5f * vu.y, -0.5f * vu.x);
        const float2 pA = cmulc(Ad, Au), pB = cmulc(Bd, Bu);
        T[ea + 2] = make_float2(pA.x - pB.y, pA.y + pB.x);
        if (eb != ea) {
            const float2 qA = cmulc(Au, Ad), qB = cmulc(Bu, Bd);  // conj(A_d) A_u, conj(B_d) B_u
            T[eb + 2] = make_float2(qA.x - qB.y, qA.y + qB.x);
        }
    }
}

// Backward out axis, one (channel, tile) per workgroup, looping over the B
// batch entries (the kernel spectrum tile is read once per workgroup):
//   DY_b = forward out-axis FFT of the output-gradient columns,
//   du_b = pruned inverse of DY_b conj(Khat), written back in place,
// and with DK also
//   U_b  = forward out-axis FFT of the gated-input columns,
//   P   += DY_b conj(U_b)   (registers; k_in = 0 lines through out_slot0_corr)
// followed by the full inverse of P (all N_out positions: the kernel gradient
// lives on every offset) into the kernel-gradient planes dkw.
// CIRC (circular mode): all L positions read and written.
template <int L, int NR, bool DK, bool CIRC, class Ctx>
__host__ __device__ __forceinline__ void col_out_bwd_body(const Ctx& ctx, int bid, const ConvArgs& a, float2* T)
{
    constexpr int TW = bwd_tw(L, NR);
    constexpr int NL = NR * TW, NT = bwd_nt(L, NR);
    constexpr int R0 = pass_radix<L, false>(0);
    constexpr int RL = pass_radix<L, false>(plan_passes(L) - 1);
    static_assert(TW >= 3, "the k_in = 0 staging uses three columns per row block");
    const Geom& g = a.g;
    const int tid = ctx.tid();
    const OutTile o = out_tile<NR, TW>(g, 1, a.nch, bid);
    const int k0 = o.t * TW, u0 = k0 & (g.lt - 1);
    const long long tile = k0 >> g.lt_log;
    // Position stride of the planes (workspace, kernel spectrum and dkw alike);
    // lane offsets as in col_out_body.
    const long long PS = (long long)g.N_mid * g.lt;
    const float2* kc = a.khat + (long long)(a.c0 + o.c_local) * g.ksz;
    const float2* kt = kc + tile * ((long long)g.N_out * g.N_mid * g.lt);
    auto lane_bytes = [&](int j, int l) -> unsigned {
        return 8u * ((unsigned)j * (unsigned)PS + (unsigned)o.rows[l / TW] * (unsigned)g.lt + (unsigned)(u0 + l % TW));
    };
    auto at = [](auto* p, long long q_elems, unsigned bytes) { return add_bytes(p + q_elems, bytes); };
    auto lvalid = [&](int l) { return k0 + l % TW < g.S; };
    using P0 = PassRegs<L, R0, NL, NT>;
    using PL = PassRegs<L, RL, NL, NT>;
    auto load_cols = [&](const float2* base, P0& s) {
        pass_load_fn<L, R0, NL, NT, !CIRC>(ctx, [&](int j, int q, int l) -> float2 {
            const bool ok = lvalid(l);
            const float2 x = *at(base, q * PS, ok ? lane_bytes(j, l) : 0u);
            return ok ? x : make_float2(0.f, 0.f);
        }, s);
    };
    float2 kv[PL::PER][RL];
    bool kok[PL::PER];
    const auto tw_staged = ctx.stage_load();
#pragma unroll
    for (int i = 0; i < PL::PER; ++i) {
        const int gi = tid + i * NT, l = gi % NL, j = gi / NL;
        kok[i] = bf_valid<PL::NB, NT>(gi) && lvalid(l) && k0 + l % TW != 0;
        const unsigned lb = kok[i] ? lane_bytes(j, l) : 8u;
#pragma unroll
        for (int r = 0; r < RL; ++r) kv[i][r] = *at(kt, (long long)r * (L / RL) * PS, lb);
    }
    ctx.stage_store(tw_staged);
    PL P;
    if constexpr (DK) {
#pragma unroll
        for (int i = 0; i < PL::PER; ++i)
#pragma unroll
            for (int r = 0; r < RL; ++r) P.v[i][r] = make_float2(0.f, 0.f);
    }
    for (int b = 0; b < a.B; ++b) {
        const long long poff = ((long long)o.c_local * a.B + b) * g.wsp + tile * ws_tile_stride(g);
        float2* bdy = a.ws + poff;
        P0 s;
        load_cols(bdy, s);
        PL t = fwd_from_regs<L, NL, NT, !CIRC>(ctx, T, s);
        ctx.sync();  // every LDS read of the transform is done: T is free
        PL tu;
        if constexpr (DK) {
            P0 s2;
            load_cols(a.ws_u + poff, s2);
            tu = fwd_from_regs<L, NL, NT, !CIRC>(ctx, T, s2);
            ctx.sync();
        }
        if (o.t == 0) {
            pass_visit<L, RL, NL, NT, false>(ctx, t, [&](int pos, int l, float2& x) {
                if (l % TW == 0) T[pos * NL + l] = x;
            });
            if constexpr (DK) {
                pass_visit<L, RL, NL, NT, false>(ctx, tu, [&](int pos, int l, float2& x) {
                    if (l % TW == 0) T[pos * NL + l + 1] = x;
                });
                ctx.sync();
                out_slot0_corr<L, NR, TW, NT>(ctx, o, T);
            }
            ctx.sync();
            out_slot0_product<L, NR, TW, NT, true>(ctx, g, o, kc, T);
            ctx.sync();
            pass_visit<L, RL, NL, NT, false>(ctx, t, [&](int pos, int l, float2& x) {
                if (l % TW == 0) x = T[pos * NL + l];
            });
            if constexpr (DK) {
                pass_visit<L, RL, NL, NT, false>(ctx, P, [&](int pos, int l, float2& x) {
                    if (l % TW == 0) x = cadd(x, T[pos * NL + l + 2]);
                });
            }
            ctx.sync();
        }
        // Lines outside the grid and the k_in = 0 lines (done above) keep their values.
#pragma unroll
        for (int i = 0; i < PL::PER; ++i) {
#pragma unroll
            for (int r = 0; r < RL; ++r) {
                if constexpr (DK) {
                    const float2 pc = cadd(P.v[i][r], cmulc(t.v[i][r], tu.v[i][r]));
                    P.v[i][r] = kok[i] ? pc : P.v[i][r];
                }
                const float2 m = cmulc(t.v[i][r], kv[i][r]);
                t.v[i][r] = kok[i] ? m : t.v[i][r];
            }
        }
        inv_to_fn<L, NL, NT, !CIRC>(ctx, T, t, [&](int j, int q, int l, const float2& x) {
            if (lvalid(l)) *at(bdy, q * PS, lane_bytes(j, l)) = x;
        });
        ctx.sync();  // the inverse's last LDS reads are done: T is free
    }
    if constexpr (DK) {
        float2* dk = a.dkw + (long long)o.c_local * g.kmain + tile * ((long long)g.N_out * g.N_mid * g.lt);
        inv_to_fn<L, NL, NT, false>(ctx, T, P, [&](int j, int q, int l, const float2& x) {
            if (lvalid(l)) *at(dk, q * PS, lane_bytes(j, l)) = x;
        });
    }
}

// ---------------------------------------------------------------- conv1d
// d = 1: the two signals of a line belong to consecutive pair slots (possibly
// different channels), so the product is applied to the separated half spectra.
// RowMeta: w0 / w1 hold the kernel spectrum offsets of the two channels.
// BWD: the line carries the output gradients dy (no gate), the product takes
// the conjugate spectrum (a correlation with K), and the backward epilogue
// turns du into dx and the dalpha / dbeta partial sums.
// CIRC (circular mode): lines of n = L samples, nothing pruned or cropped.
template <int L, bool BF16, bool BWD, bool CIRC, class Ctx>
__host__ __device__ __forceinline__ void conv1d_body(const Ctx& ctx, int bid, const ConvArgs& a, float2* T,
                                                     RowMeta* M)
{
    constexpr int NP = row_np(L), LP = row_lp(L), NT = row_nt(L), n = CIRC ? L : L / 2, S = L / 2;
    const Geom& g = a.g;
    const int P = a.nch * a.B;
    const int H = (P + 1) / 2;
    const int tid = ctx.tid();
    ctx.stage();
    for (int lp = tid; lp < NP; lp += NT) {
        const int h = bid * NP + lp;
        RowMeta m{};
        m.valid = h < H;
        if (m.valid) {
            const int qa = 2 * h, qb = 2 * h + 1;
            m.valid1 = qb < P;
            const int ca = a.c0 + qa / a.B, ba = qa % a.B;
            const int cb = m.valid1 ? a.c0 + qb / a.B : ca, bb = m.valid1 ? qb % a.B : ba;
            m.o0 = ((long long)ba * a.C + ca) * g.vox;
            m.o1 = ((long long)bb * a.C + cb) * g.vox;
            m.w0 = (long long)ca * g.ksz + (long long)ba * a.khat_bstride;
            m.w1 = (long long)cb * g.ksz + (long long)bb * a.khat_bstride;
            m.al0 = a.alpha[ca]; m.be0 = a.beta[ca];
            m.al1 = a.alpha[cb]; m.be1 = a.beta[cb];
        }
        M[lp] = m;
    }
    ctx.sync();
    constexpr int ITER = NP * n / NT;
    static_assert(NP * n % NT == 0, "whole element loops");
    float xa[BWD ? ITER : 1], xb[BWD ? ITER : 1];
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
        const int idx = tid + i * NT, lp = idx / n, m = idx % n;
        const RowMeta& md = M[lp];
        float2 z = make_float2(0.f, 0.f);
        if (md.valid) {
            if constexpr (BWD) {
                xa[i] = load_x<BF16>(a, md.o0 + m);
                xb[i] = md.valid1 ? load_x<BF16>(a, md.o1 + m) : 0.f;
                z.x = load_in<BF16>(a.dy, md.o0 + m);
                if (md.valid1) z.y = load_in<BF16>(a.dy, md.o1 + m);
            } else {
                z.x = ctx.gate(load_x<BF16>(a, md.o0 + m), md.al0, md.be0);
                if (md.valid1) z.y = ctx.gate(load_x<BF16>(a, md.o1 + m), md.al1, md.be1);
            }
        } else if constexpr (BWD) {
            xa[i] = 0.f;
            xb[i] = 0.f;
        }
        T[m * LP + lp] = z;
    }
    ctx.sync();
    tile_fft<L, NP, LP, NT, false, !CIRC, false>(ctx, T);
    for (int idx = tid; idx < NP * S; idx += NT) {
        const int lp = idx / S, k = idx % S;
        const RowMeta& md = M[lp];
        if (!md.valid) continue;
        const float2* ka = a.khat + md.w0;
        const float2* kb = a.khat + md.w1;
        // the spectrum value, conjugated for the backward
        auto kv = [](const float2* p, int i) { const float2 v = p[i]; return BWD ? cconj(v) : v; };
        if (k == 0) {
            const float2 Z0 = T[lp], ZS = T[S * LP + lp];
            const float2 Xa = make_float2(2.f * Z0.x, 2.f * ZS.x), Xb = make_float2(2.f * Z0.y, 2.f * ZS.y);
            const float2 Wa = cadd(cmul(Xa, kv(ka, 0)), cmul(cconj(Xa), kv(ka, S)));
            float2 Wb = cadd(cmul(Xb, kv(kb, 0)), cmul(cconj(Xb), kv(kb, S)));
            if (!md.valid1) Wb = make_float2(0.f, 0.f);
            T[lp] = make_float2(Wa.x, Wb.x);
            T[S * LP + lp] = make_float2(Wa.y, Wb.y);
        } else {
            const float2 Z = T[k * LP + lp], Zm = T[(L - k) * LP + lp];
            const float2 Xa = make_float2(Z.x + Zm.x, Z.y - Zm.y), Xb = make_float2(Z.y + Zm.y, Zm.x - Z.x);
            const float2 Ya = cmul(Xa, kv(ka, k));
            float2 Yb = cmul(Xb, kv(kb, k));
            if (!md.valid1) Yb = make_float2(0.f, 0.f);
            T[k * LP + lp] = make_float2(Ya.x - Yb.y, Ya.y + Yb.x);
            T[(L - k) * LP + lp] = make_float2(Ya.x + Yb.y, Yb.x - Ya.y);
        }
    }
    ctx.sync();
    tile_fft<L, NP, LP, NT, true, false, !CIRC>(ctx, T);
    if constexpr (BWD) {
        bwd_epilogue<L, n, BF16, ITER, LP, L * LP>(ctx, bid, a, T, M, xa, xb);
    } else {
        for (int idx = tid; idx < NP * n; idx += NT) {
            const int lp = idx / n, m = idx % n;
            const RowMeta& md = M[lp];
            if (!md.valid) continue;
            const float2 z = T[m * LP + lp];
            store_y<BF16>(a, md.o0 + m, z.x);
            if (md.valid1) store_y<BF16>(a, md.o1 + m, z.y);
        }
    }
}

// ======================================================== kernel spectrum
// Wrap placement: offset delta of an axis with grid n and padded length N sits
// at index delta mod N; index n is never reached and stays zero.
constexpr int kEmpty = 1 << 30;
__host__ __device__ __forceinline__ int unwrap(int m, int n, int N)
{
    if (N == 1) return 0;
    if (m < n) return m;
    if (m == n) return kEmpty;
    return m - N;
}

__host__ __device__ __forceinline__ float kernel_at(const ConvArgs& a, int c, int m_out, int m_mid, int t)
{
    const Geom& g = a.g;
    if (g.circ)  // periodic: the kernel is stored by offset mod n, which is the index itself
        return a.K[(long long)c * g.ke_out * g.ke_mid * g.ke_in + ((long long)m_out * g.ke_mid + m_mid) * g.ke_in + t];
    const int d0 = unwrap(m_out, g.n_out, g.N_out), d1 = unwrap(m_mid, g.n_mid, g.N_mid),
              d2 = unwrap(t, g.n_in, g.N_in);
    if (d0 == kEmpty || d1 == kEmpty || d2 == kEmpty) return 0.f;
    const long long kl = (long long)g.ke_out * g.ke_mid * g.ke_in;
    return a.K[(long long)c * kl +
               ((long long)(d0 + g.n_out - 1) * g.ke_mid + (d1 + g.n_mid - 1)) * g.ke_in + (d2 + g.n_in - 1)];
}

// Rows of the innermost axis, every row of the padded (out, mid) grid, paired
// within a channel (d >= 2) or across channels (d = 1).  Writes the packed
// half spectrum (true DFT values) into the main block; for d = 1 this is the
// final spectrum and is scaled and split here.
template <int L, class Ctx>
__host__ __device__ __forceinline__ void spec_row_body(const Ctx& ctx, int bid, const ConvArgs& a, float2* T)
{
    constexpr int NP = row_np(L), LP = row_lp(L), NT = row_nt(L), S = L / 2;
    const Geom& g = a.g;
    const bool one_d = g.d == 1;
    const int rc = g.N_out * g.N_mid;
    const int hp = one_d ? 1 : rc / 2;
    const int H = one_d ? (a.C + 1) / 2 : a.C * hp;
    const int h0 = bid * NP;
    const int tid = ctx.tid();
    ctx.stage();
    float2* khat = const_cast<float2*>(a.khat);
    for (int idx = tid; idx < NP * L; idx += NT) {
        const int lp = idx / L, t = idx % L;
        const int h = h0 + lp;
        float2 z = make_float2(0.f, 0.f);
        if (h < H) {
            if (one_d) {
                z.x = kernel_at(a, 2 * h, 0, 0, t);
                if (2 * h + 1 < a.C) z.y = kernel_at(a, 2 * h + 1, 0, 0, t);
            } else {
                const int c = h / hp, r = (h % hp) * 2;
                z.x = kernel_at(a, c, r / g.N_mid, r % g.N_mid, t);
                z.y = kernel_at(a, c, (r + 1) / g.N_mid, (r + 1) % g.N_mid, t);
            }
        }
        T[t * LP + lp] = z;
    }
    ctx.sync();
    tile_fft<L, NP, LP, NT, false, false, false>(ctx, T);
    const float gsc = 1.0f / (2.0f * (float)g.N_in);  // only used for d = 1
    for (int idx = tid; idx < NP * S; idx += NT) {
        const int lp = idx / S, k = idx % S;
        const int h = h0 + lp;
        if (h >= H) continue;
        const float2 Z = T[k * LP + lp];
        float2 Xa, Xb;
        if (k == 0) {
            const float2 ZN = T[S * LP + lp];
            Xa = make_float2(Z.x, ZN.x);
            Xb = make_float2(Z.y, ZN.y);
        } else {
            const float2 Zm = T[(L - k) * LP + lp];
            Xa = make_float2(0.5f * (Z.x + Zm.x), 0.5f * (Z.y - Zm.y));
            Xb = make_float2(0.5f * (Z.y + Zm.y), 0.5f * (Zm.x - Z.x));
        }
        if (one_d) {
            for (int s = 0; s < 2; ++s) {
                const int c = 2 * h + s;
                if (c >= a.C) break;
                const float2 X = s ? Xb : Xa;
                float2* kc = khat + (long long)c * g.ksz;
                if (k == 0) {
                    kc[0] = make_float2(0.5f * (X.x + X.y) * gsc, 0.f);
                    kc[S] = make_float2(0.5f * (X.x - X.y) * gsc, 0.f);
                } else {
                    kc[k] = cscale(X, gsc);
                }
            }
        } else {
            const int c = h / hp, r = (h % hp) * 2;
            float2* kc = khat + (long long)c * g.ksz;
            kc[tm_index(g, rc, r, k)] = Xa;
            kc[tm_index(g, rc, r + 1, k)] = Xb;
        }
    }
}

// Full FFT (forward, or inverse with INV) along the middle axis of 3-D planes
// of N_out * N_mid * S values in the tile-major layout of the kernel
// spectrum's main block, in place; plane p starts at planes + p * pstride.
template <int L, bool INV, class Ctx>
__host__ __device__ __forceinline__ void plane_mid_body(const Ctx& ctx, int bid, const Geom& g, float2* planes,
                                                        long long pstride, float2* T)
{
    constexpr int TW = col_tw(L), NT = col_nt(L);
    const int lines = g.N_out * g.S;
    const int tpc = (lines + TW - 1) / TW;
    const int c = bid / tpc, lam0 = (bid % tpc) * TW;
    float2* base = planes + (long long)c * pstride;
    const long long rows = (long long)g.N_out * g.N_mid;
    const int tid = ctx.tid();
    ctx.stage();
    for (int idx = tid; idx < L * TW; idx += NT) {
        const int pos = idx / TW, l = idx % TW, lam = lam0 + l;
        float2 z = make_float2(0.f, 0.f);
        if (lam < lines) z = base[tm_index(g, rows, (long long)(lam / g.S) * g.N_mid + pos, lam % g.S)];
        T[pos * TW + l] = z;
    }
    ctx.sync();
    tile_fft<L, TW, TW, NT, INV, false, false>(ctx, T);
    for (int idx = tid; idx < L * TW; idx += NT) {
        const int pos = idx / TW, l = idx % TW, lam = lam0 + l;
        if (lam < lines) base[tm_index(g, rows, (long long)(lam / g.S) * g.N_mid + pos, lam % g.S)] = T[pos * TW + l];
    }
}

// Forward middle-axis FFT of the kernel spectrum's main block (3-D).
template <int L, class Ctx>
__host__ __device__ __forceinline__ void spec_mid_body(const Ctx& ctx, int bid, const ConvArgs& a, float2* T)
{
    plane_mid_body<L, false>(ctx, bid, a.g, const_cast<float2*>(a.khat), a.g.ksz, T);
}

// Full forward FFT along the out axis, then scale by g = 1/(2 prod N) and, for
// the k_in = 0 lines, split Z = A + iB into Sv = (A+B)/2 g (main slot 0) and
// Dv = (A-B)/2 g (dblk), with A = (Z + conj Z(-k))/2, B = (Z - conj Z(-k))/(2i).
template <int L, int NR, class Ctx>
__host__ __device__ __forceinline__ void spec_out_body(const Ctx& ctx, int bid, const ConvArgs& a, float2* T)
{
    constexpr int TW = out_tw(L, NR);
    constexpr int NL = NR * TW, NT = out_nt(L, NR);
    const Geom& g = a.g;
    const OutTile o = out_tile<NR, TW>(g, 1, a.C, bid);
    const long long rows = (long long)g.N_out * g.N_mid;
    float2* kc = const_cast<float2*>(a.khat) + (long long)o.c_local * g.ksz;
    const float gsc = 1.0f / (2.0f * (float)g.N_out * (float)g.N_mid * (float)g.N_in);
    const int tid = ctx.tid();
    ctx.stage();
    for (int idx = tid; idx < L * NL; idx += NT) {
        const int pos = idx / NL, l = idx % NL, row = l / TW, col = l % TW;
        const int k = o.t * TW + col;
        float2 z = make_float2(0.f, 0.f);
        if (k < g.S) z = kc[tm_index(g, rows, (long long)pos * g.N_mid + o.rows[row], k)];
        T[pos * NL + l] = z;
    }
    ctx.sync();
    tile_fft<L, NL, NL, NT, false, false, false>(ctx, T);
    for (int idx = tid; idx < L * NL; idx += NT) {
        const int pos = idx / NL, l = idx % NL, col = l % TW;
        const int k = o.t * TW + col;
        if (k >= g.S || k == 0) continue;
        T[pos * NL + l] = cscale(T[pos * NL + l], gsc);
    }
    if (o.t == 0) {
        const int njobs = o.self_mirror ? NR * (L / 2 + 1) : L;
        for (int job = tid; job < njobs; job += NT) {
            int ra, rb, pa, pb;
            if (o.self_mirror) {
                ra = job / (L / 2 + 1); rb = ra;
                pa = job % (L / 2 + 1); pb = (L - pa) % L;
            } else {
                ra = 0; rb = 1; pa = job; pb = (L - job) % L;
            }
            const int ea = pa * NL + ra * TW, eb = pb * NL + rb * TW;
            const float2 Za = T[ea], Zb = T[eb];
            // A = (Z + conj Zm)/2, B = (Z - conj Zm)/(2i); S = (A+B)/2 g, D = (A-B)/2 g.
            const float2 Aa = cscale(cadd(Za, cconj(Zb)), 0.5f);
            const float2 Va = csub(Za, cconj(Zb));
            const float2 Ba = make_float2(0.5f * Va.y, -0.5f * Va.x);
            const float2 Ab = cscale(cadd(Zb, cconj(Za)), 0.5f);
            const float2 Vb = csub(Zb, cconj(Za));
            const float2 Bb = make_float2(0.5f * Vb.y, -0.5f * Vb.x);
            T[ea] = cscale(cadd(Aa, Ba), 0.5f * gsc);
            const int rwa = ra == 0 ? o.rows[0] : o.rows[1], rwb = rb == 0 ? o.rows[0] : o.rows[1];
            kc[g.kmain + (long long)pa * g.N_mid + rwa] = cscale(csub(Aa, Ba), 0.5f * gsc);
            if (eb != ea) {
                T[eb] = cscale(cadd(Ab, Bb), 0.5f * gsc);
                kc[g.kmain + (long long)pb * g.N_mid + rwb] = cscale(csub(Ab, Bb), 0.5f * gsc);
            }
        }
    }
    ctx.sync();
    for (int idx = tid; idx < L * NL; idx += NT) {
        const int pos = idx / NL, l = idx % NL, row = l / TW, col = l % TW;
        const int k = o.t * TW + col;
        if (k < g.S) kc[tm_index(g, rows, (long long)pos * g.N_mid + o.rows[row], k)] = T[pos * NL + l];
    }
}

// ======================================================== backward tails
// dalpha, dbeta of the chunk's channel `bid`: the sum of its B * pair_lines
// partial sums, in a fixed order (each thread sums a strided subset into
// U independent fp64 accumulators, so that U loads are in flight at once;
// then an LDS tree).  R: LDS scratch of 2 * NT doubles.  accum: the sums are
// added to the values already in dalpha, dbeta (the per-sample backward runs
// one batch entry after the other).
template <int NT, class Ctx>
__host__ __device__ __forceinline__ void gate_reduce_body(const Ctx& ctx, int bid, const ConvArgs& a, double* R)
{
    constexpr int U = 8;
    const int per = a.B * pair_lines(a.g);
    const float2* p = a.part + (long long)bid * per;
    const int tid = ctx.tid();
    double sa[U], sb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) sa[u] = sb[u] = 0.0;
    int e = tid;
    for (; e + (U - 1) * NT < per; e += U * NT) {
        float2 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = p[e + u * NT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            sa[u] += (double)v[u].x;
            sb[u] += (double)v[u].y;
        }
    }
    for (int u = 0; e < per; e += NT, ++u) {
        const float2 v = p[e];
        sa[u] += (double)v.x;
        sb[u] += (double)v.y;
    }
    double ta = 0.0, tb = 0.0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        ta += sa[u];
        tb += sb[u];
    }
    R[tid] = ta;
    R[NT + tid] = tb;
    ctx.sync();
    for (int h = NT / 2; h >= 1; h /= 2) {
        if (tid < h) {
            R[tid] += R[tid + h];
            R[NT + tid] += R[NT + tid + h];
        }
        ctx.sync();
    }
    if (tid == 0) {
        const int c = a.c0 + bid;
        a.dalpha[c] = (float)(R[0] + (a.accum ? (double)a.dalpha[c] : 0.0));
        a.dbeta[c] = (float)(R[NT] + (a.accum ? (double)a.dbeta[c] : 0.0));
    }
}

// d = 1 kernel gradient, first step: the line u_q + i dy_q of pair q (gated
// input and output gradient of one signal) -> FFT -> separated 2U, 2DY ->
// P_q = 2DY conj(2U) on the S slots (slot 0 packs the real bins 0 and S) into
// dkw[q][S].
template <int L, bool BF16, bool CIRC, class Ctx>
__host__ __device__ __forceinline__ void corr1d_body(const Ctx& ctx, int bid, const ConvArgs& a, float2* T,
                                                     RowMeta* M)
{
    constexpr int NP = row_np(L), LP = row_lp(L), NT = row_nt(L), n = CIRC ? L : L / 2, S = L / 2;
    const Geom& g = a.g;
    const int P = a.nch * a.B;
    const int tid = ctx.tid();
    ctx.stage();
    for (int lp = tid; lp < NP; lp += NT) {
        const int q = bid * NP + lp;
        RowMeta m{};
        m.valid = q < P;
        if (m.valid) {
            const int c = a.c0 + q / a.B, b = q % a.B;
            m.o0 = ((long long)b * a.C + c) * g.vox;
            m.w0 = (long long)q * S;
            m.al0 = a.alpha[c];
            m.be0 = a.beta[c];
        }
        M[lp] = m;
    }
    ctx.sync();
    for (int idx = tid; idx < NP * n; idx += NT) {
        const int lp = idx / n, m = idx % n;
        const RowMeta& md = M[lp];
        float2 z = make_float2(0.f, 0.f);
        if (md.valid)
            z = make_float2(ctx.gate(load_x<BF16>(a, md.o0 + m), md.al0, md.be0), load_in<BF16>(a.dy, md.o0 + m));
        T[m * LP + lp] = z;
    }
    ctx.sync();
    tile_fft<L, NP, LP, NT, false, !CIRC, false>(ctx, T);
    for (int idx = tid; idx < NP * S; idx += NT) {
        const int lp = idx / S, k = idx % S;
        const RowMeta& md = M[lp];
        if (!md.valid) continue;
        const float2 Z = T[k * LP + lp];
        float2 p;
        if (k == 0) {
            const float2 ZS = T[S * LP + lp];
            p = make_float2(4.f * Z.x * Z.y, 4.f * ZS.x * ZS.y);
        } else {
            const float2 Zm = T[(L - k) * LP + lp];
            const float2 ou = make_float2(Z.x + Zm.x, Z.y - Zm.y), od = make_float2(Z.y + Zm.y, Zm.x - Z.x);
            p = cmulc(od, ou);
        }
        a.dkw[md.w0 + k] = p;
    }
}

// Kernel gradient, last step: inverse real FFT of the innermost axis over the
// full length (every offset is kept), scaled by 1 / (4 prod N) (the planes
// hold 4 DY conj(U) summed over the batch) and written to dK at the offsets
// delta = unwrap(index); the wrap slot n of every axis carries nothing.  In
// circular mode the index is the offset mod n, which is K's own index.
// d >= 2: rows r, r+1 of a channel's dkw plane (N_out * N_mid rows, after the
// outer inverse transforms); d = 1: the line pairs channels 2h, 2h+1 of the
// chunk, each summing its B per-pair spectra.
template <int L, class Ctx>
__host__ __device__ __forceinline__ void dk_row_body(const Ctx& ctx, int bid, const ConvArgs& a, float2* T,
                                                     RowMeta* M)
{
    constexpr int NP = row_np(L), LP = row_lay(L), NT = row_nt(L), S = L / 2;
    const Geom& g = a.g;
    const bool one_d = g.d == 1;
    const int rc = g.N_out * g.N_mid;
    const int hp = one_d ? 1 : rc / 2;
    const int H = one_d ? (a.nch + 1) / 2 : a.nch * hp;
    const int tid = ctx.tid();
    ctx.stage();
    for (int lp = tid; lp < NP; lp += NT) {
        const int h = bid * NP + lp;
        RowMeta m{};
        m.valid = h < H;
        if (m.valid) {
            if (one_d) {
                m.w0 = 2 * h;
                m.w1 = 2 * h + 1;
                m.valid1 = 2 * h + 1 < a.nch;
            } else {
                m.w0 = m.w1 = h / hp;
                m.o0 = (h % hp) * 2;
                m.o1 = m.o0 + 1;
                m.valid1 = 1;
            }
        }
        M[lp] = m;
    }
    ctx.sync();
    for (int idx = tid; idx < NP * S; idx += NT) {
        const int lp = idx / S, k = idx % S;
        const RowMeta& md = M[lp];
        float2 ya = make_float2(0.f, 0.f), yb = make_float2(0.f, 0.f);
        if (md.valid) {
            if (one_d) {
                for (int b = 0; b < a.B; ++b) {
                    ya = cadd(ya, a.dkw[((long long)md.w0 * a.B + b) * S + k]);
                    if (md.valid1) yb = cadd(yb, a.dkw[((long long)md.w1 * a.B + b) * S + k]);
                }
            } else {
                const float2* pl = a.dkw + md.w0 * g.kmain;
                ya = pl[tm_index(g, rc, md.o0, k)];
                yb = pl[tm_index(g, rc, md.o1, k)];
            }
        }
        if (k == 0) {
            T[tile_idx<LP>(0, lp)] = make_float2(ya.x, yb.x);
            T[tile_idx<LP>(S, lp)] = make_float2(ya.y, yb.y);
        } else {
            T[tile_idx<LP>(k, lp)] = make_float2(ya.x - yb.y, ya.y + yb.x);
            T[tile_idx<LP>(L - k, lp)] = make_float2(ya.x + yb.y, yb.x - ya.y);
        }
    }
    ctx.sync();
    tile_fft<L, NP, LP, NT, true, false, false>(ctx, T);
    const float sc = 1.0f / (4.0f * (float)g.N_out * (float)g.N_mid * (float)g.N_in);
    const long long kl = (long long)g.ke_out * g.ke_mid * g.ke_in;
    for (int idx = tid; idx < NP * L; idx += NT) {
        const int lp = idx / L, t = idx % L;
        const RowMeta& md = M[lp];
        // index into K's extent of padded-grid position m on an axis (kEmpty: the wrap slot)
        auto kidx = [&](int m, int n, int N) {
            if (g.circ) return m;
            const int dl = unwrap(m, n, N);
            return dl == kEmpty ? kEmpty : dl + n - 1;
        };
        const int e2 = kidx(t, g.n_in, g.N_in);
        if (!md.valid || e2 == kEmpty) continue;
        const float2 z = T[tile_idx<LP>(t, lp)];
        for (int s2 = 0; s2 < 2; ++s2) {
            if (s2 == 1 && !md.valid1) break;
            const long long c = s2 ? md.w1 : md.w0;
            int e0 = 0, e1 = 0;
            if (!one_d) {
                const int row = (int)(s2 ? md.o1 : md.o0);
                e0 = kidx(row / g.N_mid, g.n_out, g.N_out);
                e1 = kidx(row % g.N_mid, g.n_mid, g.N_mid);
                if (e0 == kEmpty || e1 == kEmpty) continue;
            }
            a.dK[(a.c0 + c) * kl + ((long long)e0 * g.ke_mid + e1) * g.ke_in + e2] = (s2 ? z.y : z.x) * sc;
        }
    }
}

// ============================================================= long 1-D
// Signals longer than one workgroup's transform (n > 1024): the padded length
// N = 2n is factored as N1 x N2 (sample m = N2 n1 + n2), and
//   X[k1 + N1 k2] = sum_n2 W_N2^(n2 k2) W_N^(n2 k1) sum_n1 x[N2 n1 + n2] W_N1^(n1 k1)
// (the four-step decomposition of a length-N DFT): column transforms of N1
// points, the twiddle W_N^(n2 k1), row transforms of N2 points; the inverse
// runs the same steps backwards with conjugate twiddles.  Zero padding makes
// the rows n1 >= N1/2 zero on input and unused on output, so the column
// transforms prune their first / last pass.  Arithmetic is complex throughout
// (the real input occupies the real parts).  The spectrum of frequency
// k1 + N1 k2 is stored at row k1, column k2, scaled by 1/N: the workspace and
// the spectrum share the N1 x N2 layout, so the product is elementwise.

// Work item of column workgroup `bid` among W: workgroups are dispatched
// round-robin over the eight XCDs, so item w goes to id (w mod W8/8)*8 + w/(W8/8)
// and each XCD runs a contiguous range of column tiles, whose narrow row
// segments share cache lines in that XCD's L2 (2M tokens, 8 channels: 0.577
// -> 0.534 ms per call; 8M tokens, 4 channels: 1.687 -> 1.308 ms).
__host__ __device__ __forceinline__ int lng_col_item(int bid, int W)
{
    const int W8 = W & ~7;
    return bid < W8 ? (bid % 8) * (W8 / 8) + bid / 8 : bid;
}

// Step 1 (and the spectrum's first step with SPEC): TW adjacent columns per
// workgroup, N1-point forward transforms, twiddled, into rows k1.
// Forward: gated x, rows n1 < N1/2 read (pruned), workspace of pair q.
// SPEC: the kernel wrap-placed at offset delta -> delta mod N (index n empty),
// all rows read, into the spectrum of channel q.
// GATE = false (backward): the signal read through a.x is taken as it is (the
// output gradient dy).
template <int L, bool SPEC, bool BF16, bool GATE = true, class Ctx>
__host__ __device__ __forceinline__ void lng_col_fwd_body(const Ctx& ctx, int bid, const ConvArgs& a, float2* T)
{
    constexpr int TW = col_tw(L), NT = col_nt(L);
    const Geom& g = a.g;
    const int N2 = g.N2;
    const int tpp = N2 / TW;
    const int w = lng_col_item(bid, (SPEC ? a.C : a.nch * a.B) * tpp);
    const int q = w / tpp, n20 = (w % tpp) * TW;
    const unsigned nmask = (1u << g.logN) - 1u;
    float2* dst = SPEC ? const_cast<float2*>(a.khat) + (long long)q * g.ksz : a.ws + (long long)q * g.wsp;
    long long xo = 0;
    float al = 0.f, be = 0.f;
    if constexpr (!SPEC) {
        const int c = a.c0 + q / a.B, b = q % a.B;
        xo = ((long long)b * a.C + c) * g.vox;
        al = a.alpha[c];
        be = a.beta[c];
    }
    auto ld = [&](int pos, int l) -> float2 {
        const long long m = (long long)N2 * pos + n20 + l;
        if constexpr (SPEC) {
            const int dl = unwrap((int)m, g.n_in, g.N_in);
            return make_float2(dl == kEmpty ? 0.f : a.K[(long long)q * g.ke_in + dl + g.n_in - 1], 0.f);
        } else {
            const float v = load_x<BF16>(a, xo + m);
            return make_float2(GATE ? ctx.gate(v, al, be) : v, 0.f);
        }
    };
    auto st = [&](int pos, int l, const float2& v) {
        const unsigned e = ((unsigned)(n20 + l) * (unsigned)pos) & nmask;
        dst[(long long)pos * N2 + n20 + l] = cmul(v, ctx.twiddle(e, g.logN));
    };
    auto after_load = [&]() { ctx.stage(); };
    fwd_fn_to_fn<L, TW, NT, !SPEC>(ctx, T, ld, st, after_load);
}

// Spectrum, step 2: NP rows k1 per workgroup, N2 points each: the forward
// row transform scaled by 1/N, in place in the spectrum (the convolution's row
// passes are lng_prod_body and lng_prod_dk_body below).
template <int L, class Ctx>
__host__ __device__ __forceinline__ void lng_spec_row_body(const Ctx& ctx, int bid, const ConvArgs& a, float2* T)
{
    constexpr int NP = row_np(L), LP = row_lp(L), NT = row_nt(L);
    constexpr int ITER = NP * L / NT;
    static_assert(NP * L % NT == 0, "whole element loops");
    const Geom& g = a.g;
    const int N1 = g.N1;
    const int H = a.C * N1;
    const int tid = ctx.tid();
    ctx.stage();
    auto row_base = [&](int lp) -> float2* {
        const int h = bid * NP + lp, q = h / N1, k1 = h % N1;
        return const_cast<float2*>(a.khat) + (long long)q * g.ksz + (long long)k1 * L;
    };
    float2 v[ITER];
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
        const int idx = tid + i * NT, lp = idx / L, pos = idx % L;
        v[i] = bid * NP + lp < H ? row_base(lp)[pos] : make_float2(0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
        const int idx = tid + i * NT, lp = idx / L, pos = idx % L;
        T[pos * LP + lp] = v[i];
    }
    ctx.sync();
    tile_fft<L, NP, LP, NT, false, false, false>(ctx, T);
    const float sc = 1.0f / (float)(1ll << g.logN);
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
        const int idx = tid + i * NT, lp = idx / L, pos = idx % L;
        if (bid * NP + lp < H) row_base(lp)[pos] = cscale(T[pos * LP + lp], sc);
    }
}

// Long 1-D, step 2: the product rows, with the transforms' ends in registers:
// the forward's first pass reads the row from the workspace, its last pass
// leaves each thread holding the positions the inverse's first pass takes
// (the reversed plan), the product with the kernel spectrum happens there,
// and the inverse's last pass writes the row back (two LDS round trips per
// transform of 4096 points).  One line of L points per workgroup (two of
// 2048, four of 1024), 8 points per thread per pass, so that two workgroups
// share a CU below 8192 points (the 8192-point plan is a palindrome: its
// forward and reversed plans share 64 KiB of tables beside the 64 KiB line).
// CONJ (backward, du): the product takes the conjugate spectrum (a
// correlation with K).
template <int L, bool CONJ, class Ctx>
__host__ __device__ __forceinline__ void lng_prod_body(const Ctx& ctx, int bid, const ConvArgs& a, float2* T)
{
    constexpr int NL = lngp_nl(L), NT = lngp_nt(L), LP = lngp_lay(L);
    constexpr int RL = pass_radix<L, false>(plan_passes(L) - 1);
    using PL = PassRegs<L, RL, NL, NT>;
    const Geom& g = a.g;
    const int N1 = g.N1;
    const int H = a.nch * a.B * N1;
    const int tid = ctx.tid();
    // Row h = bid*NL + l: signal q = h / N1 of the chunk (channel c0 + q / B,
    // batch entry q % B), row k1 = h % N1 of its N1 x L array.
    auto row_off = [&](int l) -> long long {
        const int h = bid * NL + l;
        return (long long)(h / N1) * g.wsp + (long long)(h % N1) * L;
    };
    auto khat_off = [&](int l) -> long long {
        const int h = bid * NL + l, q = h / N1, k1 = h % N1;
        const int c = a.c0 + q / a.B, b = q % a.B;
        return (long long)c * g.ksz + (long long)b * a.khat_bstride + (long long)k1 * L;
    };
    auto live = [&](int l) { return bid * NL + l < H; };
    float2 kv[PL::PER][RL];
    auto after_load = [&]() {
        ctx.stage();
#pragma unroll
        for (int i = 0; i < PL::PER; ++i) {
            const int gi = tid + i * NT, l = gi % NL, j = gi / NL;
            const bool ok = bf_valid<PL::NB, NT>(gi) && live(l);
            const long long base = ok ? khat_off(l) + j : 0;
#pragma unroll
            for (int r = 0; r < RL; ++r) kv[i][r] = ok ? a.khat[base + r * (L / RL)] : make_float2(0.f, 0.f);
        }
    };
    auto t = fwd_from_fn<L, NL, NT, false, LP>(ctx, T, [&](int pos, int l) -> float2 {
        return live(l) ? a.ws[row_off(l) + pos] : make_float2(0.f, 0.f);
    }, after_load);
#pragma unroll
    for (int i = 0; i < PL::PER; ++i)
#pragma unroll
        for (int r = 0; r < RL; ++r) t.v[i][r] = cmul(t.v[i][r], CONJ ? cconj(kv[i][r]) : kv[i][r]);
    ctx.sync();  // every LDS read of the forward transform is done: T is free
    inv_to_fn<L, NL, NT, false, LP>(ctx, T, t, [&](int pos, int l, const float2& x) {
        if (live(l)) a.ws[row_off(l) + pos] = x;
    });
}

// Backward, kernel gradient, step 2, with the transforms' ends in registers
// (as lng_prod_body): for each batch entry the forward row
// transforms of dy and u end in registers, P += DY conj(U) there, and, where
// lng_dk_fuses_du, the du row DY conj(Khat) is inverse-transformed straight
// back to the workspace; then the inverse of P goes to the kernel-gradient
// plane dkw.
template <int L, class Ctx>
__host__ __device__ __forceinline__ void lng_prod_dk_body(const Ctx& ctx, int bid, const ConvArgs& a, float2* T)
{
    constexpr bool DU = lng_dk_fuses_du(L);
    constexpr int NL = lngp_nl(L), NT = lngp_nt(L), LP = lngp_lay(L);
    constexpr int RL = pass_radix<L, false>(plan_passes(L) - 1);
    using PL = PassRegs<L, RL, NL, NT>;
    const Geom& g = a.g;
    const int N1 = g.N1;
    const int H = a.nch * N1;
    const int tid = ctx.tid();
    auto live = [&](int l) { return bid * NL + l < H; };
    auto row_off = [&](int l, int b) -> long long {  // row k1 of pair (channel, b) in the workspace
        const int h = bid * NL + l;
        return ((long long)(h / N1) * a.B + b) * g.wsp + (long long)(h % N1) * L;
    };
    auto none = []() {};
    auto fwd_rows = [&](const float2* ws, int b) {
        return fwd_from_fn<L, NL, NT, false, LP>(ctx, T, [&](int pos, int l) -> float2 {
            return live(l) ? ws[row_off(l, b) + pos] : make_float2(0.f, 0.f);
        }, none);
    };
    ctx.stage();
    PL P;
    float2 kv[PL::PER][DU ? RL : 1];
#pragma unroll
    for (int i = 0; i < PL::PER; ++i) {
        const int gi = tid + i * NT, l = gi % NL, j = gi / NL, h = bid * NL + l;
        const bool ok = bf_valid<PL::NB, NT>(gi) && live(l);
#pragma unroll
        for (int r = 0; r < RL; ++r) {
            P.v[i][r] = make_float2(0.f, 0.f);
            if constexpr (DU)
                kv[i][r] = ok ? a.khat[(long long)(a.c0 + h / N1) * g.ksz + (long long)(h % N1) * L + j + r * (L / RL)]
                              : make_float2(0.f, 0.f);
        }
    }
    for (int b = 0; b < a.B; ++b) {
        auto DY = fwd_rows(a.ws, b);
        ctx.sync();  // T is free for the next transform
        auto U = fwd_rows(a.ws_u, b);
        ctx.sync();
#pragma unroll
        for (int i = 0; i < PL::PER; ++i)
#pragma unroll
            for (int r = 0; r < RL; ++r) P.v[i][r] = cadd(P.v[i][r], cmulc(DY.v[i][r], U.v[i][r]));
        if constexpr (DU) {
#pragma unroll
            for (int i = 0; i < PL::PER; ++i)
#pragma unroll
                for (int r = 0; r < RL; ++r) DY.v[i][r] = cmulc(DY.v[i][r], kv[i][r]);
            inv_to_fn<L, NL, NT, false, LP>(ctx, T, DY, [&](int pos, int l, const float2& x) {
                if (live(l)) a.ws[row_off(l, b) + pos] = x;
            });
            ctx.sync();  // T is free for the next transform
        }
    }
    inv_to_fn<L, NL, NT, false, LP>(ctx, T, P, [&](int pos, int l, const float2& x) {
        const int h = bid * NL + l;
        if (live(l)) a.dkw[(long long)(h / N1) * g.kmain + (long long)(h % N1) * L + pos] = x;
    });
}

// Step 3: TW adjacent columns per workgroup: conjugate twiddle, inverse
// N1-point transforms keeping rows n1 < N1/2 (the crop), real part to y.
// BWD: the transforms carry du; each output becomes dx (stored through y) and
// the workgroup's sums of the dalpha / dbeta terms (each thread's in the
// order it visits its outputs, then an LDS tree) go to part[w], the
// partials of pair q laid out [q][N2 / TW].
template <int L, bool BF16, bool BWD = false, class Ctx>
__host__ __device__ __forceinline__ void lng_col_inv_body(const Ctx& ctx, int bid, const ConvArgs& a, float2* T)
{
    constexpr int TW = col_tw(L), NT = col_nt(L);
    const Geom& g = a.g;
    const int N2 = g.N2;
    const int tpp = N2 / TW;
    const int w = lng_col_item(bid, a.nch * a.B * tpp);
    const int q = w / tpp, n20 = (w % tpp) * TW;
    const unsigned nmask = (1u << g.logN) - 1u;
    const float2* src = a.ws + (long long)q * g.wsp;
    const int c = a.c0 + q / a.B, b = q % a.B;
    const long long yo = ((long long)b * a.C + c) * g.vox;
    auto ld = [&](int pos, int l) -> float2 {
        const unsigned e = ((unsigned)(n20 + l) * (unsigned)pos) & nmask;
        return cmulc(src[(long long)pos * N2 + n20 + l], ctx.twiddle(e, g.logN));
    };
    auto after_load = [&]() { ctx.stage(); };
    if constexpr (!BWD) {
        auto st = [&](int pos, int l, const float2& v) { store_y<BF16>(a, yo + (long long)N2 * pos + n20 + l, v.x); };
        inv_fn_to_fn<L, TW, NT, true>(ctx, T, ld, st, after_load);
    } else {
        static_assert((NT & (NT - 1)) == 0, "power-of-two workgroup for the tree");
        const float al = a.alpha[c], be = a.beta[c];
        float2 acc = make_float2(0.f, 0.f);
        auto st = [&](int pos, int l, const float2& v) {
            const long long m = yo + (long long)N2 * pos + n20 + l;
            float2 terms;
            store_y<BF16>(a, m, gate_vjp(ctx, v.x, load_x<BF16>(a, m), al, be, terms));
            acc = cadd(acc, terms);
        };
        inv_fn_to_fn<L, TW, NT, true>(ctx, T, ld, st, after_load);
        ctx.sync();  // the transform's last LDS reads are done: T is scratch
        const int tid = ctx.tid();
        T[tid] = acc;
        ctx.sync();
        for (int h = NT / 2; h >= 1; h /= 2) {
            if (tid < h) T[tid] = cadd(T[tid], T[tid + h]);
            ctx.sync();
        }
        if (tid == 0) a.part[w] = T[0];
    }
}

// Backward, kernel gradient, last step: TW adjacent columns of a channel's
// dkw plane per workgroup: conjugate twiddle, inverse N1-point transforms over
// every row (the kernel gradient lives on all offsets), scaled by 1/N, written
// to dK at the offset delta = unwrap(m) of position m = N2 n1 + n2 (index n
// carries nothing).
template <int L, class Ctx>
__host__ __device__ __forceinline__ void lng_col_dk_body(const Ctx& ctx, int bid, const ConvArgs& a, float2* T)
{
    constexpr int TW = col_tw(L), NT = col_nt(L);
    const Geom& g = a.g;
    const int N2 = g.N2;
    const int tpp = N2 / TW;
    const int w = lng_col_item(bid, a.nch * tpp);
    const int cl = w / tpp, n20 = (w % tpp) * TW;
    const unsigned nmask = (1u << g.logN) - 1u;
    const float2* src = a.dkw + (long long)cl * g.kmain;
    float* dst = a.dK + (long long)(a.c0 + cl) * g.ke_in;
    const float sc = 1.0f / (float)(1ll << g.logN);
    auto ld = [&](int pos, int l) -> float2 {
        const unsigned e = ((unsigned)(n20 + l) * (unsigned)pos) & nmask;
        return cmulc(src[(long long)pos * N2 + n20 + l], ctx.twiddle(e, g.logN));
    };
    auto st = [&](int pos, int l, const float2& v) {
        const int dl = unwrap(N2 * pos + n20 + l, g.n_in, g.N_in);
        if (dl != kEmpty) dst[dl + g.n_in - 1] = v.x * sc;
    };
    auto after_load = [&]() { ctx.stage(); };
    inv_fn_to_fn<L, TW, NT, false>(ctx, T, ld, st, after_load);
}

}  // namespace hyenand
