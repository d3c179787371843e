// plan.h -- geometry, layouts and tiling of the gated N-D FFT convolution.
//
// No device code.  Shared by the C ABI (validation, workspace sizing, launch
// grids) and the kernel bodies (argument struct).
//
// Axis naming.  A d-dimensional grid [n_0 .. n_{d-1}] is handled as
// (out, mid, in):  d = 3 -> (n_0, n_1, n_2);  d = 2 -> (n_0, 1, n_1);
// d = 1 -> (1, 1, n_0).  Every present axis is zero-padded to N = 2n (the
// non-circular boundary of the gist.science summary, "Methodology",
// "Boundary handling"); absent axes keep N = 1.
//
// Frequency layout.  The innermost axis is real: its spectrum has N_in/2 + 1
// bins, of which bins 0 and N_in/2 are real.  Rows are stored with S = N_in/2
// complex slots; slot 0 packs (bin 0, bin N_in/2) as (re, im).  After the outer
// axes are transformed, slot 0 of every line holds Z = A + iB with A, B the
// (Hermitian) spectra of those two real planes; the product step separates
// them with the mirror bin -k.
//
// Kernel spectrum layout (per channel, complex64):
//   main[k_out][k_mid][k_in], k_in in [0, S):  Khat(k) * g for k_in >= 1;
//        slot k_in = 0 holds Sv = (Khat(k, 0) + Khat(k, N_in/2)) / 2 * g
//   dblk[k_out][k_mid]:                        Dv = (Khat(k, 0) - Khat(k, N_in/2)) / 2 * g
// with g = 1 / (2 prod N) and Khat the true DFT of the wrap-placed kernel.
// The product step for slot-0 lines is then W(k) = Z(k) Sv(k) + conj(Z(-k)) Dv(k).
//
// Workspace layout (per (b,c) pair, complex64): [n_out][N_mid][S].
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hyenand {

// ---------------------------------------------------------------- tiling
// Row kernels: NP line pairs of length L per workgroup (2 <= NP <= 64),
// tile L x row_lp(L) (line stride padded so that the transposed accesses of the
// load and store phases spread over the LDS banks).
// 8192-point rows (long 1-D signals beyond 2^23 samples) take one line per
// workgroup, unpadded: a 64 KiB tile beside the 64 KiB twiddle table.
constexpr int row_np(int L) { return L >= 8192 ? 1 : (4096 / L < 2 ? 2 : (4096 / L > 64 ? 64 : 4096 / L)); }
constexpr int row_lp(int L) { return row_np(L) == 1 ? 1 : row_np(L) + 1; }
// Layout code of the tiles of the forward / inverse row kernels: element
// (pos, lp) at pos * P + lp + D * (pos >> SH), the code P | D << 8 | SH << 12
// (a plain line stride when D = 0).  512-, 1024- and 2048-point rows take
// D extra slots after every 2^SH positions instead of a padded line stride:
// fewer bank conflicts on the strided Stockham stores (2048-point rows 4.2 ->
// about 0.6 conflict cycles per LDS instruction in a 32-bank model that
// reproduces the measured counts) and smaller tiles (2048 points: 49 -> 34
// KiB, three workgroups per CU instead of two; 512 points: four instead of
// three).  1024^2 forward 4.12 -> 3.59 ms, 256^2 0.318 -> 0.303 ms.
constexpr int row_lay(int L)
{
    return L == 2048 ? (2 | 1 << 8 | 3 << 12) : L == 1024 ? (4 | 1 << 8 | 2 << 12)
         : L == 512 ? (8 | 2 << 8 | 2 << 12) : row_lp(L);
}
constexpr int lay_p(int lay) { return lay & 255; }
constexpr int lay_d(int lay) { return (lay >> 8) & 15; }
constexpr int lay_sh(int lay) { return (lay >> 12) & 15; }
// Elements of an L-position tile of layout lay with NL lines.
constexpr int lay_elems(int L, int NL, int lay) { return (L - 1) * lay_p(lay) + NL + lay_d(lay) * ((L - 1) >> lay_sh(lay)); }
// Column kernels along the middle axis / the out axis of a 2-D grid:
// TW adjacent lines, tile L x TW of up to 128 KiB (gfx950 gives a workgroup
// up to 160 KiB of LDS), so that even 2048-point lines read row segments of
// 64 bytes; narrower tiles waste most of each fetched cache line.
// 512-point lines take 8 (three workgroups per CU instead of two; neighbouring
// tiles share their cache lines in L2, see the out-axis workgroup order).
constexpr int col_tw(int L) { return L == 512 ? 8 : (16384 / L > 16 ? 16 : (16384 / L < 1 ? 1 : 16384 / L)); }
// Out-axis kernel of a 3-D grid: two mirrored k_mid rows x TW lines.
// 1024-point lines take 4 (a 64 KiB tile plus 16 KiB of twiddles: two
// workgroups per CU instead of one; 512^3 k_col_out 3.08 -> 2.78 ms per call).
constexpr int mul3_tw(int L) { return L == 1024 ? 4 : (8192 / L > 16 ? 16 : (8192 / L < 1 ? 1 : 8192 / L)); }

// Threads of a workgroup for a tile of `points` complex values: 16 points per
// thread per pass (two radix-8 butterflies), between 64 and 1024 threads.
// The row kernels take 8 points per thread: twice the waves to hide HBM
// latency (they are the memory-bound passes).
constexpr int tile_threads(int points) { return points / 16 < 64 ? 64 : (points / 16 > 1024 ? 1024 : points / 16); }
constexpr int row_nt(int L) { return tile_threads(2 * L * row_np(L)); }
constexpr int col_nt(int L) { return tile_threads(L * col_tw(L)); }
// 2-D out-axis lines of 1024 points take 8 (64 KiB: two workgroups per CU
// that run one item each, instead of one looping workgroup; 512^2, B = 8,
// C = 16: k_col_out 260 -> 201 us per call).  The middle-axis kernel keeps 16
// for them (with 8, 512^3 k_col_mid 730 -> 840 us per call).
constexpr int out_tw(int L, int NR) { return NR == 1 ? (L == 1024 ? 8 : col_tw(L)) : mul3_tw(L); }
constexpr int out_nt(int L, int NR) { return tile_threads(L * NR * out_tw(L, NR)); }
// Layout code (row_lay) of the forward out-axis kernel's tile: 512-point 2-D
// lines take two extra slots after every two positions (no bank conflicts on
// the strided stores in the 32-bank model, 1.0 cycle per instruction before;
// 40,880 bytes with the twiddles, still four workgroups per CU): 256^2
// k_col_out 148-154 -> 144-146 us per launch.
constexpr int out_lay(int L, int NR) { return (NR == 1 && L == 512) ? (8 | 2 << 8 | 1 << 12) : NR * out_tw(L, NR); }
// 2-D out-axis tiles above 80 KiB leave room for one workgroup per CU: such
// kernels run one workgroup per CU that loops over the work items (1024^2:
// 4.29 -> 4.08 ms per call).  The 3-D kernel of the same tile size lost with
// the loop (512^3: 24.8 -> 29.2 ms), and smaller tiles rely on several
// workgroups per CU; those run one item per workgroup.
// Backward out-axis kernel: it holds four tile-sized register arrays (the
// output-gradient and gated-input spectra, the kernel-gradient accumulator and
// the kernel spectrum values), so its tile is capped at 64 KiB (4 x 128 KiB
// would fill a CU's whole 512 KiB register file: 1024^2 22.8 -> 10.9 ms,
// 512^3 104.6 -> 79.9 ms per call).  Points per thread per pass: 8 for 2-D
// lines (256^2: 0.88 -> 0.80 ms against 16), 16 for the two-row 3-D tiles
// (128^3: 6.7 against 7.8 ms with 8).  The two-row tiles of 256-point lines
// take 8 slots (32 KiB; the kernel spectrum's slot tiles stay 16 wide for the
// forward): 128^3 k_col_out_bwd 238 -> 187 us per launch, backward 6.73 ->
// 6.16 ms.
constexpr int bwd_tw(int L, int NR)
{
    if (NR == 2 && L == 256) return 8;
    const int cap = 65536 / (8 * L * NR);
    return out_tw(L, NR) < cap ? out_tw(L, NR) : (cap < 4 ? 4 : cap);
}
constexpr int bwd_nt(int L, int NR)
{
    const int t = L * NR * bwd_tw(L, NR) / (NR == 1 ? 8 : 16);
    return t < 64 ? 64 : (t > 1024 ? 1024 : t);
}
constexpr bool out_looped(int L, int NR) { return NR == 1 && (long long)L * NR * out_tw(L, NR) * 8 > 80 * 1024; }
// Twiddled passes whose factors the forward out-axis kernel keeps in registers
// for both of its transforms (fft_core.h TwCache).  512-point 2-D lines keep
// the first (7 factors, shared by a thread's two butterflies; 106 -> 126
// VGPRs, four workgroups per CU still): 256^2 k_col_out 145 -> 141 us.  Both
// twiddled passes (140 VGPRs, three workgroups per CU) took 155 us.
constexpr int out_tw_regs(int L, int NR) { return (NR == 1 && L == 512) ? 1 : 0; }

struct Geom {
    int d;
    int n_out, n_mid, n_in;
    int N_out, N_mid, N_in;
    int S;                 // N_in / 2
    long long vox;         // voxels per (b,c): n_out * n_mid * n_in
    long long wsp;         // workspace complex per pair: n_out * N_mid * S (0 for d = 1)
    long long kmain;       // main block complex per channel: N_out * N_mid * S
    long long ksz;         // kmain + N_out * N_mid
    int ke_out, ke_mid, ke_in;  // kernel extents 2n-1 (1 for absent axes); n when circular
    int lt, lt_log;        // slot tile of the tile-major planes (a power of two <= S)
    int circ;              // circular mode: periodic grid, N = n, no padding or crop
    // Long 1-D signals (n > 1024): the padded length N = 2n is transformed as an
    // N1 x N2 array (sample m = N2 * n1 + n2) -- column transforms of N1
    // points, a twiddle, row transforms of N2 points -- and the spectrum value
    // of frequency k1 + N1 k2 sits at row k1, column k2.
    int lng;               // 1 for the long 1-D path
    int N1, N2, logN;      // column / row transform lengths, log2 N
};

// Slot tile of the kernel spectrum and the workspace: the out-axis kernel's
// tile width (capped at S), so that each out-axis workgroup's block of a 2-D
// plane is contiguous.  In 3-D the workgroup's two mirrored k_mid rows stay
// apart whatever the tile, and consecutive out-axis positions of a tile are
// N_mid * T slots apart: there tiles of 16 slots (128-byte runs) serve the
// 16-line out-axis tiles (128^3: 1.97 -> 1.91 ms against plain rows; 32 or 64
// slots give no gain), and the 8-line tiles of 1024-point lines take 64-slot
// tiles (512^3 per call: plain rows 25.5, 16 slots 23.8, 32 slots 22.0,
// 64 slots 21.3, 128 slots 21.7, 256 slots 23.9 ms).
constexpr int slot_tile(int d, int N_out, int S)
{
    int tw = S;
    if (d == 2) tw = out_tw(N_out, 1);
    if (d == 3) tw = out_tw(N_out, 2) >= 16 ? out_tw(N_out, 2) : 64;
    return tw < S ? tw : S;
}

// A plane of `rows` rows (row = k_out * N_mid + k_mid) x S slots stored
// tile-major: slot tiles of lt consecutive slots, each holding every row,
//   element (row, slot) at ((slot / lt) * rows + row) * lt + slot % lt.
__host__ __device__ __forceinline__ long long tm_index(const Geom& g, long long rows, long long row, int slot)
{
    return ((long long)(slot >> g.lt_log) * rows + row) * g.lt + (slot & (g.lt - 1));
}

inline bool is_pow2(long long v) { return v > 0 && (v & (v - 1)) == 0; }

// Returns false for an unsupported shape: d in {1,2,3}, every n a power of two
// in [2, 1024] ([4, 1024] in circular mode, whose transforms have length n);
// d = 1 (zero-padded) also takes n up to 2^24 through the long 1-D path.
//
// Circular mode (gist.science summary, "Methodology", "Boundary handling":
// circular convolutions for periodic systems): every axis keeps N = n, the
// kernel lives on the n offsets modulo n ([C][n_0]..[n_{d-1}], index = offset
// mod n), no transform is pruned and every output is kept.
inline bool make_geom(int d, const int64_t* dims, Geom* g, bool circ = false)
{
    if (d < 1 || d > 3 || !dims) return false;
    *g = Geom{};
    if (d == 1 && !circ && dims[0] > 1024) {
        // Long 1-D: n a power of two up to 2^24.  Rows of N2 = min(N/4, 2048)
        // points up to N = 2^22, then rows and columns of up to 4096 points up
        // to N = 2^24, then 8192-point rows (N = 2^25: 4096 x 8192).
        const long long n = dims[0];
        if (!is_pow2(n) || n > (1ll << 24)) return false;
        const long long N = 2 * n;
        g->d = 1;
        g->lng = 1;
        g->N2 = (int)(N <= (1ll << 22) ? (N / 4 < 2048 ? N / 4 : 2048) : (N <= (1ll << 24) ? 4096 : 8192));
        g->N1 = (int)(N / g->N2);
        g->logN = 0;
        while ((1ll << g->logN) < N) ++g->logN;
        g->n_out = g->n_mid = 1;
        g->n_in = (int)n;
        g->N_out = g->N_mid = 1;
        g->N_in = (int)N;
        g->S = (int)n;
        g->vox = n;
        g->wsp = N;
        g->kmain = N;
        g->ksz = N;
        g->ke_out = g->ke_mid = 1;
        g->ke_in = (int)(2 * n - 1);
        g->lt = 1;
        g->lt_log = 0;
        return true;
    }
    for (int a = 0; a < d; ++a)
        if (dims[a] < (circ ? 4 : 2) || dims[a] > 1024 || !is_pow2(dims[a])) return false;
    g->d = d;
    g->circ = circ ? 1 : 0;
    if (d == 3) { g->n_out = (int)dims[0]; g->n_mid = (int)dims[1]; g->n_in = (int)dims[2]; }
    else if (d == 2) { g->n_out = (int)dims[0]; g->n_mid = 1; g->n_in = (int)dims[1]; }
    else { g->n_out = 1; g->n_mid = 1; g->n_in = (int)dims[0]; }
    const int pad = circ ? 1 : 2;
    g->N_out = d >= 2 ? pad * g->n_out : 1;
    g->N_mid = d >= 3 ? pad * g->n_mid : 1;
    g->N_in = pad * g->n_in;
    g->S = g->N_in / 2;
    g->vox = (long long)g->n_out * g->n_mid * g->n_in;
    g->wsp = d >= 2 ? (long long)g->n_out * g->N_mid * g->S : 0;
    g->kmain = (long long)g->N_out * g->N_mid * g->S;
    g->ksz = g->kmain + (long long)g->N_out * g->N_mid;
    g->ke_out = circ ? g->n_out : 2 * g->n_out - 1;
    g->ke_mid = circ ? g->n_mid : 2 * g->n_mid - 1;
    g->ke_in = circ ? g->n_in : 2 * g->n_in - 1;
    g->lt = slot_tile(d, g->N_out, g->S);
    g->lt_log = 0;
    while ((1 << g->lt_log) < g->lt) ++g->lt_log;
    return true;
}

// The on-chip 2-D forward (one workgroup per (b, c) pair, the half spectrum in
// LDS, no workspace): zero-padded 2-D grids with both padded lengths in
// [8, 128], i.e. n_out, n_in in [4, 64] (64 x 64: 32 KiB of half spectrum, up
// to four workgroups per CU).  A 128 x 128 half spectrum (128 KiB) also fits a
// workgroup's 160 KiB, but it leaves one 4-wave workgroup per CU, whose every
// LDS access and barrier is exposed: measured on MI355X (128^2, B = 8, C = 64)
// 157 us per call on chip against 82 us for the three-pass path, while at 64^2
// the on-chip kernel wins (24 against 38 us; 32^2 16 against 32 us).
constexpr int kFused2dMaxLen = 128;
inline bool fused2d_fits(const Geom& g)
{
    return g.d == 2 && !g.circ && !g.lng && g.N_out >= 8 && g.N_out <= kFused2dMaxLen && g.N_in >= 8 &&
           g.N_in <= kFused2dMaxLen;
}

// Arguments shared by every kernel of one call (passed by value).
struct ConvArgs {
    const void* x;          // [B][C][vox], fp32 or bf16
    void* y;                // same layout and dtype as x
    const float* alpha;     // [C]
    const float* beta;      // [C]
    const float2* khat;     // [C][ksz] (kernel spectrum) -- written by the spectrum kernels
    long long khat_bstride; // complex values between batch entries of a per-sample spectrum
                            // ([B][C][ksz]: C * ksz), 0 when one spectrum serves the batch
    float2* ws;             // workspace, [pairs in chunk][wsp]
    const float* K;         // spectrum input: [C][ke_out][ke_mid][ke_in] fp32
    Geom g;
    int B, C;
    int c0;                 // first channel of this chunk
    int nch;                // channels in this chunk (pairs = nch * B, channel-major)
    int bf16;               // I/O dtype: 0 fp32, 1 bf16
    int accum;              // backward: add dalpha / dbeta to what the output holds (later batch entries
                            // of the per-sample backward)
    // Backward only (y then holds dx):
    const void* dy;         // [B][C][vox], dtype of x
    float2* ws_u;           // gated-input planes, like ws (when dK is wanted)
    float2* dkw;            // d >= 2: per chunk channel, N_out * N_mid * S kernel-gradient
                            // spectrum (tile-major like K_hat's main block); d = 1: per
                            // pair, S values
    float2* part;           // per line pair (d >= 2) or per pair (d = 1): (dalpha, dbeta) terms
    float* dalpha;          // [C]
    float* dbeta;           // [C]
    float* dK;              // [C][ke_out][ke_mid][ke_in]
};

// Per-line data of a row workgroup, computed once per line: element offsets of
// the two signals of the line in x / y (o0, o1) and in the workspace or the
// kernel spectrum (w0, w1), their gate parameters, and validity.
struct RowMeta {
    long long o0, o1, w0, w1;
    float al0, be0, al1, be1;
    int valid, valid1;
};

// Recommended workspace: whole channels (all B pairs of a channel are processed
// together), up to about 256 MiB, at least one channel.  Measured on MI355X
// (ms per call for 64 / 128 / 256 MiB): 256x256 B=8 C=64 0.363 / 0.324 /
// 0.324; 1024^2 B=2 C=128 4.67 / 4.39 / 4.29; 128^3 B=1 C=32 2.15 / 1.90 /
// 1.82.  Smaller chunks lose to launch tails; the workspace does not need to
// fit in the 256 MB Infinity Cache.
inline int chunk_channels(const Geom& g, int B, int C, size_t ws_bytes_available)
{
    const size_t per_ch = (size_t)B * (size_t)g.wsp * 8u;
    if (per_ch == 0) return C;
    size_t n = ws_bytes_available / per_ch;
    if (n > (size_t)C) n = (size_t)C;
    return (int)n;
}

inline size_t recommended_workspace(const Geom& g, int B, int C)
{
    const size_t per_ch = (size_t)B * (size_t)g.wsp * 8u;
    if (per_ch == 0) return 0;
    const size_t target = (size_t)256 << 20;
    size_t n = target / per_ch;
    if (n < 1) n = 1;
    if (n > (size_t)C) n = (size_t)C;
    return n * per_ch;
}

// Long 1-D backward with dK: the kernel-gradient row kernel also writes the du
// rows (the du row pass fused) for rows of 4096 and 8192 points (one line per
// workgroup); with 1024- and 2048-point rows, four or two lines per
// workgroup, the fused product's registers would spill 94-108 VGPRs.
constexpr bool lng_dk_fuses_du(int N2) { return N2 >= 4096; }
// Long 1-D product rows in registers (lng_prod_body): lines per workgroup
// (4096 points each, one line of 8192) and threads (8 points per thread per
// pass); workgroups per CU the kernel-gradient row kernel is held to (a line
// of 8192 points and its 64 KiB of twiddles leave room for one).
constexpr int lngp_nl(int L) { return L >= 4096 ? 1 : 4096 / L; }
constexpr int lngp_nt(int L) { return L * lngp_nl(L) / 8; }
constexpr int lngp_wgs(int L) { return L >= 8192 ? 1 : 2; }
// Layout code (row_lay) of the register-flow row kernels' tiles: one extra
// slot after every 16 positions for one-line tiles of 4096 and 8192 points,
// two after every 8 for 2048-point tiles of two lines, two after every 4 for
// 1024-point tiles of four lines (LDS conflict cycles per instruction of
// k_lng_prod 2.7 and 4.4 on the plain tiles; 2^24 tokens: row pass 262 ->
// 252 us, 2^21 tokens: 179 -> 168 us).
constexpr int lngp_lay(int L)
{
    return L >= 4096 ? (1 | 1 << 8 | 4 << 12) : L == 2048 ? (2 | 2 << 8 | 3 << 12)
         : L == 1024 ? (4 | 2 << 8 | 2 << 12) : lngp_nl(L);
}

// Backward partial sums of dalpha / dbeta per (b, c) pair: one per line pair
// of the row kernels (d >= 2), one per pair (d = 1), one per inverse-column
// workgroup (long 1-D).
__host__ __device__ __forceinline__ int pair_lines(const Geom& g)
{
    if (g.lng) return g.N2 / col_tw(g.N1);  // long 1-D: one per inverse-column workgroup
    return g.d == 1 ? 1 : g.n_out * g.n_mid / 2;
}

// Backward workspace per channel of a chunk (bytes): the planes of dy and, for
// dK, of the gated input (B * wsp complex each), the kernel-gradient spectrum
// (N_out N_mid S complex for d >= 2; B S for d = 1; N for long 1-D) and the partial sums of
// dalpha and dbeta (B * pair_lines float2).
inline size_t bwd_channel_bytes(const Geom& g, int B, bool dk)
{
    size_t v = (size_t)B * (size_t)g.wsp * (dk ? 2u : 1u);
    if (dk) v += (g.d == 1 && !g.lng) ? (size_t)B * (size_t)g.S : (size_t)g.kmain;
    v += (size_t)B * (size_t)pair_lines(g);
    return v * 8u;
}

inline int bwd_chunk_channels(const Geom& g, int B, int C, bool dk, size_t ws_bytes_available)
{
    size_t n = ws_bytes_available / bwd_channel_bytes(g, B, dk);
    if (n > (size_t)C) n = (size_t)C;
    return (int)n;
}

// Recommended backward workspace: whole channels up to about 512 MiB (two
// planes per pair instead of the forward's one).
inline size_t recommended_bwd_workspace(const Geom& g, int B, int C, bool dk)
{
    const size_t per_ch = bwd_channel_bytes(g, B, dk);
    size_t n = ((size_t)512 << 20) / per_ch;
    if (n < 1) n = 1;
    if (n > (size_t)C) n = (size_t)C;
    return n * per_ch;
}

}  // namespace hyenand
