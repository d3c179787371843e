// kernels_dev.h -- gfx950 kernels of the gated N-D FFT convolution and the
// chains that launch them.  The workgroup bodies are in conv_bodies.h; this
// header binds them to the device (thread index, barrier, LDS tile, twiddle
// table) and picks the template instance for each transform length.
//
// Every kernel translation unit (k_*.hip) includes this header and
// instantiates only the kernels its chains launch.  Everything here sits in an
// unnamed namespace, so a kernel instantiated by two units is two distinct
// symbols, one in each unit's code object.
#pragma once

#include <hip/hip_runtime.h>

#include "conv_bodies.h"
#include "launch.h"

namespace hyenand {
namespace {
template <int L, int PLANS>
constexpr int twl_size() { return tw_table_alloc<L, PLANS>(); }

// Per-(length, plans) twiddle tables, built at compile time.
template <int L, int PLANS>
__constant__ const PlanTwiddles<L, PLANS> g_plan_tw = make_plan_twiddles<L, PLANS>();

// Device execution context of a kernel of NT threads whose transforms have
// length L and use the plans PLANS.  The bodies call stage() to copy the
// twiddle tables (fft_core.h) into LDS before a barrier that precedes their
// first transform pass with twiddles.
template <int L, int NT, int PLANS>
struct DevCtx {
    static constexpr int kRevBase = tw_rev_base<L, PLANS>();
    float2* twl;
    __device__ int tid() const { return (int)threadIdx.x; }
    __device__ void sync() const { __syncthreads(); }
    // phi(x) x = x / (1 + exp(-(alpha x + beta))) with the hardware exp2 and reciprocal.
    __device__ float gate(float x, float al, float be) const
    {
        const float e = __builtin_amdgcn_exp2f(-(al * x + be) * 1.44269504088896341f);
        return x * __builtin_amdgcn_rcpf(1.0f + e);
    }
    __device__ float sigmoid(float v) const
    {
        return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * 1.44269504088896341f));
    }
    // exp(-2 pi i e / N), N = 2^logN, e < N: the exact fraction e / N through
    // sincospi (accurate to a few ulp over the whole circle).
    __device__ float2 twiddle(unsigned e, int logN) const
    {
        float sn, cs;
        sincospif(2.0f * __builtin_ldexpf((float)e, -logN), &sn, &cs);
        return make_float2(cs, -sn);
    }
    // Two halves so that callers can issue other loads in between: every
    // load of the copy is issued before the first store.
    static constexpr int kTwSize = tw_table_size<L, PLANS>();
    static constexpr int kTwIter = kTwSize > 0 ? (kTwSize + NT - 1) / NT : 1;
    struct Staged {
        float2 v[kTwIter];
    };
    __device__ Staged stage_load() const
    {
        Staged st;
        if constexpr (kTwSize > 0) {
            const int t0 = (int)threadIdx.x;
#pragma unroll
            for (int i = 0; i < kTwIter; ++i) {
                const int e = t0 + i * NT;
                st.v[i] = g_plan_tw<L, PLANS>.w[e < kTwSize ? e : kTwSize - 1];
            }
        }
        return st;
    }
    __device__ void stage_store(const Staged& st) const
    {
        if constexpr (kTwSize > 0) {
            const int t0 = (int)threadIdx.x;
#pragma unroll
            for (int i = 0; i < kTwIter; ++i) {
                const int e = t0 + i * NT;
                if (e < kTwSize) twl[e] = st.v[i];
            }
        }
    }
    __device__ void stage() const { stage_store(stage_load()); }
};

template <int L, int NT, int PLANS>
__device__ __forceinline__ DevCtx<L, NT, PLANS> make_ctx(float2* twl)
{
    return DevCtx<L, NT, PLANS>{twl};
}

template <int L, bool BF16, bool GATE, bool CIRC = false>
__global__ __launch_bounds__(row_nt(L)) void k_row_fwd(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, kPlanF>()];
    __shared__ float2 T[lay_elems(L, row_np(L), row_lay(L))];
    __shared__ RowMeta M[row_np(L)];
    row_fwd_body<L, BF16, GATE, CIRC>(make_ctx<L, row_nt(L), kPlanF>(TWL), (int)blockIdx.x, a, T, M);
}

template <int L, bool BF16, bool BWD, bool CIRC = false>
__global__ __launch_bounds__(row_nt(L)) void k_row_inv(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, kPlanF>()];
    __shared__ float2 T[lay_elems(L, row_np(L), row_lay(L))];
    __shared__ RowMeta M[row_np(L)];
    row_inv_body<L, BF16, BWD, CIRC>(make_ctx<L, row_nt(L), kPlanF>(TWL), (int)blockIdx.x, a, T, M);
}

template <int L, bool BF16, bool BWD, bool CIRC = false>
__global__ __launch_bounds__(row_nt(L)) void k_conv1d(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, kPlanF>()];
    __shared__ float2 T[L * row_lp(L)];
    __shared__ RowMeta M[row_np(L)];
    conv1d_body<L, BF16, BWD, CIRC>(make_ctx<L, row_nt(L), kPlanF>(TWL), (int)blockIdx.x, a, T, M);
}

// Waves per SIMD the compiler must leave room for: two workgroups per CU for
// the 512-point 2-D tiles (at most 128 VGPRs; 256^2 backward 0.80 -> 0.71 ms
// per call); one elsewhere.
template <int L, int NR>
constexpr int bwd_min_waves() { return (NR == 1 && L == 512) ? 2 * bwd_nt(L, NR) / 64 / 4 : 1; }

template <int L, int NR, bool DK, bool CIRC>
__global__ __launch_bounds__(bwd_nt(L, NR), (bwd_min_waves<L, NR>())) void k_col_out_bwd(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, (kPlanF | kPlanR)>()];
    __shared__ float2 T[L * NR * bwd_tw(L, NR)];
    col_out_bwd_body<L, NR, DK, CIRC>(make_ctx<L, bwd_nt(L, NR), (kPlanF | kPlanR)>(TWL), (int)blockIdx.x, a, T);
}

template <int L>
__global__ __launch_bounds__(col_nt(L)) void k_plane_mid_inv(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, kPlanF>()];
    __shared__ float2 T[L * col_tw(L)];
    plane_mid_body<L, true>(make_ctx<L, col_nt(L), kPlanF>(TWL), (int)blockIdx.x, a.g, a.dkw, a.g.kmain, T);
}

template <int L, bool BF16, bool CIRC>
__global__ __launch_bounds__(row_nt(L)) void k_corr1d(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, kPlanF>()];
    __shared__ float2 T[L * row_lp(L)];
    __shared__ RowMeta M[row_np(L)];
    corr1d_body<L, BF16, CIRC>(make_ctx<L, row_nt(L), kPlanF>(TWL), (int)blockIdx.x, a, T, M);
}

template <int L>
__global__ __launch_bounds__(row_nt(L)) void k_dk_row(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, kPlanF>()];
    __shared__ float2 T[lay_elems(L, row_np(L), row_lay(L))];
    __shared__ RowMeta M[row_np(L)];
    dk_row_body<L>(make_ctx<L, row_nt(L), kPlanF>(TWL), (int)blockIdx.x, a, T, M);
}

template <int L, bool SPEC, bool BF16, bool GATE = true>
__global__ __launch_bounds__(col_nt(L)) void k_lng_col_fwd(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, kPlanF>()];
    __shared__ float2 T[L * col_tw(L)];
    lng_col_fwd_body<L, SPEC, BF16, GATE>(make_ctx<L, col_nt(L), kPlanF>(TWL), (int)blockIdx.x, a, T);
}

template <int L>
__global__ __launch_bounds__(row_nt(L)) void k_lng_spec_row(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, kPlanF>()];
    __shared__ float2 T[L * row_lp(L)];
    lng_spec_row_body<L>(make_ctx<L, row_nt(L), kPlanF>(TWL), (int)blockIdx.x, a, T);
}

template <int L, bool CONJ>
__global__ __launch_bounds__(lngp_nt(L)) void k_lng_prod(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, (kPlanF | kPlanR)>()];
    __shared__ float2 T[lay_elems(L, lngp_nl(L), lngp_lay(L))];
    lng_prod_body<L, CONJ>(make_ctx<L, lngp_nt(L), (kPlanF | kPlanR)>(TWL), (int)blockIdx.x, a, T);
}

// Two workgroups per CU below 8192 points (at most 128 VGPRs): the dy, u, P and
// kernel spectrum registers otherwise take 135 and leave room for one.  8192
// points: one workgroup per CU (its LDS), 128 VGPRs too.
template <int L>
__global__ __launch_bounds__(lngp_nt(L), lngp_wgs(L) * lngp_nt(L) / 64 / 4) void k_lng_prod_dk(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, (kPlanF | kPlanR)>()];
    __shared__ float2 T[lay_elems(L, lngp_nl(L), lngp_lay(L))];
    lng_prod_dk_body<L>(make_ctx<L, lngp_nt(L), (kPlanF | kPlanR)>(TWL), (int)blockIdx.x, a, T);
}

template <int L, bool BF16, bool BWD = false>
__global__ __launch_bounds__(col_nt(L)) void k_lng_col_inv(ConvArgs a)
{
    static_assert(col_nt(L) <= L * col_tw(L), "the backward's tree fits in the tile");
    __shared__ float2 TWL[twl_size<L, kPlanR>()];
    __shared__ float2 T[L * col_tw(L)];
    lng_col_inv_body<L, BF16, BWD>(make_ctx<L, col_nt(L), kPlanR>(TWL), (int)blockIdx.x, a, T);
}

template <int L>
__global__ __launch_bounds__(col_nt(L)) void k_lng_col_dk(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, kPlanR>()];
    __shared__ float2 T[L * col_tw(L)];
    lng_col_dk_body<L>(make_ctx<L, col_nt(L), kPlanR>(TWL), (int)blockIdx.x, a, T);
}

constexpr int kReduceNT = 1024;

__global__ __launch_bounds__(kReduceNT) void k_gate_reduce(ConvArgs a)
{
    __shared__ double R[2 * kReduceNT];
    gate_reduce_body<kReduceNT>(make_ctx<4, kReduceNT, kPlanF>(nullptr), (int)blockIdx.x, a, R);
}

// Zero fill (the gradients of an empty batch), n floats.
__global__ __launch_bounds__(256) void k_zero(float* p, long long n)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

template <int L, bool INV, bool CIRC = false>
__global__ __launch_bounds__(col_nt(L)) void k_col_mid(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, (INV ? kPlanR : kPlanF)>()];
    __shared__ float2 T[L * col_tw(L)];
    col_mid_body<L, INV, CIRC>(make_ctx<L, col_nt(L), (INV ? kPlanR : kPlanF)>(TWL), (int)blockIdx.x, a, T);
}

template <int L, int NR, bool CIRC = false>
__global__ __launch_bounds__(out_nt(L, NR)) void k_col_out(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, (kPlanF | kPlanR)>()];
    __shared__ float2 T[lay_elems(L, NR * out_tw(L, NR), out_lay(L, NR))];
    col_out_body<L, NR, CIRC>(make_ctx<L, out_nt(L, NR), (kPlanF | kPlanR)>(TWL), (int)blockIdx.x, (int)gridDim.x, a, T);
}

template <int L>
__global__ __launch_bounds__(row_nt(L)) void k_spec_row(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, kPlanF>()];
    __shared__ float2 T[L * row_lp(L)];
    spec_row_body<L>(make_ctx<L, row_nt(L), kPlanF>(TWL), (int)blockIdx.x, a, T);
}

template <int L>
__global__ __launch_bounds__(col_nt(L)) void k_spec_mid(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, kPlanF>()];
    __shared__ float2 T[L * col_tw(L)];
    spec_mid_body<L>(make_ctx<L, col_nt(L), kPlanF>(TWL), (int)blockIdx.x, a, T);
}

template <int L, int NR>
__global__ __launch_bounds__(out_nt(L, NR)) void k_spec_out(ConvArgs a)
{
    __shared__ float2 TWL[twl_size<L, kPlanF>()];
    __shared__ float2 T[L * NR * out_tw(L, NR)];
    spec_out_body<L, NR>(make_ctx<L, out_nt(L, NR), kPlanF>(TWL), (int)blockIdx.x, a, T);
}

inline unsigned ceil_div(long long a, long long b) { return (unsigned)((a + b - 1) / b); }

// Grid of an item-looping kernel: one workgroup per item up to the number
// resident at once (resident_wgs, launch.h).
template <class K>
unsigned loop_grid(K kernel, int nt, long long items)
{
    const unsigned r = resident_wgs(reinterpret_cast<const void*>(kernel), nt);
    return r > 0 && items > (long long)r ? r : (unsigned)items;
}

// Calls F.template operator()<L>() for the runtime length L in {4, ..., 2048}.
template <class F>
hipError_t with_length(int L, F&& f)
{
    switch (L) {
    case 4: return f.template operator()<4>();
    case 8: return f.template operator()<8>();
    case 16: return f.template operator()<16>();
    case 32: return f.template operator()<32>();
    case 64: return f.template operator()<64>();
    case 128: return f.template operator()<128>();
    case 256: return f.template operator()<256>();
    case 512: return f.template operator()<512>();
    case 1024: return f.template operator()<1024>();
    case 2048: return f.template operator()<2048>();
    default: return hipErrorInvalidValue;
    }
}

hipError_t last_error() { return hipGetLastError(); }

template <bool CIRC>
hipError_t forward_chunk(const ConvArgs& a, hipStream_t st, LaunchTrace* tr)
{
    auto mark = [&]() { if (tr) tr->mark(st); };
    const Geom& g = a.g;
    hipError_t e;
    if (g.d == 1) {
        return with_length(g.N_in, [&]<int L>() {
            const long long H = ((long long)a.nch * a.B + 1) / 2;
            mark();
            if (a.bf16) hipLaunchKernelGGL((k_conv1d<L, true, false, CIRC>), dim3(ceil_div(H, row_np(L))), dim3(row_nt(L)), 0, st, a);
            else hipLaunchKernelGGL((k_conv1d<L, false, false, CIRC>), dim3(ceil_div(H, row_np(L))), dim3(row_nt(L)), 0, st, a);
            return last_error();
        });
    }
    const long long H = (long long)a.nch * a.B * (g.n_out * g.n_mid / 2);
    e = with_length(g.N_in, [&]<int L>() {
        mark();
        if (a.bf16) hipLaunchKernelGGL((k_row_fwd<L, true, true, CIRC>), dim3(ceil_div(H, row_np(L))), dim3(row_nt(L)), 0, st, a);
        else hipLaunchKernelGGL((k_row_fwd<L, false, true, CIRC>), dim3(ceil_div(H, row_np(L))), dim3(row_nt(L)), 0, st, a);
        return last_error();
    });
    if (e != hipSuccess) return e;
    if (g.d == 3) {
        e = with_length(g.N_mid, [&]<int L>() {
            const long long grid = (long long)a.nch * a.B * ceil_div((long long)g.n_out * g.S, col_tw(L));
            mark();
            hipLaunchKernelGGL((k_col_mid<L, false, CIRC>), dim3((unsigned)grid), dim3(col_nt(L)), 0, st, a);
            return last_error();
        });
        if (e != hipSuccess) return e;
        e = with_length(g.N_out, [&]<int L>() {
            const long long items = out_items<2, out_tw(L, 2)>(g, a.B, a.nch);
            const unsigned grid = out_looped(L, 2) ? loop_grid(k_col_out<L, 2, CIRC>, out_nt(L, 2), items) : (unsigned)items;
            mark();
            hipLaunchKernelGGL((k_col_out<L, 2, CIRC>), dim3(grid), dim3(out_nt(L, 2)), 0, st, a);
            return last_error();
        });
        if (e != hipSuccess) return e;
        e = with_length(g.N_mid, [&]<int L>() {
            const long long grid = (long long)a.nch * a.B * ceil_div((long long)g.n_out * g.S, col_tw(L));
            mark();
            hipLaunchKernelGGL((k_col_mid<L, true, CIRC>), dim3((unsigned)grid), dim3(col_nt(L)), 0, st, a);
            return last_error();
        });
    } else {
        e = with_length(g.N_out, [&]<int L>() {
            const long long items = out_items<1, out_tw(L, 1)>(g, a.B, a.nch);
            const unsigned grid = out_looped(L, 1) ? loop_grid(k_col_out<L, 1, CIRC>, out_nt(L, 1), items) : (unsigned)items;
            mark();
            hipLaunchKernelGGL((k_col_out<L, 1, CIRC>), dim3(grid), dim3(out_nt(L, 1)), 0, st, a);
            return last_error();
        });
    }
    if (e != hipSuccess) return e;
    return with_length(g.N_in, [&]<int L>() {
        mark();
        if (a.bf16) hipLaunchKernelGGL((k_row_inv<L, true, false, CIRC>), dim3(ceil_div(H, row_np(L))), dim3(row_nt(L)), 0, st, a);
        else hipLaunchKernelGGL((k_row_inv<L, false, false, CIRC>), dim3(ceil_div(H, row_np(L))), dim3(row_nt(L)), 0, st, a);
        return last_error();
    });
}

// Transform lengths of the long 1-D path: rows N2 in {1024, 2048, 4096, 8192},
// columns N1 in {4, ..., 4096}.
template <class F>
hipError_t with_row_length(int L, F&& f)
{
    switch (L) {
    case 1024: return f.template operator()<1024>();
    case 2048: return f.template operator()<2048>();
    case 4096: return f.template operator()<4096>();
    case 8192: return f.template operator()<8192>();
    default: return hipErrorInvalidValue;
    }
}

template <class F>
hipError_t with_col_length(int L, F&& f)
{
    if (L == 4096) return f.template operator()<4096>();
    return with_length(L, f);
}

template <bool CIRC>
hipError_t backward_chunk(const ConvArgs& a, bool dk, hipStream_t st, LaunchTrace* tr)
{
    auto mark = [&]() { if (tr) tr->mark(st); };
    const Geom& g = a.g;
    hipError_t e;
    auto reduce = [&]() {
        mark();
        hipLaunchKernelGGL(k_gate_reduce, dim3((unsigned)a.nch), dim3(kReduceNT), 0, st, a);
        return last_error();
    };
    auto dk_rows = [&](long long lines) {
        return with_length(g.N_in, [&]<int L>() {
            mark();
            hipLaunchKernelGGL(k_dk_row<L>, dim3(ceil_div(lines, row_np(L))), dim3(row_nt(L)), 0, st, a);
            return last_error();
        });
    };
    if (g.d == 1) {
        e = with_length(g.N_in, [&]<int L>() {
            const long long H = ((long long)a.nch * a.B + 1) / 2;
            mark();
            if (a.bf16) hipLaunchKernelGGL((k_conv1d<L, true, true, CIRC>), dim3(ceil_div(H, row_np(L))), dim3(row_nt(L)), 0, st, a);
            else hipLaunchKernelGGL((k_conv1d<L, false, true, CIRC>), dim3(ceil_div(H, row_np(L))), dim3(row_nt(L)), 0, st, a);
            return last_error();
        });
        if (e != hipSuccess) return e;
        if ((e = reduce()) != hipSuccess || !dk) return e;
        e = with_length(g.N_in, [&]<int L>() {
            mark();
            const unsigned grid = ceil_div((long long)a.nch * a.B, row_np(L));
            if (a.bf16) hipLaunchKernelGGL((k_corr1d<L, true, CIRC>), dim3(grid), dim3(row_nt(L)), 0, st, a);
            else hipLaunchKernelGGL((k_corr1d<L, false, CIRC>), dim3(grid), dim3(row_nt(L)), 0, st, a);
            return last_error();
        });
        if (e != hipSuccess) return e;
        return dk_rows(((long long)a.nch + 1) / 2);
    }
    ConvArgs ady = a;  // the row pass reads the output gradient in place of x
    ady.x = a.dy;
    ConvArgs au = a;   // the gated input's planes
    au.ws = a.ws_u;
    const long long H = (long long)a.nch * a.B * (g.n_out * g.n_mid / 2);
    e = with_length(g.N_in, [&]<int L>() {
        mark();
        if (ady.bf16) hipLaunchKernelGGL((k_row_fwd<L, true, false, CIRC>), dim3(ceil_div(H, row_np(L))), dim3(row_nt(L)), 0, st, ady);
        else hipLaunchKernelGGL((k_row_fwd<L, false, false, CIRC>), dim3(ceil_div(H, row_np(L))), dim3(row_nt(L)), 0, st, ady);
        if (last_error() != hipSuccess || !dk) return last_error();
        mark();
        if (au.bf16) hipLaunchKernelGGL((k_row_fwd<L, true, true, CIRC>), dim3(ceil_div(H, row_np(L))), dim3(row_nt(L)), 0, st, au);
        else hipLaunchKernelGGL((k_row_fwd<L, false, true, CIRC>), dim3(ceil_div(H, row_np(L))), dim3(row_nt(L)), 0, st, au);
        return last_error();
    });
    if (e != hipSuccess) return e;
    auto col_mid = [&]<bool INV>(const ConvArgs& arg) {
        return with_length(g.N_mid, [&]<int L>() {
            const long long grid = (long long)arg.nch * arg.B * ceil_div((long long)g.n_out * g.S, col_tw(L));
            mark();
            hipLaunchKernelGGL((k_col_mid<L, INV, CIRC>), dim3((unsigned)grid), dim3(col_nt(L)), 0, st, arg);
            return last_error();
        });
    };
    if (g.d == 3) {
        if ((e = col_mid.template operator()<false>(a)) != hipSuccess) return e;
        if (dk && (e = col_mid.template operator()<false>(au)) != hipSuccess) return e;
    }
    auto col_out = [&]<int NR>() {
        return with_length(g.N_out, [&]<int L>() {
            const long long grid = (long long)a.nch * (NR == 1 ? 1 : g.N_mid / 2) * ceil_div(g.S, bwd_tw(L, NR));
            mark();
            if (dk) hipLaunchKernelGGL((k_col_out_bwd<L, NR, true, CIRC>), dim3((unsigned)grid), dim3(bwd_nt(L, NR)), 0, st, a);
            else hipLaunchKernelGGL((k_col_out_bwd<L, NR, false, CIRC>), dim3((unsigned)grid), dim3(bwd_nt(L, NR)), 0, st, a);
            return last_error();
        });
    };
    e = g.d == 3 ? col_out.template operator()<2>() : col_out.template operator()<1>();
    if (e != hipSuccess) return e;
    if (g.d == 3 && (e = col_mid.template operator()<true>(a)) != hipSuccess) return e;
    e = with_length(g.N_in, [&]<int L>() {
        mark();
        if (a.bf16) hipLaunchKernelGGL((k_row_inv<L, true, true, CIRC>), dim3(ceil_div(H, row_np(L))), dim3(row_nt(L)), 0, st, a);
        else hipLaunchKernelGGL((k_row_inv<L, false, true, CIRC>), dim3(ceil_div(H, row_np(L))), dim3(row_nt(L)), 0, st, a);
        return last_error();
    });
    if (e != hipSuccess) return e;
    if ((e = reduce()) != hipSuccess || !dk) return e;
    if (g.d == 3) {
        e = with_length(g.N_mid, [&]<int L>() {
            const long long grid = (long long)a.nch * ceil_div((long long)g.N_out * g.S, col_tw(L));
            mark();
            hipLaunchKernelGGL(k_plane_mid_inv<L>, dim3((unsigned)grid), dim3(col_nt(L)), 0, st, a);
            return last_error();
        });
        if (e != hipSuccess) return e;
    }
    return dk_rows((long long)a.nch * (g.N_out * g.N_mid / 2));
}

}  // namespace
}  // namespace hyenand
