// kernels.hip -- gfx950 kernels of the gated N-D FFT convolution and their
// launchers.  The workgroup bodies are in conv_bodies.h; this file binds them
// to the device (thread index, barrier, LDS tile, twiddle table) and picks the
// template instance for each transform length.
#include <hip/hip_runtime.h>

#include "conv_bodies.h"
#include "launch.h"

namespace hyenand {

// W_2048^t, computed at compile time (fft_core.h) and placed in constant memory.
__constant__ const TwTable g_twiddles = make_twiddles();

struct DevCtx {
    __device__ int tid() const { return (int)threadIdx.x; }
    __device__ void sync() const { __syncthreads(); }
    __device__ float2 tw(int t) const { return g_twiddles.w[t]; }
};

template <int L>
__global__ __launch_bounds__(kThreads) void k_row_fwd(ConvArgs a)
{
    __shared__ float2 T[L * (row_np(L) + 1)];
    row_fwd_body<L>(DevCtx{}, (int)blockIdx.x, a, T);
}

template <int L>
__global__ __launch_bounds__(kThreads) void k_row_inv(ConvArgs a)
{
    __shared__ float2 T[L * (row_np(L) + 1)];
    row_inv_body<L>(DevCtx{}, (int)blockIdx.x, a, T);
}

template <int L>
__global__ __launch_bounds__(kThreads) void k_conv1d(ConvArgs a)
{
    __shared__ float2 T[L * (row_np(L) + 1)];
    conv1d_body<L>(DevCtx{}, (int)blockIdx.x, a, T);
}

template <int L, bool INV>
__global__ __launch_bounds__(kThreads) void k_col_mid(ConvArgs a)
{
    __shared__ float2 T[L * col_tw(L)];
    col_mid_body<L, INV>(DevCtx{}, (int)blockIdx.x, a, T);
}

template <int L, int NR>
__global__ __launch_bounds__(kThreads) void k_col_out(ConvArgs a)
{
    __shared__ float2 T[L * NR * (NR == 1 ? col_tw(L) : mul3_tw(L))];
    col_out_body<L, NR>(DevCtx{}, (int)blockIdx.x, a, T);
}

template <int L>
__global__ __launch_bounds__(kThreads) void k_spec_row(ConvArgs a)
{
    __shared__ float2 T[L * (row_np(L) + 1)];
    spec_row_body<L>(DevCtx{}, (int)blockIdx.x, a, T);
}

template <int L>
__global__ __launch_bounds__(kThreads) void k_spec_mid(ConvArgs a)
{
    __shared__ float2 T[L * col_tw(L)];
    spec_mid_body<L>(DevCtx{}, (int)blockIdx.x, a, T);
}

template <int L, int NR>
__global__ __launch_bounds__(kThreads) void k_spec_out(ConvArgs a)
{
    __shared__ float2 T[L * NR * (NR == 1 ? col_tw(L) : mul3_tw(L))];
    spec_out_body<L, NR>(DevCtx{}, (int)blockIdx.x, a, T);
}

static inline unsigned ceil_div(long long a, long long b) { return (unsigned)((a + b - 1) / b); }

// Calls F.template operator()<L>() for the runtime length L in {4, ..., 2048}.
template <class F>
static hipError_t with_length(int L, F&& f)
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

static hipError_t last_error() { return hipGetLastError(); }

hipError_t launch_forward_chunk(const ConvArgs& a, hipStream_t st, LaunchTrace* tr)
{
    auto mark = [&]() { if (tr) tr->mark(st); };
    const Geom& g = a.g;
    const dim3 blk(kThreads);
    hipError_t e;
    if (g.d == 1) {
        return with_length(g.N_in, [&]<int L>() {
            const long long H = ((long long)a.nch * a.B + 1) / 2;
            mark();
            hipLaunchKernelGGL(k_conv1d<L>, dim3(ceil_div(H, row_np(L))), blk, 0, st, a);
            return last_error();
        });
    }
    const long long H = (long long)a.nch * a.B * (g.n_out * g.n_mid / 2);
    e = with_length(g.N_in, [&]<int L>() {
        mark();
        hipLaunchKernelGGL(k_row_fwd<L>, dim3(ceil_div(H, row_np(L))), blk, 0, st, a);
        return last_error();
    });
    if (e != hipSuccess) return e;
    if (g.d == 3) {
        e = with_length(g.N_mid, [&]<int L>() {
            const long long grid = (long long)a.nch * a.B * ceil_div((long long)g.n_out * g.S, col_tw(L));
            mark();
            hipLaunchKernelGGL((k_col_mid<L, false>), dim3((unsigned)grid), blk, 0, st, a);
            return last_error();
        });
        if (e != hipSuccess) return e;
        e = with_length(g.N_out, [&]<int L>() {
            const long long grid = (long long)a.nch * (g.N_mid / 2) * ceil_div(g.S, mul3_tw(L));
            mark();
            hipLaunchKernelGGL((k_col_out<L, 2>), dim3((unsigned)grid), blk, 0, st, a);
            return last_error();
        });
        if (e != hipSuccess) return e;
        e = with_length(g.N_mid, [&]<int L>() {
            const long long grid = (long long)a.nch * a.B * ceil_div((long long)g.n_out * g.S, col_tw(L));
            mark();
            hipLaunchKernelGGL((k_col_mid<L, true>), dim3((unsigned)grid), blk, 0, st, a);
            return last_error();
        });
    } else {
        e = with_length(g.N_out, [&]<int L>() {
            const long long grid = (long long)a.nch * ceil_div(g.S, col_tw(L));
            mark();
            hipLaunchKernelGGL((k_col_out<L, 1>), dim3((unsigned)grid), blk, 0, st, a);
            return last_error();
        });
    }
    if (e != hipSuccess) return e;
    return with_length(g.N_in, [&]<int L>() {
        mark();
        hipLaunchKernelGGL(k_row_inv<L>, dim3(ceil_div(H, row_np(L))), blk, 0, st, a);
        return last_error();
    });
}

hipError_t launch_spectrum(const ConvArgs& a, hipStream_t st)
{
    const Geom& g = a.g;
    const dim3 blk(kThreads);
    hipError_t e;
    const long long H = g.d == 1 ? ((long long)a.C + 1) / 2 : (long long)a.C * (g.N_out * g.N_mid / 2);
    e = with_length(g.N_in, [&]<int L>() {
        hipLaunchKernelGGL(k_spec_row<L>, dim3(ceil_div(H, row_np(L))), blk, 0, st, a);
        return last_error();
    });
    if (e != hipSuccess || g.d == 1) return e;
    if (g.d == 3) {
        e = with_length(g.N_mid, [&]<int L>() {
            const long long grid = (long long)a.C * ceil_div((long long)g.N_out * g.S, col_tw(L));
            hipLaunchKernelGGL(k_spec_mid<L>, dim3((unsigned)grid), blk, 0, st, a);
            return last_error();
        });
        if (e != hipSuccess) return e;
        return with_length(g.N_out, [&]<int L>() {
            const long long grid = (long long)a.C * (g.N_mid / 2) * ceil_div(g.S, mul3_tw(L));
            hipLaunchKernelGGL((k_spec_out<L, 2>), dim3((unsigned)grid), blk, 0, st, a);
            return last_error();
        });
    }
    return with_length(g.N_out, [&]<int L>() {
        const long long grid = (long long)a.C * ceil_div(g.S, col_tw(L));
        hipLaunchKernelGGL((k_spec_out<L, 1>), dim3((unsigned)grid), blk, 0, st, a);
        return last_error();
    });
}

}  // namespace hyenand
