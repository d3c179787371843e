// k_long.hip -- the four-step chains of long 1-D signals (forward, spectrum,
// backward).
#include "kernels_dev.h"

namespace hyenand {
namespace {

// Long 1-D forward (and, with SPEC, the spectrum): column pass, row pass, column pass.
hipError_t long1d_chunk(const ConvArgs& a, bool spec, hipStream_t st, LaunchTrace* tr)
{
    auto mark = [&]() { if (tr) tr->mark(st); };
    const Geom& g = a.g;
    const long long sigs = spec ? a.C : (long long)a.nch * a.B;
    hipError_t e = with_col_length(g.N1, [&]<int L>() {
        const unsigned grid = (unsigned)(sigs * (g.N2 / col_tw(L)));
        mark();
        if (spec) hipLaunchKernelGGL((k_lng_col_fwd<L, true, false>), dim3(grid), dim3(col_nt(L)), 0, st, a);
        else if (a.bf16) hipLaunchKernelGGL((k_lng_col_fwd<L, false, true>), dim3(grid), dim3(col_nt(L)), 0, st, a);
        else hipLaunchKernelGGL((k_lng_col_fwd<L, false, false>), dim3(grid), dim3(col_nt(L)), 0, st, a);
        return last_error();
    });
    if (e != hipSuccess) return e;
    e = with_row_length(g.N2, [&]<int L>() {
        mark();
        if (spec)
            hipLaunchKernelGGL((k_lng_spec_row<L>), dim3(ceil_div(sigs * g.N1, row_np(L))), dim3(row_nt(L)), 0, st, a);
        else
            hipLaunchKernelGGL((k_lng_prod<L, false>), dim3(ceil_div(sigs * g.N1, lngp_nl(L))), dim3(lngp_nt(L)), 0,
                               st, a);
        return last_error();
    });
    if (e != hipSuccess || spec) return e;
    return with_col_length(g.N1, [&]<int L>() {
        const unsigned grid = (unsigned)(sigs * (g.N2 / col_tw(L)));
        mark();
        if (a.bf16) hipLaunchKernelGGL((k_lng_col_inv<L, true>), dim3(grid), dim3(col_nt(L)), 0, st, a);
        else hipLaunchKernelGGL((k_lng_col_inv<L, false>), dim3(grid), dim3(col_nt(L)), 0, st, a);
        return last_error();
    });
}

// Long 1-D backward: column transforms of dy (and of the gated input for dK),
// the kernel-gradient row pass (for dK; for 4096-point rows it also writes
// the du rows), the du row pass (unless fused), the inverse columns with the dx
// epilogue, the dalpha / dbeta reduction and the kernel gradient's inverse
// columns.
hipError_t long1d_bwd_chunk(const ConvArgs& a, bool dk, hipStream_t st, LaunchTrace* tr)
{
    auto mark = [&]() { if (tr) tr->mark(st); };
    const Geom& g = a.g;
    const long long sigs = (long long)a.nch * a.B;
    ConvArgs ady = a;
    ady.x = a.dy;
    ConvArgs au = a;
    au.ws = a.ws_u;
    auto col_fwd = [&](const ConvArgs& arg, bool gate) {
        return with_col_length(g.N1, [&]<int L>() {
            const unsigned grid = (unsigned)(sigs * (g.N2 / col_tw(L)));
            mark();
            if (gate) {
                if (a.bf16) hipLaunchKernelGGL((k_lng_col_fwd<L, false, true, true>), dim3(grid), dim3(col_nt(L)), 0, st, arg);
                else hipLaunchKernelGGL((k_lng_col_fwd<L, false, false, true>), dim3(grid), dim3(col_nt(L)), 0, st, arg);
            } else {
                if (a.bf16) hipLaunchKernelGGL((k_lng_col_fwd<L, false, true, false>), dim3(grid), dim3(col_nt(L)), 0, st, arg);
                else hipLaunchKernelGGL((k_lng_col_fwd<L, false, false, false>), dim3(grid), dim3(col_nt(L)), 0, st, arg);
            }
            return last_error();
        });
    };
    hipError_t e = col_fwd(ady, false);
    if (e == hipSuccess && dk) e = col_fwd(au, true);
    if (e == hipSuccess && dk)
        e = with_row_length(g.N2, [&]<int L>() {
            mark();
            hipLaunchKernelGGL((k_lng_prod_dk<L>), dim3(ceil_div((long long)a.nch * g.N1, lngp_nl(L))),
                               dim3(lngp_nt(L)), 0, st, a);
            return last_error();
        });
    if (e == hipSuccess && !(dk && lng_dk_fuses_du(g.N2)))  // else the kernel-gradient row pass wrote du
        e = with_row_length(g.N2, [&]<int L>() {
            mark();
            hipLaunchKernelGGL((k_lng_prod<L, true>), dim3(ceil_div(sigs * g.N1, lngp_nl(L))), dim3(lngp_nt(L)), 0,
                               st, a);
            return last_error();
        });
    if (e == hipSuccess)
        e = with_col_length(g.N1, [&]<int L>() {
            const unsigned grid = (unsigned)(sigs * (g.N2 / col_tw(L)));
            mark();
            if (a.bf16) hipLaunchKernelGGL((k_lng_col_inv<L, true, true>), dim3(grid), dim3(col_nt(L)), 0, st, a);
            else hipLaunchKernelGGL((k_lng_col_inv<L, false, true>), dim3(grid), dim3(col_nt(L)), 0, st, a);
            return last_error();
        });
    if (e == hipSuccess) {
        mark();
        hipLaunchKernelGGL(k_gate_reduce, dim3((unsigned)a.nch), dim3(kReduceNT), 0, st, a);
        e = last_error();
    }
    if (e == hipSuccess && dk)
        e = with_col_length(g.N1, [&]<int L>() {
            mark();
            hipLaunchKernelGGL((k_lng_col_dk<L>), dim3((unsigned)((long long)a.nch * (g.N2 / col_tw(L)))), dim3(col_nt(L)), 0, st, a);
            return last_error();
        });
    return e;
}

}  // namespace

hipError_t long1d_forward(const ConvArgs& a, bool spec, hipStream_t st, LaunchTrace* tr)
{
    return long1d_chunk(a, spec, st, tr);
}

hipError_t long1d_backward(const ConvArgs& a, bool dk, hipStream_t st, LaunchTrace* tr)
{
    return long1d_bwd_chunk(a, dk, st, tr);
}

}  // namespace hyenand
