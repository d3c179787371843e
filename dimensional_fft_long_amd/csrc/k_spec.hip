// k_spec.hip -- the kernel-spectrum chains (zero-padded mode; the circular
// mode reads the kernel by offset mod n inside the same kernels).
#include "kernels_dev.h"

namespace hyenand {

hipError_t launch_spectrum(const ConvArgs& a, hipStream_t st)
{
    const Geom& g = a.g;
    if (g.lng) return long1d_forward(a, true, st, nullptr);
    hipError_t e;
    const long long H = g.d == 1 ? ((long long)a.C + 1) / 2 : (long long)a.C * (g.N_out * g.N_mid / 2);
    e = with_length(g.N_in, [&]<int L>() {
        hipLaunchKernelGGL(k_spec_row<L>, dim3(ceil_div(H, row_np(L))), dim3(row_nt(L)), 0, st, a);
        return last_error();
    });
    if (e != hipSuccess || g.d == 1) return e;
    if (g.d == 3) {
        e = with_length(g.N_mid, [&]<int L>() {
            const long long grid = (long long)a.C * ceil_div((long long)g.N_out * g.S, col_tw(L));
            hipLaunchKernelGGL(k_spec_mid<L>, dim3((unsigned)grid), dim3(col_nt(L)), 0, st, a);
            return last_error();
        });
        if (e != hipSuccess) return e;
        return with_length(g.N_out, [&]<int L>() {
            const long long grid = (long long)a.C * (g.N_mid / 2) * ceil_div(g.S, out_tw(L, 2));
            hipLaunchKernelGGL((k_spec_out<L, 2>), dim3((unsigned)grid), dim3(out_nt(L, 2)), 0, st, a);
            return last_error();
        });
    }
    return with_length(g.N_out, [&]<int L>() {
        const long long grid = (long long)a.C * ceil_div(g.S, out_tw(L, 1));
        hipLaunchKernelGGL((k_spec_out<L, 1>), dim3((unsigned)grid), dim3(out_nt(L, 1)), 0, st, a);
        return last_error();
    });
}

}  // namespace hyenand

