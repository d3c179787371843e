// k_gen.hip -- the input-dependent kernel generator's passes (gen.h) and their
// launch chain: per-sample means, registers / control / FiLM, axis spectra,
// per-pair spectra.
#include "gen.h"
#include "kernels_dev.h"

namespace hyenand {
namespace {

template <bool BF16>
__global__ __launch_bounds__(kGenNT) void k_gen_stats(GenArgs a)
{
    __shared__ double R[kGenNT];
    gen_stats_body<BF16>(make_ctx<4, kGenNT, kPlanF>(nullptr), (int)blockIdx.x, a, R);
}

__global__ __launch_bounds__(kGenNT) void k_gen_film(GenArgs a)
{
    extern __shared__ float S[];
    gen_film_body(make_ctx<4, kGenNT, kPlanF>(nullptr), (int)blockIdx.x, a, S);
}

template <int L, int AX>
__global__ __launch_bounds__(row_nt(L)) void k_gen_basis(GenArgs a)
{
    __shared__ float2 TWL[twl_size<L, kPlanF>()];
    __shared__ float2 T[L * row_lp(L)];
    gen_basis_body<L, AX>(make_ctx<L, row_nt(L), kPlanF>(TWL), (int)blockIdx.x, a, T);
}

template <bool MFMA>
__global__ __launch_bounds__(kGenNT) void k_gen_spectrum(GenArgs a)
{
    __shared__ __align__(16) float2 RC[kGenRows * kGenRC];
    __shared__ float2 X0[kGenRows], XS[kGenRows], XF[kGenRC];
    const auto ctx = make_ctx<4, kGenNT, kPlanF>(nullptr);
    if constexpr (MFMA) gen_spectrum_mfma_body(ctx, (int)blockIdx.x, a, RC, XF, X0, XS);
    else gen_spectrum_body(ctx, (int)blockIdx.x, a, RC, XF, X0, XS);
}

__global__ __launch_bounds__(kGenNT) void k_gen_btab(GenArgs a)
{
    gen_btab_body(make_ctx<4, kGenNT, kPlanF>(nullptr), (int)blockIdx.x, a);
}

template <int AX>
hipError_t basis_axis(const GenArgs& a, int L, hipStream_t st)
{
    if (L == 1) return hipSuccess;
    return with_length(L, [&]<int LL>() {
        const long long lines = (long long)a.C * kGenLines;
        hipLaunchKernelGGL((k_gen_basis<LL, AX>), dim3(ceil_div(lines, row_np(LL))), dim3(row_nt(LL)), 0, st, a);
        return last_error();
    });
}

// The passes before the per-pair spectra.
hipError_t launch_generate_prep(const GenArgs& a, hipStream_t st)
{
    const long long pairs = (long long)a.B * a.C;
    const unsigned sgrid = (unsigned)(pairs * a.splits);
    if (a.bf16) hipLaunchKernelGGL((k_gen_stats<true>), dim3(sgrid), dim3(kGenNT), 0, st, a);
    else hipLaunchKernelGGL((k_gen_stats<false>), dim3(sgrid), dim3(kGenNT), 0, st, a);
    hipError_t e = last_error();
    if (e != hipSuccess) return e;
    const size_t film_lds = sizeof(float) * ((size_t)a.C + (size_t)a.R * a.D + a.R + a.D + 2 * kGenHidden);
    hipLaunchKernelGGL(k_gen_film, dim3((unsigned)a.B), dim3(kGenNT), film_lds, st, a);
    if ((e = last_error()) != hipSuccess) return e;
    if ((e = basis_axis<0>(a, a.g.N_out, st)) != hipSuccess) return e;
    if ((e = basis_axis<1>(a, a.g.N_mid, st)) != hipSuccess) return e;
    if ((e = basis_axis<2>(a, a.g.N_in, st)) != hipSuccess) return e;
    if (a.g.S >= 16) {
        hipLaunchKernelGGL(k_gen_btab, dim3((unsigned)(a.C * (a.g.S / 16))), dim3(kGenNT), 0, st, a);
        e = last_error();
    }
    return e;
}

// The spectra of the channels [a.c0, a.c0 + a.nch) of every batch entry.
hipError_t launch_generate_pairs(const GenArgs& a, hipStream_t st)
{
    const long long rows = (long long)a.g.N_out * a.g.N_mid;
    const long long grid = (long long)a.B * a.nch * ((rows + kGenRows - 1) / kGenRows);
    if (grid == 0) return hipSuccess;
    // The matrix-core engine takes 16-slot tiles.
    if (a.g.S >= 16) hipLaunchKernelGGL((k_gen_spectrum<true>), dim3((unsigned)grid), dim3(kGenNT), 0, st, a);
    else hipLaunchKernelGGL((k_gen_spectrum<false>), dim3((unsigned)grid), dim3(kGenNT), 0, st, a);
    return last_error();
}

}  // namespace

hipError_t launch_generate_spectrum(const GenArgs& a, hipStream_t st)
{
    hipError_t e = launch_generate_prep(a, st);
    if (e != hipSuccess) return e;
    GenArgs all = a;
    all.c0 = 0;
    all.nch = a.C;
    return launch_generate_pairs(all, st);
}

}  // namespace hyenand
