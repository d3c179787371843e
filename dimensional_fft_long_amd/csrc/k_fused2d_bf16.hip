// k_fused2d_bf16.hip -- the on-chip 2-D forward (fused2d.h), bf16 I/O.
#include "fused2d.h"
#include "kernels_dev.h"

namespace hyenand {
namespace {

template <int LO, int LI, bool BF16>
__global__ __launch_bounds__(f2_nt(LO, LI)) void k_fused2d(ConvArgs a)
{
    __shared__ float2 TWR[twl_size<LI, kPlanF>()];
    __shared__ float2 TWO[twl_size<LO, (kPlanF | kPlanR)>()];
    __shared__ float2 P[(LO / 2) * (LI / 2)];
    __shared__ float2 T[f2_tile(LO, LI)];
    fused2d_body<LO, LI, BF16>(make_ctx<LI, f2_nt(LO, LI), kPlanF>(TWR), make_ctx<LO, f2_nt(LO, LI), (kPlanF | kPlanR)>(TWO),
                               (int)blockIdx.x, a, P, T);
}

// Calls f.template operator()<L>() for a padded length L in {8, ..., kFused2dMaxLen}.
template <class F>
hipError_t with_fused_length(int L, F&& f)
{
    switch (L) {
    case 8: return f.template operator()<8>();
    case 16: return f.template operator()<16>();
    case 32: return f.template operator()<32>();
    case 64: return f.template operator()<64>();
    case 128: return f.template operator()<128>();
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t fused2d_forward_bf16(const ConvArgs& a, hipStream_t st, LaunchTrace* tr)
{
    const unsigned grid = (unsigned)((long long)a.B * a.C);
    return with_fused_length(a.g.N_out, [&]<int LO>() {
        return with_fused_length(a.g.N_in, [&]<int LI>() {
            if (tr) tr->mark(st);
            hipLaunchKernelGGL((k_fused2d<LO, LI, true>), dim3(grid), dim3(f2_nt(LO, LI)), 0, st, a);
            return hipGetLastError();
        });
    });
}

}  // namespace hyenand
