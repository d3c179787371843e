// k_long.hip -- the four-step chains of long 1-D signals (forward, spectrum,
// backward).
#include "kernels_dev.h"

namespace hyenand {

hipError_t long1d_forward(const ConvArgs& a, bool spec, hipStream_t st, LaunchTrace* tr)
{
    return long1d_chunk(a, spec, st, tr);
}

hipError_t long1d_backward(const ConvArgs& a, bool dk, hipStream_t st, LaunchTrace* tr)
{
    return long1d_bwd_chunk(a, dk, st, tr);
}

}  // namespace hyenand
