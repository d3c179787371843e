// k_bwd.hip -- backward chains of the zero-padded convolution (d = 1, 2, 3)
// and the dispatch of every backward call.
#include "kernels_dev.h"

namespace hyenand {

hipError_t backward_chunk_padded(const ConvArgs& a, bool dk, hipStream_t st, LaunchTrace* tr)
{
    return backward_chunk<false>(a, dk, st, tr);
}

hipError_t launch_backward_chunk(const ConvArgs& a, bool dk, hipStream_t st, LaunchTrace* tr)
{
    if (a.g.lng) return long1d_backward(a, dk, st, tr);
    return a.g.circ ? backward_chunk_circ(a, dk, st, tr) : backward_chunk_padded(a, dk, st, tr);
}

}  // namespace hyenand
