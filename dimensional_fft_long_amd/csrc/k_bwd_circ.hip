// k_bwd_circ.hip -- backward chains of the circular mode (d = 1, 2, 3).
#include "kernels_dev.h"

namespace hyenand {

hipError_t backward_chunk_circ(const ConvArgs& a, bool dk, hipStream_t st, LaunchTrace* tr)
{
    return backward_chunk<true>(a, dk, st, tr);
}

}  // namespace hyenand
