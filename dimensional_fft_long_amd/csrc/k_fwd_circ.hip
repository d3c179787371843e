// k_fwd_circ.hip -- forward chains of the circular mode (d = 1, 2, 3).
#include "kernels_dev.h"

namespace hyenand {

hipError_t forward_chunk_circ(const ConvArgs& a, hipStream_t st, LaunchTrace* tr)
{
    return forward_chunk<true>(a, st, tr);
}

}  // namespace hyenand
