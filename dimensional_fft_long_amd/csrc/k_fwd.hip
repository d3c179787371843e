// k_fwd.hip -- forward chains of the zero-padded convolution (d = 1, 2, 3),
// the dispatch of every forward call, and the occupancy query shared by the
// looping kernels.
#include <mutex>

#include "kernels_dev.h"

namespace hyenand {

hipError_t forward_chunk_padded(const ConvArgs& a, hipStream_t st, LaunchTrace* tr)
{
    return forward_chunk<false>(a, st, tr);
}

hipError_t launch_forward_chunk(const ConvArgs& a, hipStream_t st, LaunchTrace* tr)
{
    if (a.g.lng) return long1d_forward(a, false, st, tr);
    if (fused2d_fits(a.g)) return a.bf16 ? fused2d_forward_bf16(a, st, tr) : fused2d_forward_f32(a, st, tr);
    return a.g.circ ? forward_chunk_circ(a, st, tr) : forward_chunk_padded(a, st, tr);
}

hipError_t launch_zero(float* p, long long n, hipStream_t st)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_zero, dim3(ceil_div(n, 256)), dim3(256), 0, st, p, n);
    return last_error();
}

unsigned resident_wgs(const void* kernel, int nt)
{
    struct Entry {
        const void* k;
        int nt, dev;
        unsigned n;
    };
    static std::mutex mu;
    static Entry cache[64];
    static int used = 0;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    {
        std::lock_guard<std::mutex> lk(mu);
        for (int i = 0; i < used; ++i)
            if (cache[i].k == kernel && cache[i].nt == nt && cache[i].dev == dev) return cache[i].n;
    }
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, nt, 0) != hipSuccess) return 0;
    const unsigned n = (unsigned)(cus > 0 ? cus : 0) * (unsigned)(per_cu > 0 ? per_cu : 0);
    std::lock_guard<std::mutex> lk(mu);
    if (used < 64) cache[used++] = Entry{kernel, nt, dev, n};
    return n;
}

}  // namespace hyenand
