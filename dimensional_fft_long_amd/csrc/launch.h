// launch.h -- host-side launchers of the convolution and spectrum kernels.
// Each launcher validates nothing (the C ABI does) and returns hipSuccess or
// the launch error.
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

namespace hyenand {

// Optional event trace: event ev[count] is recorded on the stream before each
// kernel launch (and once more at the end of a call) while count < n.
struct LaunchTrace {
    hipEvent_t* ev;
    int n;
    int count;
    __host__ void mark(hipStream_t st)
    {
        if (count < n) (void)hipEventRecord(ev[count], st);
        ++count;
    }
};

// Gate + forward transforms + product + inverse transforms for the channels
// [a.c0, a.c0 + a.nch) of every batch entry.
hipError_t launch_forward_chunk(const ConvArgs& a, hipStream_t stream, LaunchTrace* trace = nullptr);

// Backward for the channels [a.c0, a.c0 + a.nch): dx (into a.y), dalpha,
// dbeta and, with dk, the kernel gradient a.dK, using the chunk workspace
// a.ws (output-gradient planes), a.ws_u, a.dkw (with dk) and a.part.
hipError_t launch_backward_chunk(const ConvArgs& a, bool dk, hipStream_t stream, LaunchTrace* trace = nullptr);

// Zero fill of n floats.
hipError_t launch_zero(float* p, long long n, hipStream_t stream);

// Kernel spectrum of all channels into a.khat (in place, no workspace).
hipError_t launch_spectrum(const ConvArgs& a, hipStream_t stream);

// The chains of each kernel translation unit (k_*.hip), called by the
// dispatchers above.
hipError_t forward_chunk_padded(const ConvArgs& a, hipStream_t stream, LaunchTrace* trace);
hipError_t forward_chunk_circ(const ConvArgs& a, hipStream_t stream, LaunchTrace* trace);
hipError_t backward_chunk_padded(const ConvArgs& a, bool dk, hipStream_t stream, LaunchTrace* trace);
hipError_t backward_chunk_circ(const ConvArgs& a, bool dk, hipStream_t stream, LaunchTrace* trace);
hipError_t long1d_forward(const ConvArgs& a, bool spec, hipStream_t stream, LaunchTrace* trace);
hipError_t long1d_backward(const ConvArgs& a, bool dk, hipStream_t stream, LaunchTrace* trace);
// The on-chip 2-D forward (fused2d_fits) of every pair, fp32 / bf16 I/O.
hipError_t fused2d_forward_f32(const ConvArgs& a, hipStream_t stream, LaunchTrace* trace);
hipError_t fused2d_forward_bf16(const ConvArgs& a, hipStream_t stream, LaunchTrace* trace);

// The input-dependent kernels' spectra (gen.h): means, control / FiLM, axis
// spectra, per-pair spectra into a.khat.
struct GenArgs;
hipError_t launch_generate_spectrum(const GenArgs& a, hipStream_t stream);

// Workgroups of `kernel` (nt threads per workgroup) resident at once on the
// current device: CUs x workgroups per CU, queried once per (kernel, nt,
// device) and cached.  0 if the query fails.
unsigned resident_wgs(const void* kernel, int nt);

}  // namespace hyenand
