// Measured HBM read ceiling of the device: a streaming read with 16-byte
// loads (cached or non-temporal), each byte of the buffer read once, folded into one word per
// thread that is stored only if it equals a value that never occurs (so the
// loads cannot be removed). Its bandwidth is the practical ceiling the
// decode kernels are compared against beside the nominal 8 TB/s.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/mla_hbm_probe.h"

namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, size_t n16,
                                                          unsigned* __restrict__ sink) {
    unsigned acc = 0;
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

// The same read with non-temporal loads (the caches do not allocate the
// lines), the form the decode kernels use for large caches.
__global__ __launch_bounds__(256) void stream_read_nt_kernel(const uint4* __restrict__ p,
                                                             size_t n16,
                                                             unsigned* __restrict__ sink) {
    unsigned acc = 0;
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
        typedef unsigned v4u __attribute__((ext_vector_type(4)));
        const v4u v = __builtin_nontemporal_load((const v4u*)(p + i));
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

int launch_probe(bool nt, const void* buf, size_t bytes, unsigned* sink, int grid,
                 void* stream) {
    if (!buf || !sink || bytes == 0 || (bytes & 15) != 0 || ((uintptr_t)buf & 15) != 0)
        return 1;
    if (grid <= 0 || grid > (1 << 20)) return 1;
    if (nt)
        hipLaunchKernelGGL(stream_read_nt_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                           (const uint4*)buf, bytes / 16, sink);
    else
        hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                           (const uint4*)buf, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // namespace

extern "C" int mla_hbm_read_probe(const void* buf, size_t bytes, unsigned* sink, int grid,
                                  void* stream) {
    return launch_probe(false, buf, bytes, sink, grid, stream);
}

extern "C" int mla_hbm_read_probe_nt(const void* buf, size_t bytes, unsigned* sink, int grid,
                                     void* stream) {
    return launch_probe(true, buf, bytes, sink, grid, stream);
}
