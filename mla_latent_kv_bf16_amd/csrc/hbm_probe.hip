// Measured HBM read ceiling of the device: a plain streaming read with
// 16-byte loads, each byte of the buffer read once, folded into one word per
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

}  // namespace

extern "C" int mla_hbm_read_probe(const void* buf, size_t bytes, unsigned* sink, int grid,
                                  void* stream) {
    if (!buf || !sink || bytes == 0 || (bytes & 15) != 0 || ((uintptr_t)buf & 15) != 0)
        return 1;
    if (grid <= 0 || grid > (1 << 20)) return 1;
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const uint4*)buf, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}
