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

// The same read through buffer->LDS copies with the non-temporal hint, the
// form the decode kernels stream a large cache in: each workgroup takes
// 1 MiB chunks in turn, its 4 waves issue 1 KiB copies (16 B per lane) into
// their own 16 KiB of LDS, 16 in flight per wave, and wait for them. The copies
// cannot be removed (they are asm volatile); a chunk's tail past `bytes`
// lies outside the chunk's buffer descriptor and reads nothing.
constexpr uint32_t kChunk = 1u << 20;

__global__ __launch_bounds__(256) void stream_read_lds_nt_kernel(const uint8_t* __restrict__ p,
                                                                 size_t bytes) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[64 * 1024];
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t w = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const uint32_t lds = (uint32_t)(uintptr_t)smem + w * 16384u;  // LDS offset of this wave's slots
    const size_t nchunk = (bytes + kChunk - 1) / kChunk;
    for (size_t c = blockIdx.x; c < nchunk; c += gridDim.x) {
        const size_t left = bytes - c * kChunk;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(p + c * kChunk), (short)0,
            (int)(left < kChunk ? left : kChunk), 0x00020000);
        for (uint32_t i = 0; i < 256; i += 16) {
#pragma unroll
            for (uint32_t j = 0; j < 16; ++j) {
                const uint32_t voff = ((i + j) * 4u + w) * 1024u + 16u * lane;
                asm volatile(
                    "s_mov_b32 m0, %0\n\t"
                    "buffer_load_dwordx4 %1, %2, 0 offen nt lds"
                    :
                    : "s"(lds + j * 1024u), "v"(voff), "s"(rs)
                    : "memory", "m0");
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
    }
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

extern "C" int mla_hbm_read_probe_lds_nt(const void* buf, size_t bytes, int grid, void* stream) {
    if (!buf || bytes == 0 || (bytes & 15) != 0 || ((uintptr_t)buf & 15) != 0) return 1;
    if (grid <= 0 || grid > (1 << 20)) return 1;
    hipLaunchKernelGGL(stream_read_lds_nt_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const uint8_t*)buf, bytes);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

extern "C" int mla_hbm_read_probe_nt(const void* buf, size_t bytes, unsigned* sink, int grid,
                                     void* stream) {
    return launch_probe(true, buf, bytes, sink, grid, stream);
}
