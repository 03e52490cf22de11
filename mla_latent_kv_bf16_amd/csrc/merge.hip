// Stage 2 of the split-KV decode: log-sum-exp merge of the per-split
// partials into the bf16 output (gfx950).
//
// For a sequence split into S pieces with partial outputs O_s (each already
// divided by its own softmax sum) and base-2 log-sum-exps L_s:
//   M = max_s L_s,  w_s = 2^(L_s - M),  O = sum_s w_s O_s / sum_s w_s,
//   LSE = M + log2(sum_s w_s)
// [kernelindex.com amd-mixed-mla submission 722089 `_mla_reduce`].
// An empty sequence (S = 0) gets O = 0 and LSE = -inf, the pages' empty-split
// convention [722089 `_mla_multihead_stage1`].
//
// One workgroup per merged sequence (merge_split in stage_common.h).
#include "launch.h"
#include "plan.h"
#include "stage_common.h"

namespace mla {
namespace {

__global__ __launch_bounds__(256) void merge_kernel(const int4* __restrict__ merges,
                                                    const float* __restrict__ part_o,
                                                    const float* __restrict__ part_lse,
                                                    uint16_t* __restrict__ out,
                                                    float* __restrict__ lse_out) {
    __shared__ float lds[kHeads * kMaxSplitsPerSeq + 2 * kHeads];
    const int4 mg = merges[blockIdx.x];
    const int b = mg.x;
    merge_split<256, false>(part_o, part_lse, mg.y, mg.z, out + (size_t)b * kHeads * kDv,
                            lse_out ? lse_out + (size_t)b * kHeads : nullptr, lds, threadIdx.x);
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        p[i] = 0u;
}

}  // namespace

hipError_t launch_merge(const int4* merges, int nmerge, const float* part_o,
                        const float* part_lse, uint16_t* out, float* lse_out, hipStream_t stream) {
    if (nmerge <= 0) return hipSuccess;
    hipLaunchKernelGGL(merge_kernel, dim3(nmerge), dim3(256), 0, stream, merges, part_o, part_lse,
                       out, lse_out);
    return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

}  // namespace mla
