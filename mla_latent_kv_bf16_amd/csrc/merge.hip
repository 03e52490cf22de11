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
// One workgroup per merged sequence; thread t owns head t/16 and 32
// consecutive latent dims, read and written as 16-byte vectors.
#include "device_common.h"
#include "launch.h"

namespace mla {
namespace {

__global__ __launch_bounds__(256) void merge_kernel(const int4* __restrict__ merges,
                                                    const float* __restrict__ part_o,
                                                    const float* __restrict__ part_lse,
                                                    uint16_t* __restrict__ out,
                                                    float* __restrict__ lse_out) {
    const int4 mg = merges[blockIdx.x];
    const int b = mg.x, s0 = mg.y, ns = mg.z;
    const int h = threadIdx.x >> 4;
    const int d0 = (threadIdx.x & 15) * 32;

    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, part_lse[(size_t)(s0 + s) * kHeads + h]);
    float o[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) o[j] = 0.f;
    float W = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < ns; ++s) {
            const float ls = part_lse[(size_t)(s0 + s) * kHeads + h];
            const float wgt = (ls == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ls - M);
            W += wgt;
            const float4* src = (const float4*)(part_o + ((size_t)(s0 + s) * kHeads + h) * kDv + d0);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float4 v = src[j];
                o[4 * j] += wgt * v.x;
                o[4 * j + 1] += wgt * v.y;
                o[4 * j + 2] += wgt * v.z;
                o[4 * j + 3] += wgt * v.w;
            }
        }
        const float inv = 1.0f / W;
#pragma unroll
        for (int j = 0; j < 32; ++j) o[j] *= inv;
    }
    uint4* dst = (uint4*)(out + ((size_t)b * kHeads + h) * kDv + d0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint4 u;
        u.x = f32_to_bf16_rne(o[8 * j + 0]) | (f32_to_bf16_rne(o[8 * j + 1]) << 16);
        u.y = f32_to_bf16_rne(o[8 * j + 2]) | (f32_to_bf16_rne(o[8 * j + 3]) << 16);
        u.z = f32_to_bf16_rne(o[8 * j + 4]) | (f32_to_bf16_rne(o[8 * j + 5]) << 16);
        u.w = f32_to_bf16_rne(o[8 * j + 6]) | (f32_to_bf16_rne(o[8 * j + 7]) << 16);
        dst[j] = u;
    }
    if (lse_out && (threadIdx.x & 15) == 0)
        lse_out[(size_t)b * kHeads + h] = (M == -INFINITY) ? -INFINITY : (M + __log2f(W)) * kLn2;
}

}  // namespace

hipError_t launch_merge(const int4* merges, int nmerge, const float* part_o,
                        const float* part_lse, uint16_t* out, float* lse_out, hipStream_t stream) {
    if (nmerge <= 0) return hipSuccess;
    hipLaunchKernelGGL(merge_kernel, dim3(nmerge), dim3(256), 0, stream, merges, part_o, part_lse,
                       out, lse_out);
    return hipGetLastError();
}

}  // namespace mla
