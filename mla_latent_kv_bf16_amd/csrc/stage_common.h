// Pieces shared by the quantiser, the stage-1 kernels and the merge kernel.
#pragma once
#include "device_common.h"

namespace mla {

// Four bf16 -> four e4m3fn codes with the per-tensor scale: IEEE fp32
// division, clamp to +-448 (so the conversion saturates), round to nearest
// even [kernelindex.com amd-mixed-mla submission 722089 `quantize_fp8`].
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d, float scale) {
    const float y0 = fminf(fmaxf(a / scale, -kE4m3Max), kE4m3Max);
    const float y1 = fminf(fmaxf(b / scale, -kE4m3Max), kE4m3Max);
    const float y2 = fminf(fmaxf(c / scale, -kE4m3Max), kE4m3Max);
    const float y3 = fminf(fmaxf(d / scale, -kE4m3Max), kE4m3Max);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, r, true);
    return (uint32_t)r;
}

// Eight bf16 (one 16-byte vector) -> eight codes.
__device__ __forceinline__ uint2 fp8x8(uint4 v, float scale) {
    uint2 r;
    r.x = fp8x4(bf16_to_f32(v.x & 0xffffu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xffffu),
                bf16_to_f32(v.y >> 16), scale);
    r.y = fp8x4(bf16_to_f32(v.z & 0xffffu), bf16_to_f32(v.z >> 16), bf16_to_f32(v.w & 0xffffu),
                bf16_to_f32(v.w >> 16), scale);
    return r;
}

// The absmax scale from the partial maxima: fp32(max(amax, 1e-12)) / 448.
__device__ __forceinline__ float absmax_to_scale(float amax) {
    if (amax < 1e-12f) amax = 1e-12f;
    return amax / kE4m3Max;
}

// Store 32 floats as bf16 (round to nearest even), 64 bytes.
__device__ __forceinline__ void store_bf16x32(uint16_t* dst, const float* o) {
    uint4* d4 = (uint4*)dst;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint4 u;
        u.x = f32_to_bf16_rne(o[8 * j + 0]) | (f32_to_bf16_rne(o[8 * j + 1]) << 16);
        u.y = f32_to_bf16_rne(o[8 * j + 2]) | (f32_to_bf16_rne(o[8 * j + 3]) << 16);
        u.z = f32_to_bf16_rne(o[8 * j + 4]) | (f32_to_bf16_rne(o[8 * j + 5]) << 16);
        u.w = f32_to_bf16_rne(o[8 * j + 6]) | (f32_to_bf16_rne(o[8 * j + 7]) << 16);
        d4[j] = u;
    }
}

// Cache-policy bits of a buffer access on gfx950 (sc0 | sc1): a store writes
// through to the device-wide coherence point and a load bypasses the per-CU
// and per-XCD caches. The fused decode writes split partials this way and
// reads them back this way in another workgroup, possibly on another XCD,
// with no device-scope fence (which would write back and invalidate the
// whole L2 of the XCD for every workgroup).
constexpr int kCoherentAux = 1 | 16;
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v) {
    const v4u u = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                   __float_as_uint(v.w)};
    __builtin_amdgcn_raw_buffer_store_b128(u, r, (int)off, 0, kCoherentAux);
}
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)off, 0, kCoherentAux);
}

// Log-sum-exp merge of one sequence's ns partials (slots s0 ..) for head h
// and latent dims [d0, d0 + 32), written to out (bf16) and, by the caller's
// choice, the natural-log LSE:
//   M = max_s L_s, w_s = 2^(L_s - M), O = sum_s w_s O_s / sum_s w_s,
//   LSE = M + log2(sum_s w_s)
// [kernelindex.com amd-mixed-mla submission 722089 `_mla_reduce`]. ns = 0
// (an empty sequence) gives O = 0 and LSE = -inf. The loads are issued in
// independent batches (8 LSEs, then the rows of 4 splits) because the merge
// is latency-bound. kCoherent: read the partials with coherent buffer loads
// (they were written in the same launch by other workgroups).
template <bool kCoherent>
__device__ __forceinline__ float merge_rows(const float* __restrict__ part_o,
                                            const float* __restrict__ part_lse, int s0, int ns,
                                            int h, int d0, uint16_t* __restrict__ dst) {
    constexpr int kLb = 8, kOb = 4;
    const float* po = part_o + (size_t)s0 * kHeads * kDv;
    const float* pl = part_lse + (size_t)s0 * kHeads;
    __amdgpu_buffer_rsrc_t ro, rl;
    if constexpr (kCoherent) {
        ro = make_rsrc(po, (uint32_t)ns * kHeads * kDv * 4u);
        rl = make_rsrc(pl, (uint32_t)ns * kHeads * 4u);
    }
    auto lse_at = [&](int s) -> float {
        if constexpr (kCoherent)
            return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rl, (s * kHeads + h) * 4, 0, kCoherentAux));
        else
            return pl[(size_t)s * kHeads + h];
    };
    auto row_at = [&](int s, int q) -> float4 {
        if constexpr (kCoherent) {
            const v4u u = __builtin_amdgcn_raw_buffer_load_b128(
                ro, ((s * kHeads + h) * kDv + d0) * 4 + 16 * q, 0, kCoherentAux);
            return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                               __uint_as_float(u.w));
        } else {
            return ((const float4*)(po + ((size_t)s * kHeads + h) * kDv + d0))[q];
        }
    };
    float M = -INFINITY;
    for (int sb = 0; sb < ns; sb += kLb) {
        float l[kLb];
#pragma unroll
        for (int j = 0; j < kLb; ++j) l[j] = (sb + j < ns) ? lse_at(sb + j) : -INFINITY;
#pragma unroll
        for (int j = 0; j < kLb; ++j) M = fmaxf(M, l[j]);
    }
    float o[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) o[j] = 0.f;
    float W = 0.f;
    if (M != -INFINITY) {
        for (int sb = 0; sb < ns; sb += kOb) {
            float wgt[kOb];
            float4 v[kOb][8];
#pragma unroll
            for (int j = 0; j < kOb; ++j) {
                const bool ok = sb + j < ns;
                const int sl = ok ? sb + j : 0;
                const float ls = ok ? lse_at(sl) : -INFINITY;
                wgt[j] = (ls == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ls - M);
#pragma unroll
                for (int q = 0; q < 8; ++q) v[j][q] = row_at(sl, q);
            }
#pragma unroll
            for (int j = 0; j < kOb; ++j) {
                W += wgt[j];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    o[4 * q] += wgt[j] * v[j][q].x;
                    o[4 * q + 1] += wgt[j] * v[j][q].y;
                    o[4 * q + 2] += wgt[j] * v[j][q].z;
                    o[4 * q + 3] += wgt[j] * v[j][q].w;
                }
            }
        }
        const float inv = 1.0f / W;
#pragma unroll
        for (int j = 0; j < 32; ++j) o[j] *= inv;
    }
    store_bf16x32(dst, o);
    return (M == -INFINITY) ? -INFINITY : (M + __log2f(W)) * kLn2;
}

// Kernel arguments of the stage-1 kernels (plain and fused forms).
struct Stage1Args {
    const int4* items;          // plain: 1 int4 per item; fused: 2 (see the plan)
    const uint8_t* q8_in;       // plain: Q codes (batch, 16, 576)
    const float* q_scale;       // Q scale: plain input; fused static input
    const uint8_t* kv;          // FP8 rows (576 B) or packed e2m1 rows (288 B)
    const uint8_t* kv_scales;   // MXFP4 e8m0 block scales (18 B per row)
    const float* kv_scale;      // FP8 per-tensor scale
    float sm_scale;
    float* part_o;
    float* part_lse;
    uint16_t* out;
    float* lse_out;
    // fused form only
    const uint16_t* q_bf16;     // Q (batch, 16, 576) bf16
    uint8_t* q8_out;            // Q codes written by every item of the sequence
    float* q_scale_out;         // absmax mode: written by workgroup 0
    const float* blockmax;      // absmax mode: partial maxima, else nullptr
    int nblockmax;
    uint32_t* counters;         // per-sequence arrival counters (zero between runs)
};

}  // namespace mla
