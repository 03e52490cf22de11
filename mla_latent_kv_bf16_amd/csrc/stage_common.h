// Pieces shared by the quantiser, the stage-1 kernels and the merge kernel.
#pragma once
#include <type_traits>

#include "device_common.h"

namespace mla {

// x / s in fp32, correctly rounded, for a per-tensor scale s with r = 1/s
// (itself an IEEE division). kFast: q0 = x r, then one correction with the
// exact residual q0 s - x (one FMA), which gives the IEEE quotient for every
// bf16 x and every scale in [2^-100, 2^100] (the reciprocal is a normal
// number there); the residual taken as q0 s - x keeps the sign of a zero
// quotient, and a quotient that overflows stays infinite. The identity is
// checked over all pairs of mantissas and over every bf16 value by a host
// test. Scales outside that range take the plain division (!kFast).
__device__ __forceinline__ bool fast_div_scale(float s) { return s >= 0x1p-100f && s <= 0x1p100f; }

template <bool kFast>
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
    if constexpr (!kFast) {
        return x / s;
    } else {
        const float q0 = __fmul_rn(x, r);
        const float q1 = __builtin_fmaf(__builtin_fmaf(q0, s, -x), -r, q0);
        return __builtin_isinf(q0) ? q0 : q1;
    }
}

// Clamp to +-448 so that the e4m3 conversion saturates; a NaN stays NaN (the
// pages' torch clamp propagates it; fminf/fmaxf alone would make it -448)
// and becomes the positive quiet NaN, which converts to the code 0x7F.
__device__ __forceinline__ float clamp_e4m3(float y) {
    const float c = fminf(fmaxf(y, -kE4m3Max), kE4m3Max);
    return __builtin_isnan(y) ? __builtin_nanf("") : c;
}

// The gfx950 conversion writes a NaN as 0xFF whatever its sign; the codes
// here follow torch's cast of the positive NaN an IEEE division returns,
// 0x7F. A finite value never converts to 0x7F or 0xFF (the clamp keeps it
// within +-448), so every byte whose low seven bits are all set is a NaN and
// loses its sign bit.
__device__ __forceinline__ uint32_t nan_codes_to_7f(uint32_t q) {
    const uint32_t nan = ((q & 0x7f7f7f7fu) + 0x01010101u) & 0x80808080u;
    return q & ~nan;
}

// Four bf16 -> four e4m3fn codes with the per-tensor scale: IEEE fp32
// division, clamp to +-448 (so the conversion saturates), round to nearest
// even [kernelindex.com amd-mixed-mla submission 722089 `quantize_fp8`].
template <bool kFast>
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d, float s, float r) {
    const float y0 = clamp_e4m3(div_by_scale<kFast>(a, s, r));
    const float y1 = clamp_e4m3(div_by_scale<kFast>(b, s, r));
    const float y2 = clamp_e4m3(div_by_scale<kFast>(c, s, r));
    const float y3 = clamp_e4m3(div_by_scale<kFast>(d, s, r));
    int q = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    q = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, q, true);
    return nan_codes_to_7f((uint32_t)q);
}

// Eight bf16 (one 16-byte vector) -> eight codes.
template <bool kFast>
__device__ __forceinline__ uint2 fp8x8(uint4 v, float s, float r) {
    uint2 q;
    q.x = fp8x4<kFast>(bf16_to_f32(v.x & 0xffffu), bf16_to_f32(v.x >> 16),
                       bf16_to_f32(v.y & 0xffffu), bf16_to_f32(v.y >> 16), s, r);
    q.y = fp8x4<kFast>(bf16_to_f32(v.z & 0xffffu), bf16_to_f32(v.z >> 16),
                       bf16_to_f32(v.w & 0xffffu), bf16_to_f32(v.w >> 16), s, r);
    return q;
}

// Runs f(kind) once with kind = std::true_type when the fast division holds
// for the (wave-uniform) scale s, else with std::false_type.
template <class F>
__device__ __forceinline__ void with_div_kind(float s, F&& f) {
    if (fast_div_scale(s))
        f(std::true_type{});
    else
        f(std::false_type{});
}

// The absmax scale from the partial maxima: fp32(max(amax, 1e-12)) / 448.
// A NaN amax gives a NaN scale, an infinite one an infinite scale.
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

__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v) {
    const v4u u = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                   __float_as_uint(v.w)};
    __builtin_amdgcn_raw_buffer_store_b128(u, r, (int)off, 0, kCoherentAux);
}
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)off, 0, kCoherentAux);
}

// Thread-to-data map of a 16 x 512 fp32 partial (2048 float4) for T
// threads: float4 f = t + T q (q < 2048 / T) holds head f / 128 and dims
// 4 (f % 128) .. +3, so consecutive lanes touch consecutive 16-byte pieces.
template <int T>
struct RowMap {
    static_assert(T % 128 == 0 && T <= 2048, "whole head rows per pass");
    static constexpr int kPer = 2048 / T;  // float4 per thread
    __device__ static int head(int t, int q) { return (t >> 7) + (T / 128) * q; }
    __device__ static int dim(int t) { return 4 * (t & 127); }
};

// Log-sum-exp merge of one sequence's ns partials (slots s0 ..), by all T
// threads of the workgroup:
//   M = max_s L_s, w_s = 2^(L_s - M), O = sum_s w_s O_s / sum_s w_s,
//   LSE = M + log2(sum_s w_s)
// [kernelindex.com amd-mixed-mla submission 722089 `_mla_reduce`], per head,
// with L_s the base-2 partial LSEs. ns = 0 (an empty sequence) gives O = 0
// and LSE = -inf; a NaN partial gives NaN. out points at the sequence's (16, 512) bf16 output,
// lse_out (nullable) at its 16 natural-log LSEs; lds is scratch for
// 16 ns + 32 floats. Starts and ends with a workgroup barrier's worth of
// LDS use, so the caller must not hold data in lds. kCoherent: read the
// partials with coherent buffer loads (written by other workgroups of the
// same launch).
template <int T, bool kCoherent>
__device__ __forceinline__ void merge_split(const float* __restrict__ part_o,
                                            const float* __restrict__ part_lse, int s0, int ns,
                                            uint16_t* __restrict__ out, float* __restrict__ lse_out,
                                            float* lds, int t) {
    using Map = RowMap<T>;
    constexpr int kOb = 4;  // splits whose rows are in flight together
    const float* po = part_o + (size_t)s0 * kHeads * kDv;
    const float* pl = part_lse + (size_t)s0 * kHeads;
    __amdgpu_buffer_rsrc_t ro, rl;
    if constexpr (kCoherent) {
        ro = make_rsrc(po, (uint32_t)ns * kHeads * kDv * 4u);
        rl = make_rsrc(pl, (uint32_t)ns * kHeads * 4u);
    }
    auto row_at = [&](int s, int q) -> float4 {
        const int off = (s * kHeads + Map::head(t, q)) * kDv + Map::dim(t);
        if constexpr (kCoherent) {
            const v4u u = __builtin_amdgcn_raw_buffer_load_b128(ro, off * 4, 0, kCoherentAux);
            return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                               __uint_as_float(u.w));
        } else {
            return *(const float4*)(po + off);
        }
    };
    auto lse_at = [&](int i) -> float {
        if constexpr (kCoherent)
            return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, i * 4, 0, kCoherentAux));
        else
            return pl[i];
    };
    float* wl = lds;                    // [ns][16]: L, then w = 2^(L - M)
    float* mh = lds + kHeads * ns;      // [16]: M per head
    float* iw = mh + kHeads;            // [16]: 1 / sum w per head (0 if none)
    // The first LSEs, then the first splits' rows, are requested before any
    // of them is waited for (loads complete in order).
    const float l0 = t < kHeads * ns ? lse_at(t) : 0.f;
    float4 v[kOb][Map::kPer];
#pragma unroll
    for (int j = 0; j < kOb; ++j)
#pragma unroll
        for (int q = 0; q < Map::kPer; ++q) v[j][q] = j < ns ? row_at(j, q) : float4{0, 0, 0, 0};
    if (t < kHeads * ns) wl[t] = l0;
    for (int i = t + T; i < kHeads * ns; i += T) wl[i] = lse_at(i);
    __syncthreads();
    if (t < kHeads) {
        float M = -INFINITY;
        for (int s = 0; s < ns; ++s) M = fmaxf(M, wl[s * kHeads + t]);
        float W = 0.f;
        for (int s = 0; s < ns; ++s) {
            const float l = wl[s * kHeads + t];
            W += (l == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(l - M);
        }
        // W is 0 only when every partial is empty; a NaN partial makes W NaN
        mh[t] = M;
        iw[t] = (W == 0.f) ? 0.f : 1.0f / W;
        if (lse_out) lse_out[t] = (W == 0.f) ? -INFINITY : (M + __log2f(W)) * kLn2;
    }
    __syncthreads();
    for (int i = t; i < kHeads * ns; i += T) {
        const float l = wl[i];
        wl[i] = (l == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(l - mh[i & (kHeads - 1)]);
    }
    __syncthreads();
    float4 o[Map::kPer];
#pragma unroll
    for (int q = 0; q < Map::kPer; ++q) o[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sb = 0; sb < ns; sb += kOb) {
        if (sb > 0) {
#pragma unroll
            for (int j = 0; j < kOb; ++j)
#pragma unroll
                for (int q = 0; q < Map::kPer; ++q)
                    v[j][q] = sb + j < ns ? row_at(sb + j, q) : float4{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < kOb; ++j) {
            if (sb + j < ns) {
#pragma unroll
                for (int q = 0; q < Map::kPer; ++q) {
                    const float wgt = wl[(sb + j) * kHeads + Map::head(t, q)];
                    o[q].x += wgt * v[j][q].x;
                    o[q].y += wgt * v[j][q].y;
                    o[q].z += wgt * v[j][q].z;
                    o[q].w += wgt * v[j][q].w;
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < Map::kPer; ++q) {
        const int hq = Map::head(t, q);
        const float inv = iw[hq];
        uint2 u;
        u.x = f32_to_bf16_rne(o[q].x * inv) | (f32_to_bf16_rne(o[q].y * inv) << 16);
        u.y = f32_to_bf16_rne(o[q].z * inv) | (f32_to_bf16_rne(o[q].w * inv) << 16);
        *(uint2*)(out + hq * kDv + Map::dim(t)) = u;
    }
}

// Rows of Q up to which the fused FP8 kernel reduces an absmax Q scale in
// every workgroup instead of after a separate partial-maximum launch.
constexpr int kQAbsmaxRows = 4;

// Kernel arguments of the stage-1 kernels (plain and fused forms).
struct Stage1Args {
    const int4* items;          // plain: 1 int4 per item; fused: 2 (see the plan)
    const uint8_t* q8_in;       // plain: Q codes (batch, 16, 576)
    const float* q_scale;       // Q scale: plain input; fused static input
    const uint8_t* kv;          // FP8 rows (576 B) or packed e2m1 rows (288 B)
    const uint8_t* kv_scales;   // MXFP4 e8m0 block scales (18 B per row)
    const float* kv_scale;      // FP8 per-tensor scale
    float sm_scale;
    float logit_cap;            // > 0: each scaled logit s becomes cap * tanh(s / cap)
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
    int q_absmax_rows;          // absmax mode with at most kQAbsmaxRows rows of Q: every
                                // workgroup reduces the absmax of all of Q itself
                                // (blockmax is then nullptr); 0 otherwise
    uint32_t* counters;         // per-sequence arrival counters (zero between runs)
    int kv_nt;                  // stream the cache tiles with non-temporal loads
                                // (selects the kernel instance; the shared-row
                                // kernel never does)
    // paged cache: kv (and kv_scales for MXFP4) hold num_pages << page_shift
    // rows of the cache's format, the items' row ranges are positions in
    // their sequence, and the sequence's pages are kv_pages[page_start ..)
    // (int32 page ids)
    const int32_t* kv_pages;
    int32_t page_shift;
    int32_t num_pages;
};

}  // namespace mla
