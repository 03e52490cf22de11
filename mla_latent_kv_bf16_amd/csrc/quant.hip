// Per-tensor FP8 E4M3FN quantiser and MXFP4 encoder (gfx950).
//
// FP8: scale = fp32(max(max|x|, 1e-12)) / 448 (absmax mode) or a caller
// scale (static mode); code = e4m3fn(rne(clamp(fp32(x) / scale, +-448)))
// [kernelindex.com amd-mixed-mla submission 722089 `quantize_fp8`,
// 738050 `_quantize_fp8`; the fixed scale of 663509, module docstring
// point 1]. The division is IEEE fp32 (HIP's default, correctly rounded),
// the clamp makes the hardware conversion saturate, and the conversion
// rounds to nearest even.
//
// Absmax takes two launches and no persistent state: the first writes one
// partial maximum per block, the second reduces those (at most 1024 values,
// redundantly in every block) before quantising.
//
// MXFP4 (OCP microscaling, 32-element blocks): shared exponent
// e = floor(log2(amax)) - 2 clamped to [-127, 127] (-127 for a zero block),
// element codes e2m1 nearest to x * 2^-e with ties to the even code,
// saturating at 6; element 2i in the low nibble of byte i. A block holding a
// NaN or an infinity gets the e8m0 NaN scale 0xFF and zero element bytes.
//
// Non-finite input propagates as NaN, as torch's amax in the pages'
// quantisers does: the absmax of a tensor holding a NaN is NaN (the partial
// maxima are compared as bit patterns, with NaN above +inf), of one holding
// an infinity +inf; a NaN quotient gives the code 0x7F
// [738050 `_dequantize_mxfp4_inplace` for layout and decode].
#include "launch.h"
#include "stage_common.h"

namespace mla {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t absbits_max2(uint32_t w, uint32_t m) {
    return max(max(m, w & 0x7fffu), (w >> 16) & 0x7fffu);
}

__global__ __launch_bounds__(kThreads) void absmax_partial_kernel(const uint16_t* __restrict__ x,
                                                                  size_t n,
                                                                  float* __restrict__ blockmax) {
    __shared__ uint32_t red[kThreads / 64];
    uint32_t m = 0;
    const size_t nvec = n / 8;
    const uint4* xv = (const uint4*)x;
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
        const uint4 v = xv[i];
        m = absbits_max2(v.x, m);
        m = absbits_max2(v.y, m);
        m = absbits_max2(v.z, m);
        m = absbits_max2(v.w, m);
    }
    for (size_t i = nvec * 8 + (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
        m = max(m, (uint32_t)(x[i] & 0x7fffu));
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = red[0];
        for (int i = 1; i < kThreads / 64; ++i) r = max(r, red[i]);
        blockmax[blockIdx.x] = __uint_as_float(r << 16);
    }
}

__global__ __launch_bounds__(kThreads) void quant_fp8_kernel(
    const uint16_t* __restrict__ x, size_t n, uint8_t* __restrict__ out,
    const float* __restrict__ scale_in, const float* __restrict__ blockmax, int nblockmax,
    float* __restrict__ scale_out) {
    __shared__ uint32_t red[kThreads / 64];
    float scale;
    if (blockmax) {
        // maxima compared as bit patterns, so that a NaN partial wins
        const uint32_t* bm = (const uint32_t*)blockmax;
        uint32_t m = 0;
        for (int i = threadIdx.x; i < nblockmax; i += kThreads) m = max(m, bm[i]);
        m = wave_max_u32(m);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
        __syncthreads();
        uint32_t amax = red[0];
        for (int i = 1; i < kThreads / 64; ++i) amax = max(amax, red[i]);
        scale = absmax_to_scale(__uint_as_float(amax));
        if (blockIdx.x == 0 && threadIdx.x == 0) scale_out[0] = scale;
    } else {
        scale = scale_in[0];
    }
    const size_t nvec = n / 8;
    const uint4* xv = (const uint4*)x;
    uint2* ov = (uint2*)out;
    const size_t stride = (size_t)gridDim.x * kThreads;
    scale = uniform_f32(scale);
    const float rcp = 1.0f / scale;
    with_div_kind(scale, [&](auto kind) {
        for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride)
            ov[i] = fp8x8<decltype(kind)::value>(xv[i], scale, rcp);
    });
    for (size_t i = nvec * 8 + (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
        const float y = clamp_e4m3(bf16_to_f32(x[i]) / scale);
        out[i] = (uint8_t)(nan_codes_to_7f(__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0, false)) &
                           0xffu);
    }
}

// e2m1 magnitude code of a >= 0, nearest with ties to the even code, saturating.
__device__ __forceinline__ uint32_t e2m1_code(float a) {
    return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
           (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
           (uint32_t)(a > 5.0f);
}

__global__ __launch_bounds__(kThreads) void mxfp4_encode_kernel(const uint16_t* __restrict__ x,
                                                                size_t nblocks,
                                                                uint8_t* __restrict__ packed,
                                                                uint8_t* __restrict__ scales) {
    const size_t blk = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (blk >= nblocks) return;
    const uint4* src = (const uint4*)(x + blk * 32);
    uint32_t wv[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 v = src[j];
        wv[4 * j] = v.x;
        wv[4 * j + 1] = v.y;
        wv[4 * j + 2] = v.z;
        wv[4 * j + 3] = v.w;
    }
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = absbits_max2(wv[j], amax);
    if (amax >= 0x7f80u) {
        // a NaN or an infinity: e8m0's NaN scale, zero element bytes
        ((uint4*)packed)[blk] = make_uint4(0u, 0u, 0u, 0u);
        scales[blk] = 0xff;
        return;
    }
    int e;
    if (amax == 0) {
        e = -127;
    } else {
        const int E = (int)(amax >> 7);
        const int fl = E ? (E - 127) : ((31 - __clz((int)(amax & 0x7fu))) - 133);
        e = fl - 2;
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
    }
    // 2^-e as an fp32 (a normal number unless e = 127)
    const float inv = (e <= 126) ? __uint_as_float((uint32_t)(127 - e) << 23) : __uint_as_float(0x00400000u);
    uint32_t outw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t pair = wv[4 * j + q];
            const uint32_t h0 = pair & 0xffffu, h1 = pair >> 16;
            const uint32_t c0 = e2m1_code(fabsf(bf16_to_f32(h0)) * inv) | ((h0 >> 15) << 3);
            const uint32_t c1 = e2m1_code(fabsf(bf16_to_f32(h1)) * inv) | ((h1 >> 15) << 3);
            word |= (c0 | (c1 << 4)) << (8 * q);
        }
        outw[j] = word;
    }
    ((uint4*)packed)[blk] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    scales[blk] = (uint8_t)(e + 127);
}

}  // namespace

int absmax_blocks(size_t n) {
    size_t nvec = (n + 7) / 8;
    size_t b = (nvec + kThreads - 1) / kThreads;
    if (b < 1) b = 1;
    if (b > (size_t)kMaxAbsmaxBlocks) b = kMaxAbsmaxBlocks;
    return (int)b;
}

hipError_t launch_absmax_partial(const uint16_t* x, size_t n, float* blockmax, int nblocks,
                                 hipStream_t stream) {
    hipLaunchKernelGGL(absmax_partial_kernel, dim3(nblocks), dim3(kThreads), 0, stream, x, n,
                       blockmax);
    return hipGetLastError();
}

hipError_t launch_quant_fp8(const uint16_t* x, size_t n, uint8_t* out, const float* scale_in,
                            const float* blockmax, int nblockmax, float* scale_out,
                            hipStream_t stream) {
    size_t nvec = (n + 7) / 8;
    size_t grid = (nvec + kThreads - 1) / kThreads;
    if (grid < 1) grid = 1;
    if (grid > 8192) grid = 8192;
    hipLaunchKernelGGL(quant_fp8_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, x, n,
                       out, scale_in, blockmax, nblockmax, scale_out);
    return hipGetLastError();
}

hipError_t launch_mxfp4_encode(const uint16_t* x, size_t rows, uint8_t* packed, uint8_t* scales,
                               hipStream_t stream) {
    const size_t nblocks = rows * (kDqk / 32);
    if (nblocks == 0) return hipSuccess;
    const size_t grid = (nblocks + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(mxfp4_encode_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, x,
                       nblocks, packed, scales);
    return hipGetLastError();
}

}  // namespace mla
