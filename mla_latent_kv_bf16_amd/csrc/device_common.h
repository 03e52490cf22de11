// Device-side helpers shared by the gfx950 kernels of libmla_decode.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kHeads = 16;
constexpr int kDqk = 576;            // latent dims used by QK^T
constexpr int kDv = 512;             // latent dims used as V
constexpr int kRowChunks = kDqk / 16;  // 36 sixteen-byte chunks per FP8 row
constexpr float kE4m3Max = 448.0f;
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

// bf16 <-> fp32
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t q = ((u >> 16) | 0x40u) & 0xffffu;  // NaN stays a (quiet) NaN
    return ((u & 0x7fffffffu) > 0x7f800000u) ? q : r;
}

// Two floats -> two bf16 (round to nearest even) packed low-first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Raw buffer descriptor over [base, base + bytes): loads at offsets past the
// end return zeros instead of touching memory. Word 3 is the gfx9-family
// raw-buffer format (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// One wave-wide 16-byte-per-lane copy from a buffer into LDS: lane i's 16
// bytes from byte offset `voff` of the buffer land at LDS address
// lds_base + 16*i. lds_base must be wave-uniform. The copy is asynchronous:
// it counts against vmcnt, and the caller waits with wait_vmcnt() before
// reading the LDS it fills. Issued as inline assembly so that the compiler
// does not insert a full vmcnt drain in front of every later LDS read.
// Before refilling LDS that this wave has read, drain those reads with
// wait_lgkm0() so that the copy cannot overtake a pending read.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, uint32_t lds_base,
                                          uint32_t voff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(lds_base), "v"(voff), "s"(rs)
        : "memory", "m0");
}
// The same copy with the non-temporal hint, for cache tiles that are read
// once per step: a large cache streamed with it keeps the last-level cache
// from allocating lines that are never re-read, which measured faster for
// caches well beyond that cache's 256 MB; smaller caches gain from staying
// resident between steps, so the hint is chosen per plan (lds_dma16_kv).
__device__ __forceinline__ void lds_dma16_nt(__amdgpu_buffer_rsrc_t rs, uint32_t lds_base,
                                             uint32_t voff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen nt lds"
        :
        : "s"(lds_base), "v"(voff), "s"(rs)
        : "memory", "m0");
}
// A 16-byte buffer load into registers, issued as inline assembly like the
// LDS copies, so the compiler neither tracks nor waits for it: the caller
// waits with wait_vmcnt_regs(), which names the destination registers so
// that nothing reads them before the wait. Offsets past the descriptor's
// range read as zeros.
__device__ __forceinline__ v4u load16_async(__amdgpu_buffer_rsrc_t rs, uint32_t voff) {
    v4u v;
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(voff), "s"(rs) : "memory");
    return v;
}
#pragma clang diagnostic pop

// A cache-tile copy, non-temporal in the kernels instantiated with kNt.
template <bool kNt>
__device__ __forceinline__ void lds_dma16_kv(__amdgpu_buffer_rsrc_t rs, uint32_t lds_base,
                                             uint32_t voff) {
    if constexpr (kNt)
        lds_dma16_nt(rs, lds_base, voff);
    else
        lds_dma16(rs, lds_base, voff);
}

__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Scalar load of 8 consecutive page ids at byte offset `off` of the page
// table descriptor `r` (past its range: zeros); waits for it (and for any
// pending LDS access of the wave).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ v8i load_pages8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    v8i v;
    asm volatile("s_buffer_load_dwordx8 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)"
                 : "=&s"(v)
                 : "s"(r), "s"(off)
                 : "memory");
    return v;
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most N vector-memory operations of this wave are in flight,
// then hand the K registers filled by load16_async() on to their users.
template <int N, int K>
__device__ __forceinline__ void wait_vmcnt_regs(v4u (&r)[K]) {
    wait_vmcnt<N>();
#pragma unroll
    for (int j = 0; j < K; ++j) asm volatile("" : "+v"(r[j]));
}

// max / sum over the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48), with the gfx950 lane-swap instructions instead of LDS permutes
__device__ __forceinline__ float group4_max(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float group4_sum(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// The largest of non-negative floats (or NaN with a clear sign bit) compared
// as bit patterns: for such values the integer order is the numeric order,
// with a NaN above +inf, so a NaN anywhere wins (as torch's amax, used by the
// pages' quantisers, propagates it) where fmaxf would drop it.
__device__ __forceinline__ uint32_t group4_max_u32(uint32_t u) {
    auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    u = max((uint32_t)r[0], (uint32_t)r[1]);
    auto q = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return max((uint32_t)q[0], (uint32_t)q[1]);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t u) {
    u = group4_max_u32(u);
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) u = max(u, (uint32_t)__shfl_xor((int)u, o));
    return u;
}

// Soft-capped base-2 logit of a scaled score s (cap > 0): cap * tanh(s / cap)
// * log2(e), with tanh(y) = 1 - 2 / (e^(2y) + 1) (saturates to +-1)
// [the `logit_cap` argument of the pages' decode calls; 0 on every page].
__device__ __forceinline__ float capped(float s, float cap, float inv_cap) {
    const float e = __builtin_amdgcn_exp2f(2.0f * kLog2e * s * inv_cap);
    const float th = 1.0f - 2.0f / (e + 1.0f);
    return cap * th * kLog2e;
}

// A value that every lane of the wave holds, moved to a scalar register so
// that branches on it are scalar.
__device__ __forceinline__ float uniform_f32(float x) {
    return __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)__float_as_uint(x)));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)p;
}

// Byte permute: byte k of the result is byte sel_k of the 8-byte value
// {hi = a, lo = b} (selectors 0-3 pick b, 4-7 pick a).
__device__ __forceinline__ uint32_t perm(uint32_t a, uint32_t b, uint32_t sel) {
    return __builtin_amdgcn_perm(a, b, sel);
}

// 4x4 byte transpose: x_r holds bytes (r,0..3); y_c receives bytes (0..3,c).
__device__ __forceinline__ void transpose4x4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                             uint32_t& y0, uint32_t& y1, uint32_t& y2,
                                             uint32_t& y3) {
    uint32_t a_lo = perm(x1, x0, 0x05010400u);  // x0.0 x1.0 x0.1 x1.1
    uint32_t a_hi = perm(x1, x0, 0x07030602u);  // x0.2 x1.2 x0.3 x1.3
    uint32_t b_lo = perm(x3, x2, 0x05010400u);  // x2.0 x3.0 x2.1 x3.1
    uint32_t b_hi = perm(x3, x2, 0x07030602u);  // x2.2 x3.2 x2.3 x3.3
    y0 = perm(b_lo, a_lo, 0x05040100u);
    y1 = perm(b_lo, a_lo, 0x07060302u);
    y2 = perm(b_hi, a_hi, 0x05040100u);
    y3 = perm(b_hi, a_hi, 0x07060302u);
}

}  // namespace mla
