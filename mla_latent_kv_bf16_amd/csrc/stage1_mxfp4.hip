// Stage 1 of the split-KV decode for an MXFP4 latent cache (gfx950).
//
// Same organisation as the FP8 kernel (one workgroup per work item, four
// waves streaming disjoint 32-token tiles through private LDS rings, all 16
// heads per tile, online softmax in base 2, LDS merge of the waves), with the
// cache format of kernelindex.com amd-mixed-mla submission 738050
// (`_dequantize_mxfp4_inplace`): per token 288 bytes of e2m1 pairs (element
// 2i in the low nibble of byte i) and 18 e8m0 scales, one per 32 latent dims.
//
//   - QK^T: S^T = K Q^T on the MX-scaled 16x16x128 MFMA with K as the fp4 A
//     operand (lane group g carries latent dims 32g..32g+31 of its K step,
//     low nibble first) and its per-token e8m0 block scales as the A scales,
//     and Q as the fp8 B operand at unit scale. For fp8 operands of this
//     instruction lane group g carries dims 16g..16g+15 and 64+16g..64+16g+15
//     of the K step, so Q is loaded in that split order. (Both layouts were
//     measured on the GPU; FP4 x FP8 scaled products follow 722089
//     `_mla_multihead_stage1`, which uses `dot_scaled` e4m3 x e2m1.)
//   - P.V: V's block scales vary per token, i.e. along P.V's reduction axis,
//     so they cannot ride on the MFMA. V is decoded to bf16 in registers
//     (`v_cvt_scalef32_pk_bf16_fp4`, exact for every e8m0 exponent), byte-pair
//     transposed, and multiplied with bf16 P on the 16x16x32 bf16 MFMA.
//   - Four LDS stages per wave (the rows are 306 B, so the ring fits), each
//     9,216 B of packed rows plus the tile's 576 scale bytes read through a
//     16-byte aligned window.
#include "device_common.h"
#include "launch.h"

namespace mla {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kTok = 32;
constexpr int kNst = 4;                              // LDS stages per wave
constexpr int kRowPacked = kDqk / 2;                 // 288
constexpr int kRowScales = kDqk / 32;                // 18
constexpr int kPackedChunks = kRowPacked / 16;       // 18
constexpr int kPackedBytes = kTok * kRowPacked;      // 9216
constexpr int kScaleWindow = 37 * 16;                // 576 scale bytes + up to 15 of alignment
constexpr int kStageBytes = kPackedBytes + kScaleWindow;  // 9808
constexpr int kDmaPerStage = kPackedBytes / 1024 + 1;     // 9 packed + 1 scales
constexpr int kRingBytes = kWaves * kNst * kStageBytes;
constexpr int kXoStride = kDv + 4;
static_assert(kRingBytes <= 160 * 1024, "LDS budget");
static_assert(kWaves * kHeads * kXoStride * 4 + 2 * kWaves * kHeads * 4 <= kRingBytes,
              "merge buffers must fit in the ring");

// packed chunk c of row t sits at c ^ fx(t) within its aligned pair
__device__ __forceinline__ int fx(int t) { return (t >> 2) & 1; }
__device__ __forceinline__ int pchunk_off(int t, int c) {
    return (t * kPackedChunks + (c ^ fx(t))) * 16;
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
    return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

__device__ __forceinline__ v8i cat8(uint4 a, uint4 b) {
    v8i r;
    r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
    r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
    return r;
}

__device__ __forceinline__ uint32_t bf2_bits(v2bf v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ v8bf as_v8bf(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    uint4 u = make_uint4(a, b, c, d);
    return __builtin_bit_cast(v8bf, u);
}

__device__ __forceinline__ void wait_stages(int n) {
    // wait until at most n later stages (kDmaPerStage copies each) are pending
    if (n >= 3) wait_vmcnt<3 * kDmaPerStage>();
    else if (n == 2) wait_vmcnt<2 * kDmaPerStage>();
    else if (n == 1) wait_vmcnt<kDmaPerStage>();
    else wait_vmcnt<0>();
}

__global__ __launch_bounds__(256) void stage1_mxfp4_kernel(
    const int4* __restrict__ items, const uint8_t* __restrict__ q8,
    const float* __restrict__ q_scale, const uint8_t* __restrict__ kv_packed,
    const uint8_t* __restrict__ kv_scales, float sm_scale, float* __restrict__ part_o,
    float* __restrict__ part_lse, uint16_t* __restrict__ out, float* __restrict__ lse_out) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kRingBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15;
    const int g = lane >> 4;

    const int4 it = items[blockIdx.x];
    const int b = it.x, kb = it.y, ke = it.z, slot = it.w;
    const int ntok = ke - kb;
    const int ntile = (ntok + kTok - 1) / kTok;
    const int nt_w = ntile > w ? (ntile - w + kWaves - 1) / kWaves : 0;

    const float c = q_scale[0] * sm_scale * kLog2e;

    // Q as the fp8 B operand in the instruction's split order: bytes 0..15
    // are dims 128ks + 16g + (0..15), bytes 16..31 are 128ks + 64 + 16g + (0..15).
    // The 64-dim tail holds dims 512 + 16g + (0..15) and zeros above.
    v8i qb[5];
    {
        const uint8_t* qrow = q8 + ((size_t)b * kHeads + n16) * kDqk;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint4 lo = *(const uint4*)(qrow + 128 * ks + 16 * g);
            const uint4 hi = *(const uint4*)(qrow + 128 * ks + 64 + 16 * g);
            qb[ks] = cat8(lo, hi);
        }
        const uint4 lo = *(const uint4*)(qrow + 512 + 16 * g);
        qb[4] = cat8(lo, make_uint4(0u, 0u, 0u, 0u));
    }

    // DMA source offsets of the 9 packed copies of one stage.
    uint32_t dma_off[kDmaPerStage - 1];
#pragma unroll
    for (int i = 0; i < kDmaPerStage - 1; ++i) {
        const int s = i * 64 + lane;
        const int t = s / kPackedChunks;
        const int cp = s - t * kPackedChunks;
        dma_off[i] = (uint32_t)(t * kRowPacked + ((cp ^ fx(t)) * 16));
    }

    const uint32_t ring = lds_addr(smem) + (uint32_t)(w * kNst * kStageBytes);
    const uint8_t* item_p = kv_packed + (size_t)kb * kRowPacked;
    const uint32_t item_pbytes = (uint32_t)ntok * kRowPacked;
    // The buffer range check works per dword, so the window ends at the dword
    // holding the item's last scale byte (18 * rows is only even). That
    // dword lies in the same page as the byte, so the read is always mapped;
    // bytes past the item are never used for a valid token.
    const uintptr_t scales_end =
        ((uintptr_t)(kv_scales + (size_t)ke * kRowScales) + 3) & ~(uintptr_t)3;

    // scale-window misalignment of my k-th tile (tile start & 15)
    auto scale_delta = [&](int k) -> int {
        const uintptr_t a = (uintptr_t)(kv_scales + ((size_t)kb + (size_t)(w + kWaves * k) * kTok) *
                                                        kRowScales);
        return (int)(a & 15u);
    };

    auto issue = [&](int k, int s) {
        const int tile = w + kWaves * k;
        const uint32_t toff = (uint32_t)tile * kPackedBytes;
        const __amdgpu_buffer_rsrc_t rp = make_rsrc(item_p + toff, item_pbytes - toff);
        const uint32_t dst = ring + (uint32_t)(s * kStageBytes);
#pragma unroll
        for (int i = 0; i < kDmaPerStage - 1; ++i) lds_dma16(rp, dst + 1024u * i, dma_off[i]);
        // the tile's scale rows, from the 16-byte boundary at or below their start
        const uintptr_t a = (uintptr_t)(kv_scales + ((size_t)kb + (size_t)tile * kTok) * kRowScales);
        const uintptr_t a0 = a & ~(uintptr_t)15;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc((const void*)a0, (uint32_t)(scales_end - a0));
        if (lane < kScaleWindow / 16) lds_dma16(rs, dst + kPackedBytes, 16u * lane);
    };

    const int npre = nt_w < kNst ? nt_w : kNst;
    for (int k = 0; k < npre; ++k) issue(k, k);

    float m_run = -INFINITY, l_run = 0.0f;
    v4f acc[4][8];
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
#pragma unroll
        for (int c8 = 0; c8 < 8; ++c8) acc[ch][c8] = (v4f){0.f, 0.f, 0.f, 0.f};

    for (int k = 0; k < nt_w; ++k) {
        const int s = k % kNst;
        const int later = nt_w - 1 - k;
        wait_stages(later < kNst - 1 ? later : kNst - 1);
        const uint8_t* st = smem + (w * kNst + s) * kStageBytes;
        const uint8_t* ssc = st + kPackedBytes + scale_delta(k);  // row t's scales at ssc + 18 t
        const int tok0 = (w + kWaves * k) * kTok;

        // ---- S^T = K Q^T (fp4 x fp8, K block scales per token)
        v4f sc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int t = 16 * mb + n16;
            v4f a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const uint4 kd = *(const uint4*)(st + pchunk_off(t, 4 * ks + g));
                const int sa = ssc[t * kRowScales + 4 * ks + g];
                a4 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    cat8(kd, make_uint4(0u, 0u, 0u, 0u)), qb[ks], a4, 4, 0, 0, sa, 0, 127);
            }
            const int gt = g & 1;
            const uint4 kd = *(const uint4*)(st + pchunk_off(t, 16 + gt));
            const int sa = ssc[t * kRowScales + 16 + gt];
            const uint4 z = make_uint4(0u, 0u, 0u, 0u);
            sc[mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                cat8(g < 2 ? kd : z, z), qb[4], a4, 4, 0, 0, g < 2 ? sa : 127, 0, 127);
        }

        // ---- online softmax; lane holds head n16, tokens 16mb + 4g + i
        float x[2][4];
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = tok0 + 16 * mb + 4 * g + i;
                x[mb][i] = tok < ntok ? sc[mb][i] * c : -INFINITY;
                mx = fmaxf(mx, x[mb][i]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float p[2][4];
        float psum = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[mb][i] = __builtin_amdgcn_exp2f(x[mb][i] - m_new);
                psum += p[mb][i];
            }
        l_run = l_run * alpha + psum;
        v8bf pb;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) pb[4 * mb + i] = (__bf16)p[mb][i];

        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int ch = 0; ch < 4; ++ch)
#pragma unroll
                for (int c8 = 0; c8 < 8; ++c8) acc[ch][c8] *= alpha;
        }

        // ---- O^T += V^T P^T: lane decodes 8 dims x 8 tokens of V per chunk
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
            uint32_t d[8][4];  // token r, dim pair j
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int tau = (r < 4) ? (4 * g + r) : (16 + 4 * g + (r - 4));
                const uint32_t wv =
                    *(const uint32_t*)(st + pchunk_off(tau, 4 * ch + (n16 >> 2)) + 4 * (n16 & 3));
                // rows past the item decode as +-0 whatever byte sits there
                const uint32_t sb = (tok0 + tau < ntok) ? ssc[tau * kRowScales + 4 * ch + (n16 >> 2)] : 127u;
                const float scl = e8m0_to_f32(sb);
                d[r][0] = bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv, scl, 0));
                d[r][1] = bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv, scl, 1));
                d[r][2] = bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv, scl, 2));
                d[r][3] = bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv, scl, 3));
            }
#pragma unroll
            for (int c8 = 0; c8 < 8; ++c8) {
                const int j = c8 >> 1;
                const uint32_t sel = (c8 & 1) ? 0x07060302u : 0x05040100u;
                const v8bf va = as_v8bf(perm(d[1][j], d[0][j], sel), perm(d[3][j], d[2][j], sel),
                                        perm(d[5][j], d[4][j], sel), perm(d[7][j], d[6][j], sel));
                acc[ch][c8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[ch][c8], 0, 0, 0);
            }
        }

        if (k + kNst < nt_w) {
            wait_lgkm0();
            issue(k + kNst, s);
        }
    }

    // ---- merge the 4 waves (acc[ch][c8][i] is dim 128ch + 32g + 8i + c8, head n16)
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    __syncthreads();
    float* xo = (float*)smem;
    float* mw = xo + kWaves * kHeads * kXoStride;
    float* lw = mw + kWaves * kHeads;
    {
        float* row = xo + (w * kHeads + n16) * kXoStride;
#pragma unroll
        for (int ch = 0; ch < 4; ++ch)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float* dd = row + 128 * ch + 32 * g + 8 * i;
                *(float4*)dd = make_float4(acc[ch][0][i], acc[ch][1][i], acc[ch][2][i], acc[ch][3][i]);
                *(float4*)(dd + 4) =
                    make_float4(acc[ch][4][i], acc[ch][5][i], acc[ch][6][i], acc[ch][7][i]);
            }
        if (g == 0) {
            mw[w * kHeads + n16] = m_run;
            lw[w * kHeads + n16] = l_run;
        }
    }
    __syncthreads();

    const int h = tid >> 4;
    const int d0 = (tid & 15) * 32;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, mw[ww * kHeads + h]);
    float e[kWaves];
    float L = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
        const float mv = mw[ww * kHeads + h];
        e[ww] = (mv == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mv - M);
        L += e[ww] * lw[ww * kHeads + h];
    }
    const float inv = 1.0f / L;
    float o[32];
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
        float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float4 a = *(const float4*)(xo + (ww * kHeads + h) * kXoStride + d0 + j);
            s4.x += e[ww] * a.x;
            s4.y += e[ww] * a.y;
            s4.z += e[ww] * a.z;
            s4.w += e[ww] * a.w;
        }
        o[j] = s4.x * inv;
        o[j + 1] = s4.y * inv;
        o[j + 2] = s4.z * inv;
        o[j + 3] = s4.w * inv;
    }
    const float lse2 = M + __log2f(L);
    if (slot < 0) {
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
        if (lse_out && (tid & 15) == 0) lse_out[(size_t)b * kHeads + h] = lse2 * kLn2;
    } else {
        float4* dst = (float4*)(part_o + ((size_t)slot * kHeads + h) * kDv + d0);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            dst[j] = make_float4(o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]);
        if ((tid & 15) == 0) part_lse[(size_t)slot * kHeads + h] = lse2;
    }
}

}  // namespace

hipError_t launch_stage1_mxfp4(const int4* items, int nitems, const uint8_t* q8,
                               const float* q_scale, const uint8_t* kv_packed,
                               const uint8_t* kv_scales, float sm_scale, float* part_o,
                               float* part_lse, uint16_t* out, float* lse_out,
                               hipStream_t stream) {
    if (nitems <= 0) return hipSuccess;
    hipLaunchKernelGGL(stage1_mxfp4_kernel, dim3(nitems), dim3(256), 0, stream, items, q8,
                       q_scale, kv_packed, kv_scales, sm_scale, part_o, part_lse, out, lse_out);
    return hipGetLastError();
}

}  // namespace mla
