// Stage 1 of the split-KV decode for a bf16 latent cache (the pages' bf16
// path: bf16 Q and bf16 cache, no quantisation), gfx950, with an optional
// logit soft-cap.
//
// [kernelindex.com amd-mixed-mla submission 722089, `_aiter_path`: bf16 Q
// against the bf16 cache for small batches; the `logit_cap` argument of the
// decode calls (0 on every page). A positive cap bounds each scaled logit
// s to cap * tanh(s / cap) before the softmax.]
//
// Structure of the single-row FP8 kernel (stage1_fp8.hip): one workgroup of
// 4 waves per work item, each wave streaming its own tiles through a private
// two-stage LDS ring by direct buffer->LDS copies, its own online-softmax
// state, and the LDS merge of the 4 waves at the end. A bf16 row is 1,152 B,
// so a stage holds 16 tokens (18,432 B, 18 wave-wide 1 KiB copies).
//   - QK^T as S^T = K Q^T on the 16x16x32 bf16 MFMA: M = 16 tokens, N = 16
//     heads, 18 steps of 32 dims. Lane group g carries dims 8g..8g+7 of a
//     step in both operands (any mapping shared by A and B gives the same
//     dot product). Q (16 x 576) stays in registers.
//   - Online softmax in base 2, lazy reference maximum (slack 8: bf16 P up
//     to 2^8 is exact in range), P rounded to bf16.
//   - P.V as O^T = V^T P^T on the 16x16x16 bf16 MFMA (K = the tile's 16
//     tokens): V^T comes from the transposing LDS read ds_read_b64_tr_b16
//     (lanes 4r..4r+3 of a 16-lane group address row r, lane i receives
//     element i of the group's 4 rows: measured on the GPU), and P already
//     has the B layout (lane: head n16, tokens 4g..4g+3).
//   - LDS rows are swizzled in 16-B chunks: chunk c of row t sits at
//     position c ^ (t & 7) within its aligned group of eight.
// The fused form quantises nothing; split sequences are merged by their
// last workgroup, as in the FP8 kernel. Paged form (fused only): the cache
// is a pool of pages and a tile's rows are found through the sequence's
// page ids, as in the FP8 kernel's paged form with 16-row tiles.
#include "launch.h"
#include "stage_common.h"

namespace mla {
namespace {

constexpr int kWaves = 4;
constexpr int kTok = 16;                          // tokens per stage
constexpr int kRowBytes = kDqk * 2;               // 1152
constexpr int kRowChunks16 = kRowBytes / 16;      // 72
constexpr int kStageBytes = kTok * kRowBytes;     // 18432
constexpr int kDmaPerStage = kStageBytes / 1024;  // 18
constexpr int kRingBytes = kWaves * 2 * kStageBytes;
constexpr int kXoStride = kDv + 4;
constexpr int kMergeBytes = kWaves * kHeads * kXoStride * 4 + 3 * kWaves * kHeads * 4 + kHeads * 4;
constexpr int kLdsBytes = kRingBytes > kMergeBytes ? kRingBytes : kMergeBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
constexpr float kSlack = 8.0f;                    // lazy-max slack, log2 units

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int sw8(int t) { return t & 7; }

__device__ __forceinline__ int detach(int x) {
    int y;
    asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
    return y;
}

__device__ __forceinline__ v8bf as_v8bf(uint4 u) { return __builtin_bit_cast(v8bf, u); }

template <bool kFused, bool kNt, bool kPaged>
__global__ __launch_bounds__(256) void stage1_bf16_kernel(Stage1Args a, float logit_cap) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15;
    const int g = lane >> 4;

    constexpr int kItemWords = (kFused || kPaged) ? 2 : 1;  // int4 per item
    const int4 it = a.items[kItemWords * blockIdx.x];
    const int b = it.x, kb = it.y, slot = it.w;
    const int ntok = it.z - it.y;
    const int ntile = (ntok + kTok - 1) / kTok;
    const int nt_w = ntile > w ? (ntile - w + kWaves - 1) / kWaves : 0;

    // ---- Q row of head n16 into registers: dims 32 ks + 8 g .. +8, ks < 18
    uint4 qb[18];
    {
        const uint16_t* q = a.q_bf16 + ((size_t)b * kHeads + n16) * kDqk + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
            uint4 v = *(const uint4*)(q + 32 * ks);
            v.x = (uint32_t)detach((int)v.x);
            v.y = (uint32_t)detach((int)v.y);
            v.z = (uint32_t)detach((int)v.z);
            v.w = (uint32_t)detach((int)v.w);
            qb[ks] = v;
        }
    }
    const float sm = a.sm_scale;
    const float c = sm * kLog2e;
    const bool use_cap = logit_cap > 0.0f;
    const float inv_cap = use_cap ? 1.0f / logit_cap : 0.0f;

    // ---- tile copies
    uint32_t dma_off[kDmaPerStage];
#pragma unroll
    for (int i = 0; i < kDmaPerStage; ++i) {
        const int s = i * 64 + lane;
        const int t = s / kRowChunks16;
        const int cp = s - t * kRowChunks16;
        dma_off[i] = (uint32_t)(t * kRowBytes + ((cp ^ sw8(t)) * 16));
    }
    const uint32_t ring = lds_addr(smem) + (uint32_t)(w * 2 * kStageBytes);
    const uint8_t* item_kv = a.kv + (size_t)kb * kRowBytes;
    const uint32_t item_bytes = (uint32_t)ntok * kRowBytes;
    // paged cache: the item's page-table slice (kb and the item's end are
    // positions in the sequence)
    __amdgpu_buffer_rsrc_t pages_rs;
    if constexpr (kPaged) {
        const int4 ex = a.items[2 * blockIdx.x + 1];  // {first slot, splits, page start, pages}
        // (uniform: kept in scalar registers for the scalar page-id loads)
        const int pstart = __builtin_amdgcn_readfirstlane(ex.z);
        const int npages = __builtin_amdgcn_readfirstlane(ex.w);
        pages_rs = make_rsrc(a.kv_pages + pstart, (uint32_t)npages * 4u);
    }
    auto issue = [&](int k, int s) {
        const uint32_t dst = ring + (uint32_t)(s * kStageBytes);
        if constexpr (!kPaged) {
            const uint32_t toff = (uint32_t)(w + kWaves * k) * kStageBytes;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(item_kv + toff, item_bytes - toff);
#pragma unroll
            for (int i = 0; i < kDmaPerStage; ++i)
                lds_dma16_kv<kNt>(rs, dst + 1024u * i, dma_off[i]);
        } else {
            const int shift = a.page_shift;
            const int tt = (w + kWaves * k) * kTok;  // first row of the tile in the item
            const int tile_tok = kb + tt;            // ... and in its sequence (a multiple of 16)
            const int rem = ntok - tt;               // rows of the tile inside the item
            if (shift >= 4) {
                // the whole tile lies in one page (a page id outside the
                // pool gives an empty descriptor: zero rows)
                const v8i pg = load_pages8(pages_rs, (uint32_t)(tile_tok >> shift) * 4u);
                const uint32_t pid = (uint32_t)__builtin_amdgcn_readfirstlane(pg[0]);
                const bool in_pool = pid < (uint32_t)a.num_pages;
                const size_t row0 =
                    in_pool ? ((size_t)pid << shift) + (size_t)(tile_tok & ((1 << shift) - 1)) : 0;
                const uint32_t nrow = in_pool ? (uint32_t)(rem < kTok ? rem : kTok) : 0u;
                const __amdgpu_buffer_rsrc_t rs =
                    make_rsrc(a.kv + row0 * kRowBytes, nrow * (uint32_t)kRowBytes);
#pragma unroll
                for (int i = 0; i < kDmaPerStage; ++i)
                    lds_dma16_kv<kNt>(rs, dst + 1024u * i, dma_off[i]);
            } else {
                // up to 16 pages: lane j < 16 holds the id of the tile's j-th
                // page; each copy's lanes address their rows in the whole
                // pool (below 4 GiB: checked by the host)
                const uint32_t first = (uint32_t)(tile_tok >> shift) * 4u;
                int tbl = 0;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const v8i pg = load_pages8(pages_rs, first + 32u * q);
#pragma unroll
                    for (int e = 0; e < 8; ++e) tbl = (lane == 8 * q + e) ? pg[e] : tbl;
                }
                const uint32_t pool = ((uint32_t)a.num_pages << shift) * (uint32_t)kRowBytes;
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.kv, pool);
#pragma unroll
                for (int i = 0; i < kDmaPerStage; ++i) {
                    const int t = (64 * i + lane) / kRowChunks16;  // row of this lane's chunk
                    const uint32_t pid =
                        (uint32_t)__builtin_amdgcn_ds_bpermute((t >> shift) * 4, tbl);
                    const uint32_t phys = (pid << shift) | (uint32_t)(t & ((1 << shift) - 1));
                    const bool ok = t < rem && pid < (uint32_t)a.num_pages;
                    const uint32_t voff = ok ? dma_off[i] + (phys - (uint32_t)t) * (uint32_t)kRowBytes
                                             : 0xfffffff0u;  // past the pool: zeros
                    lds_dma16_kv<kNt>(rs, dst + 1024u * i, voff);
                }
            }
        }
    };
    if (nt_w > 0) issue(0, 0);
    if (nt_w > 1) issue(1, 1);

    float m_run = -INFINITY, l_run = 0.0f;
    v4f acc[32];  // acc[blk][r]: latent dim 16 blk + 4 g + r, head n16
#pragma unroll
    for (int blk = 0; blk < 32; ++blk) acc[blk] = (v4f){0.f, 0.f, 0.f, 0.f};

    for (int k = 0; k < nt_w; ++k) {
        const int s = k & 1;
        if (k + 1 < nt_w)
            wait_vmcnt<kDmaPerStage>();
        else
            wait_vmcnt<0>();
        const uint8_t* st = smem + (w * 2 + s) * kStageBytes;
        const int tok0 = (w + kWaves * k) * kTok;

        // ---- S^T = K Q^T: token n16 of the tile, dims 32 ks + 8 g. The
        // swizzle flips the low three bits of the chunk index, so chunk
        // 4 ks + g lies at 128 (ks / 2) + 16 ((4 (ks & 1) + g) ^ sw8(n16)) of
        // the row: two per-lane bases plus constants.
        v4f s4 = {0.f, 0.f, 0.f, 0.f};
        {
            const uint8_t* row = st + n16 * kRowBytes;
            const uint8_t* kb0 = row + 16 * (g ^ sw8(n16));
            const uint8_t* kb1 = row + 16 * ((4 + g) ^ sw8(n16));
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) {
                const uint4 kv4 = *(const uint4*)(((ks & 1) ? kb1 : kb0) + 128 * (ks >> 1));
                s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(kv4), as_v8bf(qb[ks]), s4, 0,
                                                              0, 0);
            }
        }

        // ---- online softmax: head n16, tokens 4g + i (only the last tile
        // of the item can hold tokens past its end)
        float x[4];
        float mx = -INFINITY;
        const bool full = tok0 + kTok <= ntok;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = tok0 + 4 * g + i;
            float v = use_cap ? capped(s4[i] * sm, logit_cap, inv_cap) : s4[i] * c;
            x[i] = (full || tok < ntok) ? v : -INFINITY;
            mx = fmaxf(mx, x[i]);
        }
        mx = group4_max(mx);
        const float m_new = (mx > m_run + kSlack) ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float p[4];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = __builtin_amdgcn_exp2f(x[i] - m_new);
            psum += p[i];
        }
        l_run = l_run * alpha + psum;
        v4s pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) pb[i] = (short)f32_to_bf16_rne(p[i]);

        // (the first tile's accumulators are still zero)
        if (k > 0 && __any(alpha != 1.0f)) {
#pragma unroll
            for (int blk = 0; blk < 32; ++blk) acc[blk] *= alpha;
        }

        // ---- O^T += V^T P^T: lane 16 G + 4 r + j addresses token 4 G + r,
        // dims 16 blk + 4 j; it receives dim 16 blk + (lane & 15) of the group's
        // 4 tokens
        // Chunk 2 blk + h (h = (n16 & 3) / 2) of row tt lies at
        // 128 (blk / 4) + 16 ((2 (blk & 3) + h) ^ sw8(tt)): four per-lane
        // bases plus constants.
        {
            const int tt = 4 * g + (n16 >> 2);
            const uint8_t* vrow = st + tt * kRowBytes + 8 * ((n16 & 3) & 1);
            const int sw = sw8(tt);
            const int h = (n16 & 3) >> 1;
            const uint8_t* vb[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) vb[b] = vrow + 16 * ((2 * b + h) ^ sw);
#pragma unroll
            for (int b8 = 0; b8 < 32; b8 += 8) {
                v4s va[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int blk = b8 + q;
                    va[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4s*)(vb[blk & 3] + 128 * (blk >> 2)));
                }
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    acc[b8 + q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[q], pb, acc[b8 + q],
                                                                          0, 0, 0);
            }
        }

        if (k + 2 < nt_w) {
            wait_lgkm0();
            issue(k + 2, s);
        }
    }

    // ---- merge the 4 waves (as in the FP8 kernel, with unit scales)
    l_run = group4_sum(l_run);
    __syncthreads();
    float* xo = (float*)smem;
    float* mw = xo + kWaves * kHeads * kXoStride;
    float* lw = mw + kWaves * kHeads;
    float* fw = lw + kWaves * kHeads;
    float* hl = fw + kWaves * kHeads;
    {
        float* row = xo + (w * kHeads + n16) * kXoStride + 4 * g;
#pragma unroll
        for (int blk = 0; blk < 32; ++blk)
            *(float4*)(row + 16 * blk) =
                make_float4(acc[blk][0], acc[blk][1], acc[blk][2], acc[blk][3]);
        if (g == 0) {
            mw[w * kHeads + n16] = m_run;
            lw[w * kHeads + n16] = l_run;
        }
    }
    __syncthreads();
    if (tid < kWaves * kHeads) {
        const int hh = tid & (kHeads - 1), ww = tid >> 4;
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) M = fmaxf(M, mw[v * kHeads + hh]);
        float L = 0.f, ew = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const float mv = mw[v * kHeads + hh];
            const float e = (mv == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mv - M);
            L += e * lw[v * kHeads + hh];
            if (v == ww) ew = e;
        }
        // only for a sequence with no rows (NaN scores leave M at -inf but L NaN)
        const bool empty = (M == -INFINITY) && (L == 0.f);
        fw[tid] = empty ? 0.f : ew / L;
        if (ww == 0) hl[hh] = empty ? -INFINITY : M + __log2f(L);
    }
    __syncthreads();
    using Map = RowMap<256>;
    const int dq = Map::dim(tid);
    float4 o[Map::kPer];
#pragma unroll
    for (int q = 0; q < Map::kPer; ++q) {
        const int hq = Map::head(tid, q);
        float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float f = fw[ww * kHeads + hq];
            const float4 v = *(const float4*)(xo + (ww * kHeads + hq) * kXoStride + dq);
            s4.x += f * v.x;
            s4.y += f * v.y;
            s4.z += f * v.z;
            s4.w += f * v.w;
        }
        o[q] = s4;
    }
    if (slot < 0) {
        uint16_t* ob = a.out + (size_t)b * kHeads * kDv;
#pragma unroll
        for (int q = 0; q < Map::kPer; ++q)
            *(uint2*)(ob + Map::head(tid, q) * kDv + dq) =
                make_uint2(pack_bf16x2(o[q].x, o[q].y), pack_bf16x2(o[q].z, o[q].w));
        if (a.lse_out && tid < kHeads) a.lse_out[(size_t)b * kHeads + tid] = hl[tid] * kLn2;
    } else if constexpr (!kFused) {
        float* pb = a.part_o + (size_t)slot * kHeads * kDv;
#pragma unroll
        for (int q = 0; q < Map::kPer; ++q) *(float4*)(pb + Map::head(tid, q) * kDv + dq) = o[q];
        if (tid < kHeads) a.part_lse[(size_t)slot * kHeads + tid] = hl[tid];
    } else {
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(a.part_o + (size_t)slot * kHeads * kDv, kHeads * kDv * 4);
#pragma unroll
        for (int q = 0; q < Map::kPer; ++q)
            store_coherent(ro, (uint32_t)((Map::head(tid, q) * kDv + dq) * 4), o[q]);
        if (tid < kHeads)
            store_coherent(make_rsrc(a.part_lse + (size_t)slot * kHeads, kHeads * 4),
                           (uint32_t)(tid * 4), hl[tid]);
        const int4 ex = a.items[2 * blockIdx.x + 1];  // {first slot, splits, -, -}
        wait_vmcnt<0>();
        __syncthreads();
        uint32_t* flag = (uint32_t*)smem;
        if (tid == 0) flag[0] = (atomicAdd(&a.counters[b], 1u) == (uint32_t)ex.y - 1u);
        __syncthreads();
        if (flag[0]) {
            merge_split<256, true>(a.part_o, a.part_lse, ex.x, ex.y,
                                   a.out + (size_t)b * kHeads * kDv,
                                   a.lse_out ? a.lse_out + (size_t)b * kHeads : nullptr,
                                   (float*)(smem + 16), tid);
            if (tid == 0)
                __hip_atomic_store(&a.counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

hipError_t launch_stage1_bf16(const Stage1Args& args, float logit_cap, int nitems, bool fused,
                              hipStream_t stream) {
    if (nitems <= 0) return hipSuccess;
    const dim3 grid(nitems), block(256);
#define MLA_BF_LAUNCH(F, N, P) \
    hipLaunchKernelGGL((stage1_bf16_kernel<F, N, P>), grid, block, 0, stream, args, logit_cap)
    if (args.kv_pages) {  // the paged cache runs fused only
        if (!fused) return hipErrorInvalidValue;
        if (args.kv_nt) MLA_BF_LAUNCH(true, true, true);
        else MLA_BF_LAUNCH(true, false, true);
    } else {
        if (fused && args.kv_nt) MLA_BF_LAUNCH(true, true, false);
        else if (fused) MLA_BF_LAUNCH(true, false, false);
        else if (args.kv_nt) MLA_BF_LAUNCH(false, true, false);
        else MLA_BF_LAUNCH(false, false, false);
    }
#undef MLA_BF_LAUNCH
    return hipGetLastError();
}

}  // namespace mla
