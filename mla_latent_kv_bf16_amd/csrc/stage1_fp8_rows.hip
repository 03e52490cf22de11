// Stage 1 of the split-KV decode, FP8 cache, for sequences with several query
// rows (multi-token prediction or speculative rows), gfx950.
//
// A sequence's R query rows attend causally, bottom-right aligned, to the
// same cache: row i sees its first kv_len - (R - 1 - i) rows [kernelindex.com
// amd-mixed-mla pages: the causal flag and max_seqlen_qo passed to the
// metadata calls of submissions 663509, 722089 and 738050]. Every KV tile
// is read from HBM once and serves all R x 16 (row, head) pairs: the 4 waves
// form 4 / Rp groups of Rp waves (Rp = R rounded up to 1, 2 or 4), one wave
// per row; group g streams tiles g, g + G, ... through its own LDS stages,
// each wave of the group issuing a share of every tile's copies, and the
// waves advance in step with one workgroup barrier per tile (after it every
// copy of the tile has landed and every wave is done with the previous tile,
// whose stage is then refilled). The per-tile arithmetic is that of the
// single-row kernel (stage1_fp8_tile.h). A wave beyond the sequence's rows
// (R = 3) only helps with the copies.
//
// Q comes straight into registers (each wave its own row); in the fused form
// the wave converts its row's bf16 Q with the standalone quantiser's
// arithmetic and stores the codes. Work items are three int4:
//   {sequence, kv_begin, kv_end, split (-1: the item covers the sequence)},
//   {first query row, R, end of the sequence's cache rows, splits},
//   {first partial slot of the sequence, 0, 0, 0};
// row r of split s writes partial slot first + r * splits + s, so the
// partials of one row are contiguous for the merge. Paged cache: positions
// are in the sequence, the third int4 is {first partial slot, first
// page-table entry of the sequence, its pages, 0}, and each tile's copies
// find their rows through the page ids as in the single-row kernel (rebased
// on the tile's page from 32 rows per page, gathered row by row below).
#include "launch.h"
#include "stage1_fp8_tile.h"
#include "stage_common.h"

namespace mla {
namespace {

using namespace f8tile;
constexpr int kWaves = 4;
constexpr int kStages = 8;                         // LDS tile stages in all
constexpr int kRingBytes = kStages * kStageBytes;  // 147,456
constexpr int kQBytes = kHeads * kDqk;             // one row's 16 x 576 codes
constexpr int kXoStride = kDv + 4;
// wave rows, then per (wave, head) m, l, output weight, then per (row, head) LSE
constexpr int kMergeBytes = kWaves * kHeads * kXoStride * 4 + 4 * kWaves * kHeads * 4;
constexpr int kLdsBytes = kRingBytes > kMergeBytes ? kRingBytes : kMergeBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

// A register copy the compiler cannot trace back to its load: the wait for
// the load is placed here, before any tile copy is in flight, and not at a
// later use inside the main loop (where it would drain the copies).
__device__ __forceinline__ int detach(int x) {
    int y;
    asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
    return y;
}

// Wait until at most `later` tiles of C copies each are still in flight.
template <int C, int N>
__device__ __forceinline__ void wait_tiles(int later) {
    if constexpr (N > 1) {
        if (later >= N - 1) {
            wait_vmcnt<(N - 1) * C>();
            return;
        }
        wait_tiles<C, N - 1>(later);
    } else {
        wait_vmcnt<0>();
    }
}

template <bool kFused, bool kPaged, int Rp>
__device__ __forceinline__ void rows_body(const Stage1Args& a, uint8_t* smem, float q_scale_in) {
    constexpr int G = kWaves / Rp;    // groups, each one wave per row
    constexpr int NS = kStages / G;   // LDS stages per group
    constexpr int C0 = (kDmaPerStage + Rp - 1) / Rp;  // copies per tile of wave 0

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int gi = w / Rp, r = w % Rp;
    const int n16 = lane & 15, g = lane >> 4;

    const int4 it = a.items[3 * blockIdx.x];
    const int4 ex = a.items[3 * blockIdx.x + 1];
    const int4 ex2 = a.items[3 * blockIdx.x + 2];
    const int b = it.x, kb = it.y, split = it.w;
    const int ntok = it.z - it.y;
    const int q_row0 = ex.x, R = ex.y, seq_end = ex.z, S = ex.w, base = ex2.x;
    const int ntile = (ntok + kTok - 1) / kTok;
    const int kmax = (ntile + G - 1) / G;
    const int nt_g = ntile > gi ? (ntile - gi + G - 1) / G : 0;
    const bool live = r < R;
    // cache rows of this item the wave's row may see
    int vis = seq_end - (R - 1 - r) - kb;
    vis = live ? (vis < 0 ? 0 : (vis > ntok ? ntok : vis)) : 0;
    const float ksc = a.kv_scale[0];

    // ---- this wave's Q row into registers
    float q_scale;
    v8i qb[5];
    const v8i z8 = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (!kFused) {
        q_scale = q_scale_in;
        if (live) {
            const uint8_t* q = a.q8_in + (size_t)(q_row0 + r) * kQBytes + n16 * kDqk;
#pragma unroll
            for (int ks = 0; ks < 5; ++ks) {
                const int d = ks < 4 ? 128 * ks + 32 * g : 512 + 32 * (g & 1);
                const uint4 p0 = *(const uint4*)(q + d);
                const uint4 p1 = *(const uint4*)(q + d + 16);
                v8i v = cat8(p0, p1);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = detach(v[e]);
                qb[ks] = (ks < 4 || g < 2) ? v : z8;
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 5; ++ks) qb[ks] = z8;
        }
    } else {
        if (a.blockmax) {
            // every wave reduces the absmax partials itself (as bit
            // patterns, so that a NaN partial wins)
            const uint32_t* bm = (const uint32_t*)a.blockmax;
            uint32_t m = 0;
            for (int i = lane; i < a.nblockmax; i += 64) m = max(m, bm[i]);
            q_scale = absmax_to_scale(__uint_as_float(wave_max_u32(m)));
            if (blockIdx.x == 0 && tid == 0) a.q_scale_out[0] = q_scale;
        } else {
            q_scale = q_scale_in;
        }
        q_scale = uniform_f32(q_scale);
        const float q_rcp = 1.0f / q_scale;
        if (live) {
            const uint16_t* qs = a.q_bf16 + ((size_t)(q_row0 + r) * kHeads + n16) * kDqk;
            uint8_t* qd = a.q8_out + ((size_t)(q_row0 + r) * kHeads + n16) * kDqk;
            with_div_kind(q_scale, [&](auto kind) {
#pragma unroll
                for (int ks = 0; ks < 5; ++ks) {
                    const int d = ks < 4 ? 128 * ks + 32 * g : 512 + 32 * (g & 1);
                    uint2 c[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        c[j] = fp8x8<decltype(kind)::value>(*(const uint4*)(qs + d + 8 * j),
                                                            q_scale, q_rcp);
                    v8i v;
                    v[0] = (int)c[0].x; v[1] = (int)c[0].y; v[2] = (int)c[1].x; v[3] = (int)c[1].y;
                    v[4] = (int)c[2].x; v[5] = (int)c[2].y; v[6] = (int)c[3].x; v[7] = (int)c[3].y;
                    // every code of the row stored once, by the first split
                    if ((ks < 4 || g < 2) && split <= 0) {
                        *(uint4*)(qd + d) = make_uint4(c[0].x, c[0].y, c[1].x, c[1].y);
                        *(uint4*)(qd + d + 16) = make_uint4(c[2].x, c[2].y, c[3].x, c[3].y);
                    }
                    qb[ks] = (ks < 4 || g < 2) ? v : z8;
                }
            });
        } else {
#pragma unroll
            for (int ks = 0; ks < 5; ++ks) qb[ks] = z8;
        }
    }
    // computed (and the scale loads waited for) before any tile copy is issued
    const float c_nat = q_scale * ksc * a.sm_scale;
    const LogitScale ls{__int_as_float(detach(__float_as_int(c_nat * kLog2e))), c_nat, a.logit_cap,
                        a.logit_cap > 0.f ? 1.0f / a.logit_cap : 0.f};

    // ---- tile copies: this wave issues copies i = r (mod Rp) of its group's tiles
    // source offsets of this wave's copies i = r + Rp j of a tile (the
    // swizzled layout of dma_offsets, for this wave's share only)
    uint32_t dma_off[C0];
#pragma unroll
    for (int j = 0; j < C0; ++j) {
        const int sidx = (r + Rp * j) * 64 + lane;
        const int t = sidx / kRowChunks;
        const int cp = sidx - t * kRowChunks;
        dma_off[j] = (uint32_t)(t * kDqk + ((cp ^ swz(t)) * 16));
    }
    const uint32_t ring = lds_addr(smem) + (uint32_t)(gi * NS * kStageBytes);
    const uint8_t* item_kv = a.kv + (size_t)kb * kDqk;
    const uint32_t item_bytes = (uint32_t)ntok * kDqk;
    const int cr = (kDmaPerStage - r + Rp - 1) / Rp;  // this wave's copies per tile
    // paged cache: the sequence's page-table slice (uniform: kept in scalar
    // registers for the scalar page-id loads)
    __amdgpu_buffer_rsrc_t pages_rs;
    if constexpr (kPaged) {
        const int pstart = __builtin_amdgcn_readfirstlane(ex2.y);
        const int npages = __builtin_amdgcn_readfirstlane(ex2.z);
        pages_rs = make_rsrc(a.kv_pages + pstart, (uint32_t)npages * 4u);
    }
    auto issue = [&](int k, int s) {
        const uint32_t dst = ring + (uint32_t)(s * kStageBytes);
        if constexpr (!kPaged) {
            const uint32_t toff = (uint32_t)(gi + G * k) * kStageBytes;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(item_kv + toff, item_bytes - toff);
#pragma unroll
            for (int j = 0; j < C0; ++j) {
                const int i = r + Rp * j;
                if (i < kDmaPerStage) lds_dma16(rs, dst + 1024u * (uint32_t)i, dma_off[j]);
            }
        } else {
            const int tt = (gi + G * k) * kTok;  // first row of the tile in the item
            const int tile_tok = kb + tt;        // ... and in its sequence (a multiple of 32)
            const int rem = ntok - tt;
            const int shift = a.page_shift;
            if (shift >= 5) {
                // the tile's page (a page id outside the pool gives an
                // empty descriptor: zero codes)
                const v8i pg = load_pages8(pages_rs, (uint32_t)(tile_tok >> shift) * 4u);
                const uint32_t pid = (uint32_t)__builtin_amdgcn_readfirstlane(pg[0]);
                const bool in_pool = pid < (uint32_t)a.num_pages;
                const size_t row0 =
                    in_pool ? ((size_t)pid << shift) + (size_t)(tile_tok & ((1 << shift) - 1)) : 0;
                const uint32_t nrow = in_pool ? (uint32_t)(rem < kTok ? rem : kTok) : 0u;
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.kv + row0 * kDqk, nrow * (uint32_t)kDqk);
#pragma unroll
                for (int j = 0; j < C0; ++j) {
                    const int i = r + Rp * j;
                    if (i < kDmaPerStage) lds_dma16(rs, dst + 1024u * (uint32_t)i, dma_off[j]);
                }
            } else {
                // up to 32 pages: lane j < 32 holds the id of the tile's j-th
                // page; each copy's lanes address their rows in the whole
                // pool (below 4 GiB: checked by the host)
                const uint32_t first = (uint32_t)(tile_tok >> shift) * 4u;
                int tbl = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const v8i pg = load_pages8(pages_rs, first + 32u * q);
#pragma unroll
                    for (int e = 0; e < 8; ++e) tbl = (lane == 8 * q + e) ? pg[e] : tbl;
                }
                const uint32_t pool = ((uint32_t)a.num_pages << shift) * (uint32_t)kDqk;
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.kv, pool);
#pragma unroll
                for (int j = 0; j < C0; ++j) {
                    const int i = r + Rp * j;
                    if (i < kDmaPerStage) {
                        const int t = (64 * i + lane) / kRowChunks;  // row of this lane's chunk
                        const uint32_t pid =
                            (uint32_t)__builtin_amdgcn_ds_bpermute((t >> shift) * 4, tbl);
                        const uint32_t phys =
                            (pid << shift) | (uint32_t)(t & ((1 << shift) - 1));
                        const bool ok = t < rem && pid < (uint32_t)a.num_pages;
                        const uint32_t voff = ok ? dma_off[j] + (phys - (uint32_t)t) * (uint32_t)kDqk
                                                 : 0xfffffff0u;  // past the pool: zeros
                        lds_dma16(rs, dst + 1024u * (uint32_t)i, voff);
                    }
                }
            }
        }
    };
    const int npre = nt_g < NS ? nt_g : NS;
    for (int k = 0; k < npre; ++k) issue(k, k);

    float m_run = -INFINITY, l_run = 0.0f;
    v4f acc[32];
#pragma unroll
    for (int blk = 0; blk < 32; ++blk) acc[blk] = (v4f){0.f, 0.f, 0.f, 0.f};

    for (int k = 0; k < kmax; ++k) {
        const int s = k % NS;
        if (k < nt_g) {
            const int issued = (k == 0) ? npre : (nt_g < NS + k - 1 ? nt_g : NS + k - 1);
            const int later = issued - k - 1;
            if (cr == C0)
                wait_tiles<C0, NS>(later);
            else
                wait_tiles<(C0 > 1 ? C0 - 1 : 1), NS>(later);
        }
        __syncthreads();
        // every wave is done with tile k - 1: refill its stage
        if (k >= 1 && k - 1 + NS < nt_g) issue(k - 1 + NS, (k - 1) % NS);
        const int tok0 = (gi + G * k) * kTok;
        if (k < nt_g && tok0 < vis)
            tile(smem + (gi * NS + s) * kStageBytes, qb, tok0, vis, ls, m_run, l_run, acc, n16,
                 g, k > 0);
    }

    // ---- per row, merge the G waves that streamed its tiles
    l_run = group4_sum(l_run);
    __syncthreads();
    float* xo = (float*)smem;
    float* mw = xo + kWaves * kHeads * kXoStride;
    float* lw = mw + kWaves * kHeads;
    float* fw = lw + kWaves * kHeads;  // [wave][head]: weight of the wave's rows
    float* hl = fw + kWaves * kHeads;  // [row][head]: base-2 LSE of the item
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
        const int hh = tid & (kHeads - 1), ww = tid >> 4, rr = ww % Rp;
        float M = -INFINITY;
#pragma unroll
        for (int gj = 0; gj < G; ++gj) M = fmaxf(M, mw[(gj * Rp + rr) * kHeads + hh]);
        float L = 0.f, ew = 0.f;
#pragma unroll
        for (int gj = 0; gj < G; ++gj) {
            const int v = gj * Rp + rr;
            const float mv = mw[v * kHeads + hh];
            const float e = (mv == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mv - M);
            L += e * lw[v * kHeads + hh];
            if (v == ww) ew = e;
        }
        // the row sees no cache row of the item (NaN scores leave M at -inf but L NaN)
        const bool empty = (M == -INFINITY) && (L == 0.f);
        fw[tid] = empty ? 0.f : ew * (ksc / L);
        if (ww < Rp) hl[rr * kHeads + hh] = empty ? -INFINITY : M + __log2f(L) - kPScaleLog2;
    }
    __syncthreads();
    using Map = RowMap<256>;
    const int dq = Map::dim(tid);
#pragma unroll
    for (int rr = 0; rr < Rp; ++rr) {
        if (rr >= R) break;
        float4 o[Map::kPer];
#pragma unroll
        for (int q = 0; q < Map::kPer; ++q) {
            const int hq = Map::head(tid, q);
            float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int gj = 0; gj < G; ++gj) {
                const int v = gj * Rp + rr;
                const float f = fw[v * kHeads + hq];
                const float4 x = *(const float4*)(xo + (v * kHeads + hq) * kXoStride + dq);
                s4.x += f * x.x;
                s4.y += f * x.y;
                s4.z += f * x.z;
                s4.w += f * x.w;
            }
            o[q] = s4;
        }
        const int qrow = q_row0 + rr;
        if (split < 0) {
            uint16_t* ob = a.out + (size_t)qrow * kHeads * kDv;
#pragma unroll
            for (int q = 0; q < Map::kPer; ++q)
                *(uint2*)(ob + Map::head(tid, q) * kDv + dq) =
                    make_uint2(pack_bf16x2(o[q].x, o[q].y), pack_bf16x2(o[q].z, o[q].w));
            if (a.lse_out && tid < kHeads)
                a.lse_out[(size_t)qrow * kHeads + tid] = hl[rr * kHeads + tid] * kLn2;
        } else {
            const int slot = base + rr * S + split;
            if constexpr (!kFused) {
                float* pb = a.part_o + (size_t)slot * kHeads * kDv;
#pragma unroll
                for (int q = 0; q < Map::kPer; ++q)
                    *(float4*)(pb + Map::head(tid, q) * kDv + dq) = o[q];
                if (tid < kHeads) a.part_lse[(size_t)slot * kHeads + tid] = hl[rr * kHeads + tid];
            } else {
                // written through to the coherence point for the merging workgroup
                const __amdgpu_buffer_rsrc_t ro =
                    make_rsrc(a.part_o + (size_t)slot * kHeads * kDv, kHeads * kDv * 4);
#pragma unroll
                for (int q = 0; q < Map::kPer; ++q)
                    store_coherent(ro, (uint32_t)((Map::head(tid, q) * kDv + dq) * 4), o[q]);
                if (tid < kHeads)
                    store_coherent(make_rsrc(a.part_lse + (size_t)slot * kHeads, kHeads * 4),
                                   (uint32_t)(tid * 4), hl[rr * kHeads + tid]);
            }
        }
    }
    if constexpr (kFused) {
        if (split >= 0) {
            // once every wave's stores have completed, the last of the
            // sequence's workgroups to arrive at its counter merges each row
            wait_vmcnt<0>();
            __syncthreads();
            uint32_t* flag = (uint32_t*)smem;
            if (tid == 0) flag[0] = (atomicAdd(&a.counters[b], 1u) == (uint32_t)S - 1u);
            __syncthreads();
            if (flag[0]) {
                for (int rr = 0; rr < R; ++rr) {
                    const int qrow = q_row0 + rr;
                    merge_split<256, true>(a.part_o, a.part_lse, base + rr * S, S,
                                           a.out + (size_t)qrow * kHeads * kDv,
                                           a.lse_out ? a.lse_out + (size_t)qrow * kHeads : nullptr,
                                           (float*)(smem + 16), tid);
                    __syncthreads();
                }
                if (tid == 0)
                    __hip_atomic_store(&a.counters[b], 0u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

template <bool kFused, bool kPaged>
__global__ __launch_bounds__(256) void stage1_fp8_rows_kernel(Stage1Args a) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];
    // read before any store so that it stays a scalar load
    const float q_scale_in = a.q_scale ? a.q_scale[0] : 0.f;
    const int R = a.items[3 * blockIdx.x + 1].y;
    if (R <= 1)
        rows_body<kFused, kPaged, 1>(a, smem, q_scale_in);
    else if (R == 2)
        rows_body<kFused, kPaged, 2>(a, smem, q_scale_in);
    else
        rows_body<kFused, kPaged, 4>(a, smem, q_scale_in);
}

}  // namespace

hipError_t launch_stage1_fp8_rows(const Stage1Args& args, int nitems, bool fused,
                                  hipStream_t stream) {
    if (nitems <= 0) return hipSuccess;
#define MLA_ROWS_LAUNCH(F, P) \
    hipLaunchKernelGGL((stage1_fp8_rows_kernel<F, P>), dim3(nitems), dim3(256), 0, stream, args)
    if (fused && args.kv_pages) MLA_ROWS_LAUNCH(true, true);
    else if (fused) MLA_ROWS_LAUNCH(true, false);
    else if (args.kv_pages) MLA_ROWS_LAUNCH(false, true);
    else MLA_ROWS_LAUNCH(false, false);
#undef MLA_ROWS_LAUNCH
    return hipGetLastError();
}

}  // namespace mla
