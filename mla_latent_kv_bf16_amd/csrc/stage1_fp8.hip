// Stage 1 of the split-KV decode for an FP8 E4M3FN latent cache (gfx950).
//
// One workgroup per work item (sequence b, cache rows [kv_begin, kv_end)).
// Every KV byte is read from HBM exactly once and serves all 16 heads: the
// heads are the N dimension of each MFMA, so one program covers the whole
// query group [kernelindex.com amd-mixed-mla submission 722089, module
// docstring and `_mla_multihead_stage1`: load the KV once per program and
// reuse it for every head].
//
// Layout of the work inside a workgroup (4 waves, one per SIMD):
//   - The item's rows are cut into 32-token tiles; wave w takes tiles
//     w, w+4, w+8, ... and keeps its own online-softmax state, so the main
//     loop needs no workgroup barrier.
//   - Each wave owns a two-stage LDS ring (2 x 18 KiB). Tiles arrive by
//     direct buffer->LDS copies (16 B per lane, one contiguous KiB per
//     instruction), with the next tile in flight while the current one is
//     consumed. Rows past the item end read as zeros (buffer range check)
//     and are masked out of the softmax.
//   - QK^T runs as S^T = K Q^T on the 16x16x128 FP8 MFMA: M = 16 tokens,
//     N = 16 heads, K = 128 latent dims (4 full steps and a 64-dim tail with
//     zeroed upper lane groups). Its output already has the layout P needs as
//     the B operand of P.V, so P never leaves registers.
//   - P.V runs as O^T = V^T P^T on the 16x16x32 FP8 MFMA: M = 16 latent
//     dims, N = 16 heads, K = 32 tokens. V^T comes straight out of LDS with
//     the gfx950 transposing read (ds_read_b64_tr_b8), one per 16 dims.
//     P is carried as two FP8 terms (P_hi = e4m3(P), P_lo = e5m2(P - P_hi)),
//     each fed to its own MFMA against the same V operand; one FP8 term alone
//     is too coarse for short sequences where a few weights dominate, and
//     the low term's e5m2 keeps weights down to 2^-22 of the maximum's.
//   - Online softmax in base 2 [722089 `_mla_multihead_stage1`]: logits are
//     scaled by q_scale * kv_scale * sm_scale * log2(e). The reference max
//     only moves when a tile exceeds it by more than 2 (log2 units), so the
//     accumulator is rarely rescaled; P = 2^(x - m) * 64 <= 256 keeps its FP8
//     codes in the normal range.
//   - At the end the 4 waves' (m, l, acc) are merged through LDS and the
//     item writes either the final bf16 output and LSE (unsplit sequence) or
//     an fp32 partial O normalised by its own sum and a base-2 LSE.
//
// Fused form (template flag kFused, one launch per call with a static Q
// scale): the workgroup quantises its sequence's Q rows itself (bf16 rows
// loaded into registers while the first tile is in flight, scale
// static or reduced from the absmax partials, the same arithmetic as the
// standalone quantiser) and writes the codes out; a split sequence is merged by whichever of its workgroups
// arrives last at a per-sequence counter, which it then resets to zero.
//
// Paged form (template flag kPaged): the cache is a pool of pages of
// P = 2^page_shift rows and each sequence lists its pages in order
// [kernelindex.com amd-mixed-mla, submission 663509 and 738050: kv_buffer
// viewed as (pages, page_size, 1, 576) with kv_indptr / kv_indices /
// kv_last_page_len]. A tile's 32 rows lie in one page when P >= 32 (the
// tile's copy descriptor is rebased on that page); for P < 32 the tile's
// page ids come in with one scalar load per 8 pages, each lane picks its
// row's page from a lane table (ds_bpermute) and the copy offsets are
// physical rows of the whole pool. Page ids outside the pool read as zeros.
//
// LDS row layout: a 576-byte token row is 36 chunks of 16 B; chunk c of row
// t is stored at chunk position c ^ f(t) within its aligned group of four,
// f(t) = ((t >> 2) & 3) ^ (((t >> 1) & 1) << 1), so that the 16-B reads of
// 8 or 16 consecutive rows at the same chunk fall in distinct bank groups.
#include "launch.h"
#include "stage1_fp8_tile.h"
#include "stage_common.h"

namespace mla {
namespace {

using namespace f8tile;
constexpr int kWaves = 4;
constexpr int kRingBytes = kWaves * 2 * kStageBytes;
constexpr int kQBytes = kHeads * kDqk;             // 9216: the item's Q codes
constexpr int kXoStride = kDv + 4;                // floats per head row when merging waves
// wave rows, then per (wave, head) m, l and output weight, then per-head LSE
constexpr int kMergeBytes = kWaves * kHeads * kXoStride * 4 + 3 * kWaves * kHeads * 4 + kHeads * 4;
constexpr int kBmBytes = kMaxAbsmaxBlocks * 4;    // absmax partials (fused form)
constexpr int kLdsBytes = (kRingBytes + kQBytes + kBmBytes > kMergeBytes)
                              ? kRingBytes + kQBytes + kBmBytes
                              : kMergeBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
static_assert(kMergeBytes <= kRingBytes, "the wave merge leaves the Q codes in place");
constexpr int kQVec = (2 * kQBytes / 16 + 255) / 256;  // 16-B bf16 Q vectors per thread
constexpr int kQAllVec = kQAbsmaxRows * 2 * kQBytes / 16 / 256;  // ... of all of Q (absmax)
static_assert(kQAllVec + kQVec + 2 * kDmaPerStage <= 63, "copies in flight within the wait counter");
static_assert(kQVec == 5, "bf16 Q rows: 4.5 vectors per thread");
static_assert(kBmBytes == kWaves * 1024, "one 1 KiB copy of absmax partials per wave");


template <bool kFused, bool kPaged, bool kNt>
__global__ __launch_bounds__(256) void stage1_fp8_kernel(Stage1Args a) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15;  // MFMA row (A) / column (B, C) index
    const int g = lane >> 4;    // lane group: which K slice this lane carries

    constexpr int kItemWords = (kFused || kPaged) ? 2 : 1;  // int4 per item
    const int4 it = a.items[kItemWords * blockIdx.x];
    const int b = it.x, kb = it.y, slot = it.w;
    const int ntok = it.z - it.y;
    const int ntile = (ntok + kTok - 1) / kTok;
    const int nt_w = ntile > w ? (ntile - w + kWaves - 1) / kWaves : 0;

    const float ksc = a.kv_scale[0];
    // read before any store so that it stays a scalar load (a vector load
    // here would make the compiler drain the tile copies at its first use)
    const float q_scale_in = a.q_scale ? a.q_scale[0] : 0.f;

    // Per-lane source offsets of the 18 copies of one stage
    uint32_t dma_off[kDmaPerStage];
    dma_offsets(lane, dma_off);

    const uint32_t ring = lds_addr(smem) + (uint32_t)(w * 2 * kStageBytes);
    const uint8_t* item_kv = a.kv + (size_t)kb * kDqk;
    const uint32_t item_bytes = (uint32_t)ntok * kDqk;

    // paged cache: the item's page table slice and the pool geometry
    __amdgpu_buffer_rsrc_t pages_rs;
    int page_shift = 0;
    if constexpr (kPaged) {
        const int4 ex = a.items[2 * blockIdx.x + 1];  // {first slot, splits, page start, pages}
        pages_rs = make_rsrc(a.kv_pages + ex.z, (uint32_t)ex.w * 4u);
        page_shift = a.page_shift;
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
            const int tt = (w + kWaves * k) * kTok;  // first row of the tile in the item
            const int tile_tok = kb + tt;            // ... and in its sequence (a multiple of 32)
            const int rem = ntok - tt;               // rows of the tile inside the item
            if (page_shift >= 5) {
                // the whole tile lies in one page
                const v8i pg = load_pages8(pages_rs, (uint32_t)(tile_tok >> page_shift) * 4u);
                const uint32_t pid = (uint32_t)__builtin_amdgcn_readfirstlane(pg[0]);
                const size_t row0 = ((size_t)pid << page_shift) +
                                    (size_t)(tile_tok & ((1 << page_shift) - 1));
                const uint32_t nrow = pid < (uint32_t)a.num_pages ? (rem < kTok ? rem : kTok) : 0;
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.kv + row0 * kDqk, nrow * kDqk);
#pragma unroll
                for (int i = 0; i < kDmaPerStage; ++i)
                    lds_dma16_kv<kNt>(rs, dst + 1024u * i, dma_off[i]);
            } else {
                // up to 32 pages: lane j < 32 holds the id of the tile's j-th page
                const uint32_t first = (uint32_t)(tile_tok >> page_shift) * 4u;
                int tbl = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const v8i pg = load_pages8(pages_rs, first + 32u * q);
#pragma unroll
                    for (int e = 0; e < 8; ++e) tbl = (lane == 8 * q + e) ? pg[e] : tbl;
                }
                const uint32_t pool = ((uint32_t)a.num_pages << page_shift) * (uint32_t)kDqk;
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.kv, pool);
#pragma unroll
                for (int i = 0; i < kDmaPerStage; ++i) {
                    const int t = (64 * i + lane) / kRowChunks;  // row of this lane's chunk
                    const uint32_t pid =
                        (uint32_t)__builtin_amdgcn_ds_bpermute((t >> page_shift) * 4, tbl);
                    const uint32_t phys = (pid << page_shift) | (uint32_t)(t & ((1 << page_shift) - 1));
                    const bool ok = t < rem && pid < (uint32_t)a.num_pages;
                    const uint32_t voff = ok ? dma_off[i] + (phys - (uint32_t)t) * (uint32_t)kDqk
                                             : 0xfffffff0u;  // past the pool: zeros
                    lds_dma16_kv<kNt>(rs, dst + 1024u * i, voff);
                }
            }
        }
    };

    const uint32_t qlds = lds_addr(smem) + (uint32_t)kRingBytes;
    float q_scale;
    if constexpr (!kFused) {
        // The item's Q codes go to LDS first (each wave copies some of the
        // nine KiB), then this wave's first tile; the second follows the
        // barrier. Bringing Q in through the same asynchronous path keeps the
        // compiler from waiting on a register load, which would drain the
        // tile prefetch.
        q_scale = q_scale_in;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q8_in + (size_t)b * kQBytes, kQBytes);
        for (int i = w; i < kQBytes / 1024; i += kWaves)
            lds_dma16(rq, qlds + 1024u * i, 1024u * i + 16u * lane);
        if (nt_w > 0) {
            issue(0, 0);
            wait_vmcnt<kDmaPerStage>();
        } else {
            wait_vmcnt<0>();
        }
        __syncthreads();
        if (nt_w > 1) issue(1, 1);
    } else {
        // The sequence's bf16 Q rows (18 KiB) come into registers, vector
        // v = tid + 256 j of 16 B in qv[j] (j = 4 lies past the rows for half
        // of the threads and reads as zeros). Those loads, the absmax
        // partials (to LDS) and this wave's first tile are issued before the
        // first wait, so the conversion overlaps the tile copy; the second
        // tile follows the conversion (issued with the first, its copies
        // hold up the Q rows and the conversion that every wave waits for).
        // With a.q_absmax_rows (at most 4 rows of Q) every row of Q comes in
        // first, vector v = tid + 256 j in qa[j], for the absmax: 18 + 5 + 18
        // copies stay within the 63 that the wait counter tracks.
        const bool qall = a.q_absmax_rows > 0;
        v4u qa[kQAllVec];
        if (qall) {
            const __amdgpu_buffer_rsrc_t ra =
                make_rsrc(a.q_bf16, (uint32_t)a.q_absmax_rows * 2u * kQBytes);
#pragma unroll
            for (int j = 0; j < kQAllVec; ++j)
                qa[j] = load16_async(ra, 16u * (uint32_t)(tid + 256 * j));
        }
        const __amdgpu_buffer_rsrc_t rq =
            make_rsrc(a.q_bf16 + (size_t)b * kHeads * kDqk, 2 * kQBytes);
        v4u qv[kQVec];
#pragma unroll
        for (int j = 0; j < kQVec; ++j) qv[j] = load16_async(rq, 16u * (uint32_t)(tid + 256 * j));
        const uint32_t bmlds = lds_addr(smem) + (uint32_t)(kRingBytes + kQBytes);
        if (a.blockmax) {
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.blockmax, (uint32_t)a.nblockmax * 4u);
            lds_dma16(rb, bmlds + 1024u * w, 1024u * w + 16u * lane);
        }
        if (nt_w > 0) {
            issue(0, 0);
            wait_vmcnt_regs<kDmaPerStage>(qv);
        } else {
            wait_vmcnt_regs<0>(qv);
        }
        if (qall) {
            // the copies before the tiles have landed: hand qa on, take the
            // largest |x| bit pattern (the order of finite bf16 magnitudes)
#pragma unroll
            for (int j = 0; j < kQAllVec; ++j) asm volatile("" : "+v"(qa[j]));
            uint32_t mb = 0;
#pragma unroll
            for (int j = 0; j < kQAllVec; ++j) {
                mb = max(max(mb, qa[j].x & 0x7fffu), (qa[j].x >> 16) & 0x7fffu);
                mb = max(max(mb, qa[j].y & 0x7fffu), (qa[j].y >> 16) & 0x7fffu);
                mb = max(max(mb, qa[j].z & 0x7fffu), (qa[j].z >> 16) & 0x7fffu);
                mb = max(max(mb, qa[j].w & 0x7fffu), (qa[j].w >> 16) & 0x7fffu);
            }
            // (a NaN's bit pattern lies above every other, so NaN propagates)
            const uint32_t m = wave_max_u32(mb << 16);
            uint32_t* red = (uint32_t*)(smem + kRingBytes);  // Q codes are not written yet
            if (lane == 0) red[w] = m;
            __syncthreads();
            q_scale = absmax_to_scale(
                __uint_as_float(max(max(red[0], red[1]), max(red[2], red[3]))));
            __syncthreads();
        } else if (a.blockmax) {
            __syncthreads();
            // rows past nblockmax read as zero, which never raises a maximum;
            // maxima compared as bit patterns, so that a NaN partial wins
            const uint32_t* bm = (const uint32_t*)(smem + kRingBytes + kQBytes);
            const uint32_t m = wave_max_u32(
                max(max(bm[tid], bm[tid + 256]), max(bm[tid + 512], bm[tid + 768])));
            uint32_t* red = (uint32_t*)(smem + kRingBytes);  // Q codes are not written yet
            if (lane == 0) red[w] = m;
            __syncthreads();
            q_scale = absmax_to_scale(
                __uint_as_float(max(max(red[0], red[1]), max(red[2], red[3]))));
            __syncthreads();
        } else {
            q_scale = q_scale_in;
        }
        // 1152 vectors of 8 bf16 -> 8 codes, into LDS (stored out to q8
        // after the main loop: stores issued here would queue behind the
        // tile copies in flight and hold up the start of the loop)
        q_scale = uniform_f32(q_scale);
        const float q_rcp = 1.0f / q_scale;
        uint2* dstl = (uint2*)(smem + kRingBytes);
        with_div_kind(q_scale, [&](auto kind) {
#pragma unroll
            for (int j = 0; j < kQVec; ++j) {
                const int v = tid + 256 * j;
                if (v < kQBytes / 8) {
                    const uint4 x = make_uint4(qv[j].x, qv[j].y, qv[j].z, qv[j].w);
                    dstl[v] = fp8x8<decltype(kind)::value>(x, q_scale, q_rcp);
                }
            }
        });
        if (nt_w > 1) issue(1, 1);
        __syncthreads();
    }
    const float c_nat = q_scale * ksc * a.sm_scale;
    const LogitScale ls{c_nat * kLog2e, c_nat, a.logit_cap,
                        a.logit_cap > 0.f ? 1.0f / a.logit_cap : 0.f};

    v8i qb[5];
    q_operand(smem + kRingBytes, n16, g, qb);

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

        f8tile::tile(st, qb, tok0, ntok, ls, m_run, l_run, acc, n16, g, k > 0);

        if (k + 2 < nt_w) {
            wait_lgkm0();
            issue(k + 2, s);
        }
    }

    if constexpr (kFused) {
        // the Q codes, still in LDS (the wave merge below stays under it),
        // stored by the sequence's first split only (every split holds the
        // same codes), and the absmax scale
        if (slot < 0 || slot == a.items[2 * blockIdx.x + 1].x) {
            const uint2* srcl = (const uint2*)(smem + kRingBytes);
            uint2* dstg = (uint2*)(a.q8_out + (size_t)b * kQBytes);
            for (int v = tid; v < kQBytes / 8; v += 256) dstg[v] = srcl[v];
        }
        if (a.q_scale_out && blockIdx.x == 0 && tid == 0) a.q_scale_out[0] = q_scale;
    }

    // ---- merge the 4 waves: rows to LDS, one weight per (wave, head), then
    // every thread combines 16-byte pieces in the lane-consecutive map (no
    // LDS bank conflicts, coalesced stores)
    l_run = group4_sum(l_run);
    __syncthreads();
    float* xo = (float*)smem;
    float* mw = xo + kWaves * kHeads * kXoStride;
    float* lw = mw + kWaves * kHeads;
    float* fw = lw + kWaves * kHeads;  // [wave][head]: weight of the wave's rows
    float* hl = fw + kWaves * kHeads;  // [head]: base-2 LSE of the item
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
        fw[tid] = empty ? 0.f : ew * (ksc / L);
        if (ww == 0) hl[hh] = empty ? -INFINITY : M + __log2f(L) - kPScaleLog2;
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
        // Partials are written through to the coherence point; once every
        // wave's stores have completed, the last of the sequence's
        // workgroups to arrive at its counter merges them.
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

namespace {
template <bool kFused, bool kPaged>
void launch_fp8(const Stage1Args& args, int nitems, hipStream_t stream) {
    if (args.kv_nt)
        hipLaunchKernelGGL((stage1_fp8_kernel<kFused, kPaged, true>), dim3(nitems), dim3(256), 0,
                           stream, args);
    else
        hipLaunchKernelGGL((stage1_fp8_kernel<kFused, kPaged, false>), dim3(nitems), dim3(256), 0,
                           stream, args);
}
}  // namespace

hipError_t launch_stage1_fp8(const Stage1Args& args, int nitems, bool fused,
                             hipStream_t stream) {
    if (nitems <= 0) return hipSuccess;
    const bool paged = args.kv_pages != nullptr;
    if (fused && paged)
        launch_fp8<true, true>(args, nitems, stream);
    else if (fused)
        launch_fp8<true, false>(args, nitems, stream);
    else if (paged)
        launch_fp8<false, true>(args, nitems, stream);
    else
        launch_fp8<false, false>(args, nitems, stream);
    return hipGetLastError();
}

}  // namespace mla
