// Stage 1 of the split-KV decode for an MXFP4 latent cache (gfx950).
//
// One workgroup per work item, all 16 heads per KV tile, online softmax in
// base 2, LDS merge of the partial states; the cache format is that of
// kernelindex.com amd-mixed-mla submission 738050 (`_dequantize_mxfp4_inplace`):
// per token 288 bytes of e2m1 pairs (element 2i in the low nibble of byte i)
// and 18 e8m0 scales, one per 32 latent dims.
//
// Decoding V costs more instructions per byte than the FP8 path, so this
// kernel runs two waves per SIMD: 8 waves, each owning a fixed share of the
// item's 32-token tiles (every eighth; of a long item waves 0-3 take the
// larger share), streaming them through a private two-stage LDS ring filled
// by direct buffer->LDS copies and keeping its own online-softmax state over
// all 512 V dims. No barrier in the main loop: the waves drift apart, so one
// wave's matrix work overlaps another's decode on the same SIMD.
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
//   - A stage is 9,216 B of packed rows plus the tile's 576 scale bytes read
//     through a 16-byte aligned window. In the plain form both of a wave's
//     first tiles are in flight from the start. The fused form issues only
//     the first before it converts Q (its codes pass through the last
//     wave's second stage) and the second once every wave holds its Q
//     operand: copies issued earlier queue in front of the bf16 Q rows and
//     stall the issuing wave, which delays the conversion that every wave
//     waits for.
//   - V decode: lane (n16, g) decodes the 32-dim block n16 of its eight
//     tokens (one 16-byte chunk and one e8m0 scale per token).
//   - At the end waves 4-7 hand their state to waves 0-3 through LDS, and
//     the four remaining states are merged as in the FP8 kernel.
//
// Fused form (template flag kFused): the workgroup turns its sequence's bf16
// Q rows into codes itself (rows loaded into registers, codes into wave 7's
// second stage, same arithmetic as the standalone quantiser; an absmax scale
// is reduced from the partial maxima by every wave; the codes are written
// out after the main loop) and a split
// sequence is merged by the last of its workgroups to arrive at the
// sequence's counter, which it resets to zero.
//
// Shared-row form (stage1_mxfp4_rows_kernel): a sequence's 1-4 query rows
// (multi-token prediction) read each tile from HBM once. The 8 waves form
// tile groups of one wave per row; each wave runs the one-row loop above on
// its group's tiles, for its own row up to that row's causal end, and each
// row's group states are merged at the end.
#include "launch.h"
#include "stage_common.h"

namespace mla {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kTok = 32;
constexpr int kNst = 2;                              // LDS stages per wave
constexpr int kRowPacked = kDqk / 2;                 // 288
constexpr int kRowScales = kDqk / 32;                // 18
constexpr int kPackedChunks = kRowPacked / 16;       // 18
constexpr int kPackedBytes = kTok * kRowPacked;      // 9216
constexpr int kScaleWindow = 37 * 16;                // 576 scale bytes + up to 15 of alignment
constexpr int kStageBytes = kPackedBytes + kScaleWindow;  // 9808
constexpr int kPackedCopies = kPackedBytes / 1024;   // 9
constexpr int kDmaPerStage = kPackedCopies + 1;      // + the scale window
constexpr int kRingBytes = kWaves * kNst * kStageBytes;
constexpr int kQBytes = kHeads * kDqk;               // 9216: the item's Q codes
constexpr int kXoStride = kDv + 4;
constexpr float kSlack = 8.0f;                       // lazy-max slack, log2 units
// rows of 4 waves, then per (wave, head) m, l and output weight, then per-head LSE
constexpr int kMergeBytes = 4 * kHeads * kXoStride * 4 + 3 * 4 * kHeads * 4 + kHeads * 4;
constexpr int kLdsBytes = kRingBytes > kMergeBytes ? kRingBytes : kMergeBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
// Pages of 1, 2 or 4 rows: a row's 18 scale bytes start at 18 x its pool
// row, 2-byte aligned, so each row's scales come in as the 5 dwords from the
// dword holding its first byte, into a 20-byte slot of the window (the
// bytes start 0 or 2 bytes into it: 2 x the pool row's lowest bit)
constexpr int kSlot3 = 20;
constexpr int kScaleDwords3 = kTok * kSlot3 / 4;  // 160: three copies of 64 lanes
constexpr int kStageBytes3 = kPackedBytes + kTok * kSlot3;  // 9856
constexpr int kDmaPerStage3 = kPackedCopies + (kScaleDwords3 + 63) / 64;
constexpr int kRingBytes3 = kWaves * kNst * kStageBytes3;
constexpr int kLdsBytes3 = kRingBytes3 > kMergeBytes ? kRingBytes3 : kMergeBytes;
static_assert(kLdsBytes3 <= 160 * 1024, "LDS budget");
static_assert(kQBytes <= kStageBytes, "Q codes fit in one stage");
constexpr int kCodeWave = kWaves - 1;                // its second stage holds the Q codes
constexpr int kQChunks = 9;                          // 16-dim pieces of Q per lane
constexpr int kQVec = (2 * kQBytes / 16 + 511) / 512;  // 16-B bf16 Q vectors per thread
static_assert(kQVec == 3, "bf16 Q rows: 2.25 vectors per thread");
constexpr int kBmVec = kMaxAbsmaxBlocks / 4 / 64;    // 16-B absmax partial vectors per lane
static_assert(kBmVec == 4, "1024 partial maxima over 64 lanes");
// copies in flight at the first wait: Q, the partials, two tiles
static_assert(kQChunks + 2 * kDmaPerStage <= 63 && kQVec + kBmVec + 2 * kDmaPerStage <= 63,
              "within the wait counter");

// A 4-byte buffer load per lane into LDS at lds_base + 4 lane (the dword
// form of the copies above; offsets past the descriptor's range read as
// zeros), with the non-temporal hint when kNt.
template <bool kNt>
__device__ __forceinline__ void lds_dma4_kv(__amdgpu_buffer_rsrc_t rs, uint32_t lds_base,
                                            uint32_t voff) {
    if constexpr (kNt)
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen nt lds"
                     :
                     : "s"(lds_base), "v"(voff), "s"(rs)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                     :
                     : "s"(lds_base), "v"(voff), "s"(rs)
                     : "memory", "m0");
}

// packed chunk c of row t sits at chunk position c ^ fx(t) (within its
// aligned pair), byte (t * 18 + (c ^ fx(t))) * 16 of the stage
__device__ __forceinline__ int fx(int t) { return (t >> 2) & 1; }

// 2^(s - 127) for an e8m0 byte; 255 (NaN) is read as 254 so that a stray
// byte past the item can never turn a zero element into NaN
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
    return __builtin_amdgcn_ldexpf(1.0f, (int)min(s, 254u) - 127);
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

// kPg: 0 contiguous cache; 1 paged, one page per tile (pages of at least 32
// rows); 2 paged, pages of 8 or 16 rows (a separate instance: the gathers'
// registers would otherwise crowd the one-page form).
// kRows: the items of the shared-row schedule (three int4:
// {sequence, kv_begin, kv_end, split (-1: the item covers the sequence)},
// {first query row, rows R, end of the sequence's cache rows, splits S},
// {first partial slot, first page-table entry, pages, -} (the page-table
// slice of a paged sequence); row r of split s writes slot first + r S + s),
// whose R <= Rp query rows share every tile: the 8 waves form 8 / Rp tile
// groups of Rp waves, one wave per row, and every wave streams its group's
// tiles through its own stages as in the one-row form. A row sees the
// sequence's cache rows up to its causal end (row i of R: all but the last
// R - 1 - i), so a wave's tiles are those of its row.
template <bool kFused, bool kNt, int kPg, bool kRows, int Rp>
__device__ __forceinline__ void mx_body(const Stage1Args& a, uint8_t* smem) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15;
    const int g = lane >> 4;

    constexpr bool kPaged = kPg != 0;
    static_assert(!kRows || !kNt, "shared rows: cached loads");
    constexpr int kStage = kPg == 3 ? kStageBytes3 : kStageBytes;  // bytes per LDS stage
    constexpr int kDma = kPg == 3 ? kDmaPerStage3 : kDmaPerStage;   // copies per tile
    constexpr int kSr = kPg == 3 ? kSlot3 : kRowScales;              // scale row stride in LDS
    static_assert(kRows || Rp == 1, "one row per item");
    constexpr int kItemWords = kRows ? 3 : (kFused || kPaged) ? 2 : 1;  // int4 per item
    constexpr int G = kWaves / Rp;  // tile groups
    constexpr int H = G / 2;        // groups of the older wave of each SIMD
    const int tg = w / Rp, r = w % Rp;
    const int4 it = a.items[kItemWords * blockIdx.x];
    int4 rx = make_int4(0, 1, 0, 0);   // rows form: {first query row, R, end, S}
    int4 rx2 = make_int4(0, 0, 0, 0);  // ... {first partial slot, first page entry, pages, -}
    if constexpr (kRows) {
        rx = a.items[3 * blockIdx.x + 1];
        rx2 = a.items[3 * blockIdx.x + 2];
    }
    const int rbase = rx2.x;
    const int b = it.x, kb = it.y, ke = it.z;
    const int slot = kRows ? (it.w < 0 ? -1 : rbase + r * rx.w + it.w) : it.w;
    const int first_row = kRows ? rx.x : b;  // the item's first query row
    const bool live = !kRows || r < rx.y;
    const int ntok = ke - kb;
    // cache rows of the item this wave's query row sees
    int nvis = ntok;
    if constexpr (kRows) {
        const int v = rx.z - (rx.y - 1 - r) - kb;
        nvis = live ? (v < 0 ? 0 : (v > ntok ? ntok : v)) : 0;
    }
    const int ntile = (nvis + kTok - 1) / kTok;
    // This wave's tiles. The SIMD issues the older of its two waves first,
    // so while both stream, waves 4-7 progress at about a third of the rate
    // of waves 0-3. An item of at least three rounds of G tiles therefore
    // gives its last tiles to the groups of waves 0-3 alone. With cached
    // loads (the cache may sit in the last-level cache) waves 4-7 take a
    // quarter of the tiles; streamed past the caches, where both waves of a
    // SIMD wait on HBM alike, and in the shared-row form, waves 0-3 take the
    // last two rounds alone. Tile order within each wave is fixed, so results
    // stay deterministic.
    const int m8 = ntile >= 3 * G ? ((!kNt && !kRows) ? ntile / (2 * G) : ntile / G - 2)
                                  : (ntile + G - 1) / G;
    const int tail = ntile >= 3 * G ? ntile - G * m8 : 0;
    const int nt_w = tail ? (tg < H ? m8 + (tail - tg + H - 1) / H : m8)
                          : (ntile > tg ? (ntile - tg + G - 1) / G : 0);
    auto tidx = [&](int k) { return k < m8 ? tg + G * k : G * m8 + tg + H * (k - m8); };
    // read before any store so that it stays a scalar load (a vector load
    // here would make the compiler drain the tile copies at its first use)
    const float q_scale_in = a.q_scale ? a.q_scale[0] : 0.f;

    // DMA source offsets of the 9 packed copies of a tile, matching the
    // swizzled layout (copy i puts lane l's 16 bytes at 1024 i + 16 l)
    uint32_t dma_off[kPackedCopies];
#pragma unroll
    for (int i = 0; i < kPackedCopies; ++i) {
        const int s = i * 64 + lane;
        const int t = s / kPackedChunks;
        const int cp = s - t * kPackedChunks;
        dma_off[i] = (uint32_t)(t * kRowPacked + ((cp ^ fx(t)) * 16));
    }

    auto stage_off = [](int wv, int s) { return (wv * kNst + s) * kStage; };
    const uint32_t ring = lds_addr(smem) + (uint32_t)stage_off(w, 0);
    const uint8_t* item_p = a.kv + (size_t)kb * kRowPacked;
    const uint32_t item_pbytes = (uint32_t)ntok * kRowPacked;
    // The buffer range check works per dword, so the scale window ends at the
    // dword holding the item's last scale byte (18 * rows is only even). That
    // dword lies in the same page as the byte, so the read is always mapped;
    // bytes past the item are never used for a valid token.
    const uintptr_t scales_end =
        ((uintptr_t)(a.kv_scales + (size_t)ke * kRowScales) + 3) & ~(uintptr_t)3;

    auto tile_scales = [&](int k) -> uintptr_t {
        return (uintptr_t)(a.kv_scales + ((size_t)kb + (size_t)tidx(k) * kTok) * kRowScales);
    };

    // paged cache (pages of 8, 16 or at least 32 rows): the item's
    // page-table slice; kb and ke are positions in the sequence
    __amdgpu_buffer_rsrc_t pages_rs;
    if constexpr (kPaged && kRows) {
        pages_rs = make_rsrc(a.kv_pages + rx2.y, (uint32_t)rx2.z * 4u);
    } else if constexpr (kPaged) {
        const int4 ex = a.items[2 * blockIdx.x + 1];  // {first slot, splits, page start, pages}
        pages_rs = make_rsrc(a.kv_pages + ex.z, (uint32_t)ex.w * 4u);
    }

    // pages of 1, 2 or 4 rows: per stage, bit t set when row t's scale bytes
    // start 2 bytes into their slot
    uint32_t msk0 = 0u, msk1 = 0u;

    // this wave's k-th tile into its stage s
    auto issue = [&](int k, int s) {
        const uint32_t dst = ring + (uint32_t)(s * kStage);
        if constexpr (!kPaged) {
            const uint32_t toff = (uint32_t)tidx(k) * kPackedBytes;
            const __amdgpu_buffer_rsrc_t rp = make_rsrc(item_p + toff, item_pbytes - toff);
#pragma unroll
            for (int i = 0; i < kPackedCopies; ++i)
                lds_dma16_kv<kNt>(rp, dst + 1024u * i, dma_off[i]);
            const uintptr_t a0 = tile_scales(k) & ~(uintptr_t)15;
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc((const void*)a0, (uint32_t)(scales_end - a0));
            if (lane < kScaleWindow / 16) lds_dma16_kv<kNt>(rs, dst + kPackedBytes, 16u * lane);
        } else if constexpr (kPg == 1) {
            // the tile's page, then both descriptors rebased on its first row
            // (a page id outside the pool reads as zero codes: no rows)
            const int tt = tidx(k) * kTok;  // first row of the tile in the item
            const int tile_tok = kb + tt;   // ... and in its sequence (a multiple of 32)
            const int rem = ntok - tt;      // rows of the tile inside the item
            const v8i pg = load_pages8(pages_rs, (uint32_t)(tile_tok >> a.page_shift) * 4u);
            const uint32_t pid = (uint32_t)__builtin_amdgcn_readfirstlane(pg[0]);
            const bool in_pool = pid < (uint32_t)a.num_pages;
            const size_t row0 = in_pool ? ((size_t)pid << a.page_shift) +
                                              (size_t)(tile_tok & ((1 << a.page_shift) - 1))
                                        : 0;
            const uint32_t nrow = in_pool ? (uint32_t)(rem < kTok ? rem : kTok) : 0u;
            const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.kv + row0 * kRowPacked, nrow * kRowPacked);
#pragma unroll
            for (int i = 0; i < kPackedCopies; ++i)
                lds_dma16_kv<kNt>(rp, dst + 1024u * i, dma_off[i]);
            // row0 is a multiple of 32, so the tile's scales start 16-byte
            // aligned (576 B per 32 rows); the window ends at the dword of
            // the last row's last scale byte
            const uintptr_t a0 = (uintptr_t)(a.kv_scales + row0 * kRowScales);
            const uintptr_t end = (a0 + (uintptr_t)nrow * kRowScales + 3) & ~(uintptr_t)3;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc((const void*)a0, (uint32_t)(end - a0));
            if (lane < kScaleWindow / 16) lds_dma16_kv<kNt>(rs, dst + kPackedBytes, 16u * lane);
        } else if constexpr (kPg == 2) {
            // pages of 8 or 16 rows: the tile's 2 or 4 page ids come in as
            // scalars; each code copy's lanes gather their rows from the
            // whole pool (a lane's row is its offset / 288, recomputed here
            // rather than kept across the loop), and a page's P x 18 scale
            // bytes (a multiple of 16, so 16-byte aligned in the pool) are
            // 9P/8 of the window's 16-byte pieces, in page order. Rows past
            // the item and pages outside the pool read as zeros (the scale
            // bytes of a page's rows past the item are never used for a
            // valid token).
            const int shift = a.page_shift;
            const int tt = tidx(k) * kTok;
            const int tile_tok = kb + tt;
            const int rem = ntok - tt;
            const v8i pg = load_pages8(pages_rs, (uint32_t)(tile_tok >> shift) * 4u);
            auto page = [&](uint32_t j) -> uint32_t {
                return j == 0u ? (uint32_t)pg[0] : j == 1u ? (uint32_t)pg[1]
                                                 : j == 2u ? (uint32_t)pg[2] : (uint32_t)pg[3];
            };
            const uint32_t pool_rows = (uint32_t)a.num_pages << shift;
            const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.kv, pool_rows * (uint32_t)kRowPacked);
#pragma unroll
            for (int i = 0; i < kPackedCopies; ++i) {
                uint32_t d = dma_off[i];
                asm volatile("" : "+v"(d));
                const uint32_t t = d / (uint32_t)kRowPacked;  // row of this lane's chunk
                const uint32_t pid = page(t >> shift);
                const uint32_t phys = (pid << shift) | (t & ((1u << shift) - 1u));
                const bool ok = (int)t < rem && pid < (uint32_t)a.num_pages;
                const uint32_t voff = ok ? d + (phys - t) * (uint32_t)kRowPacked
                                         : 0xfffffff0u;  // past the pool: zeros
                lds_dma16_kv<kNt>(rp, dst + 1024u * i, voff);
            }
            uint32_t ln = (uint32_t)lane;  // (recomputed per tile, as the rows are)
            asm volatile("" : "+v"(ln));
            const uint32_t per = (9u << shift) / 8u;  // 16-byte pieces of scales per page
            const uint32_t piece = ln / per;
            const uint32_t spid = page(piece & 3u);
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc(a.kv_scales, pool_rows * (uint32_t)kRowScales);
            const bool sok = ln < (uint32_t)(kTok * kRowScales / 16) &&
                             (int)(piece << shift) < rem && spid < (uint32_t)a.num_pages;
            const uint32_t soff = sok ? spid * ((uint32_t)kRowScales << shift) +
                                            16u * (ln - piece * per)
                                      : 0xfffffff0u;
            if (lane < kScaleWindow / 16) lds_dma16_kv<kNt>(rs, dst + kPackedBytes, soff);
        } else {
            // pages of 1, 2 or 4 rows: lane j < 32 holds the id of the
            // tile's j-th page; each copy's lanes find their rows' pages
            // through it (rows past the item and pages outside the pool read
            // as zeros)
            const int shift = a.page_shift;
            const int tt = tidx(k) * kTok;
            const int tile_tok = kb + tt;
            const int rem = ntok - tt;
            const uint32_t first = (uint32_t)(tile_tok >> shift) * 4u;
            int tbl = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const v8i pg = load_pages8(pages_rs, first + 32u * q);
#pragma unroll
                for (int e = 0; e < 8; ++e) tbl = (lane == 8 * q + e) ? pg[e] : tbl;
            }
            const uint32_t low = (1u << shift) - 1u;
            const uint32_t pool_rows = (uint32_t)a.num_pages << shift;
            const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.kv, pool_rows * (uint32_t)kRowPacked);
#pragma unroll
            for (int i = 0; i < kPackedCopies; ++i) {
                uint32_t d = dma_off[i];
                asm volatile("" : "+v"(d));
                const uint32_t t = d / (uint32_t)kRowPacked;  // row of this lane's chunk
                const uint32_t pid =
                    (uint32_t)__builtin_amdgcn_ds_bpermute((int)((t >> shift) * 4u), tbl);
                const uint32_t phys = (pid << shift) | (t & low);
                const bool ok = (int)t < rem && pid < (uint32_t)a.num_pages;
                const uint32_t voff = ok ? d + (phys - t) * (uint32_t)kRowPacked
                                         : 0xfffffff0u;  // past the pool: zeros
                lds_dma16_kv<kNt>(rp, dst + 1024u * i, voff);
            }
            // the scale pool's range ends at the dword holding its last byte
            // (in the same page as that byte, so always mapped)
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc(a.kv_scales, (pool_rows * (uint32_t)kRowScales + 3u) & ~3u);
#pragma unroll
            for (int j = 0; j < (kScaleDwords3 + 63) / 64; ++j) {
                uint32_t dw = (uint32_t)(64 * j + lane);  // dword of the window
                asm volatile("" : "+v"(dw));
                const uint32_t t = dw / 5u, wd = dw - 5u * t;
                const uint32_t pid =
                    (uint32_t)__builtin_amdgcn_ds_bpermute((int)(((t & 31u) >> shift) * 4u), tbl);
                const uint32_t phys = (pid << shift) | (t & low);
                const bool ok = (int)t < rem && pid < (uint32_t)a.num_pages;
                const uint32_t soff = ok ? ((phys * (uint32_t)kRowScales) & ~3u) + 4u * wd
                                         : 0xfffffffcu;
                if (dw < (uint32_t)kScaleDwords3)
                    lds_dma4_kv<kNt>(rs, dst + kPackedBytes + 256u * j, soff);
            }
            // a row's scales start 2 bytes into its slot when its pool row is
            // odd: with pages of 2 or 4 rows that is every odd row of the tile
            const uint32_t m =
                shift == 0 ? (uint32_t)__builtin_amdgcn_ballot_w64(lane < 32 && (tbl & 1))
                           : 0xaaaaaaaau;
            if (s)
                msk1 = m;
            else
                msk0 = m;
        }
    };

    // Prologue. Plain form: the lane's share of the item's Q codes (the B
    // operand of S^T = K Q^T: head n16, dims 128 ks + 16 g + (0..15) and
    // 128 ks + 64 + 16 g + (0..15) for ks < 4, and 512 + 16 g + (0..15))
    // comes straight into registers, and both of the wave's first tiles are
    // issued behind it; no barrier. Fused form: the workgroup converts its
    // sequence's bf16 Q rows once (2.25 vectors per thread) into wave 7's
    // second stage, every wave reads its operand from there, and the second
    // tiles follow the barrier after that read.
    auto q_dim = [&](int c) { return c < 8 ? 128 * (c >> 1) + 64 * (c & 1) + 16 * g : 512 + 16 * g; };
    float q_scale;
    v8i qb[5];
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (!kFused) {
        q_scale = q_scale_in;
        const __amdgpu_buffer_rsrc_t rq =
            make_rsrc(a.q8_in + (size_t)(first_row + (live ? r : 0)) * kQBytes, live ? kQBytes : 0);
        v4u qc[kQChunks];
#pragma unroll
        for (int c = 0; c < kQChunks; ++c)
            qc[c] = load16_async(rq, (uint32_t)(n16 * kDqk + q_dim(c)));
        if (nt_w > 0) issue(0, 0);
        if (nt_w > 1) issue(1, 1);
        if (nt_w > 1)
            wait_vmcnt_regs<2 * kDma>(qc);
        else if (nt_w == 1)
            wait_vmcnt_regs<kDma>(qc);
        else
            wait_vmcnt_regs<0>(qc);
        auto u4 = [](v4u v) { return make_uint4(v.x, v.y, v.z, v.w); };
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qb[ks] = cat8(u4(qc[2 * ks]), u4(qc[2 * ks + 1]));
        qb[4] = cat8(u4(qc[8]), z4);
    } else {
        const int qcodes = stage_off(kCodeWave, 1);  // LDS offset of the item's Q codes
        // bf16 Q rows into registers, vector v = tid + 512 j of 16 B in qv[j]
        // (j = 2 lies past the rows for most threads and reads as zeros); an
        // absmax scale's partial maxima into registers too, then this wave's
        // first tile (its second follows the conversion)
        // (shared rows: the item's Rp rows, those past its R reading as
        // zeros, row i's codes into wave 7 - i's second stage)
        constexpr int kQv = (Rp * 2 * kQBytes / 16 + 511) / 512;
        static_assert(kQv + kBmVec + 2 * kDma <= 63, "within the wait counter");
        const __amdgpu_buffer_rsrc_t rq =
            make_rsrc(a.q_bf16 + (size_t)first_row * kHeads * kDqk,
                      (uint32_t)(kRows ? rx.y : 1) * 2u * kQBytes);
        // offsets from a copy of tid the compiler cannot see through, so that
        // it does not share them with the split merge's equal ones (it kept
        // those live across the kernel and spilled them)
        uint32_t qtid = (uint32_t)tid;
        asm volatile("" : "+v"(qtid));
        v4u qv[kQv];
#pragma unroll
        for (int j = 0; j < kQv; ++j) qv[j] = load16_async(rq, 16u * (qtid + 512u * j));
        // every wave reduces all partial maxima itself (at most 1024: lane l
        // holds 4 l .. 4 l + 3 + 256 j; past nblockmax they read as zero,
        // which never raises a maximum)
        v4u bm[kBmVec];
        if (a.blockmax) {
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.blockmax, (uint32_t)a.nblockmax * 4u);
#pragma unroll
            for (int j = 0; j < kBmVec; ++j) bm[j] = load16_async(rb, 16u * (uint32_t)(lane + 64 * j));
        } else {
#pragma unroll
            for (int j = 0; j < kBmVec; ++j) bm[j] = v4u{0u, 0u, 0u, 0u};
        }
        if (nt_w > 0) {
            issue(0, 0);
            wait_vmcnt<kDma>();
        } else {
            wait_vmcnt<0>();
        }
#pragma unroll
        for (int j = 0; j < kQv; ++j) asm volatile("" : "+v"(qv[j]));
#pragma unroll
        for (int j = 0; j < kBmVec; ++j) asm volatile("" : "+v"(bm[j]));
        if (a.blockmax) {
            // maxima compared as bit patterns, so that a NaN partial wins
            uint32_t m = 0;
#pragma unroll
            for (int j = 0; j < kBmVec; ++j)
                m = max(max(max(m, bm[j].x), bm[j].y), max(bm[j].z, bm[j].w));
            q_scale = absmax_to_scale(__uint_as_float(wave_max_u32(m)));
        } else {
            q_scale = q_scale_in;
        }
        // 1152 vectors of 8 bf16 -> 8 codes (q8 is written from registers
        // after the main loop: stores issued here would queue behind the
        // first tile copies)
        uint2* dstl = (uint2*)(smem + qcodes);
        q_scale = uniform_f32(q_scale);
        const float q_rcp = 1.0f / q_scale;
        with_div_kind(q_scale, [&](auto kind) {
#pragma unroll
            for (int j = 0; j < kQv; ++j) {
                const int v = tid + 512 * j;
                if (v < Rp * kQBytes / 8) {
                    const uint4 x = make_uint4(qv[j].x, qv[j].y, qv[j].z, qv[j].w);
                    if constexpr (Rp == 1) {
                        dstl[v] = fp8x8<decltype(kind)::value>(x, q_scale, q_rcp);
                    } else {
                        const int qr = v / (kQBytes / 8);
                        ((uint2*)(smem + stage_off(kCodeWave - qr, 1)))[v - qr * (kQBytes / 8)] =
                            fp8x8<decltype(kind)::value>(x, q_scale, q_rcp);
                    }
                }
            }
        });
        __syncthreads();
        const uint8_t* qrow = smem + stage_off(kCodeWave - r, 1) + n16 * kDqk;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qb[ks] = cat8(*(const uint4*)(qrow + q_dim(2 * ks)), *(const uint4*)(qrow + q_dim(2 * ks + 1)));
        qb[4] = cat8(*(const uint4*)(qrow + q_dim(8)), z4);
        wait_lgkm0();
        __syncthreads();  // every wave holds Q; wave 7's second stage is free
        if (nt_w > 1) issue(1, 1);
    }
    const float c_nat = q_scale * a.sm_scale;
    const float c = c_nat * kLog2e;
    const float cap = a.logit_cap, inv_cap = cap > 0.f ? 1.0f / cap : 0.f;

    float m_run = -INFINITY, l_run = 0.0f;
    v4f acc[4][8];  // acc[cc][c8][i]: dim 32 (4 g + i) + 8 cc + c8, head n16
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int c8 = 0; c8 < 8; ++c8) acc[cc][c8] = (v4f){0.f, 0.f, 0.f, 0.f};

    for (int k = 0; k < nt_w; ++k) {
        const int s = k & 1;
        if (k + 1 < nt_w)
            wait_vmcnt<kDma>();  // tile k + 1 may still be in flight
        else
            wait_vmcnt<0>();

        const uint8_t* st = smem + stage_off(w, s);
        // row t's scales at ssc + 18 t (a paged tile's window starts at its
        // first scale: the scale pool is 16-byte aligned)
        const uint8_t* ssc =
            st + kPackedBytes + (kPaged ? 0 : (int)(tile_scales(k) & 15u));
        // pages of 1, 2 or 4 rows: row t's scales at ssc + 20 t + mis(t)
        const uint32_t msk = s ? msk1 : msk0;
        auto mis = [&](int t) -> int {
            if constexpr (kPg == 3)
                return (int)((msk >> t) & 1u) * 2;
            else
                return 0;
        };
        const int tok0 = tidx(k) * kTok;

        // ---- S^T = K Q^T (fp4 x fp8, K block scales per token). The chunk
        // swizzle flips bit 0 of the chunk index by fx(t), which for
        // t = 16 mb + n16 is fx(n16): chunk 4 ks + g of row t lies at
        // t * 288 + 64 ks + 16 (g ^ fx(n16)), the tail chunk 16 + (g & 1) at
        // t * 288 + 256 + 16 ((g & 1) ^ fx(n16)), so each read is a per-lane
        // base plus a constant.
        v4f sc[2];
        {
            const int f = fx(n16);
            const uint8_t* kbase = st + n16 * kRowPacked + 16 * (g ^ f);
            const uint8_t* ktail = st + n16 * kRowPacked + 256 + 16 * ((g & 1) ^ f);
            const uint8_t* sbase = ssc + n16 * kSr + g;
            const uint8_t* stail = ssc + n16 * kSr + 16 + (g & 1);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                v4f a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const uint4 kd = *(const uint4*)(kbase + mb * 16 * kRowPacked + 64 * ks);
                    const int sa = sbase[mb * 16 * kSr + mis(16 * mb + n16) + 4 * ks];
                    a4 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        cat8(kd, make_uint4(0u, 0u, 0u, 0u)), qb[ks], a4, 4, 0, 0, sa, 0, 127);
                }
                const uint4 kd = *(const uint4*)(ktail + mb * 16 * kRowPacked);
                const int sa = stail[mb * 16 * kSr + mis(16 * mb + n16)];
                const uint4 z = make_uint4(0u, 0u, 0u, 0u);
                sc[mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    cat8(g < 2 ? kd : z, z), qb[4], a4, 4, 0, 0, g < 2 ? sa : 127, 0, 127);
            }
        }

        // ---- online softmax; lane holds head n16, tokens 16mb + 4g + i
        // (only the item's last tile can hold tokens past its end)
        // (a soft-cap, if any, bends the natural-log logit first)
        float x[2][4];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[mb][i] = sc[mb][i] * c;
        if (cap > 0.f) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) x[mb][i] = capped(sc[mb][i] * c_nat, cap, inv_cap);
        }
        float mx = -INFINITY;
        if (tok0 + kTok <= nvis) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[mb][i]);
        } else {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = tok0 + 16 * mb + 4 * g + i;
                    x[mb][i] = tok < nvis ? x[mb][i] : -INFINITY;
                    mx = fmaxf(mx, x[mb][i]);
                }
        }
        mx = group4_max(mx);
        // lazy reference max: P = 2^(x - m) <= 2^kSlack is exact-range in bf16
        const float m_new = (mx > m_run + kSlack) ? mx : m_run;
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
            for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                for (int c8 = 0; c8 < 8; ++c8) acc[cc][c8] *= alpha;
        }

        // ---- O^T += V^T P^T over the 512 dims. MFMA (cc, c8) has the output
        // rows (dims) 32 m + 8 cc + c8, m < 16, so lane (n16, g) decodes block
        // n16 (dims 32 n16 .. 32 n16 + 31: one 16-byte chunk and one scale
        // per token) of its eight tokens tau = 4 g + r (r < 4) and
        // 12 + 4 g + r (r >= 4). They all have fx(tau) = g & 1, so the chunk
        // lies at tau * 288 + 16 (n16 ^ (g & 1)).
        const uint8_t* vbase = st + 4 * g * kRowPacked + 16 * (n16 ^ (g & 1));
        const uint8_t* vscale = ssc + 4 * g * kSr + n16;
        float vsc[8];  // token r: the block's scale
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int dt = (r < 4) ? r : 12 + r;  // tau - 4 g
            vsc[r] = e8m0_to_f32(vscale[dt * kSr + mis(4 * g + dt)]);
        }
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            // dims 32 n16 + 8 cc .. + 7 of token r; rows past the item hold
            // zero codes, so they decode to +-0
            uint32_t wv[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int dt = (r < 4) ? r : 12 + r;
                wv[r] = *(const uint32_t*)(vbase + dt * kRowPacked + 4 * cc);
            }
            // one dim pair at a time: eight tokens' bf16 pairs, then the two
            // dims' A operands (token-major pairs become dim-major eights)
            auto dim_pair = [&](auto jc) {
                constexpr int j = decltype(jc)::value;
                uint32_t d[8];
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    d[r] = bf2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv[r], vsc[r], j));
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t sel = h ? 0x07060302u : 0x05040100u;
                    const v8bf va = as_v8bf(perm(d[1], d[0], sel), perm(d[3], d[2], sel),
                                            perm(d[5], d[4], sel), perm(d[7], d[6], sel));
                    acc[cc][2 * j + h] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[cc][2 * j + h], 0, 0, 0);
                }
            };
            dim_pair(std::integral_constant<int, 0>{});
            dim_pair(std::integral_constant<int, 1>{});
            dim_pair(std::integral_constant<int, 2>{});
            dim_pair(std::integral_constant<int, 3>{});
        }

        if (k + 2 < nt_w) {
            wait_lgkm0();  // this wave's reads of the stage are done
            issue(k + 2, s);
        }
    }

    if constexpr (kFused) {
        // the Q codes out to q8 from the last wave's B operands (lane
        // (n16, g) holds head n16, dims 128 ks + 16 g and 128 ks + 64 + 16 g,
        // 16 each, and 512 + 16 g), by the sequence's first split only
        // (every split holds the same codes), and the absmax scale
        if (a.blockmax && blockIdx.x == 0 && tid == 0) a.q_scale_out[0] = q_scale;
        bool q_out;
        if constexpr (kRows)
            q_out = tg == G - 1 && live && it.w <= 0;  // one wave per row, first split
        else
            q_out = w == kWaves - 1 && (slot < 0 || slot == a.items[2 * blockIdx.x + 1].x);
        if (q_out) {
            uint8_t* qg = a.q8_out + (size_t)(first_row + r) * kQBytes + n16 * kDqk;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                *(uint4*)(qg + 128 * ks + 16 * g) =
                    make_uint4(qb[ks][0], qb[ks][1], qb[ks][2], qb[ks][3]);
                *(uint4*)(qg + 128 * ks + 64 + 16 * g) =
                    make_uint4(qb[ks][4], qb[ks][5], qb[ks][6], qb[ks][7]);
            }
            *(uint4*)(qg + 512 + 16 * g) = make_uint4(qb[4][0], qb[4][1], qb[4][2], qb[4][3]);
        }
    }

    if constexpr (!kRows || Rp == 1) {
        // ---- merge: waves 4-7 hand their state to waves 0-3, then the four
        // states are weighted and summed
        l_run = group4_sum(l_run);
        __syncthreads();
        float* xo = (float*)smem;
        float* mw = xo + 4 * kHeads * kXoStride;
        float* lw = mw + 4 * kHeads;
        const int slotw = w & 3;
        auto put = [&]() {
            float* row = xo + (slotw * kHeads + n16) * kXoStride;
    #pragma unroll
            for (int cc = 0; cc < 4; ++cc)
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float* dd = row + 128 * g + 32 * i + 8 * cc;
                    *(float4*)dd = make_float4(acc[cc][0][i], acc[cc][1][i], acc[cc][2][i], acc[cc][3][i]);
                    *(float4*)(dd + 4) =
                        make_float4(acc[cc][4][i], acc[cc][5][i], acc[cc][6][i], acc[cc][7][i]);
                }
            if (g == 0) {
                mw[slotw * kHeads + n16] = m_run;
                lw[slotw * kHeads + n16] = l_run;
            }
        };
        if (w >= 4) put();
        __syncthreads();
        if (w < 4) {
            const float mp = mw[w * kHeads + n16], lp = lw[w * kHeads + n16];
            const float M = fmaxf(m_run, mp);
            const float fo = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
            const float fp = (mp == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mp - M);
            const float* row = xo + (w * kHeads + n16) * kXoStride;
    #pragma unroll
            for (int cc = 0; cc < 4; ++cc)
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float* dd = row + 128 * g + 32 * i + 8 * cc;
                    const float4 u = *(const float4*)dd;
                    const float4 v = *(const float4*)(dd + 4);
                    const float pv[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
    #pragma unroll
                    for (int c8 = 0; c8 < 8; ++c8) acc[cc][c8][i] = acc[cc][c8][i] * fo + pv[c8] * fp;
                }
            l_run = l_run * fo + lp * fp;
            m_run = M;
        }
        __syncthreads();  // every partner row has been read
        if (w < 4) put();
        __syncthreads();

        // one weight per (wave, head), then every thread combines 16-byte pieces
        // in the lane-consecutive map (no LDS bank conflicts, coalesced stores)
        float* fw = lw + 4 * kHeads;  // [wave][head]: weight of the wave's rows
        float* hl = fw + 4 * kHeads;  // [head]: base-2 LSE of the item
        if (tid < 4 * kHeads) {
            const int hh = tid & (kHeads - 1), pp = tid >> 4;
            float M = -INFINITY;
    #pragma unroll
            for (int q = 0; q < 4; ++q) M = fmaxf(M, mw[q * kHeads + hh]);
            float L = 0.f, ep = 0.f;
    #pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float mv = mw[q * kHeads + hh];
                const float e = (mv == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mv - M);
                L += e * lw[q * kHeads + hh];
                if (q == pp) ep = e;
            }
            // only for a sequence with no rows (NaN scores leave M at -inf but L NaN)
            const bool empty = (M == -INFINITY) && (L == 0.f);
            fw[tid] = empty ? 0.f : ep / L;
            if (pp == 0) hl[hh] = empty ? -INFINITY : M + __log2f(L);
        }
        __syncthreads();
        using Map = RowMap<512>;
        const int dq = Map::dim(tid);
        float4 o[Map::kPer];
    #pragma unroll
        for (int q = 0; q < Map::kPer; ++q) {
            const int hq = Map::head(tid, q);
            float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
    #pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const float f = fw[pp * kHeads + hq];
                const float4 v = *(const float4*)(xo + (pp * kHeads + hq) * kXoStride + dq);
                s4.x += f * v.x;
                s4.y += f * v.y;
                s4.z += f * v.z;
                s4.w += f * v.w;
            }
            o[q] = s4;
        }
        if (slot < 0) {
            uint16_t* ob = a.out + (size_t)first_row * kHeads * kDv;
    #pragma unroll
            for (int q = 0; q < Map::kPer; ++q)
                *(uint2*)(ob + Map::head(tid, q) * kDv + dq) =
                    make_uint2(pack_bf16x2(o[q].x, o[q].y), pack_bf16x2(o[q].z, o[q].w));
            if (a.lse_out && tid < kHeads) a.lse_out[(size_t)first_row * kHeads + tid] = hl[tid] * kLn2;
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
            int4 ex;  // {first slot, splits, -, -}
            if constexpr (kRows)
                ex = make_int4(rbase, rx.w, 0, 0);
            else
                ex = a.items[2 * blockIdx.x + 1];
            wait_vmcnt<0>();
            __syncthreads();
            uint32_t* flag = (uint32_t*)smem;
            if (tid == 0) flag[0] = (atomicAdd(&a.counters[b], 1u) == (uint32_t)ex.y - 1u);
            __syncthreads();
            if (flag[0]) {
                merge_split<512, true>(a.part_o, a.part_lse, ex.x, ex.y,
                                       a.out + (size_t)first_row * kHeads * kDv,
                                       a.lse_out ? a.lse_out + (size_t)first_row * kHeads : nullptr,
                                       (float*)(smem + 16), tid);
                if (tid == 0)
                    __hip_atomic_store(&a.counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    } else {
        // ---- merge of shared rows: each row's G wave states, in two passes
        // of 4 / G rows (four states of 16 x 512 in LDS at a time)
        constexpr int kRpp = 4 / G;       // rows per pass
        constexpr int kPasses = Rp / kRpp;
        l_run = group4_sum(l_run);
        float* xo = (float*)smem;                 // [state][head][kXoStride]
        float* mw = xo + 4 * kHeads * kXoStride;  // [state][head]
        float* lw = mw + 4 * kHeads;
        using Map = RowMap<512>;
        const int dq = Map::dim(tid);
        const int R = rx.y, S = rx.w, split = it.w;
#pragma unroll
        for (int ps = 0; ps < kPasses; ++ps) {
            __syncthreads();  // the stages (or the previous pass's states) are free
            const int rlo = ps * kRpp;
            if (r >= rlo && r < rlo + kRpp) {
                const int sx = (r - rlo) * G + tg;
                float* row = xo + (sx * kHeads + n16) * kXoStride;
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float* dd = row + 128 * g + 32 * i + 8 * cc;
                        *(float4*)dd =
                            make_float4(acc[cc][0][i], acc[cc][1][i], acc[cc][2][i], acc[cc][3][i]);
                        *(float4*)(dd + 4) =
                            make_float4(acc[cc][4][i], acc[cc][5][i], acc[cc][6][i], acc[cc][7][i]);
                    }
                if (g == 0) {
                    mw[sx * kHeads + n16] = m_run;
                    lw[sx * kHeads + n16] = l_run;
                }
            }
            __syncthreads();
#pragma unroll
            for (int rr = 0; rr < kRpp; ++rr) {
                const int qr = rlo + rr;  // query row of the sequence
                if (qr >= R) break;
                float4 o[Map::kPer];
                float hq2[Map::kPer];
#pragma unroll
                for (int q = 0; q < Map::kPer; ++q) {
                    const int hq = Map::head(tid, q);
                    float M = -INFINITY;
#pragma unroll
                    for (int gj = 0; gj < G; ++gj) M = fmaxf(M, mw[(rr * G + gj) * kHeads + hq]);
                    float e[G], L = 0.f;
#pragma unroll
                    for (int gj = 0; gj < G; ++gj) {
                        const float mv = mw[(rr * G + gj) * kHeads + hq];
                        e[gj] = (mv == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mv - M);
                        L += e[gj] * lw[(rr * G + gj) * kHeads + hq];
                    }
                    // the row sees no cache row of the item (NaN scores leave
                    // M at -inf but L NaN)
                    const bool empty = (M == -INFINITY) && (L == 0.f);
                    hq2[q] = empty ? -INFINITY : M + __log2f(L);
                    float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                    for (int gj = 0; gj < G; ++gj) {
                        const float f = empty ? 0.f : e[gj] / L;
                        const float4 v =
                            *(const float4*)(xo + ((rr * G + gj) * kHeads + hq) * kXoStride + dq);
                        s4.x += f * v.x;
                        s4.y += f * v.y;
                        s4.z += f * v.z;
                        s4.w += f * v.w;
                    }
                    o[q] = s4;
                }
                const bool lse_lane = (tid & 127) == 0;  // heads tid / 128 + 4 q
                if (split < 0) {
                    const size_t orow = (size_t)(first_row + qr);
                    uint16_t* ob = a.out + orow * kHeads * kDv;
#pragma unroll
                    for (int q = 0; q < Map::kPer; ++q)
                        *(uint2*)(ob + Map::head(tid, q) * kDv + dq) =
                            make_uint2(pack_bf16x2(o[q].x, o[q].y), pack_bf16x2(o[q].z, o[q].w));
                    if (a.lse_out && lse_lane) {
#pragma unroll
                        for (int q = 0; q < Map::kPer; ++q)
                            a.lse_out[orow * kHeads + Map::head(tid, q)] = hq2[q] * kLn2;
                    }
                } else {
                    const int ps_slot = rbase + qr * S + split;
                    if constexpr (!kFused) {
                        float* pb = a.part_o + (size_t)ps_slot * kHeads * kDv;
#pragma unroll
                        for (int q = 0; q < Map::kPer; ++q)
                            *(float4*)(pb + Map::head(tid, q) * kDv + dq) = o[q];
                        if (lse_lane) {
#pragma unroll
                            for (int q = 0; q < Map::kPer; ++q)
                                a.part_lse[(size_t)ps_slot * kHeads + Map::head(tid, q)] = hq2[q];
                        }
                    } else {
                        // written through to the coherence point for the
                        // merging workgroup
                        const __amdgpu_buffer_rsrc_t ro =
                            make_rsrc(a.part_o + (size_t)ps_slot * kHeads * kDv, kHeads * kDv * 4);
#pragma unroll
                        for (int q = 0; q < Map::kPer; ++q)
                            store_coherent(ro, (uint32_t)((Map::head(tid, q) * kDv + dq) * 4), o[q]);
                        if (lse_lane) {
                            const __amdgpu_buffer_rsrc_t rl =
                                make_rsrc(a.part_lse + (size_t)ps_slot * kHeads, kHeads * 4);
#pragma unroll
                            for (int q = 0; q < Map::kPer; ++q)
                                store_coherent(rl, (uint32_t)(Map::head(tid, q) * 4), hq2[q]);
                        }
                    }
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
                    for (int qr = 0; qr < R; ++qr) {
                        const size_t orow = (size_t)(first_row + qr);
                        merge_split<512, true>(a.part_o, a.part_lse, rbase + qr * S, S,
                                               a.out + orow * kHeads * kDv,
                                               a.lse_out ? a.lse_out + orow * kHeads : nullptr,
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
}

template <bool kFused, bool kNt, int kPg>
__global__ __launch_bounds__(512) void stage1_mxfp4_kernel(Stage1Args a) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kPg == 3 ? kLdsBytes3 : kLdsBytes];
    mx_body<kFused, kNt, kPg, false, 1>(a, smem);
}

// The shared-row schedule's items: R query rows of one sequence per item,
// the body for Rp = R rounded up to 1, 2 or 4 chosen per workgroup; kPg as
// for the one-row kernel (a paged item keeps positions in the sequence and
// the sequence's page-table slice in its third int4).
template <bool kFused, int kPg>
__global__ __launch_bounds__(512) void stage1_mxfp4_rows_kernel(Stage1Args a) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kPg == 3 ? kLdsBytes3 : kLdsBytes];
    const int R = a.items[3 * blockIdx.x + 1].y;
    if (R <= 1)
        mx_body<kFused, false, kPg, true, 1>(a, smem);
    else if (R == 2)
        mx_body<kFused, false, kPg, true, 2>(a, smem);
    else
        mx_body<kFused, false, kPg, true, 4>(a, smem);
}

}  // namespace

hipError_t launch_stage1_mxfp4(const Stage1Args& args, int nitems, bool fused,
                               hipStream_t stream) {
    if (nitems <= 0) return hipSuccess;
    const dim3 grid(nitems), block(512);
    const bool paged = args.kv_pages != nullptr;
#define MLA_MX_LAUNCH(F, N, P) \
    hipLaunchKernelGGL((stage1_mxfp4_kernel<F, N, P>), grid, block, 0, stream, args)
    if (args.kv_pages && args.page_shift >= 5) {
        if (fused && args.kv_nt) MLA_MX_LAUNCH(true, true, 1);
        else if (fused) MLA_MX_LAUNCH(true, false, 1);
        else if (args.kv_nt) MLA_MX_LAUNCH(false, true, 1);
        else MLA_MX_LAUNCH(false, false, 1);
    } else if (args.kv_pages && args.page_shift >= 3) {
        if (fused && args.kv_nt) MLA_MX_LAUNCH(true, true, 2);
        else if (fused) MLA_MX_LAUNCH(true, false, 2);
        else if (args.kv_nt) MLA_MX_LAUNCH(false, true, 2);
        else MLA_MX_LAUNCH(false, false, 2);
    } else if (args.kv_pages) {
        if (fused && args.kv_nt) MLA_MX_LAUNCH(true, true, 3);
        else if (fused) MLA_MX_LAUNCH(true, false, 3);
        else if (args.kv_nt) MLA_MX_LAUNCH(false, true, 3);
        else MLA_MX_LAUNCH(false, false, 3);
    } else {
        if (fused && args.kv_nt) MLA_MX_LAUNCH(true, true, 0);
        else if (fused) MLA_MX_LAUNCH(true, false, 0);
        else if (args.kv_nt) MLA_MX_LAUNCH(false, true, 0);
        else MLA_MX_LAUNCH(false, false, 0);
    }
#undef MLA_MX_LAUNCH
    return hipGetLastError();
}

hipError_t launch_stage1_mxfp4_rows(const Stage1Args& args, int nitems, bool fused,
                                    hipStream_t stream) {
    if (nitems <= 0) return hipSuccess;
    const int pg = !args.kv_pages          ? 0
                   : args.page_shift >= 5 ? 1
                   : args.page_shift >= 3 ? 2
                                          : 3;
#define MLA_MXR_LAUNCH(F, P) \
    hipLaunchKernelGGL((stage1_mxfp4_rows_kernel<F, P>), dim3(nitems), dim3(512), 0, stream, args)
    if (fused) {
        if (pg == 0) MLA_MXR_LAUNCH(true, 0);
        else if (pg == 1) MLA_MXR_LAUNCH(true, 1);
        else if (pg == 2) MLA_MXR_LAUNCH(true, 2);
        else MLA_MXR_LAUNCH(true, 3);
    } else {
        if (pg == 0) MLA_MXR_LAUNCH(false, 0);
        else if (pg == 1) MLA_MXR_LAUNCH(false, 1);
        else if (pg == 2) MLA_MXR_LAUNCH(false, 2);
        else MLA_MXR_LAUNCH(false, 3);
    }
#undef MLA_MXR_LAUNCH
    return hipGetLastError();
}

}  // namespace mla
