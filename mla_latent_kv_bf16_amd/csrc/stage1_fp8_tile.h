// One 32-token tile of the FP8 stage-1 computation, shared by the kernels
// that stream tiles through LDS (one query row per workgroup, and several
// rows of one sequence sharing each tile). gfx950.
//
// Tile layout in LDS: a 576-byte token row is 36 chunks of 16 B; chunk c of
// row t is stored at chunk position c ^ f(t) within its aligned group of four,
// f(t) = ((t >> 2) & 3) ^ (((t >> 1) & 1) << 1), so that the 16-B reads of 8
// or 16 consecutive rows at the same chunk fall in distinct bank groups.
//
// The step for one wave and one 16-head query row [kernelindex.com
// amd-mixed-mla submission 722089, `_mla_multihead_stage1`: all heads per KV
// tile, base-2 online softmax]:
//   S^T = K Q^T on the 16x16x128 FP8 MFMA (M = 16 tokens, N = 16 heads,
//     K = 128 dims; 4 full steps and a 64-dim tail with zeroed upper lane
//     groups); its output already has the layout P needs as the B operand of
//     P.V, so P never leaves registers.
//   Online softmax in base 2 with a lazy reference maximum (it moves only when
//     a tile exceeds it by more than kSlack), P = 2^(x - m) * 2^(8 - kSlack).
//   O^T += V^T P^T on the 16x16x32 FP8 MFMAs, V^T from the transposing LDS
//     read (ds_read_b64_tr_b8), P carried as two FP8 terms: P_hi = e4m3(P)
//     and P_lo = e5m2(P - P_hi) (fp8 x bf8 MFMA). The low term's e5m2 keeps
//     weights far below the row maximum: with an e4m3 low term every P
//     below 2^-10 (2^-16 of the maximum's P) would round to zero, and a long
//     tail of such keys would vanish from P.V while still counted in the
//     softmax sum; e5m2 reaches down to 2^-16.
#pragma once
#include "device_common.h"

namespace mla {
namespace f8tile {

constexpr int kTok = 32;                          // tokens per tile
constexpr int kStageBytes = kTok * kDqk;          // 18432
constexpr int kDmaPerStage = kStageBytes / 1024;  // 18 wave-wide 1 KiB copies
constexpr float kSlack = 2.0f;                    // lazy-max slack, log2 units
constexpr float kPScaleLog2 = 8.0f - kSlack;      // P carries 2^(8 - kSlack)
constexpr float kPScale = 64.0f;                  // 2^kPScaleLog2
typedef int v2i __attribute__((ext_vector_type(2)));

// chunk c of row t sits at byte (t * 36 + (c ^ swz(t))) * 16 of the stage
__device__ __forceinline__ int swz(int t) { return ((t >> 2) & 3) ^ (((t >> 1) & 1) << 1); }

__device__ __forceinline__ v8i cat8(uint4 a, uint4 b) {
    v8i r;
    r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
    r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
    return r;
}

// Per-lane source offsets (relative to the tile's first row) of the 18
// wave-wide copies of one tile, matching the swizzled LDS layout: copy i puts
// lane l's 16 bytes at LDS byte 1024 i + 16 l.
__device__ __forceinline__ void dma_offsets(int lane, uint32_t (&off)[kDmaPerStage]) {
#pragma unroll
    for (int i = 0; i < kDmaPerStage; ++i) {
        const int s = i * 64 + lane;
        const int t = s / kRowChunks;
        const int cp = s - t * kRowChunks;
        off[i] = (uint32_t)(t * kDqk + ((cp ^ swz(t)) * 16));
    }
}

// Q codes of one 16-head row as the B operand of S^T = K Q^T: lane (head n16,
// lane group g) holds dims [128 ks + 32 g, +32) for ks < 4; the tail step
// holds dims 512 + 32 g for g < 2 and zeros for g >= 2. qrow points at the
// row's 16 x 576 codes (LDS or registers' source).
__device__ __forceinline__ void q_operand(const uint8_t* qrow, int n16, int g, v8i (&qb)[5]) {
    const uint8_t* q = qrow + n16 * kDqk;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const uint4* p = (const uint4*)(q + 128 * ks + 32 * g);
        qb[ks] = cat8(p[0], p[1]);
    }
    const uint4* p = (const uint4*)(q + 512 + 32 * (g & 1));
    v8i t = cat8(p[0], p[1]);
    const v8i z = {0, 0, 0, 0, 0, 0, 0, 0};
    qb[4] = g < 2 ? t : z;
}

// The tile step in four parts, which tile() runs in order. Tile at LDS `st`; tokens tok0 .. tok0 + 31 of the item, of which
// those at or past `limit` are masked out; c scales the raw products to
// base-2 logits; acc[blk][r] is latent dim 16 blk + 4 g + r of head n16.

// S^T = K Q^T for the tile's two 16-token blocks (this lane: head n16,
// tokens 16 mb + 4 g + i of block mb). The swizzle only permutes chunks
// within aligned groups of four, so every read is one of four per-lane base
// addresses plus a constant: chunk 8 ks + 2 g + e of row t lies at
// t * 576 + 64 (2 ks + g / 2) + 16 ((2 (g & 1) + e) ^ f(t)), and f(t) does not
// depend on the block (f(16 mb + n16) = f(n16)).
__device__ __forceinline__ void tile_scores(const uint8_t* st, const v8i (&qb)[5], int n16, int g,
                                            v4f (&sc)[2]) {
    const int f = swz(n16);
    const uint8_t* row = st + n16 * kDqk;
    const uint8_t* b0 = row + 64 * (g >> 1) + 16 * ((2 * (g & 1)) ^ f);      // e = 0
    const uint8_t* b1 = row + 64 * (g >> 1) + 16 * ((2 * (g & 1) + 1) ^ f);  // e = 1
    const uint8_t* t0 = row + 512 + 16 * ((2 * (g & 1)) ^ f);                // tail, e = 0
    const uint8_t* t1 = row + 512 + 16 * ((2 * (g & 1) + 1) ^ f);            // tail, e = 1
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int ro = mb * 16 * kDqk;
        v4f a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint4 lo = *(const uint4*)(b0 + ro + 128 * ks);
            const uint4 hi = *(const uint4*)(b1 + ro + 128 * ks);
            a4 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cat8(lo, hi), qb[ks], a4, 0,
                                                                  0, 0, 127, 0, 127);
        }
        const uint4 lo = *(const uint4*)(t0 + ro);
        const uint4 hi = *(const uint4*)(t1 + ro);
        const v8i z = {0, 0, 0, 0, 0, 0, 0, 0};
        const v8i at = g < 2 ? cat8(lo, hi) : z;
        sc[mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(at, qb[4], a4, 0, 0, 0, 127,
                                                                  0, 127);
    }
}

// Logit scaling of the tile step: raw products times c give base-2 logits;
// with a soft-cap (cap > 0) the natural-log logit (products times c_nat) is
// capped first.
struct LogitScale {
    float c;        // q_scale * kv_scale * sm_scale * log2(e)
    float c_nat;    // q_scale * kv_scale * sm_scale
    float cap;      // 0 = none
    float inv_cap;  // 1 / cap
};

// Online softmax of the tile: updates the running maximum and sum, returns
// the factor the accumulator must be scaled by and P as two FP8 terms (e4m3
// P_hi, e5m2 P_lo), in the B-operand layout of the P.V product.
__device__ __forceinline__ void tile_softmax(const v4f (&sc)[2], int tok0, int limit,
                                             const LogitScale& ls, int g, float& m_run,
                                             float& l_run, float& alpha, long& p_hi,
                                             long& p_lo) {
    float x[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[mb][i] = sc[mb][i] * ls.c;
    if (ls.cap > 0.f) {  // the same in every lane
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[mb][i] = capped(sc[mb][i] * ls.c_nat, ls.cap, ls.inv_cap);
    }
    float mx = -INFINITY;
    if (tok0 + kTok <= limit) {  // every tile but a range's last
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
                x[mb][i] = tok < limit ? x[mb][i] : -INFINITY;
                mx = fmaxf(mx, x[mb][i]);
            }
    }
    mx = group4_max(mx);
    // The reference max moves only when the tile's max exceeds it by more
    // than kSlack (log2 units), so the accumulator is rarely rescaled; P
    // is then at most 2^kSlack and carries a factor 2^(8 - kSlack), so the
    // largest P code is 256 and the row maximum maps to a power of two.
    const float m_new = (mx > m_run + kSlack) ? mx : m_run;
    alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float p[2][4];
    float psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[mb][i] = __builtin_amdgcn_exp2f(x[mb][i] - m_new) * kPScale;
            psum += p[mb][i];
        }
    l_run = l_run * alpha + psum;

    uint32_t ph[2], pl[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        int h = __builtin_amdgcn_cvt_pk_fp8_f32(p[mb][0], p[mb][1], 0, false);
        h = __builtin_amdgcn_cvt_pk_fp8_f32(p[mb][2], p[mb][3], h, true);
        const v2f d01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
        const v2f d23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
        int l = __builtin_amdgcn_cvt_pk_bf8_f32(p[mb][0] - d01.x, p[mb][1] - d01.y, 0, false);
        l = __builtin_amdgcn_cvt_pk_bf8_f32(p[mb][2] - d23.x, p[mb][3] - d23.y, l, true);
        ph[mb] = (uint32_t)h;
        pl[mb] = (uint32_t)l;
    }
    p_hi = (long)(((uint64_t)ph[1] << 32) | ph[0]);
    p_lo = (long)(((uint64_t)pl[1] << 32) | pl[0]);
}

// acc *= alpha, skipped when no lane's factor differs from 1 (the common case).
__device__ __forceinline__ void tile_rescale(v4f (&acc)[32], float alpha) {
    if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int blk = 0; blk < 32; ++blk) acc[blk] *= alpha;
    }
}

// O^T += V^T P^T, 16 latent dims per MFMA. A transposing LDS read gives lane
// i of lane group g dim 16 blk + i of its 8 tokens: lanes 2j and 2j+1 of the
// group address the two 8-byte halves of token tau_j's 16-byte chunk blk,
// and the read returns, to lane i, byte i of that 16-byte row for each j.
// Chunk blk of row tau lies at 64 (blk / 4) + 16 ((blk & 3) ^ f(tau)): four
// per-lane bases plus constants.
__device__ __forceinline__ void tile_pv(const uint8_t* st, long p_hi, long p_lo,
                                        v4f (&acc)[32], int n16, int g) {
    const int jj = n16 >> 1;
    const int tau = (jj < 4) ? (4 * g + jj) : (16 + 4 * g + (jj - 4));
    const uint8_t* vrow = st + tau * (kRowChunks * 16) + 8 * (n16 & 1);
    const int sw = swz(tau);
    const uint8_t* vb[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) vb[b] = vrow + 16 * (b ^ sw);
#pragma unroll
    for (int b8 = 0; b8 < 32; b8 += 8) {
        long va[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int blk = b8 + q;
            const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i*)(vb[blk & 3] + 64 * (blk >> 2)));
            va[q] = (long)(((uint64_t)(uint32_t)t[1] << 32) | (uint32_t)t[0]);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
            acc[b8 + q] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(va[q], p_hi, acc[b8 + q],
                                                                   0, 0, 0);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            acc[b8 + q] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_bf8(va[q], p_lo, acc[b8 + q],
                                                                   0, 0, 0);
    }
}

// The whole step for the wave's query row. `later`: not the wave's first
// tile (on the first, the accumulators are still zero and need no rescale;
// a NaN score still reaches them through P).
__device__ __forceinline__ void tile(const uint8_t* st, const v8i (&qb)[5], int tok0, int limit,
                                     const LogitScale& ls, float& m_run, float& l_run,
                                     v4f (&acc)[32], int n16, int g, bool later) {
    v4f sc[2];
    tile_scores(st, qb, n16, g, sc);
    float alpha;
    long p_hi, p_lo;
    tile_softmax(sc, tok0, limit, ls, g, m_run, l_run, alpha, p_hi, p_lo);
    if (later) tile_rescale(acc, alpha);
    tile_pv(st, p_hi, p_lo, acc, n16, g);
}

}  // namespace f8tile
}  // namespace mla
