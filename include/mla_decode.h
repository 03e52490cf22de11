/*
 * mla_decode.h -- C ABI of libmla_decode.so: absorbed-path Multi-head Latent
 * Attention decode on one AMD Instinct MI355X (gfx950).
 *
 * What one decode step computes (kernelindex.com "amd-mixed-mla" pages,
 * submissions 663509, 722089, 738050):
 *   16 query heads of 576 dims (one query row per sequence) attend over one
 *   shared latent KV head of 576 dims; K is all 576 dims, V is the first 512,
 *   sm_scale = 1/sqrt(576):  O = softmax(Q K^T * sm_scale) V.
 *   [738050, comment on the `mla_decode_fwd` call in `_run_a8w8`; module
 *    constants of 663509]
 *   Q arrives in bf16 and is quantised per tensor to FP8 E4M3FN before the
 *   attention, with either an absmax scale or a fixed scale.
 *   [722089 `quantize_fp8`; 663509 module docstring, point 1]
 *   The latent cache is FP8 E4M3FN with one per-tensor scale, or MXFP4
 *   (e2m1 pairs per byte plus one e8m0 scale per 32 dims).
 *   [738050 `custom_kernel` docstring and `_dequantize_mxfp4_inplace`]
 *   Work is split along each sequence's KV range and merged by log-sum-exp.
 *   [722089 `_mla_multihead_stage1`, `_mla_reduce`]
 *   Scheduling depends only on the CSR row pointers, so it is computed once
 *   per shape and reused.  [663509 module docstring, point 2]
 *
 * Conventions for every entry point:
 *   - Returns an mla_status (0 = OK). Argument checks finish before any
 *     device work is enqueued, so a failed call has no side effects.
 *   - No C++ exception or abort crosses this interface.
 *   - "device" pointers are HIP device allocations owned by the caller;
 *     "host" pointers are ordinary host memory owned by the caller.
 *   - All tensors are dense, row-major, with the stated shapes (no strides).
 *   - Enqueuing calls take a HIP stream (hipStream_t passed as void*; NULL
 *     is the default stream), enqueue asynchronously and never synchronise;
 *     device faults surface at the caller's next synchronisation.
 *   - Enqueuing calls allocate nothing and copy nothing device-to-host.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MLA_API __attribute__((visibility("default")))
#else
#define MLA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
    MLA_OK = 0,
    MLA_INVALID_ARGUMENT = 1,    /* a pointer, size or index is wrong */
    MLA_UNSUPPORTED = 2,         /* well-formed but outside what is built */
    MLA_HIP_ERROR = 3,           /* a HIP runtime call failed */
    MLA_WORKSPACE_TOO_SMALL = 4, /* workspace_bytes below the plan's need */
    MLA_OUT_OF_MEMORY = 5        /* a host or device allocation failed */
} mla_status;

enum {
    MLA_KV_FP8_E4M3FN = 0,       /* (total_kv, 576) bytes + one fp32 scale */
    MLA_KV_MXFP4 = 1,            /* (total_kv, 288) packed e2m1 + (total_kv, 18) e8m0 */
    MLA_KV_BF16 = 2              /* (total_kv, 576) bf16; runs with mla_decode_run_bf16 */
};

enum {
    MLA_Q_SCALE_STATIC = 0,      /* q_scale[0] is an input, set by the caller */
    MLA_Q_SCALE_ABSMAX = 1       /* q_scale[0] is an output: max|q| (>= 1e-12) / 448 */
};

#define MLA_NUM_HEADS 16
#define MLA_QK_DIM 576
#define MLA_V_DIM 512
#define MLA_MX_BLOCK 32

typedef struct mla_plan* mla_plan_t;  /* opaque, immutable once built */

/*
 * Build the per-shape schedule.  [663509 `_precompute_metadata`: work
 * scheduling depends only on qo_indptr / kv_indptr; K4-style split policy
 * of 722089 `_aiter_path` and 738050 `_get_num_kv_splits`, re-derived here
 * for 256 compute units]
 *   qo_indptr_host, kv_indptr_host: host int32 arrays of batch+1 entries
 *     (CSR row pointers); both start at 0 and never decrease. Sequence b
 *     has R = qo[b+1] - qo[b] query rows (R = 1 for plain decode; R > 1 for
 *     multi-token prediction or speculative rows, any mix per batch). The
 *     rows are the sequence's last R positions, already in its cache: row i
 *     (0-based) attends to the first kv_len - (R - 1 - i) cache rows
 *     (bottom-right aligned causal mask; a row with none gets O = 0 and
 *     LSE = -inf).  [663509 / 722089 / 738050: the causal flag and
 *     max_seqlen_qo passed to the metadata calls]
 *     total_q = qo_indptr[batch] rows are decoded; every per-row tensor below
 *     ("rows") has total_q rows. With 1..4 rows in every sequence (more
 *     than one in some), a sequence's rows share each cache tile, which is
 *     read once for all of them: always for the FP8 cache, and for the MXFP4
 *     cache when the per-row schedule would have more work items than
 *     num_cus (in one round of workgroups per-row items finish sooner, as a
 *     shared MXFP4 item decodes V once per row). Otherwise every query row
 *     is scheduled on its own range (the schedule mla_decode_plan_host
 *     returns).
 *   batch >= 0; num_heads must be 16; kv_format is MLA_KV_*.
 *   num_cus: compute units to schedule for; 0 queries the current device.
 *   max_splits: 0 = policy; > 0 caps the splits of any one sequence;
 *     < 0 forces -max_splits splits per sequence (clipped to at most 64
 *     and so that no split is empty), for experiments. Whatever the
 *     request, an item covers at most 2^22 cache rows (2^21 for the bf16
 *     cache, so that an item's bytes stay below 2^32), so a longer query
 *     row gets more splits than asked for (at most 512).
 *   stream: the HIP stream (hipStream_t as void*, NULL = the default
 *     stream) on which the work lists are copied to the device.
 *   *out receives the plan. The plan owns a small device copy of its work
 *   list, allocated here with hipMalloc (on the current device) and freed by
 *   mla_decode_plan_destroy. The copies are enqueued on `stream` and the call
 *   then waits for that stream (hipStreamSynchronize), and so for whatever
 *   was queued on it before; work on other streams keeps running. The plan
 *   is ready for runs on any stream when the call returns.
 * Errors: INVALID_ARGUMENT (null pointers, bad indptr, batch < 0),
 *   UNSUPPORTED (num_heads != 16, unknown kv_format, more than
 *   2^31 / 16 query rows, a bf16-cache row range of more than 2^30 rows),
 *   HIP_ERROR.
 */
MLA_API int mla_decode_plan(const int32_t* qo_indptr_host, const int32_t* kv_indptr_host,
                    int32_t batch, int32_t num_heads, int32_t kv_format, int32_t num_cus,
                    int32_t max_splits, void* stream, mla_plan_t* out);

/*
 * Host-only form of the scheduler (no HIP call; usable without a GPU).
 * Same validation as mla_decode_plan with num_cus 0 meaning 256.
 *   items_out: host int32 array with room for items_cap * 4 entries; each
 *     work item is {sequence b, kv_begin, kv_end, slot} where [kv_begin,
 *     kv_end) are absolute cache rows and slot is the partial-result slot
 *     (-1 = the item covers its whole sequence and writes the output).
 *   merge_out: host int32 array with room for merge_cap * 4 entries; each
 *     entry is {sequence b, first slot, number of slots, 0} for a sequence
 *     whose result is assembled by the merge (split sequences, and empty
 *     sequences with 0 slots).
 *   counts_out: host int32[3] = {num_items, num_merge, num_slots}.
 *   Either array may be NULL with cap 0 to query the counts only;
 *   INVALID_ARGUMENT if a non-NULL array is too small.
 */
MLA_API int mla_decode_plan_host(const int32_t* qo_indptr_host, const int32_t* kv_indptr_host,
                         int32_t batch, int32_t num_heads, int32_t kv_format,
                         int32_t num_cus, int32_t max_splits, int32_t* items_out,
                         int32_t items_cap, int32_t* merge_out, int32_t merge_cap,
                         int32_t* counts_out);

/* counts_out: host int32[4] = {num_items, num_merge, num_slots, total_q rows}. */
MLA_API int mla_decode_plan_counts(mla_plan_t plan, int32_t* counts_out);

/*
 * Device workspace needed by mla_decode_run for this plan, in bytes
 * (split partials plus the Q absmax partials).  Layout, for tests:
 *   [0, S*16*512*4): fp32 partial O, slot-major (slot, head, dim), each
 *     normalised by its own softmax sum;
 *   then S*16 fp32 partial LSE in base 2 of the logits scaled by
 *     sm_scale*log2(e) (slot, head);
 *   then the quantiser's scratch;
 *   then one uint32 arrival counter per query row, used by
 *   mla_decode_run_fused.
 * with S = num_slots and every region starting on a 256-byte boundary.
 * [722089 `_custom_multihead_path`: Mid_O, Mid_LSE]
 */
MLA_API int mla_decode_workspace_size(mla_plan_t plan, size_t* bytes);

/*
 * One decode step, enqueued on `stream`:
 *   (1) Q bf16 -> FP8 E4M3FN (absmax scale: two launches; static: one),
 *   (2) split-KV attention over the plan's work items,
 *   (3) log-sum-exp merge of split sequences (skipped if none).
 * Device pointers (all caller-owned):
 *   q_bf16       (rows, 16, 576) bf16, input.
 *   q_fp8        (rows, 16, 576) bytes, output: the e4m3fn codes.
 *   q_scale      fp32[1]: input for MLA_Q_SCALE_STATIC, output for ABSMAX.
 *   kv           FP8: (total_kv, 576) e4m3fn codes; MXFP4: (total_kv, 288)
 *                packed e2m1, element 2i in the low nibble of byte i.
 *   kv_block_scales MXFP4: (total_kv, 18) e8m0 bytes; FP8: must be NULL.
 *   q_bf16, q_fp8, kv, kv_block_scales and out_bf16 must be 16-byte aligned.
 *   kv_scale     FP8: fp32[1] per-tensor scale; MXFP4: must be NULL.
 *   sm_scale     host float, normally 1/sqrt(576); must be finite and > 0.
 *   logit_cap    host float, 0 = none; > 0 replaces each scaled logit s by
 *                logit_cap * tanh(s / logit_cap) before the softmax (also
 *                in lse_out); must be finite and >= 0. [the `logit_cap`
 *                argument of the pages' FP8 decode calls: 663509
 *                `custom_kernel`, 738050 `_run_a8w8`; 0 on every page]
 *   workspace    at least mla_decode_workspace_size bytes (may be NULL if
 *                that size is 0), 256-byte aligned.
 *   out_bf16     (rows, 16, 512) bf16, output.
 *   lse_out      optional (rows, 16) fp32 natural-log LSE of the scaled
 *                scores, or NULL.
 * Errors: INVALID_ARGUMENT, WORKSPACE_TOO_SMALL, HIP_ERROR (launch failure).
 * Concurrent runs of one plan are safe on distinct workspaces and outputs.
 */
MLA_API int mla_decode_run(mla_plan_t plan, const void* q_bf16, void* q_fp8, float* q_scale,
                   int32_t q_scale_mode, const void* kv, const void* kv_block_scales,
                   const float* kv_scale, float sm_scale, float logit_cap, void* workspace,
                   size_t workspace_bytes, void* out_bf16, float* lse_out, void* stream);

/*
 * Zero the arrival counters of a workspace for mla_decode_run_fused (a fill
 * kernel enqueued on `stream`, so it can be captured in a graph). Needed
 * once before the first fused run of `plan` on this workspace, and again if
 * the workspace has been used with another plan since: every fused run
 * leaves the counters at zero, and the other entry points do not touch them.
 * workspace: device, at least mla_decode_workspace_size bytes, 256-aligned.
 * Errors: INVALID_ARGUMENT, WORKSPACE_TOO_SMALL, HIP_ERROR.
 */
MLA_API int mla_decode_workspace_init(mla_plan_t plan, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * The decode step of mla_decode_run in one launch (static Q scale) or two
 * (absmax scale: the partial maxima, then the attention; one for an FP8
 * cache with at most 4 query rows, whose workgroups each reduce the absmax
 * of all of Q, for every finite Q the same scale): every stage-1
 * workgroup quantises its own sequence's Q rows (identical codes to the
 * standalone quantiser; the sequence's first split stores them to
 * q_fp8), and the last workgroup of a split sequence to finish, found by
 * an atomic counter per sequence, merges its partials. Arguments, outputs
 * and errors as in mla_decode_run; in addition the workspace must have been
 * prepared by mla_decode_workspace_init for this plan, and for the FP8 cache
 * kv_scale must be non-NULL whenever rows > 0. Outputs equal those of
 * mla_decode_run bit for bit. Concurrent fused runs must use distinct
 * workspaces. [663509 module docstring: fewer launches per decode step;
 * 722089 `_mla_multihead_stage1`, `_mla_reduce`]
 */
MLA_API int mla_decode_run_fused(mla_plan_t plan, const void* q_bf16, void* q_fp8, float* q_scale,
                         int32_t q_scale_mode, const void* kv, const void* kv_block_scales,
                         const float* kv_scale, float sm_scale, float logit_cap, void* workspace,
                         size_t workspace_bytes, void* out_bf16, float* lse_out, void* stream);

/*
 * mla_decode_run_fused without a workspace argument, for callers that cannot
 * allocate device memory or call hipMalloc (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). The workspace is a
 * fixed array inside the library, one per device (16,682,240 bytes, held
 * until the process ends); the call allocates nothing. Its first call on a
 * device resolves that array's address and enqueues one fill kernel on
 * `stream` that zeroes its arrival counters; every fused run leaves them at
 * zero again. All calls on one device share the array: calls that overlap
 * on one device (concurrent streams or threads) race and give wrong
 * results; order them, or use mla_decode_run_fused with distinct
 * workspaces. A call that did not complete (a device fault) leaves the
 * counters undefined.
 * Arguments, outputs and errors as mla_decode_run_fused, without workspace
 * and workspace_bytes; contiguous plans only (a paged or bf16 plan:
 * INVALID_ARGUMENT). A plan with more than 65,536 query rows or more than
 * 500 partial slots (mla_decode_plan_counts) is rejected with
 * WORKSPACE_TOO_SMALL before any launch. Outputs equal those of
 * mla_decode_run_fused bit for bit.
 */
MLA_API int mla_decode_run_fused_noalloc(mla_plan_t plan, const void* q_bf16, void* q_fp8,
                                         float* q_scale, int32_t q_scale_mode, const void* kv,
                                         const void* kv_block_scales, const float* kv_scale,
                                         float sm_scale, float logit_cap, void* out_bf16,
                                         float* lse_out, void* stream);

/*
 * One decode step for a plan made with kv_format MLA_KV_BF16 (the pages'
 * bf16 path, the counterpart of their a8w8 mode: bf16 Q against the bf16
 * cache, no quantisation), in one
 * launch: split sequences are merged by their last workgroup, so the
 * workspace must have been prepared by mla_decode_workspace_init.
 *   q_bf16       device (rows, 16, 576) bf16; kv_bf16 device (total_kv, 576)
 *                bf16; both 16-byte aligned.
 *   logit_cap    0 = none; > 0 replaces each scaled logit s by
 *                logit_cap * tanh(s / logit_cap) before the softmax.
 *   lse_out      optional, the natural-log LSE of the (capped) logits.
 * Other arguments as mla_decode_run_fused. The other run entry points reject
 * a bf16 plan (INVALID_ARGUMENT) and this one rejects other plans, paged
 * bf16 plans included (those run through mla_decode_run_bf16_paged).
 * [722089 `_aiter_path`: bf16 Q and cache below its FP8 threshold; the
 * `logit_cap` argument of the decode calls, 0 on every page]
 */
MLA_API int mla_decode_run_bf16(mla_plan_t plan, const void* q_bf16, const void* kv_bf16,
                                float sm_scale, float logit_cap, void* workspace,
                                size_t workspace_bytes, void* out_bf16, float* lse_out,
                                void* stream);

/*
 * mla_decode_run_bf16 for a paged bf16 plan (mla_decode_plan_paged with
 * kv_format MLA_KV_BF16).
 *   kv_pool      device (num_pages * page_size, 576) bf16, 16-byte aligned.
 *   kv_page_ids, num_pages  as mla_decode_run_paged. A page id outside
 *                [0, num_pages) reads as zero rows. With page_size < 16 the
 *                pool must stay below 4 GiB (num_pages * page_size * 1152
 *                bytes), else UNSUPPORTED.
 * Other arguments, outputs and errors as mla_decode_run_bf16; a plan that is
 * not a paged bf16 plan gives INVALID_ARGUMENT.
 * [663509 / 738050: the paged (pages, page_size, 1, 576) cache view;
 * 722089 `_aiter_path`: the bf16 cache]
 */
MLA_API int mla_decode_run_bf16_paged(mla_plan_t plan, const void* q_bf16, const void* kv_pool,
                                      const int32_t* kv_page_ids, int32_t num_pages,
                                      float sm_scale, float logit_cap, void* workspace,
                                      size_t workspace_bytes, void* out_bf16, float* lse_out,
                                      void* stream);

/*
 * Paged latent cache: the cache is a pool of pages of page_size rows in one
 * of the contiguous cache's row formats (FP8: (num_pages * page_size, 576)
 * e4m3fn codes; MXFP4: (num_pages * page_size, 288) packed codes beside
 * (num_pages * page_size, 18) E8M0 scales; bf16: (num_pages * page_size,
 * 576) bf16, run with mla_decode_run_bf16_paged), and sequence b owns the
 * pages kv_page_ids[kv_page_indptr[b] .. kv_page_indptr[b+1]) in order; its
 * last page holds kv_last_page_len[b] rows (1..page_size; ignored for a
 * sequence with no page).  [663509 / 738050: kv_buffer viewed as (pages,
 * page_size, 1, 576) with kv_indptr, kv_indices and kv_last_page_len]
 *   qo_indptr_host, kv_page_indptr_host: host int32 (batch + 1) row
 *     pointers (query rows as in mla_decode_plan; pages);
 *   kv_last_page_len_host: host int32 (batch);
 *   page_size: a power of two, 1 .. 65536.
 * Other arguments (stream included) and errors as mla_decode_plan. Query
 * rows are causal as in mla_decode_plan, and with 1-4 rows in every
 * sequence they share each cache tile under the same conditions (FP8
 * always, MXFP4 when per-row items would exceed num_cus); otherwise each
 * row reads its own range.
 * A paged FP8 or MXFP4 plan runs
 * only through mla_decode_run_paged, mla_decode_run_fused_paged,
 * mla_decode_attend_paged and mla_decode_stage1_paged (then mla_decode_merge,
 * which reads no cache), a paged bf16 plan only through
 * mla_decode_run_bf16_paged (the other entry points that read the cache
 * reject it with INVALID_ARGUMENT), and those reject a plan that is not paged.
 */
MLA_API int mla_decode_plan_paged(const int32_t* qo_indptr_host,
                                  const int32_t* kv_page_indptr_host,
                                  const int32_t* kv_last_page_len_host, int32_t batch,
                                  int32_t page_size, int32_t num_heads, int32_t kv_format,
                                  int32_t num_cus, int32_t max_splits, void* stream,
                                  mla_plan_t* out);

/*
 * mla_decode_run (three launches) and mla_decode_run_fused (one; two with an
 * absmax scale) for a paged plan.
 *   kv_pool      device pool of the plan's format, 16-byte aligned: FP8
 *                (num_pages * page_size, 576) e4m3fn codes; MXFP4
 *                (num_pages * page_size, 288) packed codes.
 *   kv_block_scales_pool  MXFP4: device (num_pages * page_size, 18) E8M0
 *                scales of the same rows, 16-byte aligned; FP8: NULL.
 *   kv_scale     as for the contiguous cache (FP8 only, NULL for MXFP4).
 *   kv_page_ids  device int32 page ids, indexed by the plan's page row
 *                pointers; read on the device at run time, so a caller may
 *                rewrite them between steps without a new plan.
 *   num_pages    pages in the pool. A page id outside [0, num_pages) reads
 *                as zero codes (no fault; MXFP4: zero codes and scales).
 *                With page_size < 32 the pool's codes must stay below 4 GiB
 *                (num_pages * page_size * 576 bytes for FP8, * 288 for
 *                MXFP4), else UNSUPPORTED.
 * Other arguments, outputs and errors as the contiguous forms.
 */
MLA_API int mla_decode_run_paged(mla_plan_t plan, const void* q_bf16, void* q_fp8, float* q_scale,
                                 int32_t q_scale_mode, const void* kv_pool,
                                 const void* kv_block_scales_pool, const float* kv_scale,
                                 const int32_t* kv_page_ids, int32_t num_pages, float sm_scale,
                                 float logit_cap, void* workspace, size_t workspace_bytes,
                                 void* out_bf16, float* lse_out, void* stream);
MLA_API int mla_decode_run_fused_paged(mla_plan_t plan, const void* q_bf16, void* q_fp8,
                                       float* q_scale, int32_t q_scale_mode, const void* kv_pool,
                                       const void* kv_block_scales_pool, const float* kv_scale,
                                       const int32_t* kv_page_ids,
                                       int32_t num_pages, float sm_scale, float logit_cap,
                                       void* workspace, size_t workspace_bytes, void* out_bf16,
                                       float* lse_out, void* stream);

/*
 * Steps (2) and (3) without the Q quantiser: the split-KV attention over
 * the plan's work items (writing the final output of unsplit sequences and
 * the partials of split ones), then the merge if the plan has split or
 * empty sequences. q_fp8 and q_scale are inputs here (the codes and scale
 * of a previous quantisation); other pointers as in mla_decode_run.
 * [722089 `_mla_multihead_stage1` then `_mla_reduce`]
 */
MLA_API int mla_decode_attend(mla_plan_t plan, const void* q_fp8, const float* q_scale, const void* kv,
                      const void* kv_block_scales, const float* kv_scale, float sm_scale,
                      float logit_cap, void* workspace, size_t workspace_bytes, void* out_bf16,
                      float* lse_out, void* stream);

/*
 * Step (2) alone (no merge): as mla_decode_attend, but the partials of
 * split sequences are left in the workspace for mla_decode_merge.
 */
MLA_API int mla_decode_stage1(mla_plan_t plan, const void* q_fp8, const float* q_scale, const void* kv,
                      const void* kv_block_scales, const float* kv_scale, float sm_scale,
                      float logit_cap, void* workspace, size_t workspace_bytes, void* out_bf16,
                      float* lse_out, void* stream);

/*
 * mla_decode_attend and mla_decode_stage1 for a paged FP8 or MXFP4 plan:
 * kv_pool, kv_block_scales_pool, kv_page_ids and num_pages as in
 * mla_decode_run_paged, every other argument, output and error as the
 * contiguous forms. They return INVALID_ARGUMENT for a plan that is not
 * paged (and the contiguous forms for one that is).
 * [663509 / 738050: the decode over kv_indices of a paged kv_buffer]
 */
MLA_API int mla_decode_attend_paged(mla_plan_t plan, const void* q_fp8, const float* q_scale,
                                    const void* kv_pool, const void* kv_block_scales_pool,
                                    const float* kv_scale, const int32_t* kv_page_ids,
                                    int32_t num_pages, float sm_scale, float logit_cap,
                                    void* workspace, size_t workspace_bytes, void* out_bf16,
                                    float* lse_out, void* stream);
MLA_API int mla_decode_stage1_paged(mla_plan_t plan, const void* q_fp8, const float* q_scale,
                                    const void* kv_pool, const void* kv_block_scales_pool,
                                    const float* kv_scale, const int32_t* kv_page_ids,
                                    int32_t num_pages, float sm_scale, float logit_cap,
                                    void* workspace, size_t workspace_bytes, void* out_bf16,
                                    float* lse_out, void* stream);

/*
 * Step (3) alone: merge the partials already in `workspace` (layout above)
 * into out_bf16 / lse_out for the plan's merge sequences.
 * [722089 `_mla_reduce`]  Same pointer rules as mla_decode_run.
 */
MLA_API int mla_decode_merge(mla_plan_t plan, const void* workspace, size_t workspace_bytes,
                     void* out_bf16, float* lse_out, void* stream);

/* Free a plan and its device work list. NULL is allowed. */
MLA_API void mla_decode_plan_destroy(mla_plan_t plan);

/* Static description of a status code. */
MLA_API const char* mla_status_string(int status);

/*
 * Per-tensor FP8 E4M3FN quantiser, the same one step (1) uses, exposed for
 * writing the latent cache.  [722089 `quantize_fp8`; 738050 `_quantize_fp8`]
 *   x_bf16: device, n bf16 values; out_fp8: device, n bytes.
 *   scale_mode MLA_Q_SCALE_STATIC: scale[0] (device fp32) is read;
 *   MLA_Q_SCALE_ABSMAX: scale[0] = fp32(max(max|x|, 1e-12)) / 448 is written.
 *   code = e4m3fn(round-nearest-even(clamp(fp32(x) / scale, -448, 448))).
 *   workspace: device, at least mla_quant_fp8_workspace_size(n) bytes.
 */
MLA_API int mla_quant_fp8_workspace_size(size_t n, size_t* bytes);
MLA_API int mla_quant_fp8(const void* x_bf16, size_t n, int32_t scale_mode, float* scale,
                  void* out_fp8, void* workspace, size_t workspace_bytes, void* stream);

/*
 * MXFP4 encoder for the latent cache: rows of 576 bf16 values become 288
 * packed bytes (element 2i in the low nibble) and 18 e8m0 scale bytes.
 * Per 32-element block: e = floor(log2(max|x|)) - 2 clamped to [-127, 127]
 * (-127 for an all-zero block), scale byte e + 127, each element the e2m1
 * code nearest to x * 2^-e with ties to the even code, saturating at 6.
 * [738050 `_dequantize_mxfp4_inplace` gives the layout and decode; the
 *  encoder rule is the OCP microscaling one]
 *   x_bf16: device (rows, 576); packed: device (rows, 288);
 *   block_scales: device (rows, 18).
 */
MLA_API int mla_encode_mxfp4(const void* x_bf16, size_t rows, void* packed, void* block_scales,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
