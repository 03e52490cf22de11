// C ABI of libmla_decode.so (declared in include/mla_decode.h).
//
// Host side only: argument validation, the per-shape plan (built by
// plan.cpp, copied once to the device), workspace carving and kernel
// launches on the caller's stream. Enqueuing calls allocate nothing and
// never synchronise; every check runs before the first launch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <new>
#include <vector>

#include "../../include/mla_decode.h"
#include "launch.h"
#include "noalloc.h"
#include "plan.h"
#include "stage_common.h"

struct mla_plan {
    mla::Schedule sched;      // the per-row schedule (also what mla_decode_plan_host returns)
    bool rows_mode = false;   // a sequence's query rows share each KV tile (stage1_fp8_rows)
    int32_t rows = 0;         // query rows
    int32_t num_slots = 0;    // partial slots of the schedule in use
    int32_t kv_format = 0;
    bool paged = false;       // paged cache: per-row items are two int4 (see paged_items),
                              // shared-row items three (the third holds the page slice)
    int32_t page_shift = 0;
    int4* d_items = nullptr;  // per-row mode: one int4 per item; rows mode: three
    int4* d_merges = nullptr;
    int4* d_fused = nullptr;  // per-row mode: two int4 per item (see fused_items); rows mode: three
    int32_t n_items = 0;
    int32_t n_merges = 0;
    int32_t n_fused = 0;
};

// FP8 and MXFP4 ranges (at most 2^31 rows) always fit in kMaxSplitsPerSeq
// items, and so do the policy's splits; only a bf16 range beyond 2^30 rows
// would not, and the scheduler rejects it.
static_assert((int64_t(1) << 31) / mla::max_item_tokens(0) <= mla::kMaxSplitsPerSeq &&
                  (int64_t(1) << 31) / mla::max_item_tokens(1) <= mla::kMaxSplitsPerSeq &&
                  mla::kMaxSplits <= mla::kMaxSplitsPerSeq,
              "the merge's scratch holds every partial LSE of a sequence");

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct WorkspaceLayout {
    size_t part_o = 0, part_lse = 0, blockmax = 0, counters = 0, total = 0;
};

WorkspaceLayout layout_for(int32_t nslots, int32_t batch) {
    WorkspaceLayout L;
    size_t off = 0;
    L.part_o = off;
    off += align_up((size_t)nslots * MLA_NUM_HEADS * MLA_V_DIM * sizeof(float));
    L.part_lse = off;
    off += align_up((size_t)nslots * MLA_NUM_HEADS * sizeof(float));
    L.blockmax = off;
    size_t nq = (size_t)batch * MLA_NUM_HEADS * MLA_QK_DIM;
    off += align_up((size_t)mla::absmax_blocks(nq) * sizeof(float));
    L.counters = off;
    off += align_up((size_t)batch * sizeof(uint32_t));
    L.total = off;
    return L;
}

// Work items of the fused launch: every stage-1 item followed by
// {first slot, number of splits, 0, 0} of its sequence (0 splits when the
// item writes the output itself), then one item {b, 0, 0, -1} per empty
// sequence, which writes O = 0 and LSE = -inf.
std::vector<int4> fused_items(const mla::Schedule& s) {
    std::vector<int4> seq((size_t)s.batch, int4{0, 0, 0, 0});
    for (const mla::Merge& m : s.merges) seq[m.b] = int4{m.slot_begin, m.nslots, 0, 0};
    std::vector<int4> f;
    f.reserve(2 * (s.items.size() + s.merges.size()));
    for (const mla::Item& it : s.items) {
        f.push_back(int4{it.b, it.kv_begin, it.kv_end, it.slot});
        f.push_back(it.slot < 0 ? int4{0, 0, 0, 0} : seq[it.b]);
    }
    for (const mla::Merge& m : s.merges)
        if (m.nslots == 0) {
            f.push_back(int4{m.b, 0, 0, -1});
            f.push_back(int4{0, 0, 0, 0});
        }
    return f;
}

// Work items of the paged kernel, two int4 each: {query row, first and end
// position in the sequence, slot}, {first slot, splits, first page-table
// entry of the sequence, pages of the sequence}; with_empty adds one item
// per empty row (fused form). tok: the sequences' token offsets in the
// schedule's row numbering; pi: page-table row pointers.
std::vector<int4> paged_items(const mla::Schedule& s, const std::vector<int64_t>& tok,
                              const std::vector<int32_t>& seq_of_row, const int32_t* pi,
                              bool with_empty) {
    std::vector<int4> rowinfo((size_t)s.batch, int4{0, 0, 0, 0});
    for (const mla::Merge& m : s.merges) rowinfo[m.b] = int4{m.slot_begin, m.nslots, 0, 0};
    std::vector<int4> f;
    f.reserve(2 * (s.items.size() + s.merges.size()));
    for (const mla::Item& it : s.items) {
        const int32_t q = seq_of_row[it.b];
        f.push_back(int4{it.b, (int)(it.kv_begin - tok[q]), (int)(it.kv_end - tok[q]), it.slot});
        const int4 ri = it.slot < 0 ? int4{0, 0, 0, 0} : rowinfo[it.b];
        f.push_back(int4{ri.x, ri.y, pi[q], pi[q + 1] - pi[q]});
    }
    if (with_empty)
        for (const mla::Merge& m : s.merges)
            if (m.nslots == 0) {
                const int32_t q = seq_of_row[m.b];
                f.push_back(int4{m.b, 0, 0, -1});
                f.push_back(int4{0, 0, pi[q], pi[q + 1] - pi[q]});
            }
    return f;
}

// Copies n int4 to a new device array, the copy enqueued on `st`; false on a
// HIP failure. The host source must stay alive until `st` has been
// synchronised (finish_upload).
bool upload(const int4* src, size_t n, int4** dst, hipStream_t st) {
    if (n == 0) return true;
    if (hipMalloc((void**)dst, sizeof(int4) * n) != hipSuccess) {
        *dst = nullptr;
        return false;
    }
    return hipMemcpyAsync(*dst, src, sizeof(int4) * n, hipMemcpyHostToDevice, st) == hipSuccess;
}

// Waits for the plan's copies on `st` (and for whatever the caller queued on
// that stream before them); other streams keep running.
bool finish_upload(bool ok, hipStream_t st) {
    const bool synced = hipStreamSynchronize(st) == hipSuccess;
    return ok && synced;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
    switch (status) {
        case MLA_OK: return "ok";
        case MLA_INVALID_ARGUMENT: return "invalid argument";
        case MLA_UNSUPPORTED: return "unsupported configuration";
        case MLA_HIP_ERROR: return "HIP runtime error";
        case MLA_WORKSPACE_TOO_SMALL: return "workspace too small";
        case MLA_OUT_OF_MEMORY: return "out of memory";
        default: return "unknown status";
    }
}

int mla_decode_plan(const int32_t* qo_indptr_host, const int32_t* kv_indptr_host, int32_t batch,
                    int32_t num_heads, int32_t kv_format, int32_t num_cus, int32_t max_splits,
                    void* stream, mla_plan_t* out) {
    const hipStream_t hs = (hipStream_t)stream;
    if (!out) return MLA_INVALID_ARGUMENT;
    *out = nullptr;
    if (num_cus <= 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return MLA_HIP_ERROR;
        if (hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess)
            return MLA_HIP_ERROR;
    }
    mla_plan* p = new (std::nothrow) mla_plan();
    if (!p) return MLA_OUT_OF_MEMORY;
    int st;
    try {
        st = mla::build_schedule(qo_indptr_host, kv_indptr_host, batch, num_heads, kv_format,
                                 num_cus, max_splits, &p->sched);
    } catch (...) {
        st = MLA_OUT_OF_MEMORY;
    }
    if (st) {
        delete p;
        return st;
    }
    static_assert(sizeof(mla::Item) == sizeof(int4), "item is four int32");
    static_assert(sizeof(mla::Merge) == sizeof(int4), "merge entry is four int32");
    static_assert(sizeof(mla::RowsItem) == 3 * sizeof(int4), "rows item is three int4");
    p->rows = p->sched.batch;
    p->kv_format = kv_format;
    bool ok;
    if (mla::use_rows_schedule(qo_indptr_host, batch, kv_format, false, p->sched.items.size(),
                               num_cus)) {
        mla::RowsSchedule rs;
        std::vector<mla::RowsItem> fused;
        try {
            mla::build_rows_schedule(qo_indptr_host, kv_indptr_host, batch, num_cus, max_splits,
                                     &rs);
            fused = rs.items;
            fused.insert(fused.end(), rs.empty.begin(), rs.empty.end());
        } catch (...) {
            delete p;
            return MLA_OUT_OF_MEMORY;
        }
        p->rows_mode = true;
        p->num_slots = rs.num_slots;
        p->n_items = (int32_t)rs.items.size();
        p->n_merges = (int32_t)rs.merges.size();
        p->n_fused = (int32_t)fused.size();
        ok = upload((const int4*)rs.items.data(), 3 * rs.items.size(), &p->d_items, hs) &&
             upload((const int4*)rs.merges.data(), rs.merges.size(), &p->d_merges, hs) &&
             upload((const int4*)fused.data(), 3 * fused.size(), &p->d_fused, hs);
        ok = finish_upload(ok, hs);  // before rs and fused go out of scope
    } else {
        std::vector<int4> fused;
        try {
            fused = fused_items(p->sched);
        } catch (...) {
            delete p;
            return MLA_OUT_OF_MEMORY;
        }
        p->num_slots = p->sched.num_slots;
        p->n_items = (int32_t)p->sched.items.size();
        p->n_merges = (int32_t)p->sched.merges.size();
        p->n_fused = (int32_t)(fused.size() / 2);
        ok = upload((const int4*)p->sched.items.data(), p->sched.items.size(), &p->d_items, hs) &&
             upload((const int4*)p->sched.merges.data(), p->sched.merges.size(), &p->d_merges,
                    hs) &&
             upload(fused.data(), fused.size(), &p->d_fused, hs);
        ok = finish_upload(ok, hs);  // before fused goes out of scope
    }
    if (!ok) {
        mla_decode_plan_destroy(p);
        return MLA_HIP_ERROR;
    }
    *out = p;
    return MLA_OK;
}

int mla_decode_plan_paged(const int32_t* qo_indptr_host, const int32_t* kv_page_indptr_host,
                          const int32_t* kv_last_page_len_host, int32_t batch, int32_t page_size,
                          int32_t num_heads, int32_t kv_format, int32_t num_cus,
                          int32_t max_splits, void* stream, mla_plan_t* out) {
    const hipStream_t hs = (hipStream_t)stream;
    if (!out) return MLA_INVALID_ARGUMENT;
    *out = nullptr;
    if (!qo_indptr_host || !kv_page_indptr_host || batch < 0) return MLA_INVALID_ARGUMENT;
    if (batch > 0 && !kv_last_page_len_host) return MLA_INVALID_ARGUMENT;
    if (page_size < 1 || page_size > (1 << 16) || (page_size & (page_size - 1)))
        return MLA_INVALID_ARGUMENT;
    if (kv_format != MLA_KV_FP8_E4M3FN && kv_format != MLA_KV_BF16 &&
        kv_format != MLA_KV_MXFP4)
        return MLA_INVALID_ARGUMENT;
    const int32_t* pi = kv_page_indptr_host;
    if (pi[0] != 0) return MLA_INVALID_ARGUMENT;
    // sequence lengths from the page counts and the last page's rows
    std::vector<int32_t> tok_indptr;
    std::vector<int64_t> tok;
    std::vector<int32_t> seq_of_row;
    try {
        tok_indptr.assign((size_t)batch + 1, 0);
        tok.assign((size_t)batch + 1, 0);
        for (int32_t b = 0; b < batch; b++) {
            const int64_t np = (int64_t)pi[b + 1] - pi[b];
            if (np < 0) return MLA_INVALID_ARGUMENT;
            int64_t len = 0;
            if (np > 0) {
                const int32_t last = kv_last_page_len_host[b];
                if (last < 1 || last > page_size) return MLA_INVALID_ARGUMENT;
                len = (np - 1) * page_size + last;
            }
            tok[b + 1] = tok[b] + len;
            if (tok[b + 1] > INT32_MAX) return MLA_UNSUPPORTED;
            tok_indptr[b + 1] = (int32_t)tok[b + 1];
        }
    } catch (...) {
        return MLA_OUT_OF_MEMORY;
    }
    if (num_cus <= 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return MLA_HIP_ERROR;
        if (hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess)
            return MLA_HIP_ERROR;
    }
    mla_plan* p = new (std::nothrow) mla_plan();
    if (!p) return MLA_OUT_OF_MEMORY;
    int st;
    std::vector<int4> plain, fused;
    try {
        st = mla::build_schedule(qo_indptr_host, tok_indptr.data(), batch, num_heads, kv_format,
                                 num_cus, max_splits, &p->sched);
        if (!st) {
            seq_of_row.assign((size_t)p->sched.batch, 0);
            for (int32_t b = 0; b < batch; b++)
                for (int32_t r = qo_indptr_host[b]; r < qo_indptr_host[b + 1]; r++)
                    seq_of_row[r] = b;
            plain = paged_items(p->sched, tok, seq_of_row, pi, false);
            fused = paged_items(p->sched, tok, seq_of_row, pi, true);
        }
    } catch (...) {
        st = MLA_OUT_OF_MEMORY;
    }
    if (st) {
        delete p;
        return st;
    }
    p->paged = true;
    p->page_shift = __builtin_ctz((unsigned)page_size);
    p->rows = p->sched.batch;
    p->kv_format = kv_format;
    if (mla::use_rows_schedule(qo_indptr_host, batch, kv_format, true, p->sched.items.size(),
                               num_cus)) {
        // the shared-row kernel's items, with positions in the sequence and
        // the sequence's page-table slice in the third int4
        mla::RowsSchedule rs;
        std::vector<mla::RowsItem> items, fused_rows;
        try {
            mla::build_rows_schedule(qo_indptr_host, tok_indptr.data(), batch, num_cus,
                                     max_splits, &rs);
            auto in_seq = [&](mla::RowsItem it) {
                const int32_t t0 = (int32_t)tok[(size_t)it.b];
                it.kv_begin -= t0;
                it.kv_end -= t0;
                it.seq_end -= t0;
                it.pad0 = pi[it.b];
                it.pad1 = pi[it.b + 1] - pi[it.b];
                return it;
            };
            for (const mla::RowsItem& it : rs.items) items.push_back(in_seq(it));
            fused_rows = items;
            for (const mla::RowsItem& it : rs.empty) fused_rows.push_back(in_seq(it));
        } catch (...) {
            delete p;
            return MLA_OUT_OF_MEMORY;
        }
        p->rows_mode = true;
        p->num_slots = rs.num_slots;
        p->n_items = (int32_t)items.size();
        p->n_merges = (int32_t)rs.merges.size();
        p->n_fused = (int32_t)fused_rows.size();
        bool rok = upload((const int4*)items.data(), 3 * items.size(), &p->d_items, hs) &&
                   upload((const int4*)rs.merges.data(), rs.merges.size(), &p->d_merges, hs) &&
                   upload((const int4*)fused_rows.data(), 3 * fused_rows.size(), &p->d_fused, hs);
        if (!finish_upload(rok, hs)) {  // before the host arrays go out of scope
            mla_decode_plan_destroy(p);
            return MLA_HIP_ERROR;
        }
        *out = p;
        return MLA_OK;
    }
    p->num_slots = p->sched.num_slots;
    p->n_items = (int32_t)(plain.size() / 2);
    p->n_merges = (int32_t)p->sched.merges.size();
    p->n_fused = (int32_t)(fused.size() / 2);
    const bool ok =
        upload(plain.data(), plain.size(), &p->d_items, hs) &&
        upload((const int4*)p->sched.merges.data(), p->sched.merges.size(), &p->d_merges, hs) &&
        upload(fused.data(), fused.size(), &p->d_fused, hs);
    if (!finish_upload(ok, hs)) {
        mla_decode_plan_destroy(p);
        return MLA_HIP_ERROR;
    }
    *out = p;
    return MLA_OK;
}

int mla_decode_plan_counts(mla_plan_t plan, int32_t* counts_out) {
    if (!plan || !counts_out) return MLA_INVALID_ARGUMENT;
    counts_out[0] = plan->n_items;
    counts_out[1] = plan->n_merges;
    counts_out[2] = plan->num_slots;
    counts_out[3] = plan->rows;
    return MLA_OK;
}

void mla_decode_plan_destroy(mla_plan_t plan) {
    if (!plan) return;
    if (plan->d_items) (void)hipFree(plan->d_items);
    if (plan->d_merges) (void)hipFree(plan->d_merges);
    if (plan->d_fused) (void)hipFree(plan->d_fused);
    delete plan;
}

int mla_decode_workspace_size(mla_plan_t plan, size_t* bytes) {
    if (!plan || !bytes) return MLA_INVALID_ARGUMENT;
    *bytes = layout_for(plan->num_slots, plan->rows).total;
    return MLA_OK;
}

namespace {

// Device addresses of the workspace sections one decode step uses.
struct WorkspacePtrs {
    float* part_o = nullptr;
    float* part_lse = nullptr;
    float* blockmax = nullptr;
    uint32_t* counters = nullptr;
};

WorkspacePtrs ptrs_of(const WorkspaceLayout& L, void* workspace) {
    uint8_t* ws = (uint8_t*)workspace;
    WorkspacePtrs W;
    W.part_o = (float*)(ws + L.part_o);
    W.part_lse = (float*)(ws + L.part_lse);
    W.blockmax = (float*)(ws + L.blockmax);
    W.counters = (uint32_t*)(ws + L.counters);
    return W;
}

// Checks shared by the entry points that launch the attention kernels,
// except those of the workspace.
int check_attend_core(const mla_plan* plan, const void* q_fp8, const float* q_scale,
                      const void* kv, const void* kv_block_scales, const float* kv_scale,
                      float sm_scale, float logit_cap, const void* out_bf16) {
    if (!plan) return MLA_INVALID_ARGUMENT;
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return MLA_INVALID_ARGUMENT;
    if (!std::isfinite(logit_cap) || logit_cap < 0.0f) return MLA_INVALID_ARGUMENT;
    if (!q_scale) return MLA_INVALID_ARGUMENT;
    if (plan->rows > 0 && (!q_fp8 || !out_bf16)) return MLA_INVALID_ARGUMENT;
    if (plan->rows > 0 && (!aligned16(q_fp8) || !aligned16(out_bf16))) return MLA_INVALID_ARGUMENT;
    if (plan->kv_format == MLA_KV_BF16) return MLA_INVALID_ARGUMENT;  // mla_decode_run_bf16
    if (plan->kv_format == MLA_KV_FP8_E4M3FN) {
        if (kv_block_scales) return MLA_INVALID_ARGUMENT;
        if (plan->n_items && (!kv || !kv_scale || !aligned16(kv))) return MLA_INVALID_ARGUMENT;
    } else {
        if (kv_scale) return MLA_INVALID_ARGUMENT;
        if (plan->n_items &&
            (!kv || !kv_block_scales || !aligned16(kv) || !aligned16(kv_block_scales)))
            return MLA_INVALID_ARGUMENT;
    }
    return MLA_OK;
}

// The caller's workspace against the plan's layout.
int check_workspace(const mla_plan* plan, const void* workspace, size_t workspace_bytes,
                    WorkspaceLayout* L) {
    *L = layout_for(plan->num_slots, plan->rows);
    if (workspace_bytes < L->total) return MLA_WORKSPACE_TOO_SMALL;
    if (L->total && !workspace) return MLA_INVALID_ARGUMENT;
    if (((uintptr_t)workspace & (kAlign - 1)) != 0) return MLA_INVALID_ARGUMENT;
    return MLA_OK;
}

int check_attend_args(const mla_plan* plan, const void* q_fp8, const float* q_scale,
                      const void* kv, const void* kv_block_scales, const float* kv_scale,
                      float sm_scale, float logit_cap, const void* workspace,
                      size_t workspace_bytes, const void* out_bf16, WorkspaceLayout* L) {
    const int st = check_attend_core(plan, q_fp8, q_scale, kv, kv_block_scales, kv_scale,
                                     sm_scale, logit_cap, out_bf16);
    return st ? st : check_workspace(plan, workspace, workspace_bytes, L);
}

struct Pages {
    const int32_t* ids;  // device int32 page ids, sequences' pages in order
    int32_t num_pages;   // pages in the pool
};

// Caches of at least this many bytes are streamed with non-temporal loads
// (not by the shared-row kernel, which is bound by its arithmetic and measured
// 3.6 % slower with them).
// Measured on MI355X: at 1.2 GB (FP8, bs256 kv8192) and 2.4 GB (bf16) the
// hint cut the step by 6 % and 12 %, since the 256 MB last-level cache no
// longer allocates lines that are never re-read; at 302 MB and 80 MB it cost
// 5 % and 4 %, because back-to-back steps re-read part or all of such a
// cache from the last-level cache.
constexpr int64_t kStreamNtBytes = int64_t(512) << 20;

int64_t cache_bytes(const mla_plan* plan) {
    const int64_t row = plan->kv_format == MLA_KV_FP8_E4M3FN ? MLA_QK_DIM
                        : plan->kv_format == MLA_KV_MXFP4    ? MLA_QK_DIM / 2 + MLA_QK_DIM / 32
                                                             : 2 * MLA_QK_DIM;
    return plan->sched.total_kv * row;
}

mla::Stage1Args stage1_args(const mla_plan* plan, const void* kv, const void* kv_block_scales,
                            const float* kv_scale, float sm_scale, float logit_cap,
                            const WorkspacePtrs& W, void* out_bf16, float* lse_out,
                            const Pages* pages = nullptr) {
    mla::Stage1Args a{};
    a.kv_nt = !plan->rows_mode && cache_bytes(plan) >= kStreamNtBytes;
    if (pages) {
        a.kv_pages = pages->ids;
        a.num_pages = pages->num_pages;
        a.page_shift = plan->page_shift;
    }
    a.kv = (const uint8_t*)kv;
    a.kv_scales = (const uint8_t*)kv_block_scales;
    a.kv_scale = kv_scale;
    a.sm_scale = sm_scale;
    a.logit_cap = logit_cap;
    a.part_o = W.part_o;
    a.part_lse = W.part_lse;
    a.out = (uint16_t*)out_bf16;
    a.lse_out = lse_out;
    a.counters = W.counters;
    return a;
}

hipError_t launch_stage1_any(const mla_plan* plan, const mla::Stage1Args& a, bool fused,
                             hipStream_t st) {
    const int n = fused ? plan->n_fused : plan->n_items;
    if (plan->rows_mode)
        return plan->kv_format == MLA_KV_FP8_E4M3FN ? mla::launch_stage1_fp8_rows(a, n, fused, st)
                                                    : mla::launch_stage1_mxfp4_rows(a, n, fused, st);
    if (plan->kv_format == MLA_KV_FP8_E4M3FN) return mla::launch_stage1_fp8(a, n, fused, st);
    return mla::launch_stage1_mxfp4(a, n, fused, st);
}

hipError_t launch_stage1(const mla_plan* plan, const void* q_fp8, const float* q_scale,
                         const void* kv, const void* kv_block_scales, const float* kv_scale,
                         float sm_scale, float logit_cap, const WorkspacePtrs& W, void* out_bf16,
                         float* lse_out, hipStream_t st, const Pages* pages = nullptr) {
    mla::Stage1Args a = stage1_args(plan, kv, kv_block_scales, kv_scale, sm_scale, logit_cap, W,
                                    out_bf16, lse_out, pages);
    a.items = plan->d_items;
    a.q8_in = (const uint8_t*)q_fp8;
    a.q_scale = q_scale;
    return launch_stage1_any(plan, a, false, st);
}

hipError_t launch_merge_step(const mla_plan* plan, const WorkspacePtrs& W, void* out_bf16,
                             float* lse_out, hipStream_t st) {
    return mla::launch_merge(plan->d_merges, plan->n_merges, W.part_o, W.part_lse,
                             (uint16_t*)out_bf16, lse_out, st);
}

}  // namespace

int mla_decode_workspace_init(mla_plan_t plan, void* workspace, size_t workspace_bytes,
                              void* stream) {
    if (!plan) return MLA_INVALID_ARGUMENT;
    const WorkspaceLayout L = layout_for(plan->num_slots, plan->rows);
    if (workspace_bytes < L.total) return MLA_WORKSPACE_TOO_SMALL;
    if (L.total && !workspace) return MLA_INVALID_ARGUMENT;
    if (((uintptr_t)workspace & (kAlign - 1)) != 0) return MLA_INVALID_ARGUMENT;
    if (plan->rows == 0) return MLA_OK;
    hipError_t e = mla::launch_zero_u32((uint32_t*)((uint8_t*)workspace + L.counters),
                                        (size_t)plan->rows, (hipStream_t)stream);
    return e == hipSuccess ? MLA_OK : MLA_HIP_ERROR;
}

namespace {

// Checks of a paged plan's page table against the entry point used.
int check_pages(const mla_plan* plan, const Pages* pages) {
    if (plan->paged != (pages != nullptr)) return MLA_INVALID_ARGUMENT;
    if (!pages) return MLA_OK;
    if (plan->n_items == 0) return MLA_OK;  // nothing reads the page table
    if (!pages->ids || pages->num_pages < 1) return MLA_INVALID_ARGUMENT;
    // pages smaller than a tile (FP8 and MXFP4: 32 rows, bf16: 16) are
    // gathered with 32-bit offsets into the whole pool
    const int32_t f = plan->kv_format;
    const uint64_t row_bytes = f == MLA_KV_BF16 ? 2 * MLA_QK_DIM
                               : f == MLA_KV_MXFP4 ? MLA_QK_DIM / 2 : MLA_QK_DIM;
    if (plan->page_shift < (f == MLA_KV_BF16 ? 4 : 5) &&
        ((uint64_t)pages->num_pages << plan->page_shift) * row_bytes > 0xfffffff0ull)
        return MLA_UNSUPPORTED;
    return MLA_OK;
}

// Every check of one decode step but those of the workspace.
int check_run(const mla_plan* plan, const void* q_bf16, const void* q_fp8, const float* q_scale,
              int32_t q_scale_mode, const void* kv, const void* kv_block_scales,
              const float* kv_scale, const Pages* pages, float sm_scale, float logit_cap,
              const void* out_bf16, bool fused) {
    if (q_scale_mode != MLA_Q_SCALE_STATIC && q_scale_mode != MLA_Q_SCALE_ABSMAX)
        return MLA_INVALID_ARGUMENT;
    int st = check_attend_core(plan, q_fp8, q_scale, kv, kv_block_scales, kv_scale, sm_scale,
                               logit_cap, out_bf16);
    if (st) return st;
    st = check_pages(plan, pages);
    if (st) return st;
    if (plan->rows == 0) return MLA_OK;
    if (!q_bf16 || !aligned16(q_bf16)) return MLA_INVALID_ARGUMENT;
    // every fused workgroup reads the per-tensor KV scale, also for empty sequences
    if (fused && plan->kv_format == MLA_KV_FP8_E4M3FN && !kv_scale) return MLA_INVALID_ARGUMENT;
    return MLA_OK;
}

// The launches of one decode step (arguments already checked): Q quantiser,
// stage 1 and merge (three launches), or the fused stage 1 (one launch; two
// with an absmax scale).
int run_launch(const mla_plan* plan, const void* q_bf16, void* q_fp8, float* q_scale,
               int32_t q_scale_mode, const void* kv, const void* kv_block_scales,
               const float* kv_scale, const Pages* pages, float sm_scale, float logit_cap,
               const WorkspacePtrs& W, void* out_bf16, float* lse_out, hipStream_t hs,
               bool fused) {
    float* blockmax = W.blockmax;
    if (plan->rows == 0) {
        // no rows: an absmax scale is still defined, max(0, 1e-12) / 448
        if (q_scale_mode != MLA_Q_SCALE_ABSMAX) return MLA_OK;
        hipError_t e = mla::launch_absmax_partial(nullptr, 0, blockmax, 1, hs);
        if (e == hipSuccess)
            e = mla::launch_quant_fp8(nullptr, 0, nullptr, nullptr, blockmax, 1, q_scale, hs);
        return e == hipSuccess ? MLA_OK : MLA_HIP_ERROR;
    }
    const size_t nq = (size_t)plan->rows * MLA_NUM_HEADS * MLA_QK_DIM;
    const int nb = mla::absmax_blocks(nq);
    // a small Q's absmax is reduced inside every workgroup of the fused FP8
    // kernel (one launch instead of two)
    const bool absmax_in_kernel = fused && q_scale_mode == MLA_Q_SCALE_ABSMAX &&
                                  plan->kv_format == MLA_KV_FP8_E4M3FN && !plan->rows_mode &&
                                  plan->rows <= mla::kQAbsmaxRows;
    hipError_t e;
    if (q_scale_mode == MLA_Q_SCALE_ABSMAX && !absmax_in_kernel) {
        e = mla::launch_absmax_partial((const uint16_t*)q_bf16, nq, blockmax, nb, hs);
        if (e != hipSuccess) return MLA_HIP_ERROR;
    }
    if (fused) {
        mla::Stage1Args a = stage1_args(plan, kv, kv_block_scales, kv_scale, sm_scale, logit_cap,
                                        W, out_bf16, lse_out, pages);
        a.items = plan->d_fused;
        a.q_bf16 = (const uint16_t*)q_bf16;
        a.q8_out = (uint8_t*)q_fp8;
        if (absmax_in_kernel) {
            a.q_absmax_rows = plan->rows;
            a.q_scale_out = q_scale;
        } else if (q_scale_mode == MLA_Q_SCALE_ABSMAX) {
            a.blockmax = blockmax;
            a.nblockmax = nb;
            a.q_scale_out = q_scale;
        } else {
            a.q_scale = q_scale;
        }
        e = launch_stage1_any(plan, a, true, hs);
        return e == hipSuccess ? MLA_OK : MLA_HIP_ERROR;
    }
    if (q_scale_mode == MLA_Q_SCALE_ABSMAX)
        e = mla::launch_quant_fp8((const uint16_t*)q_bf16, nq, (uint8_t*)q_fp8, nullptr, blockmax,
                                  nb, q_scale, hs);
    else
        e = mla::launch_quant_fp8((const uint16_t*)q_bf16, nq, (uint8_t*)q_fp8, q_scale, nullptr,
                                  0, nullptr, hs);
    if (e != hipSuccess) return MLA_HIP_ERROR;
    e = launch_stage1(plan, q_fp8, q_scale, kv, kv_block_scales, kv_scale, sm_scale, logit_cap, W,
                      out_bf16, lse_out, hs, pages);
    if (e != hipSuccess) return MLA_HIP_ERROR;
    e = launch_merge_step(plan, W, out_bf16, lse_out, hs);
    return e == hipSuccess ? MLA_OK : MLA_HIP_ERROR;
}

// One decode step with the caller's workspace.
int run_impl(mla_plan_t plan, const void* q_bf16, void* q_fp8, float* q_scale,
             int32_t q_scale_mode, const void* kv, const void* kv_block_scales,
             const float* kv_scale, const Pages* pages, float sm_scale, float logit_cap,
             void* workspace, size_t workspace_bytes, void* out_bf16, float* lse_out,
             void* stream, bool fused) {
    int st = check_run(plan, q_bf16, q_fp8, q_scale, q_scale_mode, kv, kv_block_scales, kv_scale,
                       pages, sm_scale, logit_cap, out_bf16, fused);
    if (st) return st;
    WorkspaceLayout L;
    st = check_workspace(plan, workspace, workspace_bytes, &L);
    if (st) return st;
    return run_launch(plan, q_bf16, q_fp8, q_scale, q_scale_mode, kv, kv_block_scales, kv_scale,
                      pages, sm_scale, logit_cap, ptrs_of(L, workspace), out_bf16, lse_out,
                      (hipStream_t)stream, fused);
}

}  // namespace

int mla_decode_run(mla_plan_t plan, const void* q_bf16, void* q_fp8, float* q_scale,
                   int32_t q_scale_mode, const void* kv, const void* kv_block_scales,
                   const float* kv_scale, float sm_scale, float logit_cap, void* workspace,
                   size_t workspace_bytes, void* out_bf16, float* lse_out, void* stream) {
    return run_impl(plan, q_bf16, q_fp8, q_scale, q_scale_mode, kv, kv_block_scales, kv_scale,
                    nullptr, sm_scale, logit_cap, workspace, workspace_bytes, out_bf16, lse_out,
                    stream, false);
}

int mla_decode_run_fused(mla_plan_t plan, const void* q_bf16, void* q_fp8, float* q_scale,
                         int32_t q_scale_mode, const void* kv, const void* kv_block_scales,
                         const float* kv_scale, float sm_scale, float logit_cap, void* workspace,
                         size_t workspace_bytes, void* out_bf16, float* lse_out, void* stream) {
    return run_impl(plan, q_bf16, q_fp8, q_scale, q_scale_mode, kv, kv_block_scales, kv_scale,
                    nullptr, sm_scale, logit_cap, workspace, workspace_bytes, out_bf16, lse_out,
                    stream, true);
}

int mla_decode_run_fused_noalloc(mla_plan_t plan, const void* q_bf16, void* q_fp8,
                                 float* q_scale, int32_t q_scale_mode, const void* kv,
                                 const void* kv_block_scales, const float* kv_scale,
                                 float sm_scale, float logit_cap, void* out_bf16, float* lse_out,
                                 void* stream) {
    int st = check_run(plan, q_bf16, q_fp8, q_scale, q_scale_mode, kv, kv_block_scales, kv_scale,
                       nullptr, sm_scale, logit_cap, out_bf16, true);
    if (st) return st;
    if (plan->rows > mla::kNoallocMaxRows || plan->num_slots > mla::kNoallocMaxSlots)
        return MLA_WORKSPACE_TOO_SMALL;
    const hipStream_t hs = (hipStream_t)stream;
    uint8_t* base = (uint8_t*)mla::noalloc_scratch(hs, &st);
    if (!base) return st;
    WorkspacePtrs W;
    W.counters = (uint32_t*)(base + mla::kNoallocCountersOff);
    W.blockmax = (float*)(base + mla::kNoallocBlockmaxOff);
    W.part_lse = (float*)(base + mla::kNoallocLseOff);
    W.part_o = (float*)(base + mla::kNoallocPartOff);
    return run_launch(plan, q_bf16, q_fp8, q_scale, q_scale_mode, kv, kv_block_scales, kv_scale,
                      nullptr, sm_scale, logit_cap, W, out_bf16, lse_out, hs, true);
}

int mla_decode_run_paged(mla_plan_t plan, const void* q_bf16, void* q_fp8, float* q_scale,
                         int32_t q_scale_mode, const void* kv_pool,
                         const void* kv_block_scales_pool, const float* kv_scale,
                         const int32_t* kv_page_ids, int32_t num_pages, float sm_scale,
                         float logit_cap, void* workspace, size_t workspace_bytes,
                         void* out_bf16, float* lse_out, void* stream) {
    const Pages pages{kv_page_ids, num_pages};
    if (!plan) return MLA_INVALID_ARGUMENT;
    return run_impl(plan, q_bf16, q_fp8, q_scale, q_scale_mode, kv_pool, kv_block_scales_pool,
                    kv_scale, &pages, sm_scale, logit_cap, workspace, workspace_bytes, out_bf16,
                    lse_out, stream, false);
}

int mla_decode_run_fused_paged(mla_plan_t plan, const void* q_bf16, void* q_fp8,
                               float* q_scale, int32_t q_scale_mode, const void* kv_pool,
                               const void* kv_block_scales_pool, const float* kv_scale,
                               const int32_t* kv_page_ids, int32_t num_pages, float sm_scale,
                               float logit_cap, void* workspace, size_t workspace_bytes,
                               void* out_bf16, float* lse_out, void* stream) {
    const Pages pages{kv_page_ids, num_pages};
    if (!plan) return MLA_INVALID_ARGUMENT;
    return run_impl(plan, q_bf16, q_fp8, q_scale, q_scale_mode, kv_pool, kv_block_scales_pool,
                    kv_scale, &pages, sm_scale, logit_cap, workspace, workspace_bytes, out_bf16,
                    lse_out, stream, true);
}

namespace {

// The bf16 decode step, contiguous (pages == nullptr) or paged.
int run_bf16_impl(mla_plan_t plan, const void* q_bf16, const void* kv_bf16, const Pages* pages,
                  float sm_scale, float logit_cap, void* workspace, size_t workspace_bytes,
                  void* out_bf16, float* lse_out, void* stream) {
    if (!plan || plan->kv_format != MLA_KV_BF16) return MLA_INVALID_ARGUMENT;
    if (const int st = check_pages(plan, pages)) return st;
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return MLA_INVALID_ARGUMENT;
    if (!std::isfinite(logit_cap) || logit_cap < 0.0f) return MLA_INVALID_ARGUMENT;
    const WorkspaceLayout L = layout_for(plan->num_slots, plan->rows);
    if (workspace_bytes < L.total) return MLA_WORKSPACE_TOO_SMALL;
    if (L.total && !workspace) return MLA_INVALID_ARGUMENT;
    if (((uintptr_t)workspace & (kAlign - 1)) != 0) return MLA_INVALID_ARGUMENT;
    if (plan->rows == 0) return MLA_OK;
    if (!q_bf16 || !out_bf16 || !aligned16(q_bf16) || !aligned16(out_bf16))
        return MLA_INVALID_ARGUMENT;
    if (plan->n_items && (!kv_bf16 || !aligned16(kv_bf16))) return MLA_INVALID_ARGUMENT;
    mla::Stage1Args a = stage1_args(plan, kv_bf16, nullptr, nullptr, sm_scale, 0.0f,
                                    ptrs_of(L, workspace), out_bf16, lse_out, pages);
    a.items = plan->d_fused;
    a.q_bf16 = (const uint16_t*)q_bf16;
    hipError_t e = mla::launch_stage1_bf16(a, logit_cap, plan->n_fused, true, (hipStream_t)stream);
    return e == hipSuccess ? MLA_OK : MLA_HIP_ERROR;
}

}  // namespace

int mla_decode_run_bf16(mla_plan_t plan, const void* q_bf16, const void* kv_bf16,
                        float sm_scale, float logit_cap, void* workspace, size_t workspace_bytes,
                        void* out_bf16, float* lse_out, void* stream) {
    return run_bf16_impl(plan, q_bf16, kv_bf16, nullptr, sm_scale, logit_cap, workspace,
                         workspace_bytes, out_bf16, lse_out, stream);
}

int mla_decode_run_bf16_paged(mla_plan_t plan, const void* q_bf16, const void* kv_pool,
                              const int32_t* kv_page_ids, int32_t num_pages, float sm_scale,
                              float logit_cap, void* workspace, size_t workspace_bytes,
                              void* out_bf16, float* lse_out, void* stream) {
    const Pages pages{kv_page_ids, num_pages};
    if (!plan) return MLA_INVALID_ARGUMENT;
    return run_bf16_impl(plan, q_bf16, kv_pool, &pages, sm_scale, logit_cap, workspace,
                         workspace_bytes, out_bf16, lse_out, stream);
}

namespace {

// Stage 1 over the plan's items from given Q codes, then (merge) the merge
// step: contiguous (pages == nullptr) or paged, as the plan was made.
int attend_impl(mla_plan_t plan, const void* q_fp8, const float* q_scale, const void* kv,
                const void* kv_block_scales, const float* kv_scale, const Pages* pages,
                float sm_scale, float logit_cap, void* workspace, size_t workspace_bytes,
                void* out_bf16, float* lse_out, void* stream, bool merge) {
    WorkspaceLayout L;
    int st = check_attend_args(plan, q_fp8, q_scale, kv, kv_block_scales, kv_scale, sm_scale,
                               logit_cap, workspace, workspace_bytes, out_bf16, &L);
    if (st) return st;
    st = check_pages(plan, pages);
    if (st) return st;
    hipStream_t hs = (hipStream_t)stream;
    const WorkspacePtrs W = ptrs_of(L, workspace);
    hipError_t e = launch_stage1(plan, q_fp8, q_scale, kv, kv_block_scales, kv_scale, sm_scale,
                                 logit_cap, W, out_bf16, lse_out, hs, pages);
    if (e == hipSuccess && merge) e = launch_merge_step(plan, W, out_bf16, lse_out, hs);
    return e == hipSuccess ? MLA_OK : MLA_HIP_ERROR;
}

}  // namespace

int mla_decode_attend(mla_plan_t plan, const void* q_fp8, const float* q_scale, const void* kv,
                      const void* kv_block_scales, const float* kv_scale, float sm_scale,
                      float logit_cap, void* workspace, size_t workspace_bytes, void* out_bf16,
                      float* lse_out, void* stream) {
    return attend_impl(plan, q_fp8, q_scale, kv, kv_block_scales, kv_scale, nullptr, sm_scale,
                       logit_cap, workspace, workspace_bytes, out_bf16, lse_out, stream, true);
}

int mla_decode_stage1(mla_plan_t plan, const void* q_fp8, const float* q_scale, const void* kv,
                      const void* kv_block_scales, const float* kv_scale, float sm_scale,
                      float logit_cap, void* workspace, size_t workspace_bytes, void* out_bf16,
                      float* lse_out, void* stream) {
    return attend_impl(plan, q_fp8, q_scale, kv, kv_block_scales, kv_scale, nullptr, sm_scale,
                       logit_cap, workspace, workspace_bytes, out_bf16, lse_out, stream, false);
}

int mla_decode_attend_paged(mla_plan_t plan, const void* q_fp8, const float* q_scale,
                            const void* kv_pool, const void* kv_block_scales_pool,
                            const float* kv_scale, const int32_t* kv_page_ids, int32_t num_pages,
                            float sm_scale, float logit_cap, void* workspace,
                            size_t workspace_bytes, void* out_bf16, float* lse_out, void* stream) {
    const Pages pages{kv_page_ids, num_pages};
    return attend_impl(plan, q_fp8, q_scale, kv_pool, kv_block_scales_pool, kv_scale, &pages,
                       sm_scale, logit_cap, workspace, workspace_bytes, out_bf16, lse_out, stream,
                       true);
}

int mla_decode_stage1_paged(mla_plan_t plan, const void* q_fp8, const float* q_scale,
                            const void* kv_pool, const void* kv_block_scales_pool,
                            const float* kv_scale, const int32_t* kv_page_ids, int32_t num_pages,
                            float sm_scale, float logit_cap, void* workspace,
                            size_t workspace_bytes, void* out_bf16, float* lse_out, void* stream) {
    const Pages pages{kv_page_ids, num_pages};
    return attend_impl(plan, q_fp8, q_scale, kv_pool, kv_block_scales_pool, kv_scale, &pages,
                       sm_scale, logit_cap, workspace, workspace_bytes, out_bf16, lse_out, stream,
                       false);
}

int mla_decode_merge(mla_plan_t plan, const void* workspace, size_t workspace_bytes,
                     void* out_bf16, float* lse_out, void* stream) {
    if (!plan) return MLA_INVALID_ARGUMENT;
    const WorkspaceLayout L = layout_for(plan->num_slots, plan->rows);
    if (workspace_bytes < L.total) return MLA_WORKSPACE_TOO_SMALL;
    if (L.total && !workspace) return MLA_INVALID_ARGUMENT;
    if (((uintptr_t)workspace & (kAlign - 1)) != 0) return MLA_INVALID_ARGUMENT;
    if (plan->rows > 0 && (!out_bf16 || !aligned16(out_bf16))) return MLA_INVALID_ARGUMENT;
    const uint8_t* ws = (const uint8_t*)workspace;
    hipError_t e = mla::launch_merge(plan->d_merges, plan->n_merges, (const float*)(ws + L.part_o),
                                     (const float*)(ws + L.part_lse), (uint16_t*)out_bf16, lse_out,
                                     (hipStream_t)stream);
    return e == hipSuccess ? MLA_OK : MLA_HIP_ERROR;
}

int mla_quant_fp8_workspace_size(size_t n, size_t* bytes) {
    if (!bytes) return MLA_INVALID_ARGUMENT;
    *bytes = align_up((size_t)mla::absmax_blocks(n) * sizeof(float));
    return MLA_OK;
}

int mla_quant_fp8(const void* x_bf16, size_t n, int32_t scale_mode, float* scale, void* out_fp8,
                  void* workspace, size_t workspace_bytes, void* stream) {
    if (!scale) return MLA_INVALID_ARGUMENT;
    if (scale_mode != MLA_Q_SCALE_STATIC && scale_mode != MLA_Q_SCALE_ABSMAX)
        return MLA_INVALID_ARGUMENT;
    if (n > 0 && (!x_bf16 || !out_fp8 || !aligned16(x_bf16) || !aligned16(out_fp8)))
        return MLA_INVALID_ARGUMENT;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (scale_mode == MLA_Q_SCALE_ABSMAX) {
        const size_t need = align_up((size_t)mla::absmax_blocks(n) * sizeof(float));
        if (workspace_bytes < need) return MLA_WORKSPACE_TOO_SMALL;
        if (!workspace) return MLA_INVALID_ARGUMENT;
        const int nb = mla::absmax_blocks(n);
        e = mla::launch_absmax_partial((const uint16_t*)x_bf16, n, (float*)workspace, nb, st);
        if (e != hipSuccess) return MLA_HIP_ERROR;
        e = mla::launch_quant_fp8((const uint16_t*)x_bf16, n, (uint8_t*)out_fp8, nullptr,
                                  (const float*)workspace, nb, scale, st);
    } else {
        e = mla::launch_quant_fp8((const uint16_t*)x_bf16, n, (uint8_t*)out_fp8, scale, nullptr, 0,
                                  nullptr, st);
    }
    return e == hipSuccess ? MLA_OK : MLA_HIP_ERROR;
}

int mla_encode_mxfp4(const void* x_bf16, size_t rows, void* packed, void* block_scales,
                     void* stream) {
    if (rows > 0 && (!x_bf16 || !packed || !block_scales || !aligned16(x_bf16) ||
                     !aligned16(packed)))
        return MLA_INVALID_ARGUMENT;
    if (rows > ((size_t)1 << 31)) return MLA_UNSUPPORTED;
    hipError_t e = mla::launch_mxfp4_encode((const uint16_t*)x_bf16, rows, (uint8_t*)packed,
                                            (uint8_t*)block_scales, (hipStream_t)stream);
    return e == hipSuccess ? MLA_OK : MLA_HIP_ERROR;
}

}  // extern "C"
