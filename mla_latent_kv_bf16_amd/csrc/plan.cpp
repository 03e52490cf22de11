// Host-side scheduler for the split-KV decode: turns the CSR row pointers
// into work items (one workgroup each) and a merge map. Pure C++, no HIP, so
// it is exercised by the CPU test suite through mla_decode_plan_host.
//
// The pages compute this once per shape because it depends only on
// qo_indptr / kv_indptr [kernelindex.com amd-mixed-mla submission 663509,
// module docstring point 2 and `_precompute_metadata`]. Their split counts
// were fixed (32) or stepped by total tokens [722089 `_aiter_path`, 738050
// `_get_num_kv_splits`]; here the split count is derived from the number of
// compute units instead: aim for about one item per CU, each item at least
// kMinChunk tokens, split boundaries on the 32-token tile grid. (Measured on
// the GPU: items shorter than 256 tokens spend more in their prologue and in
// the merge than they gain from the extra parallelism.)
#include "plan.h"

#include "../../include/mla_decode.h"

#include <algorithm>
#include <cstdint>
#include <vector>

namespace mla {

namespace {

// Workgroup i runs on XCD i mod 8 (the dispatcher hands workgroups to the
// eight XCDs in turn), and each XCD has its own L2. The items of one sequence
// read the same bf16 Q rows (a sequence with several query rows also the same
// cache rows), so they go to indices of one residue mod 8 where the counts
// allow: sequences take the residues in turn, in the order of their longest
// item, and index 8 j + r holds the j-th item of residue r's list, or, once
// that list has run out, the next item of the list with the most left. Each
// XCD still receives its items longest first. Only the order changes: every
// item computes the same result wherever it runs. (Measured: bs32 kv1024
// 15.1 -> 14.4 us per call, as three of the four splits of a sequence find
// its Q rows in L2.)
template <class It, class Key>
void xcd_order(std::vector<It>& items, int32_t nkeys, Key key) {
    constexpr int kXcds = 8;
    std::vector<std::vector<It>> lists(kXcds);
    std::vector<int32_t> res((size_t)nkeys, -1);
    int32_t next = 0;
    for (const It& it : items) {
        int32_t& r = res[(size_t)key(it)];
        if (r < 0) r = next++ % kXcds;
        lists[(size_t)r].push_back(it);
    }
    std::vector<size_t> pos(kXcds, 0);
    std::vector<It> out;
    out.reserve(items.size());
    while (out.size() < items.size()) {
        for (int r = 0; r < kXcds && out.size() < items.size(); ++r) {
            int src = r;
            if (pos[(size_t)r] == lists[(size_t)r].size()) {
                size_t most = 0;
                for (int q = 0; q < kXcds; ++q) {
                    const size_t left = lists[(size_t)q].size() - pos[(size_t)q];
                    if (left > most) {
                        most = left;
                        src = q;
                    }
                }
            }
            out.push_back(lists[(size_t)src][pos[(size_t)src]++]);
        }
    }
    items.swap(out);
}

}  // namespace

int build_schedule(const int32_t* qo, const int32_t* kv, int32_t batch, int32_t num_heads,
                   int32_t kv_format, int32_t num_cus, int32_t max_splits, Schedule* out) {
    if (!qo || !kv || !out || batch < 0) return 1;
    if (num_heads != kNumHeads) return 2;
    if (kv_format < 0 || kv_format > 2) return 2;  // FP8, MXFP4, bf16
    if (qo[0] != 0 || kv[0] != 0) return 1;
    for (int32_t b = 0; b < batch; b++) {
        if (kv[b + 1] < kv[b]) return 1;
        if (qo[b + 1] < qo[b]) return 1;
    }
    if (num_cus <= 0) num_cus = kDefaultCUs;

    // One unit of work per query row. A sequence with R rows holds its last R
    // positions; row i attends to the first len - (R - 1 - i) of its cache
    // rows (bottom-right aligned causal; the whole cache when R = 1), so each
    // row is scheduled as its own range and indexes Q and the output directly.
    const int64_t total_q = qo[batch];
    if (total_q > (int64_t)INT32_MAX / kNumHeads) return 2;
    std::vector<int32_t> rb((size_t)total_q), re((size_t)total_q);
    int64_t total = 0;
    for (int32_t b = 0; b < batch; b++) {
        const int64_t R = (int64_t)qo[b + 1] - qo[b];
        for (int64_t i = 0; i < R; i++) {
            const int64_t row = qo[b] + i;
            const int64_t end = std::max<int64_t>(kv[b], (int64_t)kv[b + 1] - (R - 1 - i));
            rb[(size_t)row] = kv[b];
            re[(size_t)row] = (int32_t)end;
            total += end - kv[b];
        }
    }
    const int32_t nrows = (int32_t)total_q;
    // chunk target: the whole cache spread over about num_cus items
    int64_t chunk = (total + num_cus - 1) / std::max<int64_t>(num_cus, 1);
    chunk = std::max<int64_t>(chunk, kMinChunk);

    const int64_t max_item = max_item_tokens(kv_format);
    Schedule s;
    s.batch = nrows;
    s.total_kv = kv[batch];
    s.kv_format = kv_format;
    std::vector<int32_t> nsplit(nrows, 0);
    for (int32_t b = 0; b < nrows; b++) {
        int64_t len = (int64_t)re[b] - rb[b];
        if (len == 0) continue;
        int64_t tiles = (len + kTileTokens - 1) / kTileTokens;
        int64_t sp;
        if (max_splits < 0)
            sp = -(int64_t)max_splits;
        else
            sp = (len + chunk - 1) / chunk;
        if (max_splits > 0) sp = std::min<int64_t>(sp, max_splits);
        sp = std::max<int64_t>(1, std::min<int64_t>({sp, tiles, kMaxSplits}));
        sp = std::max<int64_t>(sp, (len + max_item - 1) / max_item);
        // equal pieces on the tile grid; drop pieces that would be empty
        int64_t per = ((len + sp - 1) / sp + kTileTokens - 1) / kTileTokens * kTileTokens;
        sp = (len + per - 1) / per;
        if (sp > kMaxSplitsPerSeq) return 2;  // MLA_UNSUPPORTED
        nsplit[b] = (int32_t)sp;
        for (int64_t k = 0; k < sp; k++) {
            Item it;
            it.b = b;
            it.kv_begin = (int32_t)(rb[b] + k * per);
            it.kv_end = (int32_t)std::min<int64_t>(rb[b] + (k + 1) * per, re[b]);
            it.slot = (int32_t)k;  // relative for now
            s.items.push_back(it);
        }
    }
    // slots for split rows, merge entries for split and empty rows
    std::vector<int32_t> slot_base(nrows, -1);
    int32_t nslots = 0;
    for (int32_t b = 0; b < nrows; b++) {
        if (nsplit[b] >= 2) {
            slot_base[b] = nslots;
            s.merges.push_back({b, nslots, nsplit[b], 0});
            nslots += nsplit[b];
        } else if (nsplit[b] == 0) {
            s.merges.push_back({b, 0, 0, 0});
        }
    }
    for (Item& it : s.items) it.slot = (nsplit[it.b] >= 2) ? slot_base[it.b] + it.slot : -1;
    // longest items first, so the last wave of workgroups is the short one,
    // then grouped by sequence on the XCDs
    std::stable_sort(s.items.begin(), s.items.end(), [](const Item& x, const Item& y) {
        return (x.kv_end - x.kv_begin) > (y.kv_end - y.kv_begin);
    });
    std::vector<int32_t> seq_of_row((size_t)nrows);
    for (int32_t b = 0; b < batch; b++)
        for (int32_t r = qo[b]; r < qo[b + 1]; r++) seq_of_row[(size_t)r] = b;
    xcd_order(s.items, batch, [&](const Item& it) { return seq_of_row[(size_t)it.b]; });
    s.num_slots = nslots;
    *out = std::move(s);
    return 0;
}

bool use_rows_schedule(const int32_t* qo, int32_t batch, int32_t kv_format, bool paged,
                       size_t per_row_items, int32_t num_cus) {
    if (num_cus <= 0) num_cus = kDefaultCUs;
    (void)paged;
    if (!(kv_format == 0 || (kv_format == 1 && per_row_items > (size_t)num_cus))) return false;
    bool multi = false;
    for (int32_t b = 0; b < batch; b++) {
        const int32_t R = qo[b + 1] - qo[b];
        if (R < 1 || R > kMaxSharedRows) return false;
        multi |= R > 1;
    }
    return multi;
}

void build_rows_schedule(const int32_t* qo, const int32_t* kv, int32_t batch, int32_t num_cus,
                         int32_t max_splits, RowsSchedule* out) {
    if (num_cus <= 0) num_cus = kDefaultCUs;
    const int64_t total = kv[batch];
    int64_t chunk = (total + num_cus - 1) / std::max<int64_t>(num_cus, 1);
    chunk = std::max<int64_t>(chunk, kMinChunk);
    RowsSchedule s;
    s.batch = batch;
    s.rows = qo[batch];
    for (int32_t b = 0; b < batch; b++) {
        const int32_t R = qo[b + 1] - qo[b];
        const int64_t len = (int64_t)kv[b + 1] - kv[b];
        RowsItem proto{};
        proto.b = b;
        proto.q_row0 = qo[b];
        proto.rows = R;
        proto.seq_end = kv[b + 1];
        if (len == 0) {
            // rows of an empty sequence: O = 0, LSE = -inf (merge or fused item)
            proto.kv_begin = proto.kv_end = kv[b];
            proto.split = -1;
            s.empty.push_back(proto);
            for (int32_t r = 0; r < R; r++) s.merges.push_back({qo[b] + r, 0, 0, 0});
            continue;
        }
        const int64_t tiles = (len + kTileTokens - 1) / kTileTokens;
        int64_t sp = max_splits < 0 ? -(int64_t)max_splits : (len + chunk - 1) / chunk;
        if (max_splits > 0) sp = std::min<int64_t>(sp, max_splits);
        sp = std::max<int64_t>(1, std::min<int64_t>({sp, tiles, kMaxSplits}));
        sp = std::max<int64_t>(sp, (len + max_item_tokens(0) - 1) / max_item_tokens(0));
        const int64_t per = ((len + sp - 1) / sp + kTileTokens - 1) / kTileTokens * kTileTokens;
        sp = (len + per - 1) / per;
        proto.nsplit = sp >= 2 ? (int32_t)sp : 0;
        proto.slot_base = sp >= 2 ? s.num_slots : 0;
        for (int64_t k = 0; k < sp; k++) {
            RowsItem it = proto;
            it.kv_begin = (int32_t)(kv[b] + k * per);
            it.kv_end = (int32_t)std::min<int64_t>(kv[b] + (k + 1) * per, kv[b + 1]);
            it.split = sp >= 2 ? (int32_t)k : -1;
            s.items.push_back(it);
        }
        if (sp >= 2) {
            for (int32_t r = 0; r < R; r++)
                s.merges.push_back({qo[b] + r, s.num_slots + r * (int32_t)sp, (int32_t)sp, 0});
            s.num_slots += R * (int32_t)sp;
        }
    }
    // longest items first, so the last wave of workgroups is the short one,
    // then grouped by sequence on the XCDs
    std::stable_sort(s.items.begin(), s.items.end(), [](const RowsItem& x, const RowsItem& y) {
        return (x.kv_end - x.kv_begin) > (y.kv_end - y.kv_begin);
    });
    xcd_order(s.items, batch, [](const RowsItem& it) { return it.b; });
    *out = std::move(s);
}

}  // namespace mla

extern "C" int mla_decode_plan_host(const int32_t* qo_indptr_host, const int32_t* kv_indptr_host,
                                    int32_t batch, int32_t num_heads, int32_t kv_format,
                                    int32_t num_cus, int32_t max_splits, int32_t* items_out,
                                    int32_t items_cap, int32_t* merge_out, int32_t merge_cap,
                                    int32_t* counts_out) {
    try {
        mla::Schedule s;
        int st = mla::build_schedule(qo_indptr_host, kv_indptr_host, batch, num_heads,
                                     kv_format, num_cus, max_splits, &s);
        if (st) return st;
        int32_t ni = (int32_t)s.items.size(), nm = (int32_t)s.merges.size();
        if ((items_out && items_cap < ni) || (merge_out && merge_cap < nm)) return 1;
        if (items_out)
            for (int32_t i = 0; i < ni; i++) {
                items_out[4 * i + 0] = s.items[i].b;
                items_out[4 * i + 1] = s.items[i].kv_begin;
                items_out[4 * i + 2] = s.items[i].kv_end;
                items_out[4 * i + 3] = s.items[i].slot;
            }
        if (merge_out)
            for (int32_t i = 0; i < nm; i++) {
                merge_out[4 * i + 0] = s.merges[i].b;
                merge_out[4 * i + 1] = s.merges[i].slot_begin;
                merge_out[4 * i + 2] = s.merges[i].nslots;
                merge_out[4 * i + 3] = 0;
            }
        if (counts_out) {
            counts_out[0] = ni;
            counts_out[1] = nm;
            counts_out[2] = s.num_slots;
        }
        return 0;
    } catch (...) {
        return 5;  // MLA_OUT_OF_MEMORY
    }
}
