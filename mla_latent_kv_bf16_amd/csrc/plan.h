// Internal scheduler types shared by plan.cpp and api.cpp (not installed).
#pragma once
#include <cstddef>
#include <cstdint>
#include <vector>

namespace mla {

constexpr int32_t kNumHeads = 16;
constexpr int32_t kDefaultCUs = 256;   // MI355X compute units
constexpr int32_t kTileTokens = 32;    // tokens per stage-1 tile (one wave's LDS stage)
constexpr int32_t kMinChunk = 256;     // smallest split: two tiles for each of 4 waves
constexpr int32_t kMaxSplits = 64;     // policy bound on partials per sequence
// Most partials one query row can have: it sizes the merge's LDS scratch. A
// row whose range needs more items (only possible for the bf16 cache beyond
// 2^30 rows) is UNSUPPORTED.
constexpr int32_t kMaxSplitsPerSeq = 512;

// Longest item, in cache rows: the kernels address an item's rows with
// 32-bit byte offsets, so rows * (bytes per row) stays below 2^32 (576 B per
// FP8 row and 288 + 18 B per MXFP4 row: 2^22 rows; 1,152 B per bf16 row:
// 2^21). A multiple of the tile size.
constexpr int64_t max_item_tokens(int32_t kv_format) {
    return kv_format == 2 ? (int64_t(1) << 21) : (int64_t(1) << 22);
}

struct Item {          // one stage-1 workgroup
    int32_t b;         // sequence (== its query row)
    int32_t kv_begin;  // absolute cache rows [kv_begin, kv_end)
    int32_t kv_end;
    int32_t slot;      // partial slot, -1 = write the final output
};

struct Merge {         // one stage-2 workgroup
    int32_t b;
    int32_t slot_begin;
    int32_t nslots;    // 0 = empty sequence: O = 0, LSE = -inf
    int32_t pad;
};

struct Schedule {
    int32_t batch = 0;
    int64_t total_kv = 0;
    int32_t kv_format = 0;
    int32_t num_slots = 0;
    std::vector<Item> items;
    std::vector<Merge> merges;
};

// Work item of the kernels in which a sequence's query rows share every KV
// tile (FP8 or MXFP4 cache, 1-4 rows per sequence): three int4.
struct RowsItem {
    int32_t b, kv_begin, kv_end, split;  // split index, -1 = covers the sequence
    int32_t q_row0, rows, seq_end, nsplit;
    int32_t slot_base, pad0, pad1, pad2;  // row r of split s: slot_base + r * nsplit + s;
                                          // a paged plan keeps its sequence's first
                                          // page-table entry and pages in pad0, pad1
};

struct RowsSchedule {
    int32_t batch = 0;       // sequences
    int32_t rows = 0;        // query rows
    int32_t num_slots = 0;
    std::vector<RowsItem> items;
    std::vector<Merge> merges;   // per query row: {row, first slot, slots, 0}
    std::vector<RowsItem> empty; // one item per empty sequence (fused form)
};

constexpr int32_t kMaxSharedRows = 4;

// Returns an mla_status code (0 = OK).
int build_schedule(const int32_t* qo, const int32_t* kv, int32_t batch, int32_t num_heads,
                   int32_t kv_format, int32_t num_cus, int32_t max_splits, Schedule* out);

// The shared-row schedule: splits per sequence (the cache is read once for
// all of its rows). Arguments as build_schedule, already validated by it.
void build_rows_schedule(const int32_t* qo, const int32_t* kv, int32_t batch, int32_t num_cus,
                         int32_t max_splits, RowsSchedule* out);

// True when a shared-row kernel serves this batch: every sequence has
// 1..kMaxSharedRows rows, at least one has more than one, and the cache is
// FP8 or MXFP4 (contiguous or paged). For MXFP4 only when the
// per-row schedule (per_row_items items) would take more than one round of
// num_cus workgroups: a shared MXFP4 item does R rows' decode work, so in a
// single round per-row items finish sooner (measured on MI355X: bs4 kv1024
// with 4 rows 17.9 against 34.6 us, bs64 kv16384 with 2 rows 95 against
// 102 us), while several rounds of per-row items re-read the cache and pay
// each item's fixed costs again (bs256 kv8192 with 2 rows 182 against 225 us).
bool use_rows_schedule(const int32_t* qo, int32_t batch, int32_t kv_format, bool paged,
                       size_t per_row_items, int32_t num_cus);

}  // namespace mla
