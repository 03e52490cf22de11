// Internal scheduler types shared by plan.cpp and api.cpp (not installed).
#pragma once
#include <cstdint>
#include <vector>

namespace mla {

constexpr int32_t kNumHeads = 16;
constexpr int32_t kDefaultCUs = 256;   // MI355X compute units
constexpr int32_t kTileTokens = 32;    // tokens per stage-1 tile (one wave's LDS stage)
constexpr int32_t kMinChunk = 256;     // smallest split: two tiles for each of 4 waves
constexpr int32_t kMaxSplits = 64;     // policy bound on partials per sequence
constexpr int64_t kMaxItemTokens = int64_t(1) << 22;  // keeps an item's bytes below 2^32

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

// Returns an mla_status code (0 = OK).
int build_schedule(const int32_t* qo, const int32_t* kv, int32_t batch, int32_t num_heads,
                   int32_t kv_format, int32_t num_cus, int32_t max_splits, Schedule* out);

}  // namespace mla
