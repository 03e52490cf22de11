// The fixed device scratch behind mla_decode_run_fused_noalloc (internal;
// the public interface is include/mla_decode.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "launch.h"

namespace mla {

// Largest plan the scratch serves: query rows and partial slots.
constexpr int32_t kNoallocMaxRows = 65536;
constexpr int32_t kNoallocMaxSlots = 500;

// Sections of the scratch, each on a 256-byte boundary. The arrival
// counters come first, at the same place for every plan: every fused run
// leaves the counters of its rows at zero, so once zeroed they stay zero
// from one call to the next whatever the plan.
constexpr size_t kNoallocCountersOff = 0;
constexpr size_t kNoallocBlockmaxOff = kNoallocCountersOff + size_t(kNoallocMaxRows) * 4;
constexpr size_t kNoallocLseOff = kNoallocBlockmaxOff + size_t(kMaxAbsmaxBlocks) * 4;
constexpr size_t kNoallocPartOff =
    kNoallocLseOff + (size_t(kNoallocMaxSlots) * 16 * 4 + 255) / 256 * 256;
constexpr size_t kNoallocScratchBytes = kNoallocPartOff + size_t(kNoallocMaxSlots) * 16 * 512 * 4;
static_assert(kNoallocBlockmaxOff % 256 == 0 && kNoallocLseOff % 256 == 0 &&
                  kNoallocPartOff % 256 == 0 && kNoallocScratchBytes % 256 == 0,
              "sections on 256-byte boundaries");

// The scratch's address on the current device. The first call on a device
// resolves it (hipGetSymbolAddress, with that device current) and enqueues
// a fill kernel on `stream` that zeroes the counters; later calls return the
// address kept for the device. nullptr and *status = MLA_HIP_ERROR (or
// MLA_UNSUPPORTED for a device index beyond the table) on failure.
void* noalloc_scratch(hipStream_t stream, int* status);

}  // namespace mla
