// The fixed device scratch of mla_decode_run_fused_noalloc: the workspace of
// a fused decode step (arrival counters, absmax partial maxima, split
// partials) for callers that cannot allocate. One copy per device, held
// until the process ends; every call on a device shares it.
#include <mutex>

#include "../../include/mla_decode.h"
#include "noalloc.h"

namespace mla {
namespace {

// Only the device-side storage: host code never uses this name as an
// address (on the host it is a stand-in), only the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
void* g_ptr[kMaxDevices];  // the scratch's address on each device, once resolved
std::mutex g_mu;

}  // namespace

void* noalloc_scratch(hipStream_t stream, int* status) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        *status = MLA_HIP_ERROR;
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *status = MLA_UNSUPPORTED;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            *status = MLA_HIP_ERROR;
            return nullptr;
        }
        // the counters must start at zero (a fill kernel: no memset node
        // if the caller is capturing a graph)
        if (launch_zero_u32((uint32_t*)((uint8_t*)p + kNoallocCountersOff),
                            (size_t)kNoallocMaxRows, stream) != hipSuccess) {
            *status = MLA_HIP_ERROR;
            return nullptr;
        }
        g_ptr[dev] = p;
    }
    *status = MLA_OK;
    return g_ptr[dev];
}

}  // namespace mla
