// Kernel launchers of libmla_decode.so (internal; the public interface is
// include/mla_decode.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kMaxAbsmaxBlocks = 1024;

// Blocks used by the absmax pass for n elements (also the number of partial
// maxima it writes).
int absmax_blocks(size_t n);

hipError_t launch_absmax_partial(const uint16_t* x, size_t n, float* blockmax, int nblocks,
                                 hipStream_t stream);

// blockmax == nullptr: static scale read from scale_in[0].
// Otherwise the scale is fp32(max(max(blockmax), 1e-12)) / 448, and block 0
// writes it to scale_out[0].
hipError_t launch_quant_fp8(const uint16_t* x, size_t n, uint8_t* out, const float* scale_in,
                            const float* blockmax, int nblockmax, float* scale_out,
                            hipStream_t stream);

hipError_t launch_mxfp4_encode(const uint16_t* x, size_t rows, uint8_t* packed, uint8_t* scales,
                               hipStream_t stream);

hipError_t launch_stage1_fp8(const int4* items, int nitems, const uint8_t* q8,
                             const float* q_scale, const uint8_t* kv, const float* kv_scale,
                             float sm_scale, float* part_o, float* part_lse, uint16_t* out,
                             float* lse_out, hipStream_t stream);

hipError_t launch_stage1_mxfp4(const int4* items, int nitems, const uint8_t* q8,
                               const float* q_scale, const uint8_t* kv_packed,
                               const uint8_t* kv_scales, float sm_scale, float* part_o,
                               float* part_lse, uint16_t* out, float* lse_out,
                               hipStream_t stream);

hipError_t launch_merge(const int4* merges, int nmerge, const float* part_o,
                        const float* part_lse, uint16_t* out, float* lse_out, hipStream_t stream);

}  // namespace mla
