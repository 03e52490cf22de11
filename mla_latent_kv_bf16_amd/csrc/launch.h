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

struct Stage1Args;  // stage_common.h

// Stage-1 launches over nitems work items. Plain form: args.items holds one
// int4 per item and Q codes come from args.q8_in. Fused form: two int4 per
// item, Q is quantised from args.q_bf16 in the kernel and split sequences are
// merged by their last workgroup (args.counters zero on entry, zero on exit).
hipError_t launch_stage1_fp8(const Stage1Args& args, int nitems, bool fused,
                             hipStream_t stream);
hipError_t launch_stage1_mxfp4(const Stage1Args& args, int nitems, bool fused,
                               hipStream_t stream);

// FP8 stage 1 for sequences with 1-4 query rows sharing each KV tile; items
// are three int4 each (see stage1_fp8_rows.hip).
hipError_t launch_stage1_fp8_rows(const Stage1Args& args, int nitems, bool fused,
                                  hipStream_t stream);
// The same items for a contiguous MXFP4 cache (see stage1_mxfp4.hip).
hipError_t launch_stage1_mxfp4_rows(const Stage1Args& args, int nitems, bool fused,
                                    hipStream_t stream);

// bf16 cache (no quantisation), optional logit soft-cap (cap > 0); items as
// launch_stage1_fp8 (two int4 each in the fused form).
hipError_t launch_stage1_bf16(const Stage1Args& args, float logit_cap, int nitems, bool fused,
                              hipStream_t stream);

// Zero n 32-bit words (a fill kernel, so the call can sit in a captured graph).
hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t stream);

hipError_t launch_merge(const int4* merges, int nmerge, const float* part_o,
                        const float* part_lse, uint16_t* out, float* lse_out, hipStream_t stream);

}  // namespace mla
