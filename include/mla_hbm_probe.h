/*
 * mla_hbm_probe.h -- C ABI of libmla_hbm_probe.so, a measurement helper kept
 * apart from the decode library: the practical HBM read bandwidth of the
 * device, against which the decode kernels' achieved bandwidth is also
 * reported (beside the nominal peak).
 */
#ifndef MLA_HBM_PROBE_H
#define MLA_HBM_PROBE_H

#include <stddef.h>

#if defined(__GNUC__) || defined(__clang__)
#define MLA_PROBE_API __attribute__((visibility("default")))
#else
#define MLA_PROBE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Enqueue one streaming read of `bytes` bytes of device memory at `buf`
 * (16-byte aligned, bytes a non-zero multiple of 16) on `stream` (a
 * hipStream_t, NULL = default), with `grid` workgroups of 256 threads
 * (1 .. 2^20), each thread reading 16 bytes per step. `sink` is a device
 * unsigned[1] the kernel writes only for one improbable folded value.
 * Time it with events around the call. Returns 0, 1 (invalid argument) or
 * 3 (launch failure); nothing is allocated.
 */
MLA_PROBE_API int mla_hbm_read_probe(const void* buf, size_t bytes, unsigned* sink, int grid,
                                     void* stream);

/*
 * The same read with non-temporal loads (the caches do not allocate the
 * lines). Same arguments, errors and ownership.
 */
MLA_PROBE_API int mla_hbm_read_probe_nt(const void* buf, size_t bytes, unsigned* sink, int grid,
                                        void* stream);

/*
 * The same streaming read through buffer->LDS copies with the non-temporal
 * hint, the copy form of the decode kernels' large-cache path: each of the
 * `grid` workgroups (1 .. 2^20, 256 threads) takes 1 MiB chunks of `buf` in
 * turn and copies them into its own LDS, 16 KiB in flight per wave. `buf`
 * 16-byte aligned, `bytes` a non-zero multiple of 16; nothing is written to
 * device memory. Returns 0, 1 (invalid argument) or 3 (launch failure);
 * nothing is allocated.
 */
MLA_PROBE_API int mla_hbm_read_probe_lds_nt(const void* buf, size_t bytes, int grid,
                                            void* stream);

#ifdef __cplusplus
}
#endif

#endif
