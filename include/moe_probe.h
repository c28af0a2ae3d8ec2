/*
 * moe_probe.h - bandwidth probes for gfx950 (libmoe_probe.so).
 *
 * Reference kernels that the benchmark times beside the routing path, so
 * that the achievable HBM rates the finalize kernel is judged against are
 * measured in the same run, on the same access patterns: streaming reads
 * with the loads finalize uses, streaming writes with its stores, and its
 * gather without the stores. Two more give the fixed costs that bound the
 * small batches: a launch that does nothing, and one workgroup reading a
 * small buffer (after a kernel that wrote it, the latency of handing data
 * from one launch to the next). They are not part of the routing path and
 * compute nothing of the method.
 *
 * Conventions as in moe_route.h: device pointers owned by the caller,
 * asynchronous on `stream` (a hipStream_t as void*), status codes checked on
 * the host before any launch.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include "moe_route.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * moe_probe_read
 * Reads `bytes` bytes of `src` once: each wave reads 8 KiB as eight 16-byte
 * non-temporal loads per lane, all in flight together (the loads of
 * moe_finalize). Nothing is written unless the data happen to XOR to a
 * fixed 32-bit pattern, in which case one word goes to sink[0] (this keeps
 * the loads live).
 * Validation: bytes a multiple of 8192 and at most 2^40; src 16-byte
 * aligned; src and sink non-NULL when bytes > 0.
 */
moe_status_t moe_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * moe_probe_write
 * Fills `bytes` bytes of `dst` with the 32-bit `value`: each wave writes
 * 1 KiB as one 16-byte store per lane through a buffer resource, with cache
 * policy nt when `streaming` is non-zero and sc1 otherwise (the two kinds of
 * store moe_finalize makes: nt when its gathered rows exceed the 256 MiB
 * memory-side cache, sc1 below).
 * Validation: bytes a multiple of 1024 and at most 2^40; dst 16-byte
 * aligned and non-NULL when bytes > 0.
 */
moe_status_t moe_probe_write(void* dst, size_t bytes, uint32_t value, int32_t streaming,
                             void* stream);

/*
 * moe_probe_gather
 * The loads of moe_finalize alone: for each token t < T and each 1 KiB
 * column chunk of a row of `row_bytes` bytes, one wave reads that chunk of
 * rows restore[t*K + k] of `rows` (K rows, at most 8 loads in flight per
 * lane) and folds them with XOR; nothing is written unless a fixed pattern
 * appears (one word to sink[0]).
 * Validation: T >= 0, 1 <= K, T*K < 2^32, row_bytes a positive multiple of
 * 16 below 2^31, T * ceil(row_bytes / 1024) below 2^32 - 2^18; pointers
 * non-NULL and rows 16-byte aligned when T > 0. restore entries must be
 * below T*K (larger ones read row 0).
 */
moe_status_t moe_probe_gather(const void* rows, const uint32_t* restore, int64_t T, int32_t K,
                              int64_t row_bytes, uint32_t* sink, void* stream);

/*
 * moe_probe_empty
 * Launches `workgroups` workgroups of 256 threads that do nothing: the cost
 * of a launch itself.
 * Validation: 1 <= workgroups <= 65535.
 */
moe_status_t moe_probe_empty(int32_t workgroups, void* stream);

/*
 * moe_probe_consume
 * One workgroup of 1024 threads reads `bytes` bytes of `src` (each thread
 * issues all of its 16-byte loads, up to 16, before using any) and folds
 * them with XOR; nothing is written unless a fixed pattern appears (one
 * word to sink[0]).
 * Validation: bytes a multiple of 16 KiB and at most 256 KiB; src 16-byte
 * aligned; src and sink non-NULL when bytes > 0.
 */
moe_status_t moe_probe_consume(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
