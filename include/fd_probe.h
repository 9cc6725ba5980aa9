/*
 * fd_probe.h - HBM bandwidth probes that sit beside the decode kernels in
 * libfd.so. They are measurement tools, not part of decode attention: the
 * profiling checklist of the lpnh.cn memory-wall article (§5.5) judges a
 * kernel by its DRAM throughput against what the memory can deliver, and these
 * kernels measure that: a pure streaming read, a read of two row-major
 * buffers in the decode kernels' own access pattern, and a plain copy of a
 * known size whose HBM counter readings calibrate the counters taken on the
 * decode kernels.
 *
 * All run asynchronously on `stream` (a hipStream_t as void*, NULL = default),
 * allocate nothing and return FD_ERR_INVALID_ARGUMENT, having launched
 * nothing, if a pointer is NULL or not 16-byte aligned or `bytes` is not a
 * positive multiple of 16.
 */
#ifndef FD_PROBE_H
#define FD_PROBE_H

#include <stddef.h>

#include "fd.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Floats the read probe's `sink` must hold (one per work-group). */
#define FD_PROBE_SINK_FLOATS 4096

/* Reads every byte of src[0, bytes) once with 16-byte loads and writes a
 * data-dependent value per work-group to sink (device memory holding
 * FD_PROBE_SINK_FLOATS floats) so the reads cannot be elided. */
fd_status fd_probe_read(const void* src, size_t bytes, float* sink, void* stream);

/* Reads two buffers a and b of `rows` rows of `row_bytes` bytes each
 * (row_bytes a multiple of 1024; a token-major K and V cache, for instance)
 * in the pattern of the decode kernels that read whole rows: one work-group
 * of eight waves per (chunk of chunk_rows rows, column block), 1 KB of one row
 * per wave instruction, 4 rows of a and 4 of b per wave stage with the next
 * stage in flight. waves_across 0: block_bytes 1024, the eight waves split
 * the chunk's rows; waves_across 1: block_bytes 8192, wave w reads column w of
 * the block in every row; waves_across 2: as 0, but a chunk whose stages are a
 * whole multiple of the eight waves starts at a rotated stage (chunk c at
 * (7 c mod n) 8 of its n 8 stages, wrapping round), the traversal of the
 * head-rows kernel on a 16-bit cache. Any other value: FD_ERR_INVALID_ARGUMENT.
 * sink: device memory of FD_PROBE_SINK_FLOATS floats. */
fd_status fd_probe_read_rows(const void* a, const void* b, int64_t rows, int32_t row_bytes, int32_t block_bytes,
                             int32_t chunk_rows, int32_t waves_across, float* sink, void* stream);

/* Copies src[0, bytes) to dst[0, bytes) with 16-byte loads and stores. The
 * ranges must not overlap. */
fd_status fd_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FD_PROBE_H */
