/*
 * fd_probe.h - HBM bandwidth probes that sit beside the decode kernels in
 * libfd.so. They are measurement tools, not part of decode attention: the
 * profiling checklist of the lpnh.cn memory-wall article (§5.5) judges a
 * kernel by its DRAM throughput against what the memory can deliver, and these
 * two kernels measure that: a pure streaming read, and a plain copy of a known
 * size whose HBM counter readings calibrate the counters taken on the decode
 * kernels.
 *
 * Both run asynchronously on `stream` (a hipStream_t as void*, NULL = default),
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

/* Copies src[0, bytes) to dst[0, bytes) with 16-byte loads and stores. The
 * ranges must not overlap. */
fd_status fd_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FD_PROBE_H */
