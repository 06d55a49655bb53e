/*
 * hq_probe.h -- measurement helper beside libhq.so (not part of the method).
 *
 * libhq_probe.so holds a plain streaming-read kernel, the achievable-HBM
 * reference that the benchmark reports next to the nominal 8 TB/s peak.
 */
#ifndef HQ_PROBE_H
#define HQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads bytes (a multiple of 16; src 16-byte aligned, device memory) once,
 * with 16-byte loads from `grid` workgroups of 256 threads, every loaded word
 * folded into a checksum; *sink (device) is written only if the checksum
 * equals `never`, so the loads cannot be dropped.  Returns 0, or -1 for bad
 * arguments, or -6 when the launch fails.
 */
int hq_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, uint32_t never,
                         int grid, hipStream_t stream);

/* The same read with non-temporal loads (the policy of the decode scan's
 * cache loads). */
int hq_probe_stream_read_nt(const void* src, size_t bytes, uint32_t* sink, uint32_t never,
                            int grid, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
