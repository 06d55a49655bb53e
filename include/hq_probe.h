/*
 * hq_probe.h -- measurement helper beside libhq.so (not part of the method).
 *
 * libhq_probe.so holds a plain streaming-read kernel, the achievable-HBM
 * reference that the benchmark reports next to the nominal 8 TB/s peak, and
 * a matrix-core rate probe.
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

/*
 * Matrix-core rate: `grid` workgroups of 256 threads each run `iters` rounds
 * of independent fp16 MFMA chains: which = 0: v_mfma_f32_16x16x32_f16, eight
 * chains a wave; 1: v_mfma_f32_32x32x16_f16, four chains; 2 and 3: the same
 * with the column-mass work of each MFMA's outputs (fma, exp2, add per output
 * element and lane) interleaved.  FLOP per launch: grid * 4 waves * iters *
 * chains * (16384 or 32768).  *sink (device, 256 floats) is written only for
 * an impossible checksum.  Returns 0, -1 for bad arguments, -6 when the
 * launch fails.
 */
int hq_probe_mfma_rate(int which, int grid, int iters, float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
