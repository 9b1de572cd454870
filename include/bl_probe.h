/*
 * bl_probe.h -- measurement aids of the benchmark (libblprobe.so).
 *
 * Not part of the BitLinear method: two trivial gfx950 kernels that give the
 * floors the decode GEMV is measured against on the same machine and in the
 * same launch setting (HIP graphs, cold buffers).
 *
 * Conventions: device pointers owned by the caller; `stream` is a
 * hipStream_t (NULL = default); calls only enqueue work and return 0, or -1
 * for a bad argument (nothing enqueued), or -6 when the launch fails.
 */
#ifndef BL_PROBE_H
#define BL_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * blp_stream_read -- read `bytes` bytes from `src` once, as `blocks`
 * workgroups of 256 threads that each own bytes/blocks contiguous bytes,
 * with 128-bit loads (8 in flight per lane). Each workgroup writes one
 * 32-bit word to sink[block] only when a combined value matches a pattern
 * that zero-filled data never produces, so the loads cannot be elided and
 * nothing else is written. Requires bytes % (16 * blocks) == 0, blocks >= 1,
 * src 16-byte aligned, sink holding `blocks` words.
 */
int blp_stream_read(const void *src, size_t bytes, int blocks, uint32_t *sink, void *stream);

/* blp_empty -- one launch of an empty kernel of `blocks` x 256 threads. */
int blp_empty(int blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BL_PROBE_H */
