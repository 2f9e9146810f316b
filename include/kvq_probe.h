/*
 * kvq_probe.h -- streaming kernels that calibrate measurements of the kvq
 * kernels on the same device (libkvq_probe.so; not part of the kvq ABI).
 *
 * The decode kernels are bound by HBM bandwidth (NInfer KV-cache guide,
 * section on why the cache is quantized: each decode step reads the whole
 * cache, so stored bytes set the speed).  These two kernels give the
 * yardsticks such a kernel is judged by:
 *  - a read-only scan: the HBM read rate a kernel can actually reach, and a
 *    way to evict the L2 caches and the MALL between timed runs;
 *  - a copy: a known number of bytes read and written, against which the
 *    hardware's HBM byte counters are scaled.
 *
 * Both enqueue one kernel on the caller's stream and return at once.  The
 * caller owns every buffer.  Return values: 0 ok, 1 invalid argument (null
 * pointer or a size that is not a multiple of the unit below; nothing is
 * enqueued), 4 HIP error (the device query or the launch failed).
 */
#ifndef KVQ_PROBE_H
#define KVQ_PROBE_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read src[0, bytes) once (bytes a multiple of 1024, src 16-byte aligned).
 * sink: device memory of at least 4 bytes; written only if the data fold to
 * one particular 32-bit value, so that the loads cannot be optimized away. */
int kvq_probe_read(const void* src, size_t bytes, void* sink, hipStream_t stream);

/* The same read with the non-temporal hint on every load: the highest read
 * rate measured for a kernel that streams its data once (the decode
 * kernels' copies carry the same hint).  It does not evict the caches. */
int kvq_probe_read_stream(const void* src, size_t bytes, void* sink, hipStream_t stream);

/* dst[0, bytes) = src[0, bytes) (bytes a multiple of 16, both 16-byte
 * aligned, no overlap). */
int kvq_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_PROBE_H */
