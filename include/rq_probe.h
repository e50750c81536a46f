/*
 * rq_probe.h -- measurement helper in librq.so: a plain HBM read stream, the
 * attainable-bandwidth reference that decode throughput is compared with.
 * Decode over a compressed KV cache is bound by the bytes it reads
 * (ResidualQuant page, Abstract: less KV memory traffic is what speeds
 * decode up), so its roofline is the rate at which a kernel that does
 * nothing but read can stream HBM on the same device.  Conventions (device
 * pointers, validation before enqueue, stream semantics, errors) are those
 * of rq.h.
 */
#ifndef RQ_PROBE_H_
#define RQ_PROBE_H_

#include "rq.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * rq_probe_read_stream -- read `bytes` bytes of `buf` once with 128-bit
 * loads, four loads in flight per lane, and write one 32-bit XOR of what
 * each lane read to sink[n_blocks * 256], so that no load is dead.
 *   buf          device buffer, 16-byte aligned; bytes a multiple of 16, >= 16
 *   nontemporal  0: default cache policy; 1: loads with the non-temporal hint
 *                (the policy the decode kernel uses for its streamed planes)
 *   pattern      0: grid stride (consecutive lanes of the whole grid read
 *                consecutive 16 bytes); 1: chunked (workgroup b reads the
 *                b-th of n_blocks contiguous chunks, 16 KiB per iteration);
 *                2: planes (the buffer cut into 20 equal planes, workgroup b
 *                walking the b-th chunk of all of them at once, as a decode
 *                workgroup walks every plane of its (batch, head); only the
 *                whole 4 KiB segments of each chunk are read, so the bytes
 *                read are 20 * 4096 * floor(bytes / 20 / 16 / n_blocks / 256)
 *                * n_blocks)
 *   n_blocks     1 .. 65535 workgroups of 256 lanes
 *   sink         device uint32 [n_blocks * 256], 16-byte aligned; written
 * Returns RQ_ERR_INVALID_ARG for a null, misaligned or mis-sized argument,
 * RQ_ERR_DEVICE if the launch fails.
 */
rq_status rq_probe_read_stream(const void *buf, size_t bytes, int32_t nontemporal, int32_t pattern,
                               int32_t n_blocks, uint32_t *sink, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* RQ_PROBE_H_ */
