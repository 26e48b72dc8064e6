/*
 * rbq_probe.h - measurement helper beside librbq (librbq_probe.so), not part
 * of the method: a plain streaming read of device memory, the practical HBM
 * read ceiling the attention kernels are compared with.
 */
#ifndef RBQ_PROBE_H
#define RBQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * rbq_probe_stream_read - read `bytes` of device memory at `src` once with
 * 16-byte loads: `blocks` workgroups of 256 threads, each thread `unroll`
 * (1, 2, 4, 8 or 16) loads in flight per round at a grid-wide stride, with
 * the non-temporal hint when `nontemporal` is nonzero; each thread writes one
 * word of its xor-reduction to sink[blocks * 256] (device).  Enqueued on
 * `stream` (hipStream_t as void*).  Returns 0, -1 for bad arguments (null
 * pointers, bytes or src not multiples of 16, blocks <= 0, another unroll),
 * -6 for a launch failure.
 */
int rbq_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                          int32_t unroll, int32_t nontemporal, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RBQ_PROBE_H */
