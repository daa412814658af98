/*
 * nvfp4_probe.h -- measurement aid, not part of the NVFP4 library.
 *
 * libnvfp4_probe.so holds one kernel that streams a device buffer from HBM
 * and does nothing else; the benchmark times it on the byte count of its
 * headline kernel to report that kernel's bandwidth against the read
 * ceiling of a single launch on the same GPU, in the same run.
 *
 * nvfp4probe_stream_read: reads `bytes` (a multiple of 16) from device
 * pointer `buf` with `workgroups` workgroups of 512 threads, `unroll`
 * (2, 4 or 8) 16-byte non-temporal loads in flight per thread, and writes
 * one word per workgroup to device `sink` [workgroups].  Enqueued on
 * `stream` (hipStream_t, NULL = null stream).  Returns 0, 1 for invalid
 * arguments, 6 if the launch failed.
 */
#ifndef NVFP4_PROBE_H
#define NVFP4_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int32_t nvfp4probe_stream_read(const void* buf, int64_t bytes, int32_t workgroups, int32_t unroll,
                               uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif
