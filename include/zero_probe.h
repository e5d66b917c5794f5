/*
 * zero_probe.h — memory-bandwidth probes that sit beside the shard pipeline (libzero_probe.so).
 *
 * Not part of the method: these kernels move bytes in the access patterns of the pipeline's
 * kernels with trivial arithmetic, so that a benchmark run can report, next to each kernel's
 * achieved bandwidth, what the same pattern reaches on the same device in the same process.
 * They are the "achievable" ceilings against which the pipeline kernels are read (the
 * denominator of every roofline fraction stays the HBM peak).
 *
 * Every probe launches a one-shot grid (one block of 256 threads per 4 KiB of the first
 * stream, one 16-byte chunk per thread per stream, like the pipeline kernels; every
 * wavefront instruction covering whole cache lines, all loads and stores nontemporal; the
 * write and the Adam-mix probes with their blocks per CU capped at four and two through an
 * LDS reservation: the fastest form of each pattern on MI355X) on `stream`,
 * never allocates and never synchronises.  Sizes are in bytes (multiples of 16) or elements
 * (multiples of 8).  Buffers are caller-owned device memory, 16-byte aligned, and must stay
 * allocated until the launched work has finished.  Every call returns ZERO_OK, ZERO_EINVAL
 * (bad size, NULL or misaligned pointer; nothing launched) or ZERO_EHIP (launch failure);
 * zero_last_error() is not used by these calls.
 */
#ifndef ZERO_PROBE_H
#define ZERO_PROBE_H

#include <stdint.h>

#include "zero_shard.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` from d_src (16-byte nontemporal loads).  d_sink (16 bytes) is written only if the XOR of
 * all loaded words equals a fixed improbable value, so the loads cannot be dropped. */
zero_status zero_probe_read(const void* d_src, int64_t bytes, void* d_sink, void* stream);

/* Write `bytes` of a fixed pattern to d_dst (16-byte nontemporal stores). */
zero_status zero_probe_write(void* d_dst, int64_t bytes, void* stream);

/* Copy `bytes` from d_src to d_dst (one 16-byte nontemporal load and store per thread); no
 * overlap. */
zero_status zero_probe_copy(const void* d_src, void* d_dst, int64_t bytes, void* stream);

/* The Adam step's streams over n fp32 columns with trivial arithmetic: reads g, p, m, v
 * (16 bytes per column), writes p = p + g, m = m + g, v = v + g and the top 16 bits of the
 * new p into d_lp (14 bytes per column): 30 bytes per column, one block per 2048 columns,
 * in the Adam kernel's lane-strided layout (two passes; in each, a thread takes 4 consecutive
 * columns: one 16-byte access per fp32 stream, 8 bytes of the 16-bit stream).  n a multiple
 * of 2048. */
zero_status zero_probe_adam_streams(const float* d_g, float* d_p, float* d_m, float* d_v, uint16_t* d_lp, int64_t n,
                                    void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ZERO_PROBE_H */
