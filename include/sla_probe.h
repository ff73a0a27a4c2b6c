/*
 * sla_probe.h -- bandwidth-ceiling kernels of the benchmark (libsla_probe.so).
 *
 * Not part of the solver's boundary: the benchmark measures the chip's own
 * streaming and LDS ceilings with these kernels and reports the solver
 * kernels against them next to the nominal 8 TB/s HBM peak.  All d_*
 * arguments are device pointers on the current device, `stream` a
 * hipStream_t; every call is asynchronous on it and returns 0, -1 for a bad
 * argument or -5 for a launch error.
 */
#ifndef SLA_PROBE_H
#define SLA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups of the streaming kernels (d_part of sla_probe_read and
 * sla_probe_lds holds at least this many doubles). */
int32_t sla_probe_blocks(void);

/* Reads the n doubles of d_a once (n even); one partial sum per workgroup
 * into d_part.  Moves n * 8 bytes. */
int32_t sla_probe_read(const void *d_a, int64_t n, void *d_part, void *stream);

/* d_b = d_a over n doubles (n even, no overlap).  Moves 2 * n * 8 bytes. */
int32_t sla_probe_copy(const void *d_a, void *d_b, int64_t n, void *stream);

/* d_b[0..n) = v (n even).  Moves n * 8 bytes. */
int32_t sla_probe_write(void *d_b, int64_t n, double v, void *stream);

/* In-cache copy ceiling: `passes` passes over d_a and d_b (n doubles each,
 * n even, no overlap; 64 MiB each stays in the 256 MB Infinity Cache), pass
 * p reading one and writing the other with plain loads and stores
 * (d_b = d_a + 1, d_a = d_b + 1, ...); one launch of 2048 workgroups.
 * Moves passes * 2 * n * 8 bytes. */
int32_t sla_probe_copy_passes(void *d_a, void *d_b, int64_t n, int32_t passes, void *stream);

/* Many streams in one launch: d_buf holds reads + writes arrays of n doubles
 * each (n even), consecutive; arrays reads .. reads + writes - 1 get, element
 * by element, the sum of arrays 0 .. reads - 1 (16-byte plain accesses, 768
 * workgroups).  (reads, writes) is one of (2, 2), (8, 4), (9, 5), (12, 4),
 * else -1.  Moves (reads + writes) * n * 8 bytes. */
int32_t sla_probe_streams(void *d_buf, int64_t n, int32_t reads, int32_t writes, void *stream);

/* 2048 workgroups (two resident per compute unit, 1024 threads each) read
 * 16 bytes per thread from their LDS 4 * reps times; returns the bytes read
 * from LDS over the launch (< 0 on error).  d_part holds at least 2048
 * doubles. */
int64_t sla_probe_lds(int64_t reps, void *d_part, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SLA_PROBE_H */
