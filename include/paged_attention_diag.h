/*
 * paged_attention_diag.h -- measurement helpers exported by libpagedattn.so. They are not part of the decode
 * path; they exist so that a benchmark can measure, on the same device and with the same 16-byte vector loads
 * the decode kernels use, the HBM read rate a plain streaming kernel reaches (the practical ceiling the
 * attention kernels are compared with), and so that hardware counters (bytes fetched from / written to HBM)
 * can be calibrated on kernels whose traffic is known exactly.
 *
 * Conventions as in pa.h: device pointers, 16-byte aligned, `stream` is a hipStream_t, work is
 * enqueued and the call returns without synchronising; negative PA_ERR_* status on invalid arguments.
 */
#ifndef PAGED_ATTENTION_DIAG_H
#define PAGED_ATTENTION_DIAG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of floats `sink` must hold for pa_stream_read. */
#define PA_STREAM_SINK_FLOATS 8192

/*
 * Read `bytes` (a positive multiple of 16) from `src` once, with each lane consuming the 16-byte words it
 * loads, and write one float per workgroup into `sink` (PA_STREAM_SINK_FLOATS floats; the values only keep
 * the loads live). HBM traffic: `bytes` read, at most PA_STREAM_SINK_FLOATS * 4 bytes written.
 */
int pa_stream_read(const void *src, size_t bytes, float *sink, void *stream);

/* Copy `bytes` (a positive multiple of 16) from `src` to a non-overlapping `dst`: `bytes` read, `bytes` written. */
int pa_stream_copy(void *dst, const void *src, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTENTION_DIAG_H */
