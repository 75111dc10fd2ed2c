/*
 * hpc_probe.h — measurement helpers shipped with the decode library.
 *
 * Not part of the decode step.  They give the two reference points a
 * bandwidth figure needs on MI355X: the practical HBM streaming-read ceiling
 * (a read-only kernel over a buffer of known size) and a plain copy of known
 * size whose hardware byte counters calibrate FETCH_SIZE / WRITE_SIZE.
 * Conventions as in hpc_decode.h: status codes, caller-owned device buffers,
 * `stream` is a hipStream_t passed as void*.
 */
#ifndef HPC_PROBE_H
#define HPC_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Stream-read `bytes` (a positive multiple of 16) from device `buf` with
 * `n_workgroups` workgroups of 256 threads; each workgroup folds what it read
 * into one float written to device `sink[workgroup]` (so the reads cannot be
 * elided).  HPC_ERR_NULL / HPC_ERR_INVALID on bad arguments. */
int hpc_probe_read(const void* buf, int64_t bytes, float* sink, int32_t n_workgroups, void* stream);

/* As hpc_probe_read, then waits for that launch to finish and stores in *ms
 * its duration in milliseconds, from the kernel's dispatch to its end (HIP
 * events stamped by the launch itself, so host launch overhead is excluded).
 * Synchronous: returns only after the kernel has finished.  HPC_ERR_NULL /
 * HPC_ERR_INVALID on bad arguments, HPC_ERR_HIP if the launch or an event
 * call fails. */
int hpc_probe_read_timed(const void* buf, int64_t bytes, float* sink, int32_t n_workgroups, void* stream,
                         float* ms);

/* Copy `bytes` (a positive multiple of 16) from device `src` to device `dst`
 * (non-overlapping) with 16-byte accesses.  HPC_ERR_NULL / HPC_ERR_INVALID on
 * bad arguments. */
int hpc_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HPC_PROBE_H */
