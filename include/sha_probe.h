/*
 * sha_probe.h - device read-bandwidth probe used by the benchmark as a
 * secondary ceiling for the decode kernels (libsha_probe.so, separate from
 * the SHA library: it is a measurement tool, not part of the method).
 *
 * sha_probe_read streams `bytes` of device memory once: `blocks` workgroups
 * of 256 threads each read one contiguous chunk of bytes / blocks with
 * 128-bit non-temporal loads, 1 KiB per wave load and 8 loads in flight per
 * wave (the access pattern of the head-indexed decode kernel), and fold the
 * data into one word so that nothing is optimised away.
 *   buf   : device buffer of at least `bytes` bytes, 16-byte aligned.
 *   bytes : a multiple of blocks * 32 KiB (else SHA_PROBE_EINVAL).
 *   sink  : device uint32, written only if the fold hits a magic value.
 * Returns 0 on success, SHA_PROBE_EINVAL for bad arguments, or the
 * hipError_t of a failing launch.  Asynchronous on `stream`.
 */
#ifndef SHA_PROBE_H_
#define SHA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SHA_PROBE_EINVAL (-1)

int sha_probe_read(const void* buf, size_t bytes, int blocks, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SHA_PROBE_H_ */
