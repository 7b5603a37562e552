/*
 * moe_probe.h -- a measurement helper exported by libmoe.so: the HBM read
 * rate that a plain streaming kernel reaches on this GPU, to report beside
 * the published peak.  The cold scan of a buffer larger than every cache is
 * the method of "Cache-Residency Probe Results" (cism): a cold read rate is
 * measured, not taken from the vendor's figure.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` bytes at `src` once (16 bytes per lane and load, four loads
 * in flight per lane, a grid of 8 workgroups of 256 threads per compute
 * unit) and folds them with XOR; the fold is stored to *sink only when it
 * equals one particular 32-bit value, so the loads cannot be dropped and
 * almost nothing is written.
 *   src    device memory, 16-byte aligned; bytes a multiple of 16.
 *   sink   device uint32, written at most once per lane (its value is
 *          meaningless).
 * Returns MOE_ERR_INVALID for a null or misaligned pointer or a byte count
 * that is not a multiple of 16, MOE_ERR_DEVICE if the launch fails.
 * Enqueued on `stream`; time it with events around the call.
 */
moe_status moe_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
