/*
 * moe_probe.h -- measurement helpers exported by libmoe.so: the HBM read
 * rate that a plain streaming kernel reaches on this GPU, and the issue rate
 * of the scaled matrix instruction, to report beside the published peaks.
 * The cold scan of a buffer larger than every cache is the method of
 * "Cache-Residency Probe Results" (cism): a cold read rate is measured, not
 * taken from the vendor's figure.
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

/*
 * The issue rate of the scaled block-format matrix instruction: every
 * wavefront of a grid of 8 workgroups of 256 threads per compute unit runs
 * `iters` rounds of independent instructions (eight 16x16x128 or four
 * 32x32x64 accumulators, no memory traffic) on operands in registers, then
 * folds its accumulators into out.  Flops per launch: grid wavefronts x
 * iters x 8 x 2*16*16*128 (shape 16) or x 4 x 2*32*32*64 (shape 32); time
 * it with events around the call.  The ceiling of what a kernel built on
 * that instruction can issue, beside the published peak.
 *   shape   16 (v_mfma_scale_f32_16x16x128_f8f6f4) or 32 (..._32x32x64_...)
 *   fmt_a, fmt_b  operand formats: 0 E4M3, 2 E2M3 (fp6), 4 E2M1 (fp4)
 *   iters   >= 1
 *   out     device floats, at least moe_mfma_rate_out_floats() of them
 * Returns MOE_ERR_INVALID for another shape or format, iters < 1 or a null
 * out, MOE_ERR_DEVICE if the launch fails.  Enqueued on `stream`.
 */
moe_status moe_mfma_rate(int shape, int fmt_a, int fmt_b, int iters, float* out,
                         hipStream_t stream);
/* The floats moe_mfma_rate writes (one per thread of its grid); 0 when the
 * device cannot be queried. */
size_t moe_mfma_rate_out_floats(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
