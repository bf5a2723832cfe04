/*
 * Measurement probes beside the MLA library (libmla_probe.so, built from
 * probe_csrc/): not on the MLA path.  They measure the achievable rates of
 * the two roofline bounds on the device in use, so that benchmarks can report
 * fractions of what the chip sustains beside the datasheet peaks.  Status
 * codes are those of mla.h.
 */
#ifndef MLA_PROBE_H
#define MLA_PROBE_H

#include <stdint.h>

#include "mla.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * mla_probe_mfma: n_workgroups work-groups of 256 threads; every wave issues
 *   iters * 16 independent 32x32x16 bf16 MFMAs (four accumulator chains).
 *   toggle = 0 uses one fixed operand pair; toggle = 1 alternates two pairs
 *   of pseudo-random bf16 operands, so the inputs change on every
 *   instruction as with real data (the clock then settles where the power
 *   limit holds it).
 *   out [n_workgroups * 256] float (device, caller-owned) receives one value
 *   per thread (kept so the work is not removed); *flops (host, optional)
 *   receives the floating-point operations of the launch.
 * mla_probe_hbm_read: reads n_bytes (a positive multiple of 16) at src
 *   (device, 16-byte aligned) once, grid-stride with 16-byte loads over
 *   n_workgroups work-groups of 256 threads; out [n_workgroups * 256] uint32
 *   (device) receives one word per thread.
 * Errors: sizes out of range or NULL / misaligned pointers give
 * MLA_ERR_INVALID_ARG; launch failures MLA_ERR_HIP.  Both are asynchronous on
 * `stream`; time them with events on that stream.
 */
mla_status mla_probe_mfma(void* stream, int32_t n_workgroups, int32_t iters, int32_t toggle, float* out,
                          double* flops);
mla_status mla_probe_hbm_read(void* stream, const void* src, int64_t n_bytes, int32_t n_workgroups,
                              uint32_t* out);

/* Message of the last failed probe call of this thread (empty if none). */
const char* mla_probe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PROBE_H */
