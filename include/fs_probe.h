/* fs_probe.h -- throughput probes of the execution units the solver's
 * kernels are bound by, for reporting a kernel's speed against the peak that
 * this GPU reaches in the same run (next to the datasheet peak).
 *
 * The streaming log-sum-exp update is bound by the matrix cores when d is
 * large (one score contraction per pair) and by the transcendental unit when
 * d is small (one exponential per pair); see fs_sinkhorn.h.  Each probe runs a
 * kernel that does nothing but that unit's work -- independent chains of one
 * matrix instruction, or of v_exp_f32 -- on every compute unit, with no memory
 * traffic, and times it with HIP events on `stream`.
 *
 * Part of the same library as fs_sinkhorn.h, with the same status codes.
 * Allocates nothing: the caller passes `sink`, a device buffer of at least 4
 * bytes that the probe kernels may write (their results are stored there only
 * under a condition that does not hold, so that the compiler keeps the work).
 */
#ifndef FS_PROBE_H
#define FS_PROBE_H

#include <stdint.h>

#include "fs_sinkhorn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FS_PROBE_MFMA_BF16 = 1, /* v_mfma_f32_32x32x16_bf16: flop/s (2 per multiply-add) */
    FS_PROBE_MFMA_F16 = 2,  /* v_mfma_f32_32x32x16_f16: flop/s */
    FS_PROBE_MFMA_F32 = 3,  /* v_mfma_f32_32x32x2f32: flop/s */
    FS_PROBE_EXP = 4        /* v_exp_f32: exponentials per second */
} fs_probe_kind;

/* Runs the probe `kind` once untimed, then `reps` times (1..64), each launch
 * between its own pair of HIP events on `stream` (a hipStream_t; NULL: the
 * default stream), and writes the median rate over the timed launches to
 * *rate (host memory).  Each launch takes about a millisecond.  Synchronises
 * with the stream once, at the end.
 * Errors: FS_ERR_INVALID_ARG for a bad kind, reps out of range or a NULL
 * sink / rate (nothing is enqueued); FS_ERR_DEVICE for a HIP error. */
fs_status fs_probe_peak(fs_probe_kind kind, float* sink, int32_t reps, void* stream,
                        double* rate);

#ifdef __cplusplus
}
#endif

#endif /* FS_PROBE_H */
