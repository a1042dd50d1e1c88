/*
 * zero_probe.h -- achievable-bandwidth probes beside the shard step
 * (libzero_probe.so).
 *
 * A measurement aid, not part of the method.  The shard step of
 * zero_partition.h moves, per element of a rank's shard, the model states
 * that the model-states paragraph of the ZeRO explainer page ("ZeRO: Memory
 * Optimizations Toward Training Trillion Parameter Models", azimuth.plus)
 * lists: R fp16 gradient contributions read, the fp32 master, momentum and
 * variance read and written, and the fp16 parameter slot written.  These
 * probes move the same bytes with the step kernel's schedule and addressing
 * but none of its arithmetic, so their rate is what the machine gives that
 * stream mix; a plain copy is the two-stream reference.
 *
 * Conventions: plain C; every function returns 0 (ZERO_PROBE_OK) or a
 * negative status; nothing is allocated but one pair of HIP events per
 * calling thread and device; the caller owns every buffer; `stream` is a
 * hipStream_t (NULL = the null stream).  Each call launches `reps` kernels
 * back to back on `stream`, records a HIP event pair at each kernel's own
 * start and end, waits for each, and stores the mean kernel time in
 * milliseconds in *ms.  zero_probe_last_error() gives the calling thread's
 * last message.
 */
#ifndef ZERO_PROBE_H
#define ZERO_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum zero_probe_status {
    ZERO_PROBE_OK = 0,
    ZERO_PROBE_ERR_INVALID_ARG = -1,
    ZERO_PROBE_ERR_HIP = -6
};

/* The fused shard step's memory traffic over n elements, without its
 * arithmetic: reads grads[0..R-1] (fp16 bit patterns, 8-byte aligned) and
 * p, m, v (fp32, 16-byte aligned); writes p_out = p, m_out = m, v_out = v
 * (fp32, 16-byte aligned) and slot = grads[0] ^ ... ^ grads[R-1] bit by bit
 * (8-byte aligned).  26 + 2R bytes per element, one 1024-element tile per
 * wave as in the step kernel.  grads is a host array of R device pointers,
 * 1 <= R <= 16; n >= 1; reps >= 1.  Outputs must not overlap inputs.
 * Errors: INVALID_ARG (NULL, misaligned, out of range), HIP. */
int zero_probe_step_pattern(const uint16_t* const* grads, int32_t R, const float* p,
                            const float* m, const float* v, float* p_out, float* m_out,
                            float* v_out, uint16_t* slot, int64_t n, int32_t reps,
                            void* stream, float* ms);

/* dst = src over `bytes` bytes (a positive multiple of 16; both 16-byte
 * aligned, not overlapping): one read and one write stream, 4 KiB per wave.
 * Errors: INVALID_ARG, HIP. */
int zero_probe_copy(const void* src, void* dst, int64_t bytes, int32_t reps, void* stream,
                    float* ms);

/* The calling thread's last error message ("" after a successful call). */
const char* zero_probe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_PROBE_H */
