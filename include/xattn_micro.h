/*
 * xattn micro-benchmarks: achievable rates of the MI355X units that bound the
 * fused cross-attention kernel (matrix cores, v_exp_f32, fp32 VALU, LDS reads,
 * HBM copy).  Measurement helpers only; not part of the computation.
 */
#ifndef XATTN_MICRO_H
#define XATTN_MICRO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Run one micro kernel `reps` times on `stream` (a hipStream_t) and return the
 * average milliseconds per launch, or a negative value on a HIP error.
 * kind: 0 = 32x32x16 bf16 MFMA (8 independent chains per wave),
 *       1 = v_exp_f32 (16 chains per lane), 2 = fp32 FMA (16 chains per lane),
 *       3 = LDS 8-byte reads, 4 = LDS 16-byte reads, 5 = LDS transposed 8-byte
 *       reads.  Each launch has `blocks` work-groups of 256 threads and loops
 *       `iters` times; `out` is device memory of blocks*256 floats (written). */
float xattn_micro_run(int kind, int blocks, int iters, int reps, float* out, void* stream);

/* Device-to-device copy of `bytes` (a multiple of 16) from a to b, timed over
 * `reps` launches; returns average milliseconds per launch.  256 work-groups,
 * each lane keeping four 16-byte nontemporal loads in flight before storing
 * them (kernel copy_kernel). */
float xattn_micro_copy(const void* a, void* b, int64_t bytes, int reps, void* stream);

/* Reads the first 64 bytes of every 128-byte line of the `bytes` (a multiple
 * of 128, else -1) at device address a, timed over `reps` launches; `out` is
 * device memory of 524288 floats (written).  The known-size reference of the
 * read counters for 64-byte slices of 128-byte rows (kernel
 * half_line_read_kernel): bytes / 2 useful bytes per launch. */
float xattn_micro_half_line_read(const void* a, int64_t bytes, int reps, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* XATTN_MICRO_H */
