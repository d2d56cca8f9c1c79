/*
 * vdit_probe.h — a hardware rate probe shipped beside libvdit.so
 * (libvdit_probe.so, gfx950). It is no part of the attention path; the
 * benchmark uses it to state the matrix-core rate the part sustains, next to
 * the published peak, on the same device and in the same run.
 */
#ifndef VDIT_PROBE_H
#define VDIT_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Enqueue `nblocks` workgroups of 256 threads (4 wavefronts) on `stream` (a
 * hipStream_t; NULL means the default stream); returns without synchronising.
 * Every wavefront issues 8 * iters v_mfma_f32_32x32x16_bf16 (32,768 FLOP
 * each) from registers, with no memory traffic in the loop, so the launch
 * performs nblocks * 4 * 8 * iters * 32768 FLOP.
 *
 * random_operands: 0 fills the A and B operands with slowly varying,
 *   lane-invariant values (B); nonzero with independent hashed values in
 *   [-2, 2) carrying full bf16 mantissas. The instructions are the same.
 * ticks: device buffer of 2 * nblocks uint64 owned by the caller. Workgroup i
 *   writes ticks[2i] = its duration in shader clocks (s_memtime) and
 *   ticks[2i + 1] = its duration in 10 ns units (s_memrealtime, 100 MHz), so
 *   sum(ticks[2i]) / sum(ticks[2i+1]) * 100 is the mean shader clock in MHz.
 *
 * Returns 0 once enqueued; 1 if ticks is NULL; 2 if iters is outside
 * [1, 2^24] or nblocks outside [1, 65536]; 8 if the launch fails. Nothing
 * is enqueued unless it returns 0.
 */
int vdit_probe_mfma_bf16(int random_operands, int iters, int nblocks, uint64_t *ticks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VDIT_PROBE_H */
