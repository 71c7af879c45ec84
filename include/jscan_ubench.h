/*
 * libjscan_ubench -- VALU throughput measurements on MI355X (gfx950).
 *
 * A measurement library, separate from libjscan: it launches synthetic
 * kernels and reports how fast the chip issues the instruction mixes of the
 * selective scan.  The scan's prefill at d_state 16 needs 16 decays
 * exp(delta * A) per channel and token (the recurrence of the "AI Engineering
 * from Scratch" Jamba lesson, section "一页讲完 SSM"); whether that work or the
 * HBM traffic bounds it depends on these rates.
 */
#ifndef JSCAN_UBENCH_H
#define JSCAN_UBENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Times one launch of a synthetic VALU kernel on device 0 (synchronous: it
 * allocates a small output buffer, launches once to warm up, times a second
 * launch between two events and frees the buffer).
 *
 *   kind   0: plain fp32 FMA chains (v_fma_f32)
 *          1: v_exp_f32 chains
 *          2: one v_exp_f32 and four independent v_fma_f32 per group
 *             (do the transcendental and the FMAs issue in parallel?)
 *          3: the scan's token step over 16 states: per state a multiply,
 *             an exp2, a multiply and two FMAs, B and C wave-uniform
 *   waves  wavefronts of 64 lanes to launch; a multiple of 4
 *   iters  loop trips per lane (the work grows linearly with it)
 *
 * Outputs (host pointers): seconds of the timed launch, VALU lane-
 * instructions it executed, how many of those were transcendental, the
 * shader clock in MHz (s_memtime ticks over s_memrealtime ticks times the
 * wall-clock rate, read by one wave during the launch) and the wall-clock
 * rate in MHz.  Returns 0 on success, 1 for invalid arguments, 2 when a HIP
 * call fails.
 */
int jscan_ubench_valu(int kind, int64_t waves, int iters, double* seconds, double* lane_instr,
                      double* trans_lane_instr, double* clock_mhz, double* wall_mhz);

#ifdef __cplusplus
}
#endif

#endif /* JSCAN_UBENCH_H */
