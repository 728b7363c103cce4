/*
 * sinkhorn_probe.h -- instruction-rate probe of the MI355X (gfx950) streaming
 * Sinkhorn library, for the roofline figures of its measurement harness.
 *
 * The streaming update spends one exponential, one accumulation and a share of
 * a score contraction per entry; once the n x m matrix never reaches HBM, the
 * rate at which the compute units issue those instructions is the bound
 * [FS "FlashSinkhorn: IO-bewuste Entropische Optimale Transport op GPU",
 * Probleemstelling: existing solvers are bound by HBM traffic or by poor
 * instruction efficiency].  The roofline constants (exponentials, FMAs and
 * matrix-core operations per compute unit per clock, and the clock under
 * load) are measured with this probe rather than assumed.
 */
#ifndef SINKHORN_PROBE_H
#define SINKHORN_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Launches `blocks` work-groups of 256 threads (4 waves) that each run `iters`
 * iterations of one instruction mix on independent register chains:
 *   kind 0: 16 v_exp_f32 per lane            kind 3: 4 v_mfma_f32_16x16x32_bf16 per wave
 *   kind 1: 16 v_fma_f32 per lane            kind 4: one d = 3 score tile: 4 MFMA, then
 *   kind 2: 16 v_exp_f32 + 16 v_add_f32              16 exp + 16 add on their outputs
 *   kind 5: 16 v_fma_f64 per lane            kind 6: one d = 64 bf16 feature tile: 8 MFMA
 *                                                    (chained pairs), 16 fma + exp + add
 *   kind 7: 2 v_mfma_f32_32x32x16_bf16       kind 8: the feature tile with 4 chained
 *                                                    32x32x16 MFMAs, 16 fma + exp + add
 * sink [blocks * 256] (device, fp32) receives one value per thread (it keeps
 * the chains live; its contents mean nothing).  clocks [blocks][4] (device,
 * uint64) receives, per work-group, the shader-clock counter at start and end
 * and the constant-rate wall-clock counter at start and end; *wall_clock_hz
 * (host) receives that counter's frequency.  Only enqueues on `stream`.
 * Returns 0, or 1 for arguments out of range (0 <= kind <= 8,
 * 1 <= blocks <= 2^20, iters >= 1, non-NULL pointers), 5 on a HIP error.
 */
int sinkhorn_probe_rates(int kind, int blocks, int iters, float *sink,
                         unsigned long long *clocks, double *wall_clock_hz,
                         void *stream);

/*
 * Wait limit of the split stage launch, a test hook for its failure path.
 * For a small batch of pairs of at most 1024 points, sinkhorn_potentials (d = 3)
 * runs each stage of iterations in one launch whose work-groups each own a
 * slice of a pair's rows and hand their new potentials to one another between
 * half-iterations [FS Methodologie 2: fusing the update into as few launches
 * as possible].  Each hand-over is a bounded wait: when it runs out (the
 * work-groups were not all resident at once, e.g. another process held the
 * compute units), the pair's potentials come back NaN instead of the launch
 * hanging.  This sets that bound, in microseconds of wall clock, for every
 * launch enqueued after the call, process-wide (default 1000000, one second);
 * microseconds < 0 makes every wait fail at once, so that a test can see the
 * NaN results.  Returns the previous value.
 */
long long sinkhorn_probe_wait_limit(long long microseconds);

/*
 * How sinkhorn_potentials runs its iterations for these sizes on the current
 * device, so that a measurement names the kernel it times [FS Methodologie 2:
 * one fused pass per update]:
 *   0  d = 3, one launch per half-iteration, scores on the matrix cores
 *   1  d = 3, one launch per eps stage, one work-group per pair (batches of at
 *      least one pair per compute unit, clouds of at most 8192 points)
 *   2  d = 3, one launch per eps stage, each pair over 16-row work-groups that
 *      hand over their biases (clouds of at most 1024 points, the work-groups
 *      on at most half of the compute units)
 *   3  d = 3 with SK_VALU_SCORES: one launch per half-iteration, vector scores
 *   4  the feature path (d != 3)
 * Returns -1 for sizes, dtype or d that sinkhorn_potentials refuses, -2 when
 * no HIP device is current.  B, n, m, d, dtype and flags mean what they mean
 * for sinkhorn_potentials; nothing is launched.
 */
int sinkhorn_probe_potentials_path(int B, int n, int m, int d, int dtype, unsigned flags);

#ifdef __cplusplus
}
#endif

#endif /* SINKHORN_PROBE_H */
