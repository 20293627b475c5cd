/*
 * vif_selftest.h -- device-math gates of the float VIF library.
 *
 * These entry points run the device functions of the scoring kernels (the
 * same inline code, not copies) over caller-provided arrays, so a test can
 * compare the device's arithmetic with the host's bit for bit before
 * trusting the pipeline.  The pattern follows ADR-1444 "float_vif_hip runs
 * the arithmetic of the CUDA twin ...", Decision (a host comparison of the
 * device's fp64 add and divide over tens of millions of operand pairs and
 * several noise variances, on the sum, the quotient and both fp32 roundings
 * of one plus the quotient) and Consequences (a device-math test of the
 * shared arithmetic against the CPU's).
 *
 * Every pointer is a DEVICE pointer owned by the caller; n >= 0 elements;
 * stream is a hipStream_t as void* (NULL = default stream).  Each call is
 * synchronous (it waits for its kernel).  Returns VIF_OK or VIF_EINVAL (NULL
 * pointer, n < 0, an option out of range) or VIF_EHIP.
 */
#ifndef VIF_SELFTEST_H
#define VIF_SELFTEST_H

#include "vif.h"

#ifdef __cplusplus
extern "C" {
#endif

/* For each i, with a, b fp32 and nsq fp64:
 *   sum[i]   = (double)b[i] + nsq                       (fp64 add)
 *   quot[i]  = (double)a[i] / sum[i]                    (fp64 divide)
 *   rnum[i]  = (float)(1.0 + quot[i])                   (fp64 add, cvt)
 *   rden[i]  = (float)(1.0 + (double)a[i] / nsq)        (fp64 div, add, cvt)
 */
int vif_selftest_fp64(const float *a, const float *b, double nsq, long n,
                      double *sum, double *quot, float *rnum, float *rden,
                      void *stream);

/* q[i] = a[i] / b[i] in fp32 with the kernels' (correctly rounded)
 * division. */
int vif_selftest_div32(const float *a, const float *b, long n, float *q,
                       void *stream);

/* q[i] = a[i] / b[i] in fp32 with the statistic's written-out division for
 * a power-of-two noise variance, which equals the correctly rounded
 * division for a[i] == +0 or 2^-100 <= |a[i]| <= 2^17 and
 * 2^-20 <= b[i] <= 2^17 (its domain; elsewhere the result is unspecified).
 * Device arrays of n floats; VIF_EINVAL for n < 0 or a NULL array. */
int vif_selftest_div32_in_range(const float *a, const float *b, long n,
                                float *q, void *stream);

/* y[i] = the kernels' log2 polynomial of x[i] (x[i] finite, >= 1). */
int vif_selftest_log2(const float *x, long n, float *y, void *stream);

/* The kernels' one-plus-ratio values for the noise variance nsq (finite,
 * >= 0, as vif_options.sigma_nsq; else VIF_EINVAL), each through fp64 and
 * one rounding to fp32:
 *   num[i] = fl32(1 + a[i] / (sv[i] + nsq)),  den[i] = fl32(1 + a[i] / nsq).
 * A power-of-two nsq in [2^-20, 2^20] takes the kernels' power-of-two form:
 * the exact reciprocal for den, and for num the fp64 division without its
 * scaling steps, whose domain needs finite a[i] and sv[i] >= 0 (the
 * kernels' values always are); an infinite or NaN a[i] or sv[i] may then
 * give a different NaN or infinity than the general form. */
int vif_selftest_ratios(const float *a, const float *sv, double nsq, long n,
                        float *num, float *den, void *stream);

/* The kernels' per-pixel statistic: from the five filtered values
 * (mu1, mu2, xx, yy, xy, each an array of n floats) to the two terms, with
 * the noise variance nsq and the enhancement gain limit gain_limit in the
 * ranges of vif_options (else VIF_EINVAL). */
int vif_selftest_statistic(const float *mu1, const float *mu2,
                           const float *xx, const float *yy, const float *xy,
                           long n, double nsq, double gain_limit, float *num,
                           float *den, void *stream);

/* The bounded wait of scale 0's row-sum hand-over, forced from the host:
 * runs only the second tile column of a 224x16 frame of zeros, whose left
 * neighbour never hands its words over, so every waiting lane must give up
 * after its bounded number of reads (about a tenth of a second), raise the
 * error word and store NaN; the kernel still ends.  Writes *raised = the
 * error word (1 expected) and *row = the first row's numerator sum (NaN
 * expected).  Host pointers; allocates its own small device buffers. */
int vif_selftest_carry_wait(int *raised, float *row, void *stream);

/* The VALU issue rate of the scale kernels' filter step at a set occupancy,
 * the practical ceiling against which their issue rate is read: `blocks`
 * blocks of 256 threads, each thread running `iters` rounds of 32 VALU
 * instructions (16 multiplies by a uniform factor, 16 adds, in 8 independent
 * chains, as the filter's tap multiply and accumulate), with each block
 * reserving the LDS that lets waves_per_simd (3..8) blocks share a CU, one
 * wave per SIMD each.  out: DEVICE array of blocks * 256 floats (the
 * results, kept live).  *ms (HOST) = the kernel's duration from HIP events.
 * The rate follows as blocks * 4 * iters * 32 wave instructions over the
 * 1024 SIMDs and the duration (or from the VALU and cycle counters).
 * VIF_EINVAL for arguments outside those ranges (1 <= iters <= 2^24,
 * 1 <= blocks <= 2^24). */
int vif_selftest_valu_rate(int waves_per_simd, int iters, long blocks,
                           float *out, double *ms, void *stream);

/* The scale-0 kernel's input staging alone, for calibrating HBM traffic
 * counters against that kernel's own access shape: a launch with the
 * scale-0 kernel's grid, block order and staging code over the n frame
 * pairs ref[z], dist[z] (z < n; DEVICE pointers to w x h planes of bpc-bit
 * samples, row-major, one byte per sample at 8 bits, two otherwise; host
 * arrays of n pointers), whose blocks each load their tile of 32 rows x 128
 * columns of both planes (the 16 x 112 output pixels plus the radius-8 halo,
 * mirrored at the plane's edges, 8 samples per load for tiles inside a plane
 * whose width is a multiple of 8 and whose planes are aligned to 8 samples)
 * into LDS and do nothing else.  Block (frame z, strip r, tile column c)
 * then stores the sum of its tile's raw samples, both planes, at
 * out[(c * n + z) * ceil(h / 16) + r]: out is a DEVICE array of
 * n * ceil(h / 16) * ceil(w / 112) unsigned values.  Synchronous.
 * VIF_EINVAL for n outside 1..VIF_MAX_BATCH, a geometry vif_create refuses,
 * bpc not 8/10/12/16 or a NULL pointer. */
int vif_selftest_stage_loads(const void *const *ref, const void *const *dist,
                             int n, int w, int h, int bpc, unsigned *out,
                             void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VIF_SELFTEST_H */
