/*
 * fssim_oracle.h -- plain CPU oracle of the float SSIM feature with its
 * exact decimation.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this code.  The GPU library
 * never includes, links or calls it, and it includes nothing of the GPU
 * library.
 *
 * Scalar C99, single-threaded, every fp32 operation rounded on its own
 * (built with -ffp-contract=off, SSE2).  The decimation follows the page
 * "Research-2130: float_ssim decimation on the SYCL device", Question and
 * Sources; the SSIM stage, which the pages do not print, is the published
 * SSIM (Wang, Bovik, Sheikh and Simoncelli, 2004) in the readings stated in
 * fssim_oracle.c.
 *
 * Layouts: planes are row-major, pitch = width.  Samples are uint8_t for
 * bpc 8, else uint16_t.  Functions return 0 on success, -1 on bad
 * arguments.
 */
#ifndef FSSIM_ORACLE_H
#define FSSIM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FSSIMO_TAPS 11
#define FSSIMO_MAX_SCALE 128

/* Decimation factor of a w x h frame: max(1, round(min(w, h) / 256)). */
int fssimo_scale(int w, int h);

/* Size of a plane decimated by factor f: n / f + (n & 1) (per axis). */
int fssimo_decimated_size(int n, int f);

/* Index into [0, n) by the symmetric border of period 2n. */
int fssimo_symmetric(int i, int n);

/* Decimate one fp32 plane (w x h) by factor f into dst
 * (fssimo_decimated_size(w, f) x fssimo_decimated_size(h, f)): box window
 * of f x f taps fl32(1 / (f * f)), products in fp32, summed in fp64, one
 * rounding to fp32.  1 <= f <= FSSIMO_MAX_SCALE. */
int fssimo_decimate(const float *src, int w, int h, int f, float *dst);

/* The 11 fp32 Gaussian taps of the SSIM window (sigma 1.5). */
void fssimo_taps(float taps[FSSIMO_TAPS]);

/* Separable 11-tap Gaussian filter with the symmetric border: vertical
 * pass, then horizontal, taps in ascending order, each product and sum an
 * fp32 rounding.  dst is w x h. */
int fssimo_filter(const float *src, int w, int h, float *dst);

/* Per-pixel SSIM from the five filtered values. */
float fssimo_pixel(float mu1, float mu2, float xx, float yy, float xy);

/* Whole feature for one frame pair.
 *   out[0]  float_ssim: the frame mean, an fp32 value widened to double
 *   out[1]  the decimation factor used
 *   map     (optional) the w' x h' per-pixel SSIM values
 *   planes  (optional) the decimated ref then dist planes, 2 * w' * h'
 *   rows    (optional) the w'-long fp64 row sums, h' of them
 * w', h' are the decimated sizes (w, h when the factor is 1).  Requires
 * w, h >= 1, bpc in {8, 10, 12, 16} and a factor <= FSSIMO_MAX_SCALE. */
int fssimo_score(const void *ref, const void *dist, int w, int h, int bpc,
                 double out[2], float *map, float *planes, double *rows);

#ifdef __cplusplus
}
#endif

#endif
