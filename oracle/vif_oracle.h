/*
 * vif_oracle.h -- plain CPU oracle of the float VIF feature.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this code.  The GPU library
 * never includes, links or calls it, and it includes nothing of the GPU
 * library.
 *
 * It is the definition written out: scalar C99, single-threaded, every fp32
 * operation rounded on its own (built with -ffp-contract=off, SSE2 so no
 * excess precision), and the two one-plus-ratio expressions in fp64.  The
 * passages it follows are cited per function in vif_oracle.c; readings where
 * the pages are silent are marked "reading".
 *
 * Layouts: planes are row-major, pitch = width.  Samples are uint8_t for
 * bpc 8, else uint16_t.  Functions return 0 on success, -1 on bad arguments.
 */
#ifndef VIF_ORACLE_H
#define VIF_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VIFO_NSCALES 4
#define VIFO_MAX_TAPS 17

/* Gaussian taps of scale s (0..3): writes N_s floats, returns N_s (17, 9,
 * 5, 3) or -1. */
int vifo_taps(int scale, float *taps);

/* log2f_approx of one finite fp32 value x >= 1. */
float vifo_log2(float x);

/* vifo_log2 over n values (y[i] = vifo_log2(x[i])). */
void vifo_log2_array(const float *x, float *y, long n);

/* The two one-plus-ratio values, each evaluated in fp64 and rounded to
 * fp32 once: fl32(1 + a / (sv_sq + nsq)) and fl32(1 + sigma1_sq / nsq). */
float vifo_num_ratio(float num_arg, float sv_sq);
float vifo_den_ratio(float sigma1_sq);

/* The same with the noise variance nsq as an argument. */
float vifo_num_ratio_nsq(float num_arg, float sv_sq, double nsq);
float vifo_den_ratio_nsq(float sigma1_sq, double nsq);

/* vifo_num_ratio / vifo_den_ratio over arrays (den uses a only). */
void vifo_ratio_arrays(const float *a, const float *sv, float *num_out,
                       float *den_out, long n);
void vifo_ratio_arrays_nsq(const float *a, const float *sv, double nsq,
                           float *num_out, float *den_out, long n);

/* Per-pixel statistic: from the five filtered values to the two terms,
 * with nsq = 2 and the gain limit 100. */
void vifo_statistic(float mu1, float mu2, float xx, float yy, float xy,
                    float *num_t, float *den_t);

/* The same with the noise variance and the enhancement gain limit given. */
void vifo_statistic_ex(float mu1, float mu2, float xx, float yy, float xy,
                       double nsq, double gain_limit, float *num_t,
                       float *den_t);

/* vifo_statistic / vifo_statistic_ex over n pixels given as five arrays. */
void vifo_statistic_array(const float *mu1, const float *mu2, const float *xx,
                          const float *yy, const float *xy, float *num_t,
                          float *den_t, long n);
void vifo_statistic_array_ex(const float *mu1, const float *mu2,
                             const float *xx, const float *yy,
                             const float *xy, double nsq, double gain_limit,
                             float *num_t, float *den_t, long n);

/* Options of the feature (readings of the option names the pages give).
 *   sigma_nsq        noise variance, finite, >= 0 (default 2.0)
 *   enhn_gain_limit  upper bound of the gain g where it enters the
 *                    numerator, >= 0, may be +inf (default 100.0)
 *   kernelscale      filter scale; only 1.0 (widths 17/9/5/3) is defined
 *   scale_min_val    floors of the reported vif_scale1..3 (default 0.0)
 *   skip_scale0      1: scale 0 has no statistic, zero sums, score 0 */
typedef struct vifo_options {
    double sigma_nsq;
    double enhn_gain_limit;
    double kernelscale;
    double scale_min_val[3];
    int skip_scale0;
} vifo_options;

void vifo_default_options(vifo_options *o);

/* Sample normalisation of a w*h plane to fp32. */
int vifo_normalise(const void *src, int w, int h, int bpc, float *dst);

/* Separable filter with n taps and whole-sample mirrored borders; dst is
 * w*h.  Requires n odd, w and h >= (n+1)/2. */
int vifo_filter(const float *src, int w, int h, const float *taps, int n,
                float *dst);

/* Low-pass with n taps, then keep even rows and columns; dst is
 * (w/2)*(h/2). */
int vifo_decimate(const float *src, int w, int h, const float *taps, int n,
                  float *dst);

/* Ordered sums of one scale's w*h term planes (row-major): each row's terms
 * left to right into one fp32 accumulator from 0 (rowsums, optional: n_y,
 * d_y per row), then the row sums top to bottom into one fp32 accumulator
 * per plane (*n_out, *d_out).  Returns 0, or -1 for bad arguments. */
int vifo_ordered_sums(const float *num_t, const float *den_t, int w, int h,
                      float *rowsums, float *n_out, float *d_out);

/* Number of rows over all four scales for a w*h frame (h + h/2 + ...). */
int vifo_total_rows(int w, int h);

/* Whole feature for one frame pair.
 *   out[0..3] vif_scale0..3 = N_s / D_s (fp64)
 *   out[4]    num = ((N_0 + N_1) + N_2) + N_3 (fp64)
 *   out[5]    den, the same way
 *   out[6]    num / den
 *   out[7]    0.0 (reserved)
 *   sums      (optional) N_0, D_0, N_1, D_1, ..., N_3, D_3 as fp32
 *   rowsums   (optional) per scale, per row y: n_y, d_y (2 * total rows)
 * Requires w, h >= 16 and bpc in {8, 10, 12, 16}.  Default options. */
int vifo_score(const void *ref, const void *dist, int w, int h, int bpc,
               double out[8], float sums[8], float *rowsums);

/* vifo_score with options; returns -1 for options outside the ranges
 * above. */
int vifo_score_ex(const void *ref, const void *dist, int w, int h, int bpc,
                  const vifo_options *opt, double out[8], float sums[8],
                  float *rowsums);

#ifdef __cplusplus
}
#endif

#endif
