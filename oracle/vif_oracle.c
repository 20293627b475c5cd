/*
 * vif_oracle.c -- plain CPU oracle of the float VIF feature.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library.
 *
 * Build: gcc -std=c99 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (x86-64, SSE2: FLT_EVAL_METHOD 0, so every float expression below rounds
 * to binary32 at each operation, in the order written).
 *
 * Sources, cited by page title and section:
 *   [ADR-1422 Context]  "ADR-1422: float_vif_sycl computes the CPU's
 *       arithmetic without an fp64 type ...", section Context: the four
 *       CPU properties (taps from vif_get_filter, the log2f_approx
 *       polynomial, vif_sigma_nsq kept in fp64, one fp32 sum per row and
 *       then over the rows) and the two fp64 one-plus-ratio expressions,
 *       each rounded to fp32 once.
 *   [ADR-1422 Decision] same page, section Decision: taps generated at run
 *       time per scale; the fp64 comparison sigma1_sq < vif_sigma_nsq; rows
 *       summed left to right into one fp32 accumulator, rows added top to
 *       bottom in fp32.
 *   [ADR-1444 Context/Decision] "ADR-1444: float_vif_hip runs the arithmetic
 *       of the CUDA twin ...": reflected tile indices, frames under 72 px,
 *       plain operators with -ffp-contract=off, correctly rounded division,
 *       the fp64 sum, quotient and conversion.
 *   [Research-2130 Sources] "Research-2130: float_ssim decimation on the
 *       SYCL device", section Sources: picture_copy normalisation (8-bit as
 *       is; 10/12/16-bit divided by 4/16/256).
 * Readings where the pages are silent (sigma of the Gaussian, decimation
 * phase, mirror convention, content of the low-variance branch, ...) are
 * marked "reading" below.
 */
#include "vif_oracle.h"

#include <assert.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

static const int kWidths[VIFO_NSCALES] = {17, 9, 5, 3};

/* Noise variance vif_sigma_nsq, kept in binary64 [ADR-1422 Context]. */
static const double kNsq = 2.0;

/* Default enhancement gain limit.  Reading: the pages print no default for
 * vif_enhn_gain_limit; the sibling ADM option's default is 100
 * [Research-1434 Findings 1], and VIF takes the same. */
static const double kGainLimit = 100.0;

/* ---------------------------------------------------------------------- */
/* O3  Gaussian taps [ADR-1422 Decision: taps computed at run time per
 * scale].  Reading: width N_s = 17/9/5/3, sigma_s = N_s / 5 (the published
 * pixel-domain VIF window), evaluated and normalised in fp64, each tap
 * rounded to fp32 once:
 *   sigma = N / 5.0;  denom = (2.0 * sigma) * sigma;
 *   g_k = exp(-(d * d) / denom), d = k - r;   S = sum_k g_k (k ascending);
 *   t_k = (float)(g_k / S).                                               */
int vifo_taps(int scale, float *taps)
{
    if (scale < 0 || scale >= VIFO_NSCALES || taps == NULL)
        return -1;
    const int n = kWidths[scale];
    const int r = (n - 1) / 2;
    const double sigma = (double)n / 5.0;
    const double denom = 2.0 * sigma * sigma;
    double g[VIFO_MAX_TAPS];
    double sum = 0.0;
    for (int k = 0; k < n; k++) {
        const double d = (double)(k - r);
        g[k] = exp(-(d * d) / denom);
    }
    for (int k = 0; k < n; k++)
        sum = sum + g[k];
    for (int k = 0; k < n; k++)
        taps[k] = (float)(g[k] / sum);
    return n;
}

/* ---------------------------------------------------------------------- */
/* O10  log2f_approx [ADR-1422 Context: the CPU's log2 is a polynomial
 * evaluated in fp32].  Reading: the coefficients are this method's own
 * (Chebyshev interpolation of log2(1+t)/t on [0,1], degree 9, see
 * fit_log2.py); x = 2^e * m, m in [1,2), t = m - 1 (exact);
 * q = t * P(t) by Horner in fp32; result = (float)e + q.                 */
#define VIFO_LOG2_K 10
static const uint32_t kLog2Coef[VIFO_LOG2_K] = {
    0x3fb8aa3bu, 0xbf38aa21u, 0x3ef63175u, 0xbeb84ebdu, 0x3e913ea6u,
    0xbe6194f1u, 0x3e1bc356u, 0xbda6904fu, 0x3ce6f6e9u, 0xbb96254au,
};

static float bits_to_float(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

float vifo_log2(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    const int e = (int)((u >> 23) & 0xffu) - 127;
    const float m = bits_to_float((u & 0x007fffffu) | 0x3f800000u);
    const float t = m - 1.0f;
    float p = bits_to_float(kLog2Coef[VIFO_LOG2_K - 1]);
    for (int k = VIFO_LOG2_K - 2; k >= 0; k--) {
        const float pt = p * t;
        p = pt + bits_to_float(kLog2Coef[k]);
    }
    const float q = p * t;
    return (float)e + q;
}

void vifo_log2_array(const float *x, float *y, long n)
{
    for (long i = 0; i < n; i++)
        y[i] = vifo_log2(x[i]);
}

/* ---------------------------------------------------------------------- */
/* The two one-plus-ratio values [ADR-1422 Context: 1 + g*g*sigma1_sq /
 * (sv_sq + vif_sigma_nsq) and 1 + sigma1_sq / vif_sigma_nsq are evaluated
 * in fp64 and each rounded to fp32 once; ADR-1422 Decision lists the fp64
 * steps: the sum sv_sq + nsq, the quotient, the sum with one, the
 * conversion].  num_arg is the fp32 product (g*g)*sigma1_sq.              */
float vifo_num_ratio_nsq(float num_arg, float sv_sq, double nsq)
{
    const double num_den = (double)sv_sq + nsq;
    const double num_q = (double)num_arg / num_den;
    return (float)(1.0 + num_q);
}

float vifo_den_ratio_nsq(float sigma1_sq, double nsq)
{
    const double den_q = (double)sigma1_sq / nsq;
    return (float)(1.0 + den_q);
}

float vifo_num_ratio(float num_arg, float sv_sq)
{
    return vifo_num_ratio_nsq(num_arg, sv_sq, kNsq);
}

float vifo_den_ratio(float sigma1_sq)
{
    return vifo_den_ratio_nsq(sigma1_sq, kNsq);
}

void vifo_ratio_arrays_nsq(const float *a, const float *sv, double nsq,
                           float *num_out, float *den_out, long n)
{
    for (long i = 0; i < n; i++) {
        num_out[i] = vifo_num_ratio_nsq(a[i], sv[i], nsq);
        den_out[i] = vifo_den_ratio_nsq(a[i], nsq);
    }
}

void vifo_ratio_arrays(const float *a, const float *sv, float *num_out,
                       float *den_out, long n)
{
    vifo_ratio_arrays_nsq(a, sv, kNsq, num_out, den_out, n);
}

/* ---------------------------------------------------------------------- */
/* O7 (second half) and O8  per-pixel statistic.
 * sigma1_sq = xx - mu1*mu1 etc. in fp32, clamped at 0 (sigma12 is not).
 * The branch compares sigma1_sq with vif_sigma_nsq in fp64 [ADR-1422
 * Decision].  Reading: below it both terms are 1.0f.  Above it, the
 * published pixel-domain VIF rules in order: g = sigma12 / sigma1_sq,
 * sv_sq = sigma2_sq - g*sigma12; sigma2_sq < eps -> g = sv_sq = 0; g < 0 ->
 * sv_sq = sigma2_sq, g = 0; sv_sq >= eps.  Reading for the option
 * vif_enhn_gain_limit [ADR-1422 Consequences; ADR-1444 Consequences name
 * it]: it bounds the gain where the gain enters the numerator, once sv_sq
 * is settled, as C's MIN(g, limit) does with a double limit: the
 * comparison in fp64, the limit rounded to fp32 when it is taken (so a NaN
 * gain becomes the limit).  Then the two one-plus-ratio expressions in
 * fp64, each rounded to fp32 once [ADR-1422 Context; ADR-1422 Decision
 * lists the sequence fl64(sv_sq + nsq), fp64 quotient, fp64 sum,
 * conversion to fp32], and log2f_approx of each.  Reading for nsq = 0: no
 * special rule; IEEE 754 arithmetic throughout (a zero sigma1_sq then
 * divides by zero), and log2f_approx reads whatever bits arrive.         */
void vifo_statistic_ex(float mu1, float mu2, float xx, float yy, float xy,
                       double nsq, double gain_limit, float *num_t,
                       float *den_t)
{
    const float eps = 1e-10f;
    const float mu1_sq = mu1 * mu1;
    const float mu2_sq = mu2 * mu2;
    const float mu1_mu2 = mu1 * mu2;
    float sigma1_sq = xx - mu1_sq;
    float sigma2_sq = yy - mu2_sq;
    const float sigma12 = xy - mu1_mu2;
    if (sigma1_sq < 0.0f)
        sigma1_sq = 0.0f;
    if (sigma2_sq < 0.0f)
        sigma2_sq = 0.0f;

    if ((double)sigma1_sq < nsq) {
        *num_t = 1.0f;
        *den_t = 1.0f;
        return;
    }

    float g = sigma12 / sigma1_sq;
    const float g_sigma12 = g * sigma12;
    float sv_sq = sigma2_sq - g_sigma12;
    if (sigma2_sq < eps) {
        g = 0.0f;
        sv_sq = 0.0f;
    }
    if (g < 0.0f) {
        sv_sq = sigma2_sq;
        g = 0.0f;
    }
    if (sv_sq < eps)
        sv_sq = eps;
    if (!((double)g < gain_limit))
        g = (float)gain_limit;

    const float g_sq = g * g;
    const float num_arg = g_sq * sigma1_sq;
    *num_t = vifo_log2(vifo_num_ratio_nsq(num_arg, sv_sq, nsq));
    *den_t = vifo_log2(vifo_den_ratio_nsq(sigma1_sq, nsq));
}

void vifo_statistic(float mu1, float mu2, float xx, float yy, float xy,
                    float *num_t, float *den_t)
{
    vifo_statistic_ex(mu1, mu2, xx, yy, xy, kNsq, kGainLimit, num_t, den_t);
}

void vifo_statistic_array_ex(const float *mu1, const float *mu2,
                             const float *xx, const float *yy,
                             const float *xy, double nsq, double gain_limit,
                             float *num_t, float *den_t, long n)
{
    for (long i = 0; i < n; i++)
        vifo_statistic_ex(mu1[i], mu2[i], xx[i], yy[i], xy[i], nsq,
                          gain_limit, &num_t[i], &den_t[i]);
}

void vifo_statistic_array(const float *mu1, const float *mu2, const float *xx,
                          const float *yy, const float *xy, float *num_t,
                          float *den_t, long n)
{
    vifo_statistic_array_ex(mu1, mu2, xx, yy, xy, kNsq, kGainLimit, num_t,
                            den_t, n);
}

/* ---------------------------------------------------------------------- */
/* O2  normalisation [Research-2130 Sources, picture_copy]: 8-bit samples
 * as they are, 10/12/16-bit samples divided by 4/16/256.  Reading: no
 * offset.  The product with an exact power of two is exact.              */
int vifo_normalise(const void *src, int w, int h, int bpc, float *dst)
{
    if (src == NULL || dst == NULL || w <= 0 || h <= 0)
        return -1;
    const size_t n = (size_t)w * (size_t)h;
    if (bpc == 8) {
        const uint8_t *s = (const uint8_t *)src;
        for (size_t i = 0; i < n; i++)
            dst[i] = (float)s[i];
        return 0;
    }
    float scale;
    if (bpc == 10)
        scale = 0.25f;
    else if (bpc == 12)
        scale = 0.0625f;
    else if (bpc == 16)
        scale = 0.00390625f;
    else
        return -1;
    const uint16_t *s = (const uint16_t *)src;
    for (size_t i = 0; i < n; i++)
        dst[i] = (float)s[i] * scale;
    return 0;
}

/* ---------------------------------------------------------------------- */
/* O4  mirror.  Reading: whole-sample reflection about the edge sample
 * (-i -> i, n-1+i -> n-1-i), applied once.  ADR-1444 Decision adds a clamp
 * on the GPU for loads no output consumes; every index the oracle uses is
 * consumed, so one reflection must land inside the plane.                */
static int mirror(int i, int n)
{
    int m = i;
    if (m < 0)
        m = -m;
    else if (m > n - 1)
        m = 2 * (n - 1) - m;
    assert(m >= 0 && m <= n - 1);
    return m;
}

/* O5  separable filter.  Reading: vertical pass, then horizontal pass;
 * fp32 accumulator from 0.0f; taps in ascending k; each product rounded,
 * then each sum rounded (plain operators, -ffp-contract=off
 * [ADR-1444 Context]).                                                   */
int vifo_filter(const float *src, int w, int h, const float *taps, int n,
                float *dst)
{
    if (src == NULL || dst == NULL || taps == NULL || n < 1 || (n & 1) == 0)
        return -1;
    const int r = (n - 1) / 2;
    if (w < r + 1 || h < r + 1)
        return -1;
    float *v = (float *)malloc(sizeof(float) * (size_t)w * (size_t)h);
    if (v == NULL)
        return -1;
    for (int y = 0; y < h; y++) {
        for (int x = 0; x < w; x++) {
            float acc = 0.0f;
            for (int k = 0; k < n; k++) {
                const int yy = mirror(y + k - r, h);
                const float prod = taps[k] * src[(size_t)yy * w + x];
                acc = acc + prod;
            }
            v[(size_t)y * w + x] = acc;
        }
    }
    for (int y = 0; y < h; y++) {
        for (int x = 0; x < w; x++) {
            float acc = 0.0f;
            for (int k = 0; k < n; k++) {
                const int xx = mirror(x + k - r, w);
                const float prod = taps[k] * v[(size_t)y * w + xx];
                acc = acc + prod;
            }
            dst[(size_t)y * w + x] = acc;
        }
    }
    free(v);
    return 0;
}

/* O6  decimation: the next scale's plane is the low-pass of the current one
 * (with the next scale's taps) sampled at (2y, 2x); size floor(n/2).
 * Reading: even phase and floor halving; the low-pass is computed over the
 * whole plane and then subsampled, which is the definition itself.  With
 * floor halving a frame narrower than 72 px has fewer than 9 samples at
 * scale 3, which is where ADR-1444 Context places the old loader's fault. */
int vifo_decimate(const float *src, int w, int h, const float *taps, int n,
                  float *dst)
{
    if (src == NULL || dst == NULL)
        return -1;
    float *full = (float *)malloc(sizeof(float) * (size_t)w * (size_t)h);
    if (full == NULL)
        return -1;
    const int rc = vifo_filter(src, w, h, taps, n, full);
    if (rc != 0) {
        free(full);
        return rc;
    }
    const int wd = w / 2;
    const int hd = h / 2;
    for (int y = 0; y < hd; y++)
        for (int x = 0; x < wd; x++)
            dst[(size_t)y * wd + x] = full[(size_t)(2 * y) * w + 2 * x];
    free(full);
    return 0;
}

int vifo_total_rows(int w, int h)
{
    (void)w;
    int rows = 0;
    int hs = h;
    for (int s = 0; s < VIFO_NSCALES; s++) {
        rows += hs;
        hs /= 2;
    }
    return rows;
}

/* ---------------------------------------------------------------------- */
/* O9  ordered sums [ADR-1422 Context: the CPU adds the terms into one fp32
 * sum per row and then adds the rows; ADR-1422 Decision: a row's terms go
 * left to right into one fp32 accumulator that starts at zero, and the row
 * sums are added top to bottom in fp32].  num_t and den_t are w*h term
 * planes, row-major.  rowsums (optional) receives n_y, d_y for each row y;
 * *n_out and *d_out the plane's two sums.                                */
int vifo_ordered_sums(const float *num_t, const float *den_t, int w, int h,
                      float *rowsums, float *n_out, float *d_out)
{
    if (num_t == NULL || den_t == NULL || n_out == NULL || d_out == NULL ||
        w < 1 || h < 1)
        return -1;
    float n_s = 0.0f, d_s = 0.0f;
    for (int y = 0; y < h; y++) {
        float n_y = 0.0f, d_y = 0.0f;
        for (int x = 0; x < w; x++) {
            const size_t i = (size_t)y * w + x;
            n_y = n_y + num_t[i];
            d_y = d_y + den_t[i];
        }
        if (rowsums != NULL) {
            rowsums[2 * y] = n_y;
            rowsums[2 * y + 1] = d_y;
        }
        n_s = n_s + n_y;
        d_s = d_s + d_y;
    }
    *n_out = n_s;
    *d_out = d_s;
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Options.  Reading: the pages name vif_sigma_nsq, vif_enhn_gain_limit,
 * vif_skip_scale0, vif_kernelscale and vif_scale1..3_min_val (default 0)
 * [ADR-1422 Decision and Consequences; ADR-1444 Decision and Consequences]
 * without defining them beyond their names; see vif_oracle.h for the
 * meaning taken for each. */
void vifo_default_options(vifo_options *o)
{
    o->sigma_nsq = kNsq;
    o->enhn_gain_limit = kGainLimit;
    o->kernelscale = 1.0;
    o->scale_min_val[0] = 0.0;
    o->scale_min_val[1] = 0.0;
    o->scale_min_val[2] = 0.0;
    o->skip_scale0 = 0;
}

static int options_valid(const vifo_options *o)
{
    if (!(o->sigma_nsq >= 0.0) || isinf(o->sigma_nsq))
        return 0;
    if (!(o->enhn_gain_limit >= 0.0))
        return 0;
    if (o->kernelscale != 1.0)
        return 0;
    for (int i = 0; i < 3; i++)
        if (isnan(o->scale_min_val[i]))
            return 0;
    return o->skip_scale0 == 0 || o->skip_scale0 == 1;
}

/* O1-O11  whole feature for one frame pair.  Sums [ADR-1422 Context and
 * Decision]: each row's terms are added left to right into one fp32
 * accumulator starting at 0.0f; the row sums are added top to bottom into
 * one fp32 accumulator per scale.  Scores (reading): fp64 quotients of the
 * fp32 sums; num and den added over the scales in scale order in fp64.
 * A skipped scale 0 (reading) still feeds the pyramid, has no statistic,
 * zero sums and zero rows, and reports the score 0.  The floors of scales
 * 1..3 (reading) act on the reported scores only: score < floor -> floor.
 */
int vifo_score(const void *ref, const void *dist, int w, int h, int bpc,
               double out[8], float sums[8], float *rowsums)
{
    vifo_options o;
    vifo_default_options(&o);
    return vifo_score_ex(ref, dist, w, h, bpc, &o, out, sums, rowsums);
}

int vifo_score_ex(const void *ref, const void *dist, int w, int h, int bpc,
                  const vifo_options *opt, double out[8], float sums[8],
                  float *rowsums)
{
    if (ref == NULL || dist == NULL || out == NULL || opt == NULL)
        return -1;
    if (w < 16 || h < 16)
        return -1;
    if (bpc != 8 && bpc != 10 && bpc != 12 && bpc != 16)
        return -1;
    if (!options_valid(opt))
        return -1;

    const size_t n0 = (size_t)w * (size_t)h;
    float *X = (float *)malloc(sizeof(float) * n0);
    float *Y = (float *)malloc(sizeof(float) * n0);
    float *XX = (float *)malloc(sizeof(float) * n0);
    float *YY = (float *)malloc(sizeof(float) * n0);
    float *XY = (float *)malloc(sizeof(float) * n0);
    float *mu1 = (float *)malloc(sizeof(float) * n0);
    float *mu2 = (float *)malloc(sizeof(float) * n0);
    float *fxx = (float *)malloc(sizeof(float) * n0);
    float *fyy = (float *)malloc(sizeof(float) * n0);
    float *fxy = (float *)malloc(sizeof(float) * n0);
    float *Xn = (float *)malloc(sizeof(float) * n0);
    float *Yn = (float *)malloc(sizeof(float) * n0);
    int rc = -1;
    if (!X || !Y || !XX || !YY || !XY || !mu1 || !mu2 || !fxx || !fyy ||
        !fxy || !Xn || !Yn)
        goto done;

    vifo_normalise(ref, w, h, bpc, X);
    vifo_normalise(dist, w, h, bpc, Y);

    float N[VIFO_NSCALES], D[VIFO_NSCALES];
    int ws = w, hs = h;
    size_t row_base = 0;
    for (int s = 0; s < VIFO_NSCALES; s++) {
        float taps[VIFO_MAX_TAPS];
        const int nt = vifo_taps(s, taps);
        if (s > 0) {
            if (vifo_decimate(X, ws, hs, taps, nt, Xn) != 0 ||
                vifo_decimate(Y, ws, hs, taps, nt, Yn) != 0)
                goto done;
            ws /= 2;
            hs /= 2;
            memcpy(X, Xn, sizeof(float) * (size_t)ws * hs);
            memcpy(Y, Yn, sizeof(float) * (size_t)ws * hs);
        }
        if (s == 0 && opt->skip_scale0) {
            if (rowsums != NULL)
                for (int y = 0; y < hs; y++) {
                    rowsums[2 * (row_base + y)] = 0.0f;
                    rowsums[2 * (row_base + y) + 1] = 0.0f;
                }
            row_base += (size_t)hs;
            N[0] = 0.0f;
            D[0] = 0.0f;
            continue;
        }
        const size_t ns = (size_t)ws * (size_t)hs;
        for (size_t i = 0; i < ns; i++) {
            XX[i] = X[i] * X[i];
            YY[i] = Y[i] * Y[i];
            XY[i] = X[i] * Y[i];
        }
        if (vifo_filter(X, ws, hs, taps, nt, mu1) != 0 ||
            vifo_filter(Y, ws, hs, taps, nt, mu2) != 0 ||
            vifo_filter(XX, ws, hs, taps, nt, fxx) != 0 ||
            vifo_filter(YY, ws, hs, taps, nt, fyy) != 0 ||
            vifo_filter(XY, ws, hs, taps, nt, fxy) != 0)
            goto done;

        /* the products' planes are free once filtered: they take the
         * term planes (row-major, like the planes) */
        float *num_t = XX, *den_t = YY;
        for (size_t i = 0; i < ns; i++)
            vifo_statistic_ex(mu1[i], mu2[i], fxx[i], fyy[i], fxy[i],
                              opt->sigma_nsq, opt->enhn_gain_limit,
                              &num_t[i], &den_t[i]);
        float n_s, d_s;
        vifo_ordered_sums(num_t, den_t, ws, hs,
                          rowsums != NULL ? rowsums + 2 * row_base : NULL,
                          &n_s, &d_s);
        row_base += (size_t)hs;
        N[s] = n_s;
        D[s] = d_s;
    }

    for (int s = 0; s < VIFO_NSCALES; s++)
        out[s] = (double)N[s] / (double)D[s];
    if (opt->skip_scale0)
        out[0] = 0.0;
    for (int s = 1; s < VIFO_NSCALES; s++)
        if (out[s] < opt->scale_min_val[s - 1])
            out[s] = opt->scale_min_val[s - 1];
    double num = 0.0, den = 0.0;
    num = (double)N[0] + (double)N[1];
    num = num + (double)N[2];
    num = num + (double)N[3];
    den = (double)D[0] + (double)D[1];
    den = den + (double)D[2];
    den = den + (double)D[3];
    out[4] = num;
    out[5] = den;
    out[6] = num / den;
    out[7] = 0.0;
    if (sums != NULL) {
        for (int s = 0; s < VIFO_NSCALES; s++) {
            sums[2 * s] = N[s];
            sums[2 * s + 1] = D[s];
        }
    }
    rc = 0;

done:
    free(X);
    free(Y);
    free(XX);
    free(YY);
    free(XY);
    free(mu1);
    free(mu2);
    free(fxx);
    free(fyy);
    free(fxy);
    free(Xn);
    free(Yn);
    return rc;
}
