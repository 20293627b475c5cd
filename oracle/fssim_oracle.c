/*
 * fssim_oracle.c -- plain CPU oracle of the float SSIM feature with its
 * exact decimation.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library.
 *
 * Build: gcc -std=c99 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (x86-64, SSE2: every float expression rounds to binary32 at each
 * operation, in the order written).
 *
 * Sources, cited by page title and section:
 *   [R2130 Question] "Research-2130: float_ssim decimation on the SYCL
 *       device", Question: both planes are decimated by the factor
 *       max(1, round(min(w, h) / 256)) before SSIM (4 at 1920x1080, 8 at
 *       3840x2160).
 *   [R2130 Sources] same page, Sources: the box tap 1 / (scale * scale) in
 *       fp32 with the symmetric border; the decimated pixel (x, y) is the
 *       window centred on (x * factor, y * factor), offsets -k/2 ..
 *       k/2 - (k even); each product is an fp32 value, the products are
 *       added in double and the sum is rounded to fp32 once; the decimated
 *       size is n / factor + (n & 1); the symmetric border mirrors with
 *       period 2n; sample normalisation as for VIF; the frame mean is
 *       returned as fp32.
 *   [R2130 Findings] same page, Findings: the double sum is exact for
 *       factors up to 128 (every partial sum is a multiple of 2^-45 below
 *       256), and a decimated output never reads a value another output
 *       wrote, so decimating from an untouched copy is the same.
 * Readings where the pages are silent (the SSIM stage itself: window,
 * constants, separable filtering, summation order) are marked "reading".
 */
#include "fssim_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* [R2130 Question]  round() is C's: halves away from zero. */
int fssimo_scale(int w, int h)
{
    const int m = w < h ? w : h;
    const int s = (int)round((double)m / 256.0);
    return s < 1 ? 1 : s;
}

/* [R2130 Sources] */
int fssimo_decimated_size(int n, int f)
{
    return n / f + (n & 1);
}

/* [R2130 Sources]  The symmetric border: the plane repeated with its
 * mirror image, period 2n; -1 -> 0, -2 -> 1, n -> n-1, n+1 -> n-2. */
int fssimo_symmetric(int i, int n)
{
    const int p = 2 * n;
    int m = i % p;
    if (m < 0)
        m += p;
    if (m >= n)
        m = p - 1 - m;
    return m;
}

/* [R2130 Sources, Findings]  Box low-pass at (x*f, y*f) of f x f taps
 * fl32(1/(f*f)), each product fp32, the sum in fp64 from 0.0, then one
 * rounding to fp32 (the sum scaled by 1.0 first, which changes nothing). */
int fssimo_decimate(const float *src, int w, int h, int f, float *dst)
{
    if (src == NULL || dst == NULL || w < 1 || h < 1 || f < 1 ||
        f > FSSIMO_MAX_SCALE)
        return -1;
    const float tap = 1.0f / (float)(f * f);
    const int lo = -(f / 2);
    const int hi = f / 2 - (f % 2 == 0 ? 1 : 0);
    const int ow = fssimo_decimated_size(w, f);
    const int oh = fssimo_decimated_size(h, f);
    for (int y = 0; y < oh; y++) {
        for (int x = 0; x < ow; x++) {
            double sum = 0.0;
            for (int dy = lo; dy <= hi; dy++) {
                const int yy = fssimo_symmetric(y * f + dy, h);
                for (int dx = lo; dx <= hi; dx++) {
                    const int xx = fssimo_symmetric(x * f + dx, w);
                    const float prod = src[(size_t)yy * w + xx] * tap;
                    sum += (double)prod;
                }
            }
            dst[(size_t)y * ow + x] = (float)(sum * (double)1.0f);
        }
    }
    return 0;
}

/* Reading: the published SSIM window, a Gaussian of 11 taps with sigma
 * 1.5, evaluated in fp64 (libm exp), normalised by its fp64 sum in
 * ascending order, each tap rounded to fp32 once; applied separably. */
void fssimo_taps(float taps[FSSIMO_TAPS])
{
    double g[FSSIMO_TAPS];
    double sum = 0.0;
    const double sigma = 1.5;
    for (int k = 0; k < FSSIMO_TAPS; k++) {
        const double d = (double)(k - FSSIMO_TAPS / 2);
        g[k] = exp(-(d * d) / (2.0 * sigma * sigma));
    }
    for (int k = 0; k < FSSIMO_TAPS; k++)
        sum += g[k];
    for (int k = 0; k < FSSIMO_TAPS; k++)
        taps[k] = (float)(g[k] / sum);
}

/* Reading: vertical pass, then horizontal; taps in ascending order; an
 * fp32 accumulator from 0.0f, each product and sum rounded; the symmetric
 * border of the decimation [R2130 Sources] at the plane's edges. */
int fssimo_filter(const float *src, int w, int h, float *dst)
{
    if (src == NULL || dst == NULL || w < 1 || h < 1)
        return -1;
    float t[FSSIMO_TAPS];
    fssimo_taps(t);
    const int r = FSSIMO_TAPS / 2;
    float *v = (float *)malloc(sizeof(float) * (size_t)w * h);
    if (v == NULL)
        return -1;
    for (int y = 0; y < h; y++)
        for (int x = 0; x < w; x++) {
            float acc = 0.0f;
            for (int k = 0; k < FSSIMO_TAPS; k++) {
                const int yy = fssimo_symmetric(y + k - r, h);
                acc = acc + t[k] * src[(size_t)yy * w + x];
            }
            v[(size_t)y * w + x] = acc;
        }
    for (int y = 0; y < h; y++)
        for (int x = 0; x < w; x++) {
            float acc = 0.0f;
            for (int k = 0; k < FSSIMO_TAPS; k++) {
                const int xx = fssimo_symmetric(x + k - r, w);
                acc = acc + t[k] * v[(size_t)y * w + xx];
            }
            dst[(size_t)y * w + x] = acc;
        }
    free(v);
    return 0;
}

/* Reading: the published SSIM in its combined form, with K1 = 0.01,
 * K2 = 0.03 and L = 255 (the samples are normalised to the 8-bit range);
 * C1 and C2 formed in fp64 and rounded to fp32; every other operation fp32
 * in the order written.  A window against itself gives numerator and
 * denominator the same value, so exactly 1 (the pages require identical
 * windows to score exactly 1). */
float fssimo_pixel(float mu1, float mu2, float xx, float yy, float xy)
{
    const float c1 = (float)((0.01 * 255.0) * (0.01 * 255.0));
    const float c2 = (float)((0.03 * 255.0) * (0.03 * 255.0));
    const float m11 = mu1 * mu1;
    const float m22 = mu2 * mu2;
    const float m12 = mu1 * mu2;
    const float s11 = xx - m11;
    const float s22 = yy - m22;
    const float s12 = xy - m12;
    const float num = (2.0f * m12 + c1) * (2.0f * s12 + c2);
    const float den = (m11 + m22 + c1) * (s11 + s22 + c2);
    return num / den;
}

static int normalise(const void *src, int w, int h, int bpc, float *dst)
{
    const size_t n = (size_t)w * h;
    if (bpc == 8) {
        const uint8_t *s = (const uint8_t *)src;
        for (size_t i = 0; i < n; i++)
            dst[i] = (float)s[i];
        return 0;
    }
    const float scale = bpc == 10 ? 0.25f : bpc == 12 ? 0.0625f : 0.00390625f;
    const uint16_t *s = (const uint16_t *)src;
    for (size_t i = 0; i < n; i++)
        dst[i] = (float)s[i] * scale;
    return 0;
}

/* Whole feature.  Reading for the mean: each row's SSIM values added left
 * to right into an fp64 sum from 0.0, the row sums added top to bottom in
 * fp64, divided by the pixel count in fp64 and rounded to fp32 [R2130
 * Findings: the frame mean is an fp32 value]. */
int fssimo_score(const void *ref, const void *dist, int w, int h, int bpc,
                 double out[2], float *map, float *planes, double *rows)
{
    if (ref == NULL || dist == NULL || out == NULL || w < 1 || h < 1)
        return -1;
    if (bpc != 8 && bpc != 10 && bpc != 12 && bpc != 16)
        return -1;
    const int f = fssimo_scale(w, h);
    if (f > FSSIMO_MAX_SCALE)
        return -1;
    const int ow = f > 1 ? fssimo_decimated_size(w, f) : w;
    const int oh = f > 1 ? fssimo_decimated_size(h, f) : h;
    const size_t n0 = (size_t)w * h, n = (size_t)ow * oh;
    float *X0 = (float *)malloc(sizeof(float) * n0);
    float *Y0 = (float *)malloc(sizeof(float) * n0);
    float *buf = (float *)malloc(sizeof(float) * n * 10);
    int rc = -1;
    if (X0 == NULL || Y0 == NULL || buf == NULL)
        goto done;
    float *X = buf, *Y = buf + n, *XX = buf + 2 * n, *YY = buf + 3 * n,
          *XY = buf + 4 * n, *mu1 = buf + 5 * n, *mu2 = buf + 6 * n,
          *fxx = buf + 7 * n, *fyy = buf + 8 * n, *fxy = buf + 9 * n;
    normalise(ref, w, h, bpc, X0);
    normalise(dist, w, h, bpc, Y0);
    if (f > 1) {
        if (fssimo_decimate(X0, w, h, f, X) != 0 ||
            fssimo_decimate(Y0, w, h, f, Y) != 0)
            goto done;
    } else {
        memcpy(X, X0, sizeof(float) * n);
        memcpy(Y, Y0, sizeof(float) * n);
    }
    if (planes != NULL) {
        memcpy(planes, X, sizeof(float) * n);
        memcpy(planes + n, Y, sizeof(float) * n);
    }
    for (size_t i = 0; i < n; i++) {
        XX[i] = X[i] * X[i];
        YY[i] = Y[i] * Y[i];
        XY[i] = X[i] * Y[i];
    }
    if (fssimo_filter(X, ow, oh, mu1) != 0 ||
        fssimo_filter(Y, ow, oh, mu2) != 0 ||
        fssimo_filter(XX, ow, oh, fxx) != 0 ||
        fssimo_filter(YY, ow, oh, fyy) != 0 ||
        fssimo_filter(XY, ow, oh, fxy) != 0)
        goto done;
    double total = 0.0;
    for (int y = 0; y < oh; y++) {
        double row = 0.0;
        for (int x = 0; x < ow; x++) {
            const size_t i = (size_t)y * ow + x;
            const float s = fssimo_pixel(mu1[i], mu2[i], fxx[i], fyy[i],
                                         fxy[i]);
            if (map != NULL)
                map[i] = s;
            row += (double)s;
        }
        if (rows != NULL)
            rows[y] = row;
        total += row;
    }
    out[0] = (double)(float)(total / (double)n);
    out[1] = (double)f;
    rc = 0;

done:
    free(X0);
    free(Y0);
    free(buf);
    return rc;
}
