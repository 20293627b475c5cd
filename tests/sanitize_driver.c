/*
 * sanitize_driver.c -- runs both CPU oracles on edge geometries, built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_oracle_sanitizers.py.  Any out-of-bounds access, use of freed
 * memory or undefined behaviour aborts with a non-zero exit.  Test
 * infrastructure only.
 *
 * Frames come from a 64-bit linear congruential generator (Knuth's MMIX
 * constants); the values do not matter, only that every code path and
 * border runs.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "fssim_oracle.h"
#include "vif_oracle.h"

static uint64_t lcg = 88172645463325252ull;

static unsigned next_bits(void)
{
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (unsigned)(lcg >> 33);
}

static void *frame(int w, int h, int bpc, int flat)
{
    const size_t n = (size_t)w * h;
    const unsigned top = (1u << bpc) - 1u;
    if (bpc == 8) {
        uint8_t *p = malloc(n);
        for (size_t i = 0; i < n; i++)
            p[i] = (uint8_t)(flat ? 77u : next_bits() % (top + 1u));
        return p;
    }
    uint16_t *p = malloc(n * 2);
    for (size_t i = 0; i < n; i++)
        p[i] = (uint16_t)(flat ? 77u : next_bits() % (top + 1u));
    return p;
}

static int run_vif(int w, int h, int bpc, const vifo_options *opt, int flat)
{
    void *r = frame(w, h, bpc, flat), *d = frame(w, h, bpc, 0);
    double out[8];
    float sums[8];
    float *rows = malloc(sizeof(float) * 2 * (size_t)vifo_total_rows(w, h));
    const int rc = opt ? vifo_score_ex(r, d, w, h, bpc, opt, out, sums, rows)
                       : vifo_score(r, d, w, h, bpc, out, sums, rows);
    free(rows);
    free(r);
    free(d);
    if (rc != 0) {
        fprintf(stderr, "vifo_score %dx%d bpc %d: rc %d\n", w, h, bpc, rc);
        return 1;
    }
    return 0;
}

static int run_fssim(int w, int h, int bpc)
{
    void *r = frame(w, h, bpc, 0), *d = frame(w, h, bpc, 0);
    const int f = fssimo_scale(w, h);
    const int ow = f > 1 ? fssimo_decimated_size(w, f) : w;
    const int oh = f > 1 ? fssimo_decimated_size(h, f) : h;
    double out[2];
    float *map = malloc(sizeof(float) * (size_t)ow * oh);
    float *planes = malloc(sizeof(float) * 2 * (size_t)ow * oh);
    double *rows = malloc(sizeof(double) * (size_t)oh);
    const int rc = fssimo_score(r, d, w, h, bpc, out, map, planes, rows);
    free(map);
    free(planes);
    free(rows);
    free(r);
    free(d);
    if (rc != 0) {
        fprintf(stderr, "fssimo_score %dx%d bpc %d: rc %d\n", w, h, bpc, rc);
        return 1;
    }
    return 0;
}

int main(void)
{
    int bad = 0;
    static const int vif_sizes[][2] = {{16, 16}, {17, 23}, {16, 71},
                                       {40, 40}, {71, 71}, {73, 41},
                                       {113, 17}, {200, 33}};
    static const int bpcs[] = {8, 10, 12, 16};
    for (size_t i = 0; i < sizeof vif_sizes / sizeof vif_sizes[0]; i++)
        for (size_t b = 0; b < 4; b++)
            bad |= run_vif(vif_sizes[i][0], vif_sizes[i][1], bpcs[b], NULL,
                           0);
    bad |= run_vif(40, 40, 8, NULL, 1); /* flat reference: low branch */
    vifo_options o;
    vifo_default_options(&o);
    o.sigma_nsq = 0.0; /* IEEE special cases: 0/0, x/0 */
    bad |= run_vif(33, 29, 8, &o, 1);
    o.sigma_nsq = 4.7;
    o.enhn_gain_limit = 0.5;
    o.skip_scale0 = 1;
    o.scale_min_val[0] = 0.9;
    bad |= run_vif(48, 40, 10, &o, 0);

    static const int ss_sizes[][2] = {{1, 1}, {2, 3}, {3, 2}, {5, 7},
                                      {11, 11}, {16, 16}, {64, 17},
                                      {400, 384}, {1281, 721}, {1083, 720}};
    for (size_t i = 0; i < sizeof ss_sizes / sizeof ss_sizes[0]; i++)
        bad |= run_fssim(ss_sizes[i][0], ss_sizes[i][1],
                         bpcs[i % 4]);
    if (!bad)
        printf("sanitized oracle runs: ok\n");
    return bad;
}
