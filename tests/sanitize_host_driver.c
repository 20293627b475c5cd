/*
 * sanitize_host_driver.c -- runs the library's host-only entry points,
 * built with AddressSanitizer and UndefinedBehaviorSanitizer on the host side
 * by tests/test_host_sanitizers.py: the strip geometry over every strip
 * boundary of small frames, the host sums and scores from row sums under
 * every option path, the tap generators, the option and argument checks of
 * the context constructors (refused before any device call), and the error
 * strings.  No GPU is touched.  Any out-of-bounds access or undefined
 * behaviour aborts with a non-zero exit.  Test infrastructure only.
 *
 * Row sums come from a 64-bit linear congruential generator (Knuth's MMIX
 * constants); the values do not matter, only that every path runs.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "fssim.h"
#include "vif.h"

static uint64_t lcg = 88172645463325252ull;

static float next_float(void)
{
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((lcg >> 40) & 0xffffff) / 16777216.0f * 4096.0f;
}

static int fail(const char *what, int a, int b, int c)
{
    printf("FAIL %s (%d, %d, %d)\n", what, a, b, c);
    return 1;
}

/* every strip of every small frame height; owned rows must tile each scale */
static int strips(void)
{
    int bad = 0;
    for (int h = 16; h <= 140; ++h) {
        for (int row0 = -8; row0 <= h + 8; row0 += 4) {
            for (int row1 = row0 - 8; row1 <= h + 8; row1 += 4) {
                int info[VIF_STRIP_INFO];
                const int r = vif_strip_geometry(64, h, row0, row1, info);
                const int want = row0 >= 0 && row0 % 8 == 0 && row1 > row0 &&
                                 row1 <= h && (row1 % 8 == 0 || row1 == h);
                if ((r == VIF_OK) != want)
                    bad |= fail("strip acceptance", h, row0, row1);
                if (r != VIF_OK)
                    continue;
                if (info[0] < 0 || info[0] + info[1] > h || info[1] < 1)
                    bad |= fail("strip input rows", h, row0, row1);
                for (int s = 0; s < 4; ++s)
                    if (info[2 + 2 * s] < 0 || info[3 + 2 * s] < 0 ||
                        info[2 + 2 * s] + info[3 + 2 * s] > (h >> s))
                        bad |= fail("strip owned rows", h, row0, row1);
            }
            /* a NULL output array is refused */
            if (vif_strip_geometry(64, h, 0, h, NULL) != VIF_EINVAL)
                bad |= fail("strip NULL", h, 0, 0);
        }
        /* the rows of a tiling of 8-row multiples own each row once */
        int owned[4] = {0, 0, 0, 0};
        for (int row0 = 0; row0 < h; row0 += 24) {
            const int row1 = row0 + 24 < h ? row0 + 24 : h;
            int info[VIF_STRIP_INFO];
            if (vif_strip_geometry(64, h, row0, row1, info) != VIF_OK)
                return fail("tiling", h, row0, row1);
            for (int s = 0; s < 4; ++s) {
                if (info[2 + 2 * s] != owned[s])
                    bad |= fail("tiling contiguity", h, row0, s);
                owned[s] += info[3 + 2 * s];
            }
        }
        for (int s = 0; s < 4; ++s)
            if (owned[s] != (h >> s))
                bad |= fail("tiling coverage", h, s, owned[s]);
    }
    return bad;
}

/* the host sums and scores from row sums, every option path */
static int scores(void)
{
    int bad = 0;
    static float rows[2 * 4096];
    for (int h = 16; h <= 1030; h += 7) {
        const int n = 2 * (h + (h >> 1) + (h >> 2) + (h >> 3));
        for (int i = 0; i < n; ++i)
            rows[i] = next_float();
        for (int variant = 0; variant < 6; ++variant) {
            vif_options o;
            vif_default_options(&o);
            if (variant == 1)
                o.skip_scale0 = 1;
            if (variant == 2)
                o.scale_min_val[0] = o.scale_min_val[1] =
                    o.scale_min_val[2] = 2.0;
            if (variant == 3)
                o.sigma_nsq = 0.0;
            if (variant == 4)
                o.enhn_gain_limit = INFINITY;
            double out[8];
            float sums[8];
            const int r = vif_scores_from_rows(
                100, h, variant == 5 ? NULL : &o, rows, out,
                variant == 4 ? NULL : sums);
            if (r != VIF_OK)
                bad |= fail("scores_from_rows", h, variant, r);
            if (variant == 1 && out[0] != 0.0)
                bad |= fail("skip_scale0", h, 0, 0);
        }
        double out[8];
        if (vif_scores_from_rows(100, h, NULL, NULL, out, NULL) != VIF_EINVAL ||
            vif_scores_from_rows(100, h, NULL, rows, NULL, NULL) != VIF_EINVAL ||
            vif_scores_from_rows(15, h, NULL, rows, out, NULL) != VIF_EINVAL)
            bad |= fail("scores_from_rows refusals", h, 0, 0);
        vif_options o;
        vif_default_options(&o);
        o.kernelscale = 2.0;
        if (vif_scores_from_rows(100, h, &o, rows, out, NULL) != VIF_EINVAL)
            bad |= fail("scores_from_rows options", h, 0, 0);
    }
    return bad;
}

/* taps, option checks of the constructors, error strings */
static int misc(void)
{
    int bad = 0;
    float taps[VIF_MAX_TAPS + 8];
    for (int s = -2; s < 6; ++s) {
        const int n = vif_taps(s, taps);
        if ((s >= 0 && s < 4) != (n > 0))
            bad |= fail("vif_taps", s, n, 0);
    }
    if (vif_taps(0, NULL) >= 0)
        bad |= fail("vif_taps NULL", 0, 0, 0);
    float st[FSSIM_TAPS];
    if (fssim_taps(st) != FSSIM_TAPS || fssim_taps(NULL) != VIF_EINVAL)
        bad |= fail("fssim_taps", 0, 0, 0);
    /* geometry and options the constructors refuse before any device call */
    const int geoms[][3] = {{15, 64, 8}, {64, 15, 8}, {64, 64, 9},
                            {64, 64, 0}, {1 << 14, 1 << 14, 8}, {-5, 64, 8}};
    for (unsigned i = 0; i < sizeof(geoms) / sizeof(geoms[0]); ++i)
        if (vif_create(geoms[i][0], geoms[i][1], geoms[i][2]) != NULL ||
            vif_errno() != VIF_EINVAL)
            bad |= fail("vif_create refusal", geoms[i][0], geoms[i][1],
                        geoms[i][2]);
    const double nsq[] = {-1.0, NAN, INFINITY};
    for (unsigned i = 0; i < 3; ++i) {
        vif_options o;
        vif_default_options(&o);
        o.sigma_nsq = nsq[i];
        if (vif_create_ex(64, 64, 8, &o) != NULL || vif_errno() != VIF_EINVAL)
            bad |= fail("vif_create_ex options", (int)i, 0, 0);
    }
    if (vif_create_strip(64, 64, 8, NULL, 1, 4, 64) != NULL ||
        vif_create_strip(64, 64, 8, NULL, 0, 0, 64) != NULL ||
        vif_create_strip(64, 64, 8, NULL, VIF_MAX_BATCH + 1, 0, 64) != NULL)
        bad |= fail("vif_create_strip refusal", 0, 0, 0);
    if (fssim_create(0, 64, 8) != NULL || fssim_create(64, 64, 7) != NULL)
        bad |= fail("fssim_create refusal", 0, 0, 0);
    for (int c = -6; c <= 1; ++c)
        if (vif_strerror(c) == NULL)
            bad |= fail("vif_strerror", c, 0, 0);
    return bad;
}

int main(void)
{
    int bad = strips();
    bad |= scores();
    bad |= misc();
    if (bad)
        return 1;
    printf("ok\n");
    return 0;
}
