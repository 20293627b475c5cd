/*
 * score_raw.c -- a plain C program that scores one frame pair through the
 * library's C ABI (include/vif.h, include/fssim.h), with no Python and no
 * C++: the boundary as a C caller sees it.
 *
 *   score_raw W H BPC REF.raw DIST.raw
 *
 * REF.raw and DIST.raw hold one tightly packed row-major plane each: W*H
 * bytes for BPC 8, else W*H little-endian uint16 samples.  The program
 * copies both planes to the device, then prints, one per line, the outputs
 * as the hexadecimal bit patterns of the doubles:
 *   vif        out[0..7] of vif_score (device frames)
 *   vif_host   out[0..7] of vif_score_host (the same frames from host memory)
 *   fssim      out[0..1] of fssim_score (device frames)
 * Exit status 0 on success; on a failure it prints the library's error
 * string and exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fssim.h"
#include "vif.h"

static void *read_plane(const char *path, size_t bytes)
{
    FILE *f = fopen(path, "rb");
    if (f == NULL)
        return NULL;
    void *p = malloc(bytes);
    if (p != NULL && fread(p, 1, bytes, f) != bytes) {
        free(p);
        p = NULL;
    }
    fclose(f);
    return p;
}

static void print_bits(const char *name, const double *v, int n)
{
    printf("%s", name);
    for (int i = 0; i < n; i++) {
        uint64_t u;
        memcpy(&u, &v[i], sizeof u);
        printf(" %016llx", (unsigned long long)u);
    }
    printf("\n");
}

static int fail(const char *what)
{
    fprintf(stderr, "%s failed: %s\n", what, vif_strerror(vif_errno()));
    return 1;
}

int main(int argc, char **argv)
{
    if (argc != 6) {
        fprintf(stderr, "usage: %s W H BPC REF.raw DIST.raw\n", argv[0]);
        return 2;
    }
    const int w = atoi(argv[1]), h = atoi(argv[2]), bpc = atoi(argv[3]);
    if (w < 1 || h < 1 || (bpc != 8 && bpc != 10 && bpc != 12 && bpc != 16)) {
        fprintf(stderr, "bad geometry or bit depth\n");
        return 2;
    }
    const size_t bytes = (size_t)w * h * (bpc == 8 ? 1 : 2);
    void *ref = read_plane(argv[4], bytes);
    void *dist = read_plane(argv[5], bytes);
    if (ref == NULL || dist == NULL) {
        fprintf(stderr, "cannot read %zu bytes from each plane file\n", bytes);
        return 2;
    }
    void *dref = NULL, *ddist = NULL;
    if (hipMalloc(&dref, bytes) != hipSuccess ||
        hipMalloc(&ddist, bytes) != hipSuccess ||
        hipMemcpy(dref, ref, bytes, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(ddist, dist, bytes, hipMemcpyHostToDevice) != hipSuccess) {
        fprintf(stderr, "device buffers could not be set up\n");
        return 1;
    }
    int rc = 0;
    double out[8];

    vif_ctx *v = vif_create(w, h, bpc);
    if (v == NULL)
        return fail("vif_create");
    if (vif_score(v, dref, ddist, out) != VIF_OK)
        rc = fail("vif_score");
    else
        print_bits("vif", out, 8);
    if (rc == 0 && vif_score_host(v, ref, dist, out) != VIF_OK)
        rc = fail("vif_score_host");
    else if (rc == 0)
        print_bits("vif_host", out, 8);
    vif_destroy(v);

    fssim_ctx *s = fssim_create(w, h, bpc);
    if (s == NULL)
        return fail("fssim_create");
    if (rc == 0 && fssim_score(s, dref, ddist, out) != VIF_OK)
        rc = fail("fssim_score");
    else if (rc == 0)
        print_bits("fssim", out, 2);
    fssim_destroy(s);

    (void)hipFree(dref);
    (void)hipFree(ddist);
    free(ref);
    free(dist);
    return rc;
}
