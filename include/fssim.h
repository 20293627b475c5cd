/*
 * fssim.h -- C ABI of the MI355X (gfx950) float SSIM feature with its exact
 * decimation.
 *
 * One call scores one reference/distorted luma frame pair:
 *   1. both planes are normalised to fp32 (8-bit samples as they are, 10/12/
 *      16-bit samples divided by 4/16/256) and, when the factor
 *      f = max(1, round(min(w, h) / 256)) is above 1, decimated: decimated
 *      pixel (x, y) is the f x f box window centred on (x*f, y*f), offsets
 *      -f/2 .. f/2 - (f even), with the tap fl32(1 / (f*f)); each product is
 *      an fp32 value, the products are added exactly (the page proves the
 *      CPU's double sum exact for f <= 128) and the sum is rounded to fp32
 *      once; the border is the symmetric one of period 2n; a decimated side
 *      is n / f + (n & 1) samples.  The decimated planes are bit-identical to
 *      the CPU's.
 *   2. the SSIM stage on the (decimated) planes: an 11-tap Gaussian window
 *      (sigma 1.5), separable, vertical pass then horizontal, taps in
 *      ascending order, the same symmetric border, every product and sum an
 *      fp32 rounding; the combined SSIM formula per pixel in fp32 with
 *      C1 = (0.01 * 255)^2 and C2 = (0.03 * 255)^2 rounded to fp32;
 *   3. the frame mean: each row's values added left to right into an fp64
 *      sum from 0, the rows added top to bottom in fp64, divided by the
 *      pixel count in fp64 and rounded to fp32.
 * Every output is bit-identical to the CPU definition.
 *
 * Sources (page title, section):
 *   Research-2130 "float_ssim decimation on the SYCL device", Question (the
 *     factor), Sources (taps, window offsets, the double sum, the decimated
 *     size, the symmetric border, the sample normalisation, fp32 frame
 *     means) and Findings (the exactness of the double sum for factors up to
 *     128, the context check that refuses larger ones, decimation from an
 *     untouched copy giving the same planes, a submit failing cleanly
 *     instead of dereferencing NULL).
 * The SSIM stage itself (window, constants, filter order) is not printed on
 * the pages; the published SSIM of Wang, Bovik, Sheikh and Simoncelli (2004)
 * is the reading taken.
 *
 * Errors share the thread-local state of vif.h: functions return VIF_OK (0)
 * or a negative VIF_E* code, and vif_errno() / vif_strerror() report the
 * last failure on the calling thread.
 */
#ifndef FSSIM_H
#define FSSIM_H

#ifdef __cplusplus
extern "C" {
#endif

#define FSSIM_TAPS 11
#define FSSIM_MAX_FACTOR 128      /* Research-2130, Findings               */
#define FSSIM_MAX_PIXELS (1L << 27) /* largest w * h accepted              */
#define FSSIM_QUEUE_DEPTH 3

typedef struct fssim_ctx fssim_ctx;

/*
 * fssim_create -- a scoring context for w x h frames at bpc bits.
 *   w, h   >= 1, w * h <= FSSIM_MAX_PIXELS; the factor of the frame must
 *          not exceed FSSIM_MAX_FACTOR (a context check, as on the page).
 *   bpc    8, 10, 12 or 16.
 * Allocates every buffer the context needs (decimated planes, the SSIM map,
 * pinned row sums) on the device current at the call and computes the taps
 * on the host.  NULL on failure; vif_errno() gives VIF_EINVAL, VIF_ENOMEM or
 * VIF_EHIP.
 */
fssim_ctx *fssim_create(int w, int h, int bpc);

/*
 * fssim_geometry -- geom[0] = the decimation factor f, geom[1] = w',
 * geom[2] = h', the size of the plane the SSIM stage scores (w, h when f is
 * 1).  Host only.
 */
int fssim_geometry(const fssim_ctx *ctx, int geom[3]);

/*
 * fssim_score -- score one frame pair.
 *   ref, dist  DEVICE pointers to tightly packed row-major planes (pitch =
 *              w samples): uint8_t when bpc is 8, else uint16_t (2-byte
 *              aligned).  Values are used as given.  Owned by the caller and
 *              valid until the call returns.
 *   out        HOST memory for 2 doubles: out[0] = float_ssim, the fp32
 *              frame mean widened to double; out[1] = the factor f.
 * Synchronous (fssim_submit then fssim_collect); VIF_EINVAL while frames
 * submitted with fssim_submit are pending.  Allocates nothing.  On error
 * out is untouched.  A context is not thread-safe.
 */
int fssim_score(fssim_ctx *ctx, const void *ref, const void *dist,
                double out[2]);

/*
 * Asynchronous scoring, as vif_submit / vif_collect: up to
 * FSSIM_QUEUE_DEPTH frames in flight, collected in submission order; the
 * frames stay valid and unchanged until their fssim_collect returns.
 */
int fssim_submit(fssim_ctx *ctx, const void *ref, const void *dist);
int fssim_collect(fssim_ctx *ctx, double out[2]);
int fssim_pending(const fssim_ctx *ctx);

/*
 * Batched submission, as vif_create_batch / vif_submit_batch: a context from
 * fssim_create_batch (1 <= max_batch <= FSSIM_MAX_BATCH; buffers sized for
 * max_batch frames per queue slot) accepts fssim_submit_batch of n <=
 * max_batch pairs as one slot, each kernel running once for all n frames;
 * fssim_collect returns them one by one in order.  The same bits as n single
 * submissions.  VIF_EINVAL for a bad n, NULL arrays or frames, or a full
 * queue.  fssim_create makes max_batch = 1.  Allocates nothing.
 */
#define FSSIM_MAX_BATCH 16
fssim_ctx *fssim_create_batch(int w, int h, int bpc, int max_batch);
int fssim_submit_batch(fssim_ctx *ctx, int n, const void *const *refs,
                       const void *const *dists);

/*
 * fssim_set_stream -- the caller's HIP stream (hipStream_t as void*; NULL =
 * the default stream): work queued on it before a submit is ordered before
 * the frame's kernels.  VIF_EINVAL while frames are pending.
 */
int fssim_set_stream(fssim_ctx *ctx, void *hip_stream);

/*
 * Values of the last frame returned by fssim_score or fssim_collect; each
 * call needs no frame pending (VIF_EINVAL otherwise, or when no frame has
 * been returned yet).  They copy from the device synchronously.
 *   fssim_get_row_sums  the h' fp64 row sums; rows holds capacity doubles;
 *                       returns h'.
 *   fssim_get_map       the w' x h' per-pixel SSIM values, row-major;
 *                       capacity in floats; returns w' * h'.
 *   fssim_get_planes    the decimated reference then distorted planes,
 *                       row-major, 2 * w' * h' floats; returns that count.
 *                       Only when f > 1 (VIF_EINVAL at f = 1, where the
 *                       SSIM stage reads the samples themselves).
 */
int fssim_get_row_sums(const fssim_ctx *ctx, double *rows, int capacity);
long fssim_get_map(fssim_ctx *ctx, float *map, long capacity);
long fssim_get_planes(fssim_ctx *ctx, float *planes, long capacity);

/*
 * fssim_taps -- the 11 fp32 taps of the SSIM window as the context passes
 * them to its kernel (fp64 Gaussian, sigma 1.5, normalised by its sum,
 * each rounded once).  Returns FSSIM_TAPS.  Host only.
 */
int fssim_taps(float taps[FSSIM_TAPS]);

/*
 * Kernel timing, as vif_set_profiling / vif_get_kernel_times, for the kinds
 *   0  decimation (both planes; absent at f = 1)
 *   1  SSIM stage (filter and per-pixel value)
 *   2  ordered row sums
 * kinds is a bit mask (0x7 all).  fssim_get_kernel_times returns 3.  A
 * launch counted there is one kind's work for one submission: one kernel
 * launch, or several in a row for planes with more than 65535 rows of
 * blocks, timed as one.
 */
int fssim_set_profiling(fssim_ctx *ctx, int kinds);
int fssim_get_kernel_times(const fssim_ctx *ctx, double *ms, long *launches,
                           int capacity);

/* fssim_destroy -- frees everything the context owns.  NULL is a no-op. */
void fssim_destroy(fssim_ctx *ctx);

#ifdef __cplusplus
}
#endif

#endif /* FSSIM_H */
