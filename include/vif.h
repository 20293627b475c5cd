/*
 * vif.h -- C ABI of the MI355X (gfx950) float VIF feature extractor.
 *
 * One call scores one reference/distorted luma frame pair with the float
 * VIF feature: four scales, a separable Gaussian low-pass (17/9/5/3 taps)
 * with mirrored borders, 2x decimation between scales, per-pixel local
 * statistics, the two one-plus-ratio values evaluated in fp64 and rounded
 * to fp32 once, a log2 polynomial, and fp32 sums per row and then over the
 * rows.  The results are bit-identical to the CPU definition.
 *
 * Sources (page title, section):
 *   ADR-1422 "float_vif_sycl computes the CPU's arithmetic without an fp64
 *     type ...", Context and Decision: taps generated at run time and passed
 *     to each launch by value; the fp64 expressions; one fp32 accumulator
 *     per row, rows added top to bottom; two floats per row per scale read
 *     back in one copy and added on the host.
 *   ADR-1444 "float_vif_hip runs the arithmetic of the CUDA twin ...",
 *     Decision and Consequences: reflected-then-clamped tile indices, frames
 *     from 16x16 up, the frame ratio and the per-scale sums as outputs.
 *   Research-2130 "float_ssim decimation on the SYCL device", Sources
 *     (sample normalisation) and Open questions (a submit fails cleanly
 *     instead of dereferencing NULL).
 *
 * No C++ or torch types cross this boundary.  Every function is safe to call
 * from C.  Functions that return int return VIF_OK (0) on success or a
 * negative VIF_E* code; the code of the last failure on the calling thread
 * is also kept for vif_errno().
 */
#ifndef VIF_H
#define VIF_H

#ifdef __cplusplus
extern "C" {
#endif

#define VIF_OK 0
#define VIF_EINVAL (-1) /* bad geometry, bit depth, NULL pointer, state   */
#define VIF_ENOMEM (-2) /* device or pinned host allocation failed        */
#define VIF_EHIP (-3)   /* any other HIP runtime error (see vif_strerror)  */
#define VIF_ETOOBIG (-4) /* frame too large for vif_score_noalloc's array  */

#define VIF_NSCALES 4
#define VIF_MAX_TAPS 17
#define VIF_MIN_SIDE 16          /* smallest width or height accepted     */
#define VIF_MAX_PIXELS (1L << 27) /* largest w * h accepted               */

typedef struct vif_ctx vif_ctx;

/*
 * Options of the feature.  The pages name them -- vif_sigma_nsq,
 * vif_enhn_gain_limit, vif_skip_scale0, the floors vif_scale1..3_min_val
 * (default 0) and the tap generator's vif_kernelscale (ADR-1422, Decision
 * and Consequences; ADR-1444, Decision and Consequences) -- but print no
 * arithmetic for them.  The meaning taken for each:
 *   sigma_nsq        noise variance of the statistic, a double: the branch
 *                    sigma1_sq < nsq (compared in fp64) and both
 *                    one-plus-ratio expressions use it.  Finite, >= 0;
 *                    default 2.0.  At 0 nothing is special-cased: IEEE
 *                    arithmetic (a zero sigma1_sq divides by zero) and the
 *                    log2 polynomial reads the bits that arrive (exponent
 *                    field 255 counts as 128).
 *   enhn_gain_limit  bound of the gain g where it enters the numerator,
 *                    once sv_sq is settled: g = MIN(g, limit) as C computes
 *                    it with a double limit (fp64 comparison, the limit
 *                    rounded to fp32).  >= 0, may be +inf; default 100.0,
 *                    the default of the sibling ADM option (Research-1434,
 *                    Findings 1).  On samples in range no gain reaches 91,
 *                    so the default never binds.
 *   kernelscale      filter scale of the tap generator; only 1.0 (widths
 *                    17/9/5/3) is defined.
 *   scale_min_val    floors of the reported vif_scale1..3: a score below its
 *                    floor is replaced by the floor.  Sums, num, den and the
 *                    ratio are not floored.  Not NaN; default 0.0.
 *   skip_scale0      0 or 1.  1: scale 0 still feeds the pyramid but
 *                    contributes nothing: N_0 = D_0 = 0, its row sums read 0
 *                    and vif_scale0 reports 0.0.
 *   reserved         must be 0.
 */
typedef struct vif_options {
  double sigma_nsq;
  double enhn_gain_limit;
  double kernelscale;
  double scale_min_val[3];
  int skip_scale0;
  int reserved;
} vif_options;

/* vif_default_options -- fills *opt with the defaults above.  NULL-safe. */
void vif_default_options(vif_options *opt);

/*
 * vif_create -- a scoring context for frames of w x h samples at bpc bits.
 *   w, h   >= VIF_MIN_SIDE and w * h <= VIF_MAX_PIXELS.  The pages' smallest
 *          scored frame is 16x16 (ADR-1444, Consequences).
 *   bpc    8, 10, 12 or 16 (Research-2130, Sources: 8-bit samples used as
 *          they are, wider samples divided by 4, 16 or 256).
 * Allocates every device buffer the context needs (pyramid planes, the
 * row sums' hand-over words) and pinned host buffers (row sums), on the
 * device current at the call, and computes the taps on the host.  Work goes
 * to the default stream unless vif_set_stream() is called.  Returns NULL on
 * failure; vif_errno() then gives VIF_EINVAL, VIF_ENOMEM or VIF_EHIP.
 * Geometry is refused here, never in the middle of a frame.
 */
vif_ctx *vif_create(int w, int h, int bpc);

/*
 * vif_create_ex -- vif_create with options (NULL: the defaults, the same as
 * vif_create).  The options are copied.  VIF_EINVAL for options outside the
 * ranges of vif_options.
 */
vif_ctx *vif_create_ex(int w, int h, int bpc, const vif_options *opt);

/* vif_get_options -- copies the context's options to *opt. */
int vif_get_options(const vif_ctx *ctx, vif_options *opt);

/*
 * vif_score -- score one frame pair.
 *   ref, dist  DEVICE pointers to tightly packed row-major planes (pitch =
 *              w samples): uint8_t when bpc is 8, else uint16_t holding the
 *              sample in its low bits (2-byte aligned).  Sample values are
 *              used as given (no range check).  Owned by the caller, who
 *              keeps them valid until the call returns.
 *   out        HOST memory for 8 doubles, owned by the caller:
 *                out[0..3] vif_scale0..3 = N_s / D_s in fp64
 *                out[4]    num = ((N_0 + N_1) + N_2) + N_3 in fp64
 *                out[5]    den, the same way
 *                out[6]    num / den (the frame's vif ratio)
 *                out[7]    0.0 (reserved)
 *              where N_s, D_s are the fp32 sums of scale s.
 * Synchronous: returns after the results are on the host (vif_submit then
 * vif_collect); VIF_EINVAL if frames submitted with vif_submit are still
 * pending.  Allocates nothing.  A context is not thread-safe; separate
 * contexts are independent.  On error out is left untouched.
 */
int vif_score(vif_ctx *ctx, const void *ref, const void *dist, double out[8]);

/*
 * Asynchronous scoring.  A context keeps up to VIF_QUEUE_DEPTH frames in
 * flight: vif_submit enqueues one frame pair on the context's stream and
 * returns at once; vif_collect waits for the oldest submitted frame and
 * writes its outputs (the same 8 doubles as vif_score), in submission order.
 * The frames of a submitted pair must stay valid and unchanged until their
 * vif_collect returns.  vif_submit returns VIF_EINVAL when VIF_QUEUE_DEPTH
 * frames are already pending (collect first); vif_collect returns VIF_EINVAL
 * when none is.  Consecutive frames overlap on the device: one frame's
 * read-back runs while the next frame's kernels compute.
 */
#define VIF_QUEUE_DEPTH 3
int vif_submit(vif_ctx *ctx, const void *ref, const void *dist);
int vif_collect(vif_ctx *ctx, double out[8]);

/*
 * Frames in HOST memory.  vif_submit_host enqueues a pair whose planes
 * (same layout as for vif_submit) are in host memory: the context copies
 * them into device buffers of the frame's queue slot with asynchronous
 * copies on the slot's stream, then scores them as vif_submit does, so one
 * frame's upload overlaps the other frames' kernels (double buffering over
 * the VIF_QUEUE_DEPTH slots).  Host memory from hipHostMalloc makes the
 * copies asynchronous; pageable memory also works, but the runtime then
 * stages the copy and the call may wait for it.  The host planes must stay
 * valid and unchanged until the frame's vif_collect returns.  Collect with
 * vif_collect.  vif_score_host is the synchronous form (submit, collect).
 * Errors and queue limits as for vif_submit / vif_score.  The per-slot frame
 * buffers are allocated by vif_create; these calls allocate nothing.
 */
int vif_submit_host(vif_ctx *ctx, const void *ref, const void *dist);
int vif_score_host(vif_ctx *ctx, const void *ref, const void *dist,
                   double out[8]);

/*
 * Batched submission (an extension of the queue above for many frames of one
 * geometry).  vif_create_batch is vif_create_ex for a context whose
 * submissions may carry up to max_batch frame pairs (1 <= max_batch <=
 * VIF_MAX_BATCH); each queue slot's device and pinned buffers are sized for
 * max_batch frames, so memory grows with it.  vif_submit_batch enqueues n
 * pairs (1 <= n <= max_batch; refs[z], dists[z] as for vif_submit) as ONE
 * slot: every kernel of the path runs once for all n frames, which amortises
 * the launches and fills the device with small frames.  The frames count as
 * n pending frames; vif_collect returns them one by one in order, and the
 * slot is free again once all n are collected.  Results are the same bits as
 * n single submissions.  VIF_EINVAL for a bad n, NULL arrays or frames, or
 * when all VIF_QUEUE_DEPTH slots are in use.  vif_submit is a batch of one;
 * vif_create and vif_create_ex make contexts with max_batch = 1.  The frames
 * stay valid until their vif_collect returns.  Allocates nothing.
 */
#define VIF_MAX_BATCH 16
vif_ctx *vif_create_batch(int w, int h, int bpc, const vif_options *opt,
                          int max_batch);
int vif_submit_batch(vif_ctx *ctx, int n, const void *const *refs,
                     const void *const *dists);

/*
 * Row strips: one device's share of a frame split by rows across devices.
 * Every device scores its strip of every frame with no exchange; the host
 * concatenates the strips' row sums and adds them as for a whole frame.  The
 * bits are the whole frame's: the device returns each row's fp32 sum and the
 * host adds the rows top to bottom (ADR-1422 "float_vif_sycl computes the
 * CPU's arithmetic ...", Decision), so whole rows of disjoint strips,
 * concatenated, are the frame's rows; and each strip recomputes the rows
 * around it that its own rows depend on, mirroring only at the frame's top
 * and bottom (ADR-1444 "float_vif_hip runs the arithmetic of the CUDA twin
 * ...", Decision: indices reflect at the plane's edges, then clamp).
 *
 * A strip is scale-0 rows [row0, row1) of a w x h frame: row0 a multiple
 * of 8 with 0 <= row0 < row1, row1 a multiple of 8 or h, row1 <= h.  It
 * owns rows [row0 >> s, row1 >> s) of scale s's plane (floor(h / 2^s) rows;
 * the strip ending at h owns the plane's remaining rows), so strips that
 * tile [0, h) tile every scale's rows.
 *
 * vif_strip_geometry -- host only.  Writes info[0] = in0, the first frame
 * row the strip reads, max(0, row0 - 24); info[1] = the rows it reads,
 * min(h, row1 + 13) - in0; and for s = 0..3 info[2 + 2s] = the first row
 * it owns at scale s (in the frame's plane), info[3 + 2s] = how many (0 is
 * possible at the coarse scales of a strip of fewer than 8 rows at the
 * bottom).  The reach is 20 rows up and 13 down, the filter radii 8/4/2/1
 * carried through the decimations; in0 is rounded down to a multiple of 8
 * so that every scale's planes start on one of the frame's rows.  VIF_OK,
 * or VIF_EINVAL for a geometry vif_create refuses or a strip outside the
 * rules above.
 *
 * vif_create_strip -- vif_create_batch for the strip of w x h frames.  The
 * frames given to vif_score, vif_submit, vif_submit_batch and
 * vif_submit_host are the strip's input rows: info[1] rows of w samples,
 * starting at frame row info[0] (a pointer to the frame plus in0 * w
 * samples).  The outputs cover the strip's own rows only: out[8] and
 * vif_get_sums are the scores and fp32 sums of those rows, and
 * vif_get_row_sums returns them scale by scale (scale 0's own rows, then
 * scale 1's, ...; the total own rows is its return value).  A strip of
 * [0, h) is the whole frame: the same as vif_create_batch.
 *
 * vif_scores_from_rows -- host only.  The outputs of a w x h frame from
 * its row sums: rows holds, for scale s = 0..3 and each row y of that scale
 * (h >> s rows), the pair n_y, d_y -- what vif_get_row_sums returns for a
 * whole frame, or the strips' vif_get_row_sums concatenated scale by scale
 * in row order.  Each scale's rows are added top to bottom in fp32, and
 * out[8] is formed as vif_score forms it, with the options opt (NULL: the
 * defaults; skip_scale0 ignores scale 0's rows).  sums (may be NULL)
 * receives the eight fp32 sums.  VIF_OK or VIF_EINVAL.
 */
#define VIF_STRIP_INFO 10
int vif_strip_geometry(int w, int h, int row0, int row1,
                       int info[VIF_STRIP_INFO]);
vif_ctx *vif_create_strip(int w, int h, int bpc, const vif_options *opt,
                          int max_batch, int row0, int row1);
int vif_scores_from_rows(int w, int h, const vif_options *opt,
                         const float *rows, double out[8], float sums[8]);

/*
 * vif_score_noalloc -- vif_score for callers that cannot allocate memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Scores one frame pair of w x h samples at bpc bits with the
 * options opt (NULL: the defaults) on the HIP stream hip_stream (a
 * hipStream_t as void*; NULL: the default stream), without a context and
 * without allocating anything: no device, pinned or host allocation, no
 * library routine that allocates.  The kernels are vif_score's and so are
 * the bits of out.  ref, dist and out as for vif_score (device frames, host
 * out).
 * The buffers the kernels need beyond the frames and out (pyramid planes,
 * the row sums' hand-over words, row sums, the eight sums) live in one
 * array of VIF_NOALLOC_SCRATCH bytes of device memory that the library
 * defines: each
 * device the call runs on holds it from the call's first use there until
 * the process ends.  A frame whose buffers do not fit is refused with
 * VIF_ETOOBIG before any work is queued (3840x2160 needs about 22 MiB).
 * Synchronous: returns once out is written (it synchronises hip_stream).
 * Every call on one device shares that device's array, which keeps the last
 * call's contents: calls that overlap on one device (two streams or two host
 * threads at once) race, and the caller must serialise them.  VIF_EINVAL for
 * bad arguments (as vif_create_ex and vif_score), VIF_EHIP for a HIP error.
 */
#define VIF_NOALLOC_SCRATCH (32L << 20)
int vif_score_noalloc(int w, int h, int bpc, const vif_options *opt,
                      const void *ref, const void *dist, void *hip_stream,
                      double out[8]);

/* vif_pending -- frames submitted and not yet collected (or VIF_EINVAL). */
int vif_pending(const vif_ctx *ctx);

/* vif_destroy -- frees everything the context owns.  NULL is a no-op. */
void vif_destroy(vif_ctx *ctx);

/*
 * vif_set_stream -- the caller's HIP stream (a hipStream_t passed as void*,
 * e.g. torch's current stream; NULL = the default stream, the initial
 * setting): work queued on it before vif_submit (say, the copy that fills
 * the frames) is ordered before the frame's kernels, which run on the
 * streams the context owns (one per queue slot).  Those are blocking
 * streams, so work on the default stream orders itself; a non-NULL stream
 * costs one event per submission.
 * The caller keeps the stream alive while the context uses it.  VIF_EINVAL
 * while frames are pending.
 */
int vif_set_stream(vif_ctx *ctx, void *hip_stream);

/*
 * vif_get_sums -- the fp32 per-scale sums of the last frame returned by
 * vif_score or vif_collect: N_0, D_0, N_1, D_1, N_2, D_2, N_3, D_3 (the
 * eight per-scale sums of the pages' debug output, ADR-1422, Consequences).
 * VIF_EINVAL if no frame has been returned yet.
 */
int vif_get_sums(const vif_ctx *ctx, float sums[8]);

/*
 * vif_get_debug -- the values of the pages' debug mode (ADR-1444,
 * Consequences, and ADR-1422, Consequences: fifteen values, the scores with
 * the frame ratio and all eight per-scale sums) for the last frame returned
 * by vif_score or vif_collect, as doubles:
 *   [0..3]   vif_scale0..3, as in out[0..3] (floors applied)
 *   [4]      vif, the frame ratio num / den (out[6])
 *   [5], [6] num and den (out[4], out[5])
 *   [7..14]  N_0, D_0, N_1, D_1, N_2, D_2, N_3, D_3 (the fp32 sums, exact
 *            in fp64)
 * VIF_EINVAL if no frame has been returned yet.
 */
#define VIF_NDEBUG 15
int vif_get_debug(const vif_ctx *ctx, double out[VIF_NDEBUG]);

/*
 * vif_get_row_sums -- the per-row fp32 sums of the last frame returned by
 * vif_score or vif_collect, as they came back from the device: for scale
 * 0..3, for row y = 0..h_s-1, the pair (n_y, d_y) (a strip context: its own
 * rows of each scale, see vif_create_strip).  rows must hold 2 * capacity
 * floats.  Returns the total number of rows (h_0 + h_1 + h_2 + h_3, plane
 * heights halving with floor) when capacity is large enough, else
 * VIF_EINVAL.
 */
int vif_get_row_sums(const vif_ctx *ctx, float *rows, int capacity);

/*
 * vif_taps -- the fp32 Gaussian taps of scale 0..3 that the context passes
 * to its kernels (ADR-1422, Decision: taps computed on the host at run time
 * and passed by value).  Writes N floats to taps (room for VIF_MAX_TAPS)
 * and returns N (17, 9, 5 or 3), or VIF_EINVAL.  Host only; needs no GPU.
 */
int vif_taps(int scale, float *taps);

/*
 * vif_set_profiling -- kinds is a bit mask of kernel kinds (bit k = kind k
 * of vif_get_kernel_times; 0xf = all, 0 = off).  Frames submitted from
 * then on record a pair of HIP events around each launch of those kinds on
 * the stream it runs on, and vif_collect accumulates their durations (a
 * small cost per event).  Every call resets the totals; VIF_EINVAL while
 * frames are pending.
 */
int vif_set_profiling(vif_ctx *ctx, int kinds);

/*
 * vif_get_kernel_times -- accumulated kernel durations in milliseconds and
 * launch counts since profiling was enabled, one entry per kernel kind:
 *   0..3  the kernel of scale s (filter, statistic, next scale's planes,
 *         and the ordered row sums: each row's fp32 sum is carried from tile
 *         to tile inside the kernel)
 * A launch here is one kind's work for one submission (all its frames): one
 * kernel launch, or several in a row for a plane more than 65535 tiles of
 * 112 columns wide, timed as one.
 * ms and launches hold at least `capacity` entries (either may be NULL).
 * Returns the number of kinds (4) or VIF_EINVAL.
 */
int vif_get_kernel_times(const vif_ctx *ctx, double *ms, long *launches,
                         int capacity);

/* vif_errno -- the last error code set on the calling thread (0 if none). */
int vif_errno(void);

/* vif_strerror -- a static description of an error code.  For VIF_EHIP it
 * names the HIP error of the calling thread's last failure. */
const char *vif_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* VIF_H */
