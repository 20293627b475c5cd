// fssim_api.cpp -- the C ABI of include/fssim.h: context, launch sequence
// and the host mean.
//
// Each submission (one frame, or a batch of up to max_batch frames that
// every kernel processes in one launch) takes a slot of a three-slot ring;
// each slot has its own stream, decimated planes, SSIM maps and pinned row
// sums, sized for max_batch frames, so consecutive submissions overlap on
// the device.  A submission is three launches on its slot's stream
// (decimation when the factor is above 1, the SSIM stage, the ordered row
// sums, which store straight into the slot's pinned host buffer) and one
// event.  Collect waits for the event and adds the rows top
// to bottom in fp64; the mean is that sum divided by the pixel count in
// fp64, rounded to fp32 (Research-2130 "float_ssim decimation on the SYCL
// device", Sources and Findings: iqa_ssim() returns the frame mean as an
// fp32 value).
#include <hip/hip_runtime_api.h>

#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/fssim.h"
#include "../../include/vif.h"
#include "fssim_internal.h"
#include "hip_util.h"
#include "vif_status.h"

namespace {

using vifk::DeviceScope;
using vifk::destroy_event;

constexpr int kDepth = FSSIM_QUEUE_DEPTH;
constexpr int kKinds = 3; // decimation, SSIM stage, row sums

struct FSlot {
  float *dref = nullptr;  // decimated planes (factor > 1)
  float *ddist = nullptr;
  float *map = nullptr;   // column-major, pitch map_pitch(h')
  double *rows_host = nullptr; // pinned, written by the row-sum kernel
  hipStream_t stream = nullptr;
  hipEvent_t submitted = nullptr;
  hipEvent_t done = nullptr;
  hipEvent_t prof[kKinds][2] = {};
  int prof_mask = 0;
  int n = 0;     // frames of the submission in this slot
  int taken = 0; // of those, frames already collected
};

} // namespace

struct fssim_ctx {
  int w = 0, h = 0, bpc = 0;
  int f = 1, ow = 0, oh = 0, pitch = 0;
  int device = 0;
  float in_scale = 1.0f;
  float tap = 1.0f;
  fssimk::SsimArgs sa = {};
  hipStream_t stream = nullptr;
  FSlot slots[kDepth];
  int max_batch = 1;
  size_t plane = 0;          // floats of one decimated plane
  size_t map_elems = 0;      // floats of one frame's map
  long head = 0, tail = 0;   // submitted / collected frames
  long shead = 0, stail = 0; // submitted / released slots
  double *last_rows = nullptr;
  bool have = false;
  int last_slot = 0, last_z = 0; // where the last collected frame lives
  int prof_mask = 0;
  double kernel_ms[kKinds] = {};
  long kernel_launches[kKinds] = {};
};

namespace {

void free_all(fssim_ctx *c) {
  for (FSlot &sl : c->slots) {
    if (sl.dref)
      (void)hipFree(sl.dref);
    if (sl.ddist)
      (void)hipFree(sl.ddist);
    if (sl.map)
      (void)hipFree(sl.map);
    if (sl.rows_host)
      (void)hipHostFree(sl.rows_host);
    destroy_event(sl.submitted);
    destroy_event(sl.done);
    for (auto &p : sl.prof) {
      destroy_event(p[0]);
      destroy_event(p[1]);
    }
    if (sl.stream)
      (void)hipStreamDestroy(sl.stream);
  }
  std::free(c->last_rows);
}

bool bad_frame_ptrs(const fssim_ctx *ctx, const void *ref, const void *dist) {
  if (ref == nullptr || dist == nullptr)
    return true;
  return ctx->bpc != 8 && ((reinterpret_cast<uintptr_t>(ref) |
                            reinterpret_cast<uintptr_t>(dist)) & 1u);
}

int submit_frames(fssim_ctx *ctx, int n, const void *const *refs,
                  const void *const *dists) {
  FSlot &sl = ctx->slots[ctx->shead % kDepth];
  hipStream_t st = sl.stream;
  hipError_t e = hipSuccess;
  if (ctx->stream != nullptr) {
    e = hipEventRecord(sl.submitted, ctx->stream);
    if (e == hipSuccess)
      e = hipStreamWaitEvent(st, sl.submitted, 0);
  }
  sl.prof_mask = ctx->prof_mask;
  auto timed = [&](int k, auto &&launch) {
    const bool on = (sl.prof_mask >> k) & 1;
    if (e == hipSuccess && on)
      e = hipEventRecord(sl.prof[k][0], st);
    if (e == hipSuccess)
      e = launch();
    if (e == hipSuccess && on)
      e = hipEventRecord(sl.prof[k][1], st);
  };
  fssimk::FramePair in = {};
  for (int z = 0; z < n; ++z) {
    in.a[z] = refs[z];
    in.b[z] = dists[z];
  }
  if (ctx->f > 1) {
    timed(0, [&] {
      return fssimk::launch_decimate(ctx->bpc, in, n, ctx->w, ctx->h, ctx->f,
                                     ctx->tap, ctx->in_scale, ctx->ow,
                                     ctx->oh, sl.dref, sl.ddist, st);
    });
    fssimk::FramePair dec = {};
    for (int z = 0; z < n; ++z) {
      dec.a[z] = sl.dref + z * ctx->plane;
      dec.b[z] = sl.ddist + z * ctx->plane;
    }
    timed(1, [&] {
      return fssimk::launch_ssim(0, dec, n, ctx->ow, ctx->oh, 1.0f, ctx->sa,
                                 sl.map, st);
    });
  } else {
    timed(1, [&] {
      return fssimk::launch_ssim(ctx->bpc, in, n, ctx->w, ctx->h,
                                 ctx->in_scale, ctx->sa, sl.map, st);
    });
  }
  timed(2, [&] {
    return fssimk::launch_ssim_rowsum(sl.map, n, ctx->ow, ctx->oh,
                                      sl.rows_host, st);
  });
  if (e == hipSuccess)
    e = hipEventRecord(sl.done, st);
  if (e != hipSuccess)
    return vifk::status_from_hip(e);
  sl.n = n;
  sl.taken = 0;
  ctx->shead += 1;
  ctx->head += n;
  return vifk::set_status(VIF_OK);
}

int collect_frame(fssim_ctx *ctx, double out[2]) {
  const int si = static_cast<int>(ctx->stail % kDepth);
  FSlot &sl = ctx->slots[si];
  const int z = sl.taken;
  hipError_t e = hipEventSynchronize(sl.done);
  if (e != hipSuccess) {
    ctx->tail += sl.n - z;
    sl.taken = sl.n;
    ctx->stail += 1;
    return vifk::status_from_hip(e);
  }
  if (z == 0) {
    for (int k = 0; k < kKinds; ++k) {
      if (!((sl.prof_mask >> k) & 1) || (k == 0 && ctx->f == 1))
        continue;
      float ms = 0.0f;
      if (hipEventElapsedTime(&ms, sl.prof[k][0], sl.prof[k][1]) ==
          hipSuccess) {
        ctx->kernel_ms[k] += ms;
        ctx->kernel_launches[k] += 1;
      }
    }
  }
  std::memcpy(ctx->last_rows,
              sl.rows_host + static_cast<size_t>(z) * ctx->pitch,
              sizeof(double) * ctx->oh);
  double total = 0.0;
  for (int y = 0; y < ctx->oh; ++y)
    total = total + ctx->last_rows[y];
  const double n = static_cast<double>(ctx->ow) * static_cast<double>(ctx->oh);
  ctx->have = true;
  ctx->last_slot = si;
  ctx->last_z = z;
  ctx->tail += 1;
  sl.taken = z + 1;
  if (sl.taken == sl.n)
    ctx->stail += 1;
  out[0] = static_cast<double>(static_cast<float>(total / n));
  out[1] = static_cast<double>(ctx->f);
  return vifk::set_status(VIF_OK);
}

// The slot of the last returned frame, when its buffers are still its own
// (nothing submitted since).
const FSlot *last_slot(const fssim_ctx *ctx) {
  if (ctx == nullptr || !ctx->have || ctx->head != ctx->tail)
    return nullptr;
  return &ctx->slots[ctx->last_slot];
}

} // namespace

extern "C" {

__attribute__((visibility("default"))) fssim_ctx *fssim_create(int w, int h,
                                                               int bpc) {
  return fssim_create_batch(w, h, bpc, 1);
}

__attribute__((visibility("default"))) fssim_ctx *
fssim_create_batch(int w, int h, int bpc, int max_batch) {
  if (w < 1 || h < 1 || static_cast<long>(w) * h > FSSIM_MAX_PIXELS ||
      (bpc != 8 && bpc != 10 && bpc != 12 && bpc != 16) ||
      fssimk::factor(w, h) > FSSIM_MAX_FACTOR || max_batch < 1 ||
      max_batch > FSSIM_MAX_BATCH) {
    vifk::set_status(VIF_EINVAL);
    return nullptr;
  }
  fssim_ctx *c = new (std::nothrow) fssim_ctx;
  if (c == nullptr) {
    vifk::set_status(VIF_ENOMEM);
    return nullptr;
  }
  c->w = w;
  c->h = h;
  c->bpc = bpc;
  c->max_batch = max_batch;
  c->f = fssimk::factor(w, h);
  c->ow = c->f > 1 ? fssimk::decimated_size(w, c->f) : w;
  c->oh = c->f > 1 ? fssimk::decimated_size(h, c->f) : h;
  c->pitch = fssimk::map_pitch(c->oh);
  c->in_scale = bpc == 8 ? 1.0f : bpc == 10 ? 0.25f : bpc == 12 ? 0.0625f
                                                                : 0.00390625f;
  c->tap = fssimk::box_tap(c->f);
  c->sa = fssimk::make_ssim_args();
  hipError_t e = hipSuccess;
  // the kernel reads t[min(k, 10-k)]: the taps must be symmetric bit for bit
  for (int k = 0; k < fssimk::kTaps; ++k)
    if (std::memcmp(&c->sa.t[k], &c->sa.t[fssimk::kTaps - 1 - k],
                    sizeof(float)) != 0)
      e = hipErrorInvalidValue;
  if (e == hipSuccess)
    e = hipGetDevice(&c->device);
  c->last_rows = static_cast<double *>(std::calloc(c->oh, sizeof(double)));
  if (c->last_rows == nullptr && e == hipSuccess)
    e = hipErrorOutOfMemory;
  c->plane = static_cast<size_t>(c->ow) * c->oh;
  c->map_elems = static_cast<size_t>(c->ow) * c->pitch;
  const size_t nb = static_cast<size_t>(max_batch);
  for (FSlot &sl : c->slots) {
    if (c->f > 1) {
      if (e == hipSuccess)
        e = hipMalloc(reinterpret_cast<void **>(&sl.dref), nb * c->plane * 4);
      if (e == hipSuccess)
        e = hipMalloc(reinterpret_cast<void **>(&sl.ddist), nb * c->plane * 4);
    }
    if (e == hipSuccess)
      e = hipMalloc(reinterpret_cast<void **>(&sl.map), nb * c->map_elems * 4);
    // the row sums also read the map's padding rows (and drop them)
    if (e == hipSuccess)
      e = hipMemset(sl.map, 0, nb * c->map_elems * 4);
    if (e == hipSuccess)
      e = hipHostMalloc(reinterpret_cast<void **>(&sl.rows_host),
                        nb * sizeof(double) * c->pitch, hipHostMallocCoherent);
    if (e == hipSuccess)
      e = hipEventCreateWithFlags(&sl.submitted, hipEventDisableTiming);
    if (e == hipSuccess)
      e = hipEventCreateWithFlags(&sl.done, hipEventDisableTiming);
    if (e == hipSuccess)
      e = hipStreamCreate(&sl.stream); // blocking: ordered with the default
                                       // stream
    for (auto &p : sl.prof)
      for (hipEvent_t &ev : p)
        if (e == hipSuccess)
          e = hipEventCreate(&ev);
  }
  if (e == hipSuccess)
    e = hipDeviceSynchronize(); // the memsets are done before any frame
  if (e != hipSuccess) {
    free_all(c);
    delete c;
    if (e == hipErrorInvalidValue)
      vifk::set_status(VIF_EINVAL);
    else
      vifk::status_from_hip(e);
    return nullptr;
  }
  vifk::set_status(VIF_OK);
  return c;
}

__attribute__((visibility("default"))) void fssim_destroy(fssim_ctx *ctx) {
  if (ctx == nullptr)
    return;
  {
    DeviceScope scope(ctx->device);
    if (ctx->head != ctx->tail)
      for (FSlot &sl : ctx->slots)
        (void)hipStreamSynchronize(sl.stream);
    free_all(ctx);
  }
  delete ctx;
}

__attribute__((visibility("default"))) int fssim_geometry(const fssim_ctx *ctx,
                                                          int geom[3]) {
  if (ctx == nullptr || geom == nullptr)
    return vifk::set_status(VIF_EINVAL);
  geom[0] = ctx->f;
  geom[1] = ctx->ow;
  geom[2] = ctx->oh;
  return vifk::set_status(VIF_OK);
}

__attribute__((visibility("default"))) int fssim_set_stream(fssim_ctx *ctx,
                                                            void *hip_stream) {
  if (ctx == nullptr || ctx->head != ctx->tail)
    return vifk::set_status(VIF_EINVAL);
  ctx->stream = static_cast<hipStream_t>(hip_stream);
  return vifk::set_status(VIF_OK);
}

__attribute__((visibility("default"))) int
fssim_submit(fssim_ctx *ctx, const void *ref, const void *dist) {
  if (ctx == nullptr || bad_frame_ptrs(ctx, ref, dist) ||
      ctx->shead - ctx->stail >= kDepth)
    return vifk::set_status(VIF_EINVAL);
  DeviceScope scope(ctx->device);
  if (scope.error() != hipSuccess)
    return vifk::status_from_hip(scope.error());
  return submit_frames(ctx, 1, &ref, &dist);
}

__attribute__((visibility("default"))) int
fssim_submit_batch(fssim_ctx *ctx, int n, const void *const *refs,
                   const void *const *dists) {
  if (ctx == nullptr || refs == nullptr || dists == nullptr || n < 1 ||
      n > ctx->max_batch || ctx->shead - ctx->stail >= kDepth)
    return vifk::set_status(VIF_EINVAL);
  for (int z = 0; z < n; ++z)
    if (bad_frame_ptrs(ctx, refs[z], dists[z]))
      return vifk::set_status(VIF_EINVAL);
  DeviceScope scope(ctx->device);
  if (scope.error() != hipSuccess)
    return vifk::status_from_hip(scope.error());
  return submit_frames(ctx, n, refs, dists);
}

__attribute__((visibility("default"))) int fssim_collect(fssim_ctx *ctx,
                                                         double out[2]) {
  if (ctx == nullptr || out == nullptr || ctx->head == ctx->tail)
    return vifk::set_status(VIF_EINVAL);
  DeviceScope scope(ctx->device);
  if (scope.error() != hipSuccess)
    return vifk::status_from_hip(scope.error());
  return collect_frame(ctx, out);
}

__attribute__((visibility("default"))) int fssim_pending(const fssim_ctx *ctx) {
  if (ctx == nullptr)
    return vifk::set_status(VIF_EINVAL);
  vifk::set_status(VIF_OK);
  return static_cast<int>(ctx->head - ctx->tail);
}

__attribute__((visibility("default"))) int
fssim_score(fssim_ctx *ctx, const void *ref, const void *dist, double out[2]) {
  if (ctx == nullptr || out == nullptr || bad_frame_ptrs(ctx, ref, dist) ||
      ctx->head != ctx->tail)
    return vifk::set_status(VIF_EINVAL);
  DeviceScope scope(ctx->device);
  if (scope.error() != hipSuccess)
    return vifk::status_from_hip(scope.error());
  const int rc = submit_frames(ctx, 1, &ref, &dist);
  if (rc != VIF_OK)
    return rc;
  return collect_frame(ctx, out);
}

__attribute__((visibility("default"))) int
fssim_get_row_sums(const fssim_ctx *ctx, double *rows, int capacity) {
  if (last_slot(ctx) == nullptr || rows == nullptr || capacity < ctx->oh)
    return vifk::set_status(VIF_EINVAL);
  std::memcpy(rows, ctx->last_rows, sizeof(double) * ctx->oh);
  vifk::set_status(VIF_OK);
  return ctx->oh;
}

__attribute__((visibility("default"))) long
fssim_get_map(fssim_ctx *ctx, float *map, long capacity) {
  const FSlot *sl = last_slot(ctx);
  const long n = sl ? static_cast<long>(ctx->ow) * ctx->oh : 0;
  if (sl == nullptr || map == nullptr || capacity < n)
    return vifk::set_status(VIF_EINVAL);
  DeviceScope scope(ctx->device);
  if (scope.error() != hipSuccess)
    return vifk::status_from_hip(scope.error());
  std::vector<float> cm;
  try {
    cm.resize(static_cast<size_t>(ctx->ow) * ctx->pitch);
  } catch (...) {
    return vifk::set_status(VIF_ENOMEM);
  }
  const hipError_t e =
      hipMemcpy(cm.data(), sl->map + ctx->last_z * ctx->map_elems,
                cm.size() * 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess)
    return vifk::status_from_hip(e);
  for (int y = 0; y < ctx->oh; ++y)
    for (int x = 0; x < ctx->ow; ++x)
      map[static_cast<size_t>(y) * ctx->ow + x] =
          cm[static_cast<size_t>(x) * ctx->pitch + y];
  vifk::set_status(VIF_OK);
  return n;
}

__attribute__((visibility("default"))) long
fssim_get_planes(fssim_ctx *ctx, float *planes, long capacity) {
  const FSlot *sl = last_slot(ctx);
  const long n = sl ? static_cast<long>(ctx->ow) * ctx->oh : 0;
  if (sl == nullptr || ctx->f == 1 || planes == nullptr || capacity < 2 * n)
    return vifk::set_status(VIF_EINVAL);
  DeviceScope scope(ctx->device);
  if (scope.error() != hipSuccess)
    return vifk::status_from_hip(scope.error());
  hipError_t e = hipMemcpy(planes, sl->dref + ctx->last_z * ctx->plane,
                           static_cast<size_t>(n) * 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess)
    e = hipMemcpy(planes + n, sl->ddist + ctx->last_z * ctx->plane,
                  static_cast<size_t>(n) * 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess)
    return vifk::status_from_hip(e);
  vifk::set_status(VIF_OK);
  return 2 * n;
}

__attribute__((visibility("default"))) int fssim_taps(float taps[FSSIM_TAPS]) {
  if (taps == nullptr)
    return vifk::set_status(VIF_EINVAL);
  fssimk::window_taps(taps);
  vifk::set_status(VIF_OK);
  return FSSIM_TAPS;
}

__attribute__((visibility("default"))) int fssim_set_profiling(fssim_ctx *ctx,
                                                               int kinds) {
  if (ctx == nullptr || kinds < 0 || kinds > (1 << kKinds) - 1 ||
      ctx->head != ctx->tail)
    return vifk::set_status(VIF_EINVAL);
  for (int k = 0; k < kKinds; ++k) {
    ctx->kernel_ms[k] = 0.0;
    ctx->kernel_launches[k] = 0;
  }
  ctx->prof_mask = kinds;
  return vifk::set_status(VIF_OK);
}

__attribute__((visibility("default"))) int
fssim_get_kernel_times(const fssim_ctx *ctx, double *ms, long *launches,
                       int capacity) {
  if (ctx == nullptr || capacity < kKinds)
    return vifk::set_status(VIF_EINVAL);
  for (int k = 0; k < kKinds; ++k) {
    if (ms)
      ms[k] = ctx->kernel_ms[k];
    if (launches)
      launches[k] = ctx->kernel_launches[k];
  }
  vifk::set_status(VIF_OK);
  return kKinds;
}

} // extern "C"
