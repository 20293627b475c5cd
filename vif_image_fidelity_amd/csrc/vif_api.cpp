// vif_api.cpp -- the C ABI of include/vif.h: context, launch sequence, one
// read-back per frame and the host sums.
//
// Every submission (one frame, or a batch of up to max_batch frames that
// each kernel processes in one launch, its grid running over the strips of
// every frame) has a slot of a three-slot ring, and every slot its own
// stream and buffers (pyramid planes, the row sums' tile-to-tile hand-over
// words, and its row sums in pinned host memory, each sized for max_batch
// frames).  The slot's stream runs one kernel per scale; each does the
// filter, the statistic, the next scale's planes and the ordered row sums,
// carrying each row's fp32 sum from tile to tile.  The row sums go straight
// into the host buffer, two floats per row per scale: one read-back per
// frame with no copy call (ADR-1422 "float_vif_sycl computes the CPU's
// arithmetic ...", Decision: the row sums come back in one transfer and the
// host adds them).
// Frames in host memory are first copied into the slot's own frame buffers
// on the slot's stream (vif_submit_host).
// Consecutive frames rotate over the slots, so one frame's small scales
// overlap the next frame's scale 0, which fills the GPU.  When one scale-0
// kernel covers the GPU twice over, consecutive frames' scale-0 kernels run
// one after the other (a stream wait on the previous frame's scale-0
// event): two of them side by side gain nothing, and each launch's duration
// then is its own.  A submission is five runtime calls (four launches, one
// event), plus an event and that stream wait when the scale-0 kernels are
// ordered (and a launch more per scale for every 65535 tile columns beyond
// the first: see launch_scale).
//
// The slot streams are blocking streams, so they are ordered after work on
// the default stream (where a caller typically fills the frames); a caller
// stream set with vif_set_stream is joined with an event instead.
//
// vif_collect adds the rows of each scale top to bottom in fp32 on the host.
// The scores are fp64 quotients of the fp32 sums; num and den add the four
// scales in order in fp64.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <new>

#include "../../include/vif.h"
#include "vif_internal.h"
#include "hip_util.h"
#include "vif_status.h"

using vifk::kScales;

namespace {

using vifk::DeviceScope;
using vifk::destroy_event;

constexpr int kDepth = VIF_QUEUE_DEPTH;

constexpr int kKinds = kScales; // the scale kernels 0..3

struct Slot {
  float *pyr_ref[kScales] = {};   // [0] unused: scale 0 reads the frames;
  float *pyr_dist[kScales] = {};  // max_batch planes each, plane_elems apart
  void *frame_ref = nullptr;      // device copies of host frames
  void *frame_dist = nullptr;
  unsigned long long *carry[kScales] = {}; // row sums between tiles
  float *rows_host = nullptr;     // pinned, written by the kernels
  int *err_host = nullptr;        // pinned, raised by a carry wait that
                                  // gave up
  hipStream_t stream = nullptr;   // owned: all of the slot's work
  hipEvent_t submitted = nullptr; // on the caller's stream
  hipEvent_t done = nullptr;      // on the slot's stream, after scale 3
  hipEvent_t s0_end = nullptr;    // on the slot's stream, after scale 0
  hipEvent_t s0_done = nullptr;   // the event after this submission's scale
                                  // 0: s0_end, or the timing event there
  hipEvent_t prof[kKinds][2] = {};
  int prof_mask = 0; // kinds timed for the frame in this slot
  int n = 0;         // frames of the submission in this slot
  int taken = 0;     // of those, frames already collected
};

} // namespace

struct vif_ctx {
  int w = 0, h = 0, bpc = 0;
  int device = 0;
  vif_options opt = {};
  vifk::StatArgs stat = {};
  hipStream_t stream = nullptr; // caller's stream (NULL: the default stream)
  vifk::ScaleGeom geom[kScales] = {};
  vifk::TapArgs taps[kScales] = {};
  Slot slots[kDepth];
  int max_batch = 1;                   // frames one submission may carry
  size_t plane_elems[kScales] = {};    // floats per frame, pyramid plane
  size_t carry_words[kScales] = {};    // hand-over words per frame
  int total_rows = 0;             // rows of the planes, all scales
  int row_base[kScales] = {};
  // the rows the context reports: scale s's planes' rows [own0[s],
  // own0[s] + nown[s]) (all of them for a whole frame; a strip's own rows
  // for a strip context, whose planes start at input row in0 of the frame)
  int in0 = 0;
  int own0[kScales] = {};
  int nown[kScales] = {};
  int own_base[kScales] = {};
  int own_rows = 0;
  bool order_scale0 = false; // consecutive frames' scale-0 kernels ordered
  unsigned carry_tag = 0;    // tag of the last submission's carries
  long head = 0, tail = 0;   // submitted / collected frame counts
  long shead = 0, stail = 0; // submitted / released slot counts
  float sums[8] = {};
  double last_out[8] = {};
  float *last_rows = nullptr; // the last collected frame's own row sums
  bool have_sums = false;
  int prof_mask = 0;
  double kernel_ms[kKinds] = {};
  long kernel_launches[kKinds] = {};
};

namespace vifk {

namespace {
thread_local int t_status = VIF_OK;
thread_local hipError_t t_hip = hipSuccess;
} // namespace

int set_status(int code, hipError_t hip) {
  t_status = code;
  t_hip = hip;
  return code;
}

int status_from_hip(hipError_t e) {
  if (e == hipSuccess)
    return set_status(VIF_OK);
  if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation)
    return set_status(VIF_ENOMEM, e);
  return set_status(VIF_EHIP, e);
}

} // namespace vifk

namespace {

bool fault_injected_alloc() {
  const char *v = std::getenv("VIF_FAULT_INJECT");
  return v != nullptr && std::strcmp(v, "alloc") == 0;
}

void free_all(vif_ctx *c) {
  for (Slot &sl : c->slots) {
    for (int s = 0; s < kScales; ++s) {
      if (sl.pyr_ref[s])
        (void)hipFree(sl.pyr_ref[s]);
      if (sl.pyr_dist[s])
        (void)hipFree(sl.pyr_dist[s]);
      if (sl.carry[s])
        (void)hipFree(sl.carry[s]);
    }
    if (sl.err_host)
      (void)hipHostFree(sl.err_host);
    if (sl.frame_ref)
      (void)hipFree(sl.frame_ref);
    if (sl.frame_dist)
      (void)hipFree(sl.frame_dist);
    if (sl.rows_host)
      (void)hipHostFree(sl.rows_host);
    destroy_event(sl.submitted);
    destroy_event(sl.done);
    destroy_event(sl.s0_end);
    for (auto &p : sl.prof) {
      destroy_event(p[0]);
      destroy_event(p[1]);
    }
    if (sl.stream)
      (void)hipStreamDestroy(sl.stream);
  }
  std::free(c->last_rows);
}

template <typename T> hipError_t dev_alloc(T **p, size_t elems) {
  return hipMalloc(reinterpret_cast<void **>(p), elems * sizeof(T));
}

// Enqueues n frames (1 <= n <= max_batch) into the next slot: each kernel
// runs once for all n frames.
int submit_frames(vif_ctx *ctx, int n, const void *const *refs,
                  const void *const *dists) {
  Slot &sl = ctx->slots[ctx->shead % kDepth];
  hipStream_t st = sl.stream;
  hipError_t e = hipSuccess;
  // the slot's previous frames are ordered before these on its stream;
  // work on the default stream is ordered before them by the blocking stream
  if (ctx->stream != nullptr) {
    e = hipEventRecord(sl.submitted, ctx->stream);
    if (e == hipSuccess)
      e = hipStreamWaitEvent(st, sl.submitted, 0);
  }
  // consecutive submissions' scale-0 kernels run one after the other when
  // each fills the GPU (the small scales and row sums of one submission
  // still overlap the next one's scale 0)
  if (e == hipSuccess && ctx->order_scale0 && ctx->shead > 0)
    e = hipStreamWaitEvent(st, ctx->slots[(ctx->shead - 1) % kDepth].s0_done,
                           0);
  sl.prof_mask = ctx->prof_mask;
  for (int s = 0; s < kScales && e == hipSuccess; ++s) {
    vifk::ScaleIO io = {};
    for (int z = 0; z < n; ++z) {
      io.in_ref[z] = s == 0 ? refs[z] : sl.pyr_ref[s] + z * ctx->plane_elems[s];
      io.in_dist[z] =
          s == 0 ? dists[z] : sl.pyr_dist[s] + z * ctx->plane_elems[s];
    }
    if (s + 1 < kScales) {
      io.next_ref = sl.pyr_ref[s + 1];
      io.next_dist = sl.pyr_dist[s + 1];
      io.next_stride = ctx->plane_elems[s + 1];
    }
    // the row sums are chained across each row's tiles inside the kernel:
    // a fresh tag per submission marks this submission's hand-over words
    if (s == 0)
      ctx->carry_tag = ctx->carry_tag + 1 == 0 ? 1 : ctx->carry_tag + 1;
    io.carry = sl.carry[s];
    io.carry_tag = ctx->carry_tag;
    io.strips = ctx->geom[s].strips;
    io.ntx = ctx->geom[s].ntx;
    io.rows = sl.rows_host + 2 * ctx->row_base[s];
    io.rows_stride = static_cast<size_t>(2) * ctx->total_rows;
    io.err = sl.err_host;
    if (s == 0) {
      // 8 samples per load: rows start on 8-sample boundaries and the
      // planes are aligned to 8 samples' bytes
      const uintptr_t align = ctx->bpc == 8 ? 8 : 16;
      bool vec = ctx->w % 8 == 0;
      for (int z = 0; z < n; ++z)
        vec = vec && reinterpret_cast<uintptr_t>(refs[z]) % align == 0 &&
              reinterpret_cast<uintptr_t>(dists[z]) % align == 0;
      io.vec_in = vec ? 1 : 0;
    }
    const vifk::TapArgs &nt = ctx->taps[s + 1 < kScales ? s + 1 : s];
    const bool timed = (sl.prof_mask >> s) & 1;
    if (timed)
      e = hipEventRecord(sl.prof[s][0], st);
    if (e == hipSuccess)
      e = vifk::launch_scale(s, ctx->bpc, io, n, ctx->geom[s], ctx->taps[s],
                             nt, ctx->stat, st);
    if (e == hipSuccess && timed)
      e = hipEventRecord(sl.prof[s][1], st);
    // one event after scale 0 orders the next submission's: the timing
    // event when scale 0 is timed (a second record right after it would
    // delay the slot's next kernel once more)
    if (e == hipSuccess && s == 0 && ctx->order_scale0) {
      sl.s0_done = timed ? sl.prof[0][1] : sl.s0_end;
      if (!timed)
        e = hipEventRecord(sl.s0_end, st);
    }
  }
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

int submit_frame(vif_ctx *ctx, const void *ref, const void *dist) {
  return submit_frames(ctx, 1, &ref, &dist);
}

// Enqueues one frame whose planes are in host memory: two copies into the
// slot's frame buffers on the slot's stream, then the frame itself.  The
// slot's previous frame read those buffers earlier on the same stream.
int submit_host_frame(vif_ctx *ctx, const void *ref, const void *dist) {
  Slot &sl = ctx->slots[ctx->shead % kDepth];
  const size_t bytes = static_cast<size_t>(ctx->w) * ctx->geom[0].h *
                       (ctx->bpc == 8 ? 1 : 2);
  hipError_t e = hipMemcpyAsync(sl.frame_ref, ref, bytes,
                                hipMemcpyHostToDevice, sl.stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(sl.frame_dist, dist, bytes, hipMemcpyHostToDevice,
                       sl.stream);
  if (e != hipSuccess)
    return vifk::status_from_hip(e);
  return submit_frame(ctx, sl.frame_ref, sl.frame_dist);
}

// Waits for the oldest pending frame and writes its outputs.  A slot is
// released once every frame of its submission has been collected.
int collect_frame(vif_ctx *ctx, double out[8]) {
  Slot &sl = ctx->slots[ctx->stail % kDepth];
  const int z = sl.taken;
  hipError_t e = hipEventSynchronize(sl.done);
  if (e != hipSuccess) {
    // the submission is lost; keep the ring consistent
    ctx->tail += sl.n - z;
    sl.taken = sl.n;
    ctx->stail += 1;
    return vifk::status_from_hip(e);
  }
  if (*static_cast<volatile int *>(sl.err_host) != 0) {
    // a wait for a row-sum carry gave up: the submission's sums are void
    *static_cast<volatile int *>(sl.err_host) = 0;
    ctx->tail += sl.n - z;
    sl.taken = sl.n;
    ctx->stail += 1;
    return vifk::set_status(VIF_EHIP, hipErrorLaunchTimeOut);
  }
  if (z == 0) {
    for (int k = 0; k < kKinds; ++k) {
      if (!((sl.prof_mask >> k) & 1))
        continue;
      float ms = 0.0f;
      if (hipEventElapsedTime(&ms, sl.prof[k][0], sl.prof[k][1]) ==
          hipSuccess) {
        ctx->kernel_ms[k] += ms;
        ctx->kernel_launches[k] += 1;
      }
    }
  }
  // the own rows of each scale, in scale order
  const float *rows =
      sl.rows_host + static_cast<size_t>(z) * 2 * ctx->total_rows;
  for (int s = 0; s < kScales; ++s)
    std::memcpy(ctx->last_rows + 2 * ctx->own_base[s],
                rows + 2 * (ctx->row_base[s] + ctx->own0[s]),
                sizeof(float) * 2 * ctx->nown[s]);
  // a skipped scale 0 contributes nothing: its rows read 0 (the kernels
  // still build the pyramid from it)
  if (ctx->opt.skip_scale0 != 0)
    std::memset(ctx->last_rows, 0, sizeof(float) * 2 * ctx->nown[0]);
  vifk::scores_from_rows(ctx->last_rows, ctx->nown, ctx->opt, out,
                         ctx->sums);
  ctx->have_sums = true;
  ctx->tail += 1;
  sl.taken = z + 1;
  if (sl.taken == sl.n)
    ctx->stail += 1;
  std::memcpy(ctx->last_out, out, sizeof(ctx->last_out));
  return vifk::set_status(VIF_OK);
}

bool bad_frame_ptrs(const vif_ctx *ctx, const void *ref, const void *dist) {
  if (ref == nullptr || dist == nullptr)
    return true;
  return ctx->bpc != 8 && ((reinterpret_cast<uintptr_t>(ref) |
                            reinterpret_cast<uintptr_t>(dist)) & 1u);
}

} // namespace

extern "C" {

__attribute__((visibility("default"))) void
vif_default_options(vif_options *opt) {
  if (opt == nullptr)
    return;
  std::memset(opt, 0, sizeof(*opt));
  opt->sigma_nsq = 2.0;
  opt->enhn_gain_limit = 100.0;
  opt->kernelscale = 1.0;
}

__attribute__((visibility("default"))) vif_ctx *vif_create(int w, int h,
                                                           int bpc) {
  return vif_create_ex(w, h, bpc, nullptr);
}

__attribute__((visibility("default"))) vif_ctx *
vif_create_ex(int w, int h, int bpc, const vif_options *opt) {
  return vif_create_batch(w, h, bpc, opt, 1);
}

__attribute__((visibility("default"))) vif_ctx *
vif_create_batch(int w, int h, int bpc, const vif_options *opt,
                 int max_batch) {
  return vif_create_strip(w, h, bpc, opt, max_batch, 0, h);
}

__attribute__((visibility("default"))) vif_ctx *
vif_create_strip(int w, int h, int bpc, const vif_options *opt,
                 int max_batch, int row0, int row1) {
  vif_options o;
  vif_default_options(&o);
  if (opt != nullptr)
    o = *opt;
  vifk::StripRows sr;
  if (w < VIF_MIN_SIDE || h < VIF_MIN_SIDE ||
      static_cast<long>(w) * h > VIF_MAX_PIXELS ||
      (bpc != 8 && bpc != 10 && bpc != 12 && bpc != 16) ||
      !vifk::options_ok(o) || max_batch < 1 || max_batch > VIF_MAX_BATCH ||
      !vifk::strip_rows(h, row0, row1, &sr)) {
    vifk::set_status(VIF_EINVAL);
    return nullptr;
  }
  if (fault_injected_alloc()) {
    vifk::set_status(VIF_ENOMEM);
    return nullptr;
  }
  vif_ctx *c = new (std::nothrow) vif_ctx;
  if (c == nullptr) {
    vifk::set_status(VIF_ENOMEM);
    return nullptr;
  }
  c->w = w;
  c->h = h;
  c->bpc = bpc;
  c->opt = o;
  c->max_batch = max_batch;
  c->stat = vifk::make_stat_args(o.sigma_nsq, o.enhn_gain_limit);
  hipError_t e = hipGetDevice(&c->device);
  if (e != hipSuccess) {
    delete c;
    vifk::status_from_hip(e);
    return nullptr;
  }
  // the planes hold the input rows: the whole frame, or a strip's rows
  // [in0, in0 + in_rows), a multiple of 8 rows below the frame's top, so
  // that scale s's planes start at the frame's row in0 >> s
  c->in0 = sr.in0;
  int ws = w, hs = sr.in_rows, rows = 0, own = 0;
  for (int s = 0; s < kScales; ++s) {
    if (s > 0) {
      ws /= 2;
      hs /= 2;
    }
    vifk::ScaleGeom &g = c->geom[s];
    g.w = ws;
    g.h = hs;
    g.strips = (hs + vifk::kTileH - 1) / vifk::kTileH;
    g.ntx = (ws + vifk::kTileW - 1) / vifk::kTileW;
    c->row_base[s] = rows;
    rows += hs;
    c->own0[s] = sr.own0[s] - (sr.in0 >> s);
    c->nown[s] = sr.nown[s];
    c->own_base[s] = own;
    own += sr.nown[s];
    c->plane_elems[s] = static_cast<size_t>(ws) * hs;
    // one hand-over word per sequence and inner tile boundary of a row
    c->carry_words[s] = static_cast<size_t>(g.strips) *
                        (g.ntx > 1 ? g.ntx - 1 : 1) * vifk::kSeq;
    const int nt = vifk::gaussian_taps(s, c->taps[s].t);
    // the kernels rely on bitwise symmetric taps (see tap() there)
    for (int k = 0; k < nt; ++k)
      if (std::memcmp(&c->taps[s].t[k], &c->taps[s].t[nt - 1 - k],
                      sizeof(float)) != 0)
        e = hipErrorInvalidValue;
  }
  // order consecutive scale-0 kernels when one covers the device's resident
  // blocks at least twice: two side by side then gain nothing, and the wait
  // (a cross-stream dependency, a few tens of microseconds of host time) is
  // hidden behind the GPU.  Smaller frames leave CUs free and are host-bound,
  // so their scale-0 kernels may overlap.
  if (e == hipSuccess) {
    int resident = 0;
    e = vifk::scale0_resident_blocks(bpc, &resident);
    c->order_scale0 =
        e == hipSuccess &&
        c->geom[0].tiles() >= 2 * static_cast<size_t>(resident);
  }
  c->total_rows = rows;
  c->own_rows = own;
  c->last_rows = static_cast<float *>(
      std::calloc(static_cast<size_t>(2) * (own > 0 ? own : 1), 4));
  if (c->last_rows == nullptr)
    e = hipErrorOutOfMemory;

  const size_t nb = static_cast<size_t>(max_batch);
  for (Slot &sl : c->slots) {
    for (int s = 1; s < kScales && e == hipSuccess; ++s) {
      e = dev_alloc(&sl.pyr_ref[s], nb * c->plane_elems[s]);
      if (e == hipSuccess)
        e = dev_alloc(&sl.pyr_dist[s], nb * c->plane_elems[s]);
    }
    const size_t frame_bytes =
        static_cast<size_t>(w) * sr.in_rows * (bpc == 8 ? 1 : 2);
    if (e == hipSuccess)
      e = hipMalloc(&sl.frame_ref, frame_bytes);
    if (e == hipSuccess)
      e = hipMalloc(&sl.frame_dist, frame_bytes);
    // the hand-over words, cleared once: every submission writes its own
    // tag
    for (int s = 0; s < kScales && e == hipSuccess; ++s) {
      e = dev_alloc(&sl.carry[s], nb * c->carry_words[s]);
      if (e == hipSuccess)
        e = hipMemset(sl.carry[s], 0,
                      nb * c->carry_words[s] * sizeof(unsigned long long));
    }
    if (e == hipSuccess)
      e = hipHostMalloc(reinterpret_cast<void **>(&sl.err_host), sizeof(int),
                        hipHostMallocCoherent);
    if (e == hipSuccess)
      *sl.err_host = 0;
    // coherent pinned memory: the scale kernels' row-sum stores reach the host
    // without a copy, visible once the slot's event has completed
    if (e == hipSuccess)
      e = hipHostMalloc(reinterpret_cast<void **>(&sl.rows_host),
                        nb * sizeof(float) * 2 * rows, hipHostMallocCoherent);
    if (e == hipSuccess)
      e = hipEventCreateWithFlags(&sl.submitted, hipEventDisableTiming);
    if (e == hipSuccess)
      e = hipEventCreateWithFlags(&sl.done, hipEventDisableTiming);
    if (e == hipSuccess)
      e = hipEventCreateWithFlags(&sl.s0_end, hipEventDisableTiming);
    if (e == hipSuccess)
      e = hipStreamCreate(&sl.stream); // blocking: ordered with the default
                                       // stream
    for (auto &p : sl.prof)
      for (hipEvent_t &ev : p)
        if (e == hipSuccess)
          e = hipEventCreate(&ev);
  }
  if (e != hipSuccess) {
    free_all(c);
    delete c;
    vifk::status_from_hip(e);
    return nullptr;
  }
  vifk::set_status(VIF_OK);
  return c;
}

__attribute__((visibility("default"))) void vif_destroy(vif_ctx *ctx) {
  if (ctx == nullptr)
    return;
  {
    DeviceScope scope(ctx->device);
    if (ctx->head != ctx->tail) {
      for (Slot &sl : ctx->slots)
        (void)hipStreamSynchronize(sl.stream);
    }
    free_all(ctx);
  }
  delete ctx;
}

__attribute__((visibility("default"))) int vif_set_stream(vif_ctx *ctx,
                                                          void *hip_stream) {
  if (ctx == nullptr || ctx->head != ctx->tail)
    return vifk::set_status(VIF_EINVAL);
  ctx->stream = static_cast<hipStream_t>(hip_stream);
  return vifk::set_status(VIF_OK);
}

__attribute__((visibility("default"))) int
vif_submit(vif_ctx *ctx, const void *ref, const void *dist) {
  if (ctx == nullptr || bad_frame_ptrs(ctx, ref, dist) ||
      ctx->shead - ctx->stail >= kDepth)
    return vifk::set_status(VIF_EINVAL);
  DeviceScope scope(ctx->device);
  if (scope.error() != hipSuccess)
    return vifk::status_from_hip(scope.error());
  return submit_frame(ctx, ref, dist);
}

__attribute__((visibility("default"))) int
vif_submit_host(vif_ctx *ctx, const void *ref, const void *dist) {
  if (ctx == nullptr || bad_frame_ptrs(ctx, ref, dist) ||
      ctx->shead - ctx->stail >= kDepth)
    return vifk::set_status(VIF_EINVAL);
  DeviceScope scope(ctx->device);
  if (scope.error() != hipSuccess)
    return vifk::status_from_hip(scope.error());
  return submit_host_frame(ctx, ref, dist);
}

__attribute__((visibility("default"))) int
vif_score_host(vif_ctx *ctx, const void *ref, const void *dist,
               double out[8]) {
  if (ctx == nullptr || out == nullptr || bad_frame_ptrs(ctx, ref, dist) ||
      ctx->head != ctx->tail)
    return vifk::set_status(VIF_EINVAL);
  DeviceScope scope(ctx->device);
  if (scope.error() != hipSuccess)
    return vifk::status_from_hip(scope.error());
  const int rc = submit_host_frame(ctx, ref, dist);
  if (rc != VIF_OK)
    return rc;
  return collect_frame(ctx, out);
}

__attribute__((visibility("default"))) int
vif_submit_batch(vif_ctx *ctx, int n, const void *const *refs,
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

__attribute__((visibility("default"))) int vif_collect(vif_ctx *ctx,
                                                       double out[8]) {
  if (ctx == nullptr || out == nullptr || ctx->head == ctx->tail)
    return vifk::set_status(VIF_EINVAL);
  DeviceScope scope(ctx->device);
  if (scope.error() != hipSuccess)
    return vifk::status_from_hip(scope.error());
  return collect_frame(ctx, out);
}

__attribute__((visibility("default"))) int vif_pending(const vif_ctx *ctx) {
  if (ctx == nullptr)
    return vifk::set_status(VIF_EINVAL);
  vifk::set_status(VIF_OK);
  return static_cast<int>(ctx->head - ctx->tail);
}

__attribute__((visibility("default"))) int
vif_score(vif_ctx *ctx, const void *ref, const void *dist, double out[8]) {
  if (ctx == nullptr || out == nullptr || bad_frame_ptrs(ctx, ref, dist) ||
      ctx->head != ctx->tail)
    return vifk::set_status(VIF_EINVAL);
  DeviceScope scope(ctx->device);
  if (scope.error() != hipSuccess)
    return vifk::status_from_hip(scope.error());
  const int rc = submit_frame(ctx, ref, dist);
  if (rc != VIF_OK)
    return rc;
  return collect_frame(ctx, out);
}

__attribute__((visibility("default"))) int vif_get_sums(const vif_ctx *ctx,
                                                        float sums[8]) {
  if (ctx == nullptr || sums == nullptr || !ctx->have_sums)
    return vifk::set_status(VIF_EINVAL);
  std::memcpy(sums, ctx->sums, sizeof(ctx->sums));
  return vifk::set_status(VIF_OK);
}

__attribute__((visibility("default"))) int
vif_get_options(const vif_ctx *ctx, vif_options *opt) {
  if (ctx == nullptr || opt == nullptr)
    return vifk::set_status(VIF_EINVAL);
  *opt = ctx->opt;
  return vifk::set_status(VIF_OK);
}

__attribute__((visibility("default"))) int
vif_get_debug(const vif_ctx *ctx, double out[VIF_NDEBUG]) {
  if (ctx == nullptr || out == nullptr || !ctx->have_sums)
    return vifk::set_status(VIF_EINVAL);
  for (int s = 0; s < kScales; ++s)
    out[s] = ctx->last_out[s];
  out[4] = ctx->last_out[6];
  out[5] = ctx->last_out[4];
  out[6] = ctx->last_out[5];
  for (int k = 0; k < 2 * kScales; ++k)
    out[7 + k] = static_cast<double>(ctx->sums[k]);
  return vifk::set_status(VIF_OK);
}

__attribute__((visibility("default"))) int
vif_get_row_sums(const vif_ctx *ctx, float *rows, int capacity) {
  if (ctx == nullptr || rows == nullptr || !ctx->have_sums ||
      capacity < ctx->own_rows)
    return vifk::set_status(VIF_EINVAL);
  std::memcpy(rows, ctx->last_rows, sizeof(float) * 2 * ctx->own_rows);
  vifk::set_status(VIF_OK);
  return ctx->own_rows;
}

__attribute__((visibility("default"))) int vif_taps(int scale, float *taps) {
  if (taps == nullptr)
    return vifk::set_status(VIF_EINVAL);
  const int n = vifk::gaussian_taps(scale, taps);
  if (n < 0)
    return vifk::set_status(VIF_EINVAL);
  vifk::set_status(VIF_OK);
  return n;
}

__attribute__((visibility("default"))) int vif_set_profiling(vif_ctx *ctx,
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
vif_get_kernel_times(const vif_ctx *ctx, double *ms, long *launches,
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

__attribute__((visibility("default"))) int vif_errno(void) {
  return vifk::t_status;
}

__attribute__((visibility("default"))) const char *vif_strerror(int code) {
  switch (code) {
  case VIF_OK:
    return "success";
  case VIF_EINVAL:
    return "invalid argument (geometry, bit depth, pointer or state)";
  case VIF_ENOMEM:
    return "device or pinned host allocation failed";
  case VIF_EHIP:
    return vifk::t_hip != hipSuccess ? hipGetErrorString(vifk::t_hip)
                                     : "HIP runtime error";
  case VIF_ETOOBIG:
    return "frame needs more than vif_score_noalloc's device array "
           "(VIF_NOALLOC_SCRATCH bytes)";
  default:
    return "unknown error code";
  }
}

} // extern "C"
