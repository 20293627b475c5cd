// vif_api.cpp -- the C ABI of include/vif.h: context, launch sequence, one
// read-back and the host sums.
//
// Per frame, on the context's stream: for s = 0..3 the per-scale kernel
// (filter, statistic, terms, next scale's planes) and the row-sum kernel of
// that scale; then one device-to-host copy of every row sum (two floats per
// row per scale) into pinned memory, and the host adds the rows of each
// scale top to bottom in fp32 (ADR-1422 "float_vif_sycl computes the CPU's
// arithmetic ...", Decision).  The scores are fp64 quotients of the fp32
// sums; num and den add the four scales in order in fp64.
#include <hip/hip_runtime_api.h>

#include <cstdlib>
#include <cstring>
#include <new>

#include "../../include/vif.h"
#include "vif_internal.h"
#include "vif_status.h"

using vifk::kScales;

struct vif_ctx {
  int w = 0, h = 0, bpc = 0;
  int device = 0;
  hipStream_t stream = nullptr;
  vifk::ScaleGeom geom[kScales] = {};
  vifk::TapArgs taps[kScales] = {};
  float *pyr_ref[kScales] = {};  // [0] unused: scale 0 reads the frames
  float *pyr_dist[kScales] = {};
  float *terms[kScales] = {};
  float *rows_dev = nullptr;
  float *rows_host = nullptr; // pinned
  int total_rows = 0;
  int row_base[kScales] = {};
  float sums[8] = {};
  bool have_sums = false;
  int prof_mask = 0; // kernel kinds timed with events
  hipEvent_t ev[2 * 8] = {};
  double kernel_ms[8] = {};
  long kernel_launches[8] = {};
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

// Makes the context's device current for the scope of one call.
class DeviceScope {
public:
  explicit DeviceScope(int dev) {
    if (hipGetDevice(&prev_) != hipSuccess)
      prev_ = -1;
    if (prev_ != dev)
      err_ = hipSetDevice(dev);
  }
  ~DeviceScope() {
    int cur = -1;
    if (prev_ >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev_)
      (void)hipSetDevice(prev_);
  }
  hipError_t error() const { return err_; }

private:
  int prev_ = -1;
  hipError_t err_ = hipSuccess;
};

bool fault_injected_alloc() {
  const char *v = std::getenv("VIF_FAULT_INJECT");
  return v != nullptr && std::strcmp(v, "alloc") == 0;
}

void free_all(vif_ctx *c) {
  for (int s = 0; s < kScales; ++s) {
    if (c->pyr_ref[s])
      (void)hipFree(c->pyr_ref[s]);
    if (c->pyr_dist[s])
      (void)hipFree(c->pyr_dist[s]);
    if (c->terms[s])
      (void)hipFree(c->terms[s]);
  }
  if (c->rows_dev)
    (void)hipFree(c->rows_dev);
  if (c->rows_host)
    (void)hipHostFree(c->rows_host);
  for (hipEvent_t &e : c->ev)
    if (e) {
      (void)hipEventDestroy(e);
      e = nullptr;
    }
}

template <typename T> hipError_t dev_alloc(T **p, size_t elems) {
  return hipMalloc(reinterpret_cast<void **>(p), elems * sizeof(T));
}

} // namespace

extern "C" {

__attribute__((visibility("default"))) vif_ctx *vif_create(int w, int h,
                                                           int bpc) {
  if (w < VIF_MIN_SIDE || h < VIF_MIN_SIDE ||
      static_cast<long>(w) * h > VIF_MAX_PIXELS ||
      (bpc != 8 && bpc != 10 && bpc != 12 && bpc != 16)) {
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
  hipError_t e = hipGetDevice(&c->device);
  if (e != hipSuccess) {
    delete c;
    vifk::status_from_hip(e);
    return nullptr;
  }
  int ws = w, hs = h, rows = 0;
  for (int s = 0; s < kScales; ++s) {
    if (s > 0) {
      ws /= 2;
      hs /= 2;
    }
    vifk::ScaleGeom &g = c->geom[s];
    g.w = ws;
    g.h = hs;
    g.strips = (hs + vifk::kTileH - 1) / vifk::kTileH;
    g.term_elems = static_cast<size_t>(g.strips) * ws * 32;
    c->row_base[s] = rows;
    rows += hs;
    vifk::gaussian_taps(s, c->taps[s].t);
  }
  c->total_rows = rows;

  for (int s = 0; s < kScales && e == hipSuccess; ++s) {
    const size_t n = static_cast<size_t>(c->geom[s].w) * c->geom[s].h;
    if (s > 0) {
      e = dev_alloc(&c->pyr_ref[s], n);
      if (e == hipSuccess)
        e = dev_alloc(&c->pyr_dist[s], n);
    }
    if (e == hipSuccess)
      e = dev_alloc(&c->terms[s], c->geom[s].term_elems);
  }
  if (e == hipSuccess)
    e = dev_alloc(&c->rows_dev, static_cast<size_t>(2) * rows);
  if (e == hipSuccess)
    e = hipHostMalloc(reinterpret_cast<void **>(&c->rows_host),
                      sizeof(float) * 2 * rows, hipHostMallocDefault);
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
    free_all(ctx);
  }
  delete ctx;
}

__attribute__((visibility("default"))) int vif_set_stream(vif_ctx *ctx,
                                                          void *hip_stream) {
  if (ctx == nullptr)
    return vifk::set_status(VIF_EINVAL);
  ctx->stream = static_cast<hipStream_t>(hip_stream);
  return vifk::set_status(VIF_OK);
}

__attribute__((visibility("default"))) int
vif_score(vif_ctx *ctx, const void *ref, const void *dist, double out[8]) {
  if (ctx == nullptr || ref == nullptr || dist == nullptr || out == nullptr)
    return vifk::set_status(VIF_EINVAL);
  if (ctx->bpc != 8 && ((reinterpret_cast<uintptr_t>(ref) |
                         reinterpret_cast<uintptr_t>(dist)) & 1u))
    return vifk::set_status(VIF_EINVAL);
  DeviceScope scope(ctx->device);
  if (scope.error() != hipSuccess)
    return vifk::status_from_hip(scope.error());
  hipStream_t st = ctx->stream;
  hipError_t e = hipSuccess;
  // events ev[2k], ev[2k+1] bracket kernel kind k (0..3 scale kernels,
  // 4..7 row sums) when bit k of prof_mask is set
  auto mark = [&](int kind, int edge) {
    if ((ctx->prof_mask >> kind) & 1 && e == hipSuccess)
      e = hipEventRecord(ctx->ev[2 * kind + edge], st);
  };
  for (int s = 0; s < kScales && e == hipSuccess; ++s) {
    const void *in_ref = s == 0 ? ref : ctx->pyr_ref[s];
    const void *in_dist = s == 0 ? dist : ctx->pyr_dist[s];
    float *nref = s + 1 < kScales ? ctx->pyr_ref[s + 1] : nullptr;
    float *ndist = s + 1 < kScales ? ctx->pyr_dist[s + 1] : nullptr;
    const vifk::TapArgs &nt = ctx->taps[s + 1 < kScales ? s + 1 : s];
    mark(s, 0);
    if (e == hipSuccess)
      e = vifk::launch_scale(s, ctx->bpc, in_ref, in_dist, ctx->geom[s],
                             ctx->taps[s], nt, ctx->terms[s], nref, ndist, st);
    mark(s, 1);
    mark(4 + s, 0);
    if (e == hipSuccess)
      e = vifk::launch_rowsum(ctx->terms[s], ctx->geom[s],
                              ctx->rows_dev + 2 * ctx->row_base[s], st);
    mark(4 + s, 1);
  }
  if (e == hipSuccess)
    e = hipMemcpyAsync(ctx->rows_host, ctx->rows_dev,
                       sizeof(float) * 2 * ctx->total_rows,
                       hipMemcpyDeviceToHost, st);
  if (e == hipSuccess)
    e = hipStreamSynchronize(st);
  if (e != hipSuccess)
    return vifk::status_from_hip(e);

  for (int k = 0; k < 8; ++k) {
    float ms = 0.0f;
    if ((ctx->prof_mask >> k) & 1 &&
        hipEventElapsedTime(&ms, ctx->ev[2 * k], ctx->ev[2 * k + 1]) ==
            hipSuccess) {
      ctx->kernel_ms[k] += ms;
      ctx->kernel_launches[k] += 1;
    }
  }

  float N[kScales], D[kScales];
  for (int s = 0; s < kScales; ++s) {
    const float *r = ctx->rows_host + 2 * ctx->row_base[s];
    float n = 0.0f, d = 0.0f;
    for (int y = 0; y < ctx->geom[s].h; ++y) {
      n = n + r[2 * y];
      d = d + r[2 * y + 1];
    }
    N[s] = n;
    D[s] = d;
    ctx->sums[2 * s] = n;
    ctx->sums[2 * s + 1] = d;
  }
  ctx->have_sums = true;
  for (int s = 0; s < kScales; ++s)
    out[s] = static_cast<double>(N[s]) / static_cast<double>(D[s]);
  double num = static_cast<double>(N[0]) + static_cast<double>(N[1]);
  num = num + static_cast<double>(N[2]);
  num = num + static_cast<double>(N[3]);
  double den = static_cast<double>(D[0]) + static_cast<double>(D[1]);
  den = den + static_cast<double>(D[2]);
  den = den + static_cast<double>(D[3]);
  out[4] = num;
  out[5] = den;
  out[6] = num / den;
  out[7] = 0.0;
  return vifk::set_status(VIF_OK);
}

__attribute__((visibility("default"))) int vif_get_sums(const vif_ctx *ctx,
                                                        float sums[8]) {
  if (ctx == nullptr || sums == nullptr || !ctx->have_sums)
    return vifk::set_status(VIF_EINVAL);
  std::memcpy(sums, ctx->sums, sizeof(ctx->sums));
  return vifk::set_status(VIF_OK);
}

__attribute__((visibility("default"))) int
vif_get_row_sums(const vif_ctx *ctx, float *rows, int capacity) {
  if (ctx == nullptr || rows == nullptr || !ctx->have_sums ||
      capacity < ctx->total_rows)
    return vifk::set_status(VIF_EINVAL);
  std::memcpy(rows, ctx->rows_host, sizeof(float) * 2 * ctx->total_rows);
  vifk::set_status(VIF_OK);
  return ctx->total_rows;
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
  if (ctx == nullptr || kinds < 0 || kinds > 0xff)
    return vifk::set_status(VIF_EINVAL);
  for (int k = 0; k < 8; ++k) {
    ctx->kernel_ms[k] = 0.0;
    ctx->kernel_launches[k] = 0;
  }
  if (kinds != 0) {
    DeviceScope scope(ctx->device);
    for (hipEvent_t &ev : ctx->ev) {
      if (ev == nullptr) {
        hipError_t e = hipEventCreate(&ev);
        if (e != hipSuccess)
          return vifk::status_from_hip(e);
      }
    }
  }
  ctx->prof_mask = kinds;
  return vifk::set_status(VIF_OK);
}

__attribute__((visibility("default"))) int
vif_get_kernel_times(const vif_ctx *ctx, double *ms, long *launches,
                     int capacity) {
  if (ctx == nullptr || capacity < 8)
    return vifk::set_status(VIF_EINVAL);
  for (int k = 0; k < 8; ++k) {
    if (ms)
      ms[k] = ctx->kernel_ms[k];
    if (launches)
      launches[k] = ctx->kernel_launches[k];
  }
  vifk::set_status(VIF_OK);
  return 8;
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
  default:
    return "unknown error code";
  }
}

} // extern "C"
