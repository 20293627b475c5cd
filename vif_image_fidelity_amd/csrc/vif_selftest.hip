// vif_selftest.hip -- device-math gates: run the scoring kernels' own device
// functions (vif_device_math.h) over caller arrays so tests can compare the
// device's roundings with the host's bit for bit (ADR-1444 "float_vif_hip
// runs the arithmetic of the CUDA twin ...", Decision and Consequences).
#include <hip/hip_runtime.h>

#include "../../include/vif_selftest.h"
#include "vif_device_math.h"
#include "vif_internal.h"
#include "vif_status.h"

namespace {

constexpr int kBlock = 256;

__global__ void fp64_gate_kernel(const float *__restrict__ a,
                                 const float *__restrict__ b, double nsq,
                                 long n, double *__restrict__ sum,
                                 double *__restrict__ quot,
                                 float *__restrict__ rnum,
                                 float *__restrict__ rden) {
  const long i = static_cast<long>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= n)
    return;
  const double s = static_cast<double>(b[i]) + nsq;
  const double q = static_cast<double>(a[i]) / s;
  sum[i] = s;
  quot[i] = q;
  rnum[i] = static_cast<float>(1.0 + q);
  rden[i] = static_cast<float>(1.0 + static_cast<double>(a[i]) / nsq);
}

__global__ void div32_in_range_kernel(const float *__restrict__ a,
                                      const float *__restrict__ b, long n,
                                      float *__restrict__ q) {
  const long i = static_cast<long>(blockIdx.x) * kBlock + threadIdx.x;
  if (i < n)
    q[i] = vifk::div_in_range_f32(a[i], b[i]);
}

__global__ void div32_kernel(const float *__restrict__ a,
                             const float *__restrict__ b, long n,
                             float *__restrict__ q) {
  const long i = static_cast<long>(blockIdx.x) * kBlock + threadIdx.x;
  if (i < n)
    q[i] = a[i] / b[i];
}

__global__ void log2_kernel(const float *__restrict__ x, long n,
                            float *__restrict__ y) {
  const long i = static_cast<long>(blockIdx.x) * kBlock + threadIdx.x;
  if (i < n)
    y[i] = vifk::log2_poly(x[i]);
}

template <bool kPow2>
__global__ void ratios_kernel(const float *__restrict__ a,
                              const float *__restrict__ sv, long n,
                              vifk::StatArgs sa, float *__restrict__ num,
                              float *__restrict__ den) {
  const long i = static_cast<long>(blockIdx.x) * kBlock + threadIdx.x;
  if (i < n) {
    num[i] = vifk::num_ratio<kPow2>(a[i], sv[i], sa.nsq);
    den[i] = vifk::den_ratio<kPow2>(a[i], sa);
  }
}

template <bool kPow2>
__global__ void statistic_kernel(const float *__restrict__ mu1,
                                 const float *__restrict__ mu2,
                                 const float *__restrict__ xx,
                                 const float *__restrict__ yy,
                                 const float *__restrict__ xy, long n,
                                 vifk::StatArgs sa, float *__restrict__ num,
                                 float *__restrict__ den) {
  const long i = static_cast<long>(blockIdx.x) * kBlock + threadIdx.x;
  if (i < n) {
    float a, b;
    vifk::pixel_terms<kPow2>(mu1[i], mu2[i], xx[i], yy[i], xy[i], sa, a, b);
    num[i] = a;
    den[i] = b;
  }
}

// The filter's instruction pair at a chosen occupancy: each round, every
// one of 8 accumulators takes a multiply by a uniform (SGPR) factor and a
// VGPR add, twice (a += t0 * b, then b += t1 * a): 32 VALU instructions,
// 8 independent chains.  The dynamic LDS the launch reserves caps the
// blocks per CU; it is never touched.
__global__ __launch_bounds__(kBlock) void valu_rate_kernel(
    float *__restrict__ out, float t0, float t1, int iters) {
  float a[8], b[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = static_cast<float>(threadIdx.x + k);
    b[k] = static_cast<float>(k + 1);
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      a[k] = a[k] + t0 * b[k];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      b[k] = b[k] + t1 * a[k];
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    s = s + (a[k] + b[k]);
  out[static_cast<long>(blockIdx.x) * kBlock + threadIdx.x] = s;
}

dim3 grid_for(long n) {
  return dim3(static_cast<unsigned>((n + kBlock - 1) / kBlock));
}

int finish(hipStream_t s) {
  hipError_t e = hipGetLastError();
  if (e == hipSuccess)
    e = hipStreamSynchronize(s);
  return vifk::status_from_hip(e);
}

// grid.x is limited to 2^31-1 blocks; n up to 2^38 stays well inside.
bool bad_n(long n) { return n < 0 || n > (1L << 36); }

// The statistic's options as the library checks them.
bool bad_stat_options(double nsq, double gain_limit) {
  vifk::OptionValues o{};
  o.sigma_nsq = nsq;
  o.enhn_gain_limit = gain_limit;
  o.kernelscale = 1.0;
  return !vifk::options_valid(o);
}

} // namespace

extern "C" {

__attribute__((visibility("default"))) int
vif_selftest_fp64(const float *a, const float *b, double nsq, long n,
                  double *sum, double *quot, float *rnum, float *rden,
                  void *stream) {
  if (bad_n(n) || (n > 0 && (!a || !b || !sum || !quot || !rnum || !rden)))
    return vifk::set_status(VIF_EINVAL);
  if (n == 0)
    return vifk::set_status(VIF_OK);
  hipStream_t s = static_cast<hipStream_t>(stream);
  fp64_gate_kernel<<<grid_for(n), kBlock, 0, s>>>(a, b, nsq, n, sum, quot,
                                                  rnum, rden);
  return finish(s);
}

__attribute__((visibility("default"))) int
vif_selftest_div32(const float *a, const float *b, long n, float *q,
                   void *stream) {
  if (bad_n(n) || (n > 0 && (!a || !b || !q)))
    return vifk::set_status(VIF_EINVAL);
  if (n == 0)
    return vifk::set_status(VIF_OK);
  hipStream_t s = static_cast<hipStream_t>(stream);
  div32_kernel<<<grid_for(n), kBlock, 0, s>>>(a, b, n, q);
  return finish(s);
}

__attribute__((visibility("default"))) int
vif_selftest_div32_in_range(const float *a, const float *b, long n, float *q,
                            void *stream) {
  if (bad_n(n) || (n > 0 && (!a || !b || !q)))
    return vifk::set_status(VIF_EINVAL);
  if (n == 0)
    return vifk::set_status(VIF_OK);
  hipStream_t s = static_cast<hipStream_t>(stream);
  div32_in_range_kernel<<<grid_for(n), kBlock, 0, s>>>(a, b, n, q);
  return finish(s);
}

__attribute__((visibility("default"))) int
vif_selftest_log2(const float *x, long n, float *y, void *stream) {
  if (bad_n(n) || (n > 0 && (!x || !y)))
    return vifk::set_status(VIF_EINVAL);
  if (n == 0)
    return vifk::set_status(VIF_OK);
  hipStream_t s = static_cast<hipStream_t>(stream);
  log2_kernel<<<grid_for(n), kBlock, 0, s>>>(x, n, y);
  return finish(s);
}

__attribute__((visibility("default"))) int
vif_selftest_ratios(const float *a, const float *sv, double nsq, long n,
                    float *num, float *den, void *stream) {
  if (bad_n(n) || bad_stat_options(nsq, 100.0) ||
      (n > 0 && (!a || !sv || !num || !den)))
    return vifk::set_status(VIF_EINVAL);
  if (n == 0)
    return vifk::set_status(VIF_OK);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const vifk::StatArgs sa = vifk::make_stat_args(nsq, 100.0);
  if (sa.inv_nsq != 0.0)
    ratios_kernel<true><<<grid_for(n), kBlock, 0, s>>>(a, sv, n, sa, num, den);
  else
    ratios_kernel<false><<<grid_for(n), kBlock, 0, s>>>(a, sv, n, sa, num,
                                                        den);
  return finish(s);
}

__attribute__((visibility("default"))) int
vif_selftest_statistic(const float *mu1, const float *mu2, const float *xx,
                       const float *yy, const float *xy, long n, double nsq,
                       double gain_limit, float *num, float *den,
                       void *stream) {
  if (bad_n(n) || bad_stat_options(nsq, gain_limit) ||
      (n > 0 && (!mu1 || !mu2 || !xx || !yy || !xy || !num || !den)))
    return vifk::set_status(VIF_EINVAL);
  if (n == 0)
    return vifk::set_status(VIF_OK);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const vifk::StatArgs sa = vifk::make_stat_args(nsq, gain_limit);
  if (sa.inv_nsq != 0.0)
    statistic_kernel<true><<<grid_for(n), kBlock, 0, s>>>(
        mu1, mu2, xx, yy, xy, n, sa, num, den);
  else
    statistic_kernel<false><<<grid_for(n), kBlock, 0, s>>>(
        mu1, mu2, xx, yy, xy, n, sa, num, den);
  return finish(s);
}

__attribute__((visibility("default"))) int
vif_selftest_carry_wait(int *raised, float *row, void *stream) {
  if (raised == nullptr || row == nullptr)
    return vifk::set_status(VIF_EINVAL);
  // a 224 x 16 frame of zeros: two tile columns, one strip; only column 1
  // runs, so the words it waits for never carry the launch's tag
  constexpr int kW = 224, kH = 16;
  vifk::ScaleGeom g{};
  g.w = kW;
  g.h = kH;
  g.strips = 1;
  g.ntx = 2;
  vifk::TapArgs taps[2];
  vifk::gaussian_taps(0, taps[0].t);
  vifk::gaussian_taps(1, taps[1].t);
  const vifk::StatArgs stat = vifk::make_stat_args(2.0, 100.0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char *frame = nullptr;
  float *next = nullptr, *rows = nullptr;
  unsigned long long *carry = nullptr;
  int *err = nullptr;
  hipError_t e = hipMalloc(&frame, kW * kH);
  if (e == hipSuccess)
    e = hipMalloc(&next, sizeof(float) * (kW / 2) * (kH / 2) * 2);
  if (e == hipSuccess)
    e = hipMalloc(&rows, sizeof(float) * 2 * kH);
  if (e == hipSuccess)
    e = hipMalloc(&carry, sizeof(unsigned long long) * vifk::kSeq);
  if (e == hipSuccess)
    e = hipMalloc(&err, sizeof(int));
  if (e == hipSuccess)
    e = hipMemsetAsync(frame, 0, kW * kH, s);
  if (e == hipSuccess)
    e = hipMemsetAsync(carry, 0, sizeof(unsigned long long) * vifk::kSeq, s);
  if (e == hipSuccess)
    e = hipMemsetAsync(err, 0, sizeof(int), s);
  if (e == hipSuccess)
    e = hipMemsetAsync(rows, 0, sizeof(float) * 2 * kH, s);
  if (e == hipSuccess) {
    vifk::ScaleIO io{};
    io.in_ref[0] = frame;
    io.in_dist[0] = frame;
    io.next_ref = next;
    io.next_dist = next + (kW / 2) * (kH / 2);
    io.carry = carry;
    io.carry_tag = 7;
    io.strips = 1;
    io.ntx = 2;
    io.rows = rows;
    io.rows_stride = 2 * kH;
    io.err = err;
    e = vifk::launch_scale0_column(io, g, taps[0], taps[1], stat, 1, s);
  }
  if (e == hipSuccess)
    e = hipStreamSynchronize(s);
  if (e == hipSuccess)
    e = hipMemcpy(raised, err, sizeof(int), hipMemcpyDeviceToHost);
  if (e == hipSuccess)
    e = hipMemcpy(row, rows, sizeof(float), hipMemcpyDeviceToHost);
  (void)hipFree(frame);
  (void)hipFree(next);
  (void)hipFree(rows);
  (void)hipFree(carry);
  (void)hipFree(err);
  return vifk::status_from_hip(e);
}

__attribute__((visibility("default"))) int
vif_selftest_valu_rate(int waves_per_simd, int iters, long blocks, float *out,
                       double *ms, void *stream) {
  if (waves_per_simd < 3 || waves_per_simd > 8 || iters < 1 ||
      iters > (1 << 24) || blocks < 1 || blocks > (1L << 24) ||
      out == nullptr || ms == nullptr)
    return vifk::set_status(VIF_EINVAL);
  // 160 KiB of LDS per CU: a block reserving a whole number of KiB under a
  // 1/w share of 159 KiB lets w blocks (one wave per SIMD each) fit, not
  // w + 1 (exactly 32 KiB, for w = 5, fits only four times)
  const size_t lds = static_cast<size_t>(159 / waves_per_simd) * 1024;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess)
    e = hipEventCreate(&e1);
  if (e == hipSuccess)
    e = hipEventRecord(e0, s);
  if (e == hipSuccess) {
    valu_rate_kernel<<<dim3(static_cast<unsigned>(blocks)), kBlock, lds, s>>>(
        out, 1.0e-7f, -1.0e-7f, iters);
    e = hipGetLastError();
  }
  if (e == hipSuccess)
    e = hipEventRecord(e1, s);
  if (e == hipSuccess)
    e = hipEventSynchronize(e1);
  float t = 0.0f;
  if (e == hipSuccess)
    e = hipEventElapsedTime(&t, e0, e1);
  if (e == hipSuccess)
    *ms = t;
  if (e0)
    (void)hipEventDestroy(e0);
  if (e1)
    (void)hipEventDestroy(e1);
  return vifk::status_from_hip(e);
}

__attribute__((visibility("default"))) int
vif_selftest_stage_loads(const void *const *ref, const void *const *dist,
                         int n, int w, int h, int bpc, unsigned *out,
                         void *stream) {
  if (ref == nullptr || dist == nullptr || out == nullptr || n < 1 ||
      n > vifk::kMaxBatch || w < VIF_MIN_SIDE || h < VIF_MIN_SIDE ||
      static_cast<long>(w) * h > VIF_MAX_PIXELS ||
      (bpc != 8 && bpc != 10 && bpc != 12 && bpc != 16))
    return vifk::set_status(VIF_EINVAL);
  vifk::ScaleGeom g{};
  g.w = w;
  g.h = h;
  g.strips = (h + vifk::kTileH - 1) / vifk::kTileH;
  g.ntx = (w + vifk::kTileW - 1) / vifk::kTileW;
  vifk::ScaleIO io{};
  // 8 samples per load where the scale-0 kernel would take them
  const uintptr_t align = bpc == 8 ? 8 : 16;
  bool vec = w % 8 == 0;
  for (int z = 0; z < n; ++z) {
    if (ref[z] == nullptr || dist[z] == nullptr)
      return vifk::set_status(VIF_EINVAL);
    io.in_ref[z] = ref[z];
    io.in_dist[z] = dist[z];
    vec = vec && reinterpret_cast<uintptr_t>(ref[z]) % align == 0 &&
          reinterpret_cast<uintptr_t>(dist[z]) % align == 0;
  }
  io.vec_in = vec ? 1 : 0;
  io.strips = g.strips;
  io.ntx = g.ntx;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = vifk::launch_stage_probe(bpc, io, n, g, out, s);
  if (e != hipSuccess)
    return vifk::status_from_hip(e);
  return finish(s);
}

} // extern "C"
