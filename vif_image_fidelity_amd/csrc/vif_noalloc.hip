// vif_noalloc.hip -- vif_score_noalloc: one frame pair scored through the
// same kernels as vif_score, with every buffer beyond the caller's frames
// and outputs in one file-scope device array, so that the call allocates
// nothing (for callers that cannot allocate device or pinned memory).
//
// The array `scratch` holds, per call, the pyramid planes of scales 1..3,
// the row-sum hand-over words of the four scales (cleared at the start of
// every call), the row sums and the eight per-scale sums.
// Its device address comes from hipGetSymbolAddress, once per device with
// that device current (the array's name in host code is only a stand-in for
// the symbol); kernels receive that address.  Every call on a device uses
// the same array, so calls that overlap on one device race: the caller
// serialises them (one stream, or one host thread at a time).  The kernels
// write every word they read before reading it, except the hand-over words
// (a tile waits until its left neighbour's word carries the call's tag),
// which a small kernel clears first.
//
// The row sums stay on the device: a small kernel adds each scale's rows
// top to bottom in fp32, in the order the host adds them for vif_score
// (ADR-1422 "float_vif_sycl computes the CPU's arithmetic ...", Decision:
// one fp32 sum per row, then the rows top to bottom), and only the eight
// sums come back.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/vif.h"
#include "hip_util.h"
#include "vif_internal.h"
#include "vif_status.h"

static __device__ __align__(256) unsigned char scratch[VIF_NOALLOC_SCRATCH];

namespace vifk {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

// The device address of `scratch` on device dev (current): looked up on the
// first call on that device and kept.
hipError_t scratch_address(int dev, unsigned char **p) {
  if (dev < 0 || dev >= kMaxDevices)
    return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
      return e;
    g_scratch[dev] = ptr;
  }
  *p = static_cast<unsigned char *>(g_scratch[dev]);
  return hipSuccess;
}

size_t round256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// Offsets (bytes) of one call's buffers in the array: the pyramid planes of
// scales 1..3, the four scales' hand-over words (one run), the row sums, and
// the eight sums followed by the hand-over error word.
struct Layout {
  size_t pyr_ref[kScales], pyr_dist[kScales], carry[kScales], rows, sums;
  size_t carry_words; // all four scales'
  size_t total;
};

Layout layout(const ScaleGeom (&g)[kScales], int total_rows) {
  Layout L{};
  size_t off = 0;
  for (int s = 1; s < kScales; ++s) {
    const size_t plane = round256(sizeof(float) * g[s].w * g[s].h);
    L.pyr_ref[s] = off;
    off += plane;
    L.pyr_dist[s] = off;
    off += plane;
  }
  const size_t carry0 = off;
  for (int s = 0; s < kScales; ++s) {
    L.carry[s] = off;
    off += sizeof(unsigned long long) * g[s].strips *
           (g[s].ntx > 1 ? g[s].ntx - 1 : 1) * kSeq;
  }
  L.carry_words = (off - carry0) / sizeof(unsigned long long);
  off = carry0 + round256(off - carry0);
  L.rows = off;
  off += round256(sizeof(float) * 2 * total_rows);
  L.sums = off;
  off += round256(sizeof(float) * 8 + sizeof(int));
  L.total = off;
  return L;
}

struct SumArgs {
  const float *rows[kScales]; // 2 floats per row of scale s
  int h[kScales];
};

// Clears the hand-over words and the error word: the array's earlier
// contents are another call's (or another geometry's), and every word of
// this call must read as not yet written until its tile writes it (tag 1).
__global__ void clear_kernel(unsigned long long *carry, size_t words,
                             int *err) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       i < words; i += stride)
    carry[i] = 0ull;
  if (blockIdx.x == 0 && threadIdx.x == 0)
    *err = 0;
}

constexpr int kSumChunk = 2048; // rows per LDS chunk

// Lane k < 8 adds sequence (scale k / 2, component k % 2) top to bottom in
// fp32 from 0; the block stages each scale's rows through LDS in chunks
// with coalesced loads.
__global__ __launch_bounds__(256) void scale_sums_kernel(SumArgs a,
                                                         float *sums) {
  __shared__ float chunk[2 * kSumChunk];
  const int t = threadIdx.x;
  float acc = 0.0f;
  for (int s = 0; s < kScales; ++s) {
    const float *src = a.rows[s];
    for (int y0 = 0; y0 < a.h[s]; y0 += kSumChunk) {
      const int n = min(kSumChunk, a.h[s] - y0);
      __syncthreads();
      for (int i = t; i < 2 * n; i += blockDim.x)
        chunk[i] = src[2 * y0 + i];
      __syncthreads();
      if (t >> 1 == s)
        for (int y = 0; y < n; ++y)
          acc = acc + chunk[2 * y + (t & 1)];
    }
  }
  if (t < 2 * kScales)
    sums[t] = acc;
}

} // namespace
} // namespace vifk

extern "C" __attribute__((visibility("default"))) int
vif_score_noalloc(int w, int h, int bpc, const vif_options *opt,
                  const void *ref, const void *dist, void *hip_stream,
                  double out[8]) {
  using namespace vifk;
  vif_options o;
  vif_default_options(&o);
  if (opt != nullptr)
    o = *opt;
  if (w < VIF_MIN_SIDE || h < VIF_MIN_SIDE ||
      static_cast<long>(w) * h > VIF_MAX_PIXELS ||
      (bpc != 8 && bpc != 10 && bpc != 12 && bpc != 16) || !options_ok(o) ||
      ref == nullptr || dist == nullptr || out == nullptr ||
      (bpc != 8 && ((reinterpret_cast<uintptr_t>(ref) |
                     reinterpret_cast<uintptr_t>(dist)) & 1u)))
    return set_status(VIF_EINVAL);
  ScaleGeom g[kScales];
  TapArgs taps[kScales];
  SumArgs sa{};
  int ws = w, hs = h, rows = 0, row_base[kScales];
  for (int s = 0; s < kScales; ++s) {
    if (s > 0) {
      ws /= 2;
      hs /= 2;
    }
    g[s].w = ws;
    g[s].h = hs;
    g[s].strips = (hs + kTileH - 1) / kTileH;
    g[s].ntx = (ws + kTileW - 1) / kTileW;
    row_base[s] = rows;
    rows += hs;
    const int nt = gaussian_taps(s, taps[s].t);
    for (int k = 0; k < nt; ++k)
      if (taps[s].t[k] != taps[s].t[nt - 1 - k])
        return set_status(VIF_EINVAL);
    sa.h[s] = hs;
  }
  const Layout L = layout(g, rows);
  if (L.total > VIF_NOALLOC_SCRATCH)
    return set_status(VIF_ETOOBIG);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  unsigned char *base = nullptr;
  if (e == hipSuccess)
    e = scratch_address(dev, &base);
  if (e != hipSuccess)
    return status_from_hip(e);
  auto at = [base](size_t off) {
    return reinterpret_cast<float *>(base + off);
  };
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const StatArgs stat = make_stat_args(o.sigma_nsq, o.enhn_gain_limit);
  int *err = reinterpret_cast<int *>(at(L.sums) + 8);
  clear_kernel<<<256, 256, 0, st>>>(
      reinterpret_cast<unsigned long long *>(base + L.carry[0]),
      L.carry_words, err);
  e = hipGetLastError();
  for (int s = 0; s < kScales && e == hipSuccess; ++s) {
    ScaleIO io = {};
    io.in_ref[0] = s == 0 ? ref : at(L.pyr_ref[s]);
    io.in_dist[0] = s == 0 ? dist : at(L.pyr_dist[s]);
    if (s + 1 < kScales) {
      io.next_ref = at(L.pyr_ref[s + 1]);
      io.next_dist = at(L.pyr_dist[s + 1]);
    }
    io.carry = reinterpret_cast<unsigned long long *>(base + L.carry[s]);
    io.carry_tag = 1;
    io.strips = g[s].strips;
    io.ntx = g[s].ntx;
    io.rows = at(L.rows) + 2 * row_base[s];
    io.rows_stride = static_cast<size_t>(2) * rows;
    io.err = err;
    if (s == 0) {
      const uintptr_t align = bpc == 8 ? 8 : 16;
      io.vec_in = w % 8 == 0 &&
                  reinterpret_cast<uintptr_t>(ref) % align == 0 &&
                  reinterpret_cast<uintptr_t>(dist) % align == 0;
    }
    e = launch_scale(s, bpc, io, 1, g[s], taps[s],
                     taps[s + 1 < kScales ? s + 1 : s], stat, st);
  }
  for (int s = 0; s < kScales; ++s)
    sa.rows[s] = at(L.rows) + 2 * row_base[s];
  // (the sums kernel reads the rows the scale kernels wrote, in stream
  // order)
  if (e == hipSuccess) {
    scale_sums_kernel<<<1, 256, 0, st>>>(sa, at(L.sums));
    e = hipGetLastError();
  }
  float back[9]; // the eight sums and the error word
  if (e == hipSuccess)
    e = hipMemcpyAsync(back, at(L.sums), sizeof(back), hipMemcpyDeviceToHost,
                       st);
  if (e == hipSuccess)
    e = hipStreamSynchronize(st);
  if (e != hipSuccess)
    return status_from_hip(e);
  if (__builtin_bit_cast(int, back[8]) != 0)
    return set_status(VIF_EHIP, hipErrorLaunchTimeOut);
  scores_from_sums(back, o, out);
  return set_status(VIF_OK);
}
