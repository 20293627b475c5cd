// fssim_kernels.hip -- HIP kernels of the float SSIM feature for gfx950.
//
// Three kernels per frame pair:
//   decimate_kernel  both planes decimated by the factor f > 1: the f x f
//                    box window of tap fl32(1 / f^2) at (x*f, y*f), each
//                    product an fp32 value, summed exactly in fp64 and
//                    rounded to fp32 once (Research-2130 "float_ssim
//                    decimation on the SYCL device", Sources and Findings);
//                    decimate_pow2_kernel for factors 2, 4, 8, 16, where
//                    the same value is an integer sum times a power of two;
//   ssim_kernel      the 11-tap Gaussian window of x, y, x*x, y*y, x*y
//                    (vertical pass, then horizontal) and the per-pixel
//                    SSIM value, stored column-major;
//   rowsum_kernel    each row's values added left to right in fp64, one
//                    lane per row (the map staged through LDS), straight
//                    into the context's pinned host buffer.
// Every border index goes through the symmetric mirror of period 2n
// (Research-2130, Sources), so planes of any size >= 1 stay in bounds.
//
// Exactness of the decimation in any order.  Samples are multiples of 2^-8
// below 256; for f <= 128 the tap is at least 2^-14, so a non-zero product
// is at least 2^-22 and a multiple of 2^-45, and all products of a window
// add up to less than 256 (Research-2130, Findings).  Every partial sum of
// any subset of them is therefore a multiple of 2^-45 below 2^8, which fits
// the 53 bits of a double: each fp64 addition is exact whatever the order.
// The kernel adds each column's products over the window's rows first and
// then the columns; the result is the CPU's exact sum, and one conversion
// to fp32 (round to nearest even) gives the CPU's plane bit for bit.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>

#include "fssim_internal.h"

namespace fssimk {

// Index into [0, n) by the symmetric border of period 2n: -1 -> 0,
// -2 -> 1, n -> n-1, n+1 -> n-2, repeating for indices further out.
__device__ __forceinline__ int sym_index(int i, int n) {
  if (static_cast<unsigned>(i) < static_cast<unsigned>(n))
    return i;
  const int p = 2 * n;
  int m = i % p;
  m = m < 0 ? m + p : m;
  return m < n ? m : p - 1 - m;
}

// A sample normalised to fp32: 8-bit as it is, wider samples times 1/4,
// 1/16 or 1/256 (exact).
__device__ __forceinline__ float norm(uint8_t v, float) {
  return static_cast<float>(v);
}
__device__ __forceinline__ float norm(uint16_t v, float s) {
  return static_cast<float>(v) * s;
}
__device__ __forceinline__ float norm(float v, float) { return v; }

// Four consecutive samples from row + c.  kVec: one aligned 4- or 8-byte
// load (the host checked the alignment and that c + 3 < w); otherwise one
// load per sample, those at or beyond w read as 0 (never used).
template <bool kVec>
__device__ __forceinline__ void load4(const uint8_t *p, int c, int w,
                                      float s, float (&v)[4]) {
  if constexpr (kVec) {
    const uint32_t u = *reinterpret_cast<const uint32_t *>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = static_cast<float>((u >> (8 * j)) & 0xffu);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = c + j < w ? norm(p[j], s) : 0.0f;
  }
}

template <bool kVec>
__device__ __forceinline__ void load4(const uint16_t *p, int c, int w,
                                      float s, float (&v)[4]) {
  if constexpr (kVec) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    v[0] = norm(static_cast<uint16_t>(u.x & 0xffffu), s);
    v[1] = norm(static_cast<uint16_t>(u.x >> 16), s);
    v[2] = norm(static_cast<uint16_t>(u.y & 0xffffu), s);
    v[3] = norm(static_cast<uint16_t>(u.y >> 16), s);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = c + j < w ? norm(p[j], s) : 0.0f;
  }
}

// One block: decimated row y = y0 + blockIdx.y (planes with more rows than
// a grid's y dimension allows take several launches), decimated columns
// [x0, x1) with x0 = blockIdx.x * xpb.  Their windows (mirrored) read plane
// columns [lo, hi]; thread t covers columns a + 4t .. a + 4t + 3 with a = lo
// rounded down to a multiple of 4.
//   1. every thread adds, for each of its 4 columns, the products of the f
//      window rows (mirrored row indices are uniform in the block) into an
//      fp64 column sum, for both planes; the loads of up to kRowGroup rows
//      are all issued before the first of them is used; the sums go to LDS;
//   2. decimated pixel x adds the column sums of its f window columns
//      (mirrored) and rounds the sum to fp32 once.
constexpr int kRowGroup = 8;

template <typename InT, bool kVec>
__global__ __launch_bounds__(kDecThreads) void decimate_kernel(
    FramePair in, int w, int h, int f, float tap, float in_scale, int ow,
    int oh, int xpb, float *__restrict__ dref_all,
    float *__restrict__ ddist_all, int y0) {
  const int z = blockIdx.z; // frame of a batched launch
  const InT *__restrict__ ref = static_cast<const InT *>(in.a[z]);
  const InT *__restrict__ dist = static_cast<const InT *>(in.b[z]);
  const size_t plane = static_cast<size_t>(ow) * static_cast<size_t>(oh);
  float *__restrict__ dref = dref_all + z * plane;
  float *__restrict__ ddist = ddist_all + z * plane;
  __shared__ double cs[2][kDecSpan];
  const int t = threadIdx.x;
  const int y = y0 + static_cast<int>(blockIdx.y);
  const int half = f / 2;
  const int x0 = blockIdx.x * xpb;
  const int x1 = min(ow, x0 + xpb);
  // the f columns left of the first window cover the mirror images of the
  // columns right of the plane (which lie within f of its edge)
  const int lo = max(0, x0 * f - half - f);
  const int a = lo & ~3;
  const int hi = min(w - 1, (x1 - 1) * f - half + f - 1);
  const int c = a + 4 * t;
  double sr[4] = {0.0, 0.0, 0.0, 0.0};
  double sd[4] = {0.0, 0.0, 0.0, 0.0};
  if (c <= hi) {
    const int ry = y * f - half;
    for (int g = 0; g < f; g += kRowGroup) {
      // rows past the window load the last row again (in bounds, no
      // branch, so every load of the group is in flight at once) and add
      // +0.0, which leaves the non-negative sum as it is
      float vr[kRowGroup][4], vd[kRowGroup][4];
#pragma unroll
      for (int k = 0; k < kRowGroup; ++k) {
        const int dy = min(g + k, f - 1);
        const size_t off = static_cast<size_t>(sym_index(ry + dy, h)) *
                               static_cast<size_t>(w) +
                           static_cast<size_t>(c);
        load4<kVec>(ref + off, c, w, in_scale, vr[k]);
        load4<kVec>(dist + off, c, w, in_scale, vd[k]);
      }
#pragma unroll
      for (int k = 0; k < kRowGroup; ++k) {
        const bool in = g + k < f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float pr = in ? vr[k][j] * tap : 0.0f;
          const float pd = in ? vd[k][j] * tap : 0.0f;
          sr[j] = sr[j] + static_cast<double>(pr);
          sd[j] = sd[j] + static_cast<double>(pd);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    cs[0][4 * t + j] = sr[j];
    cs[1][4 * t + j] = sd[j];
  }
  __syncthreads();
  for (int xo = x0 + t; xo < x1; xo += kDecThreads) {
    const int cx = xo * f - half;
    double u = 0.0, v = 0.0;
    for (int dx = 0; dx < f; ++dx) {
      const int k = sym_index(cx + dx, w) - a;
      u = u + cs[0][k];
      v = v + cs[1][k];
    }
    const size_t o = static_cast<size_t>(y) * static_cast<size_t>(ow) +
                     static_cast<size_t>(xo);
    dref[o] = static_cast<float>(u);
    ddist[o] = static_cast<float>(v);
  }
}

// Power-of-two factors up to 16: the tap 2^-2k is exact and so is every
// product (a sample of at most 16 bits times a power of two), so the window
// sum is 2^-(bpc-8) * tap times the integer sum S of the raw samples.
// S <= 16^2 * 65535 < 2^24 is exact in fp32, and the scaling by a power of
// two is exact too: the decimated value is (float)S * iscale with no
// rounding at all, the same value the exact fp64 sum rounds to.  The block
// and LDS layout are those of decimate_kernel; the column sums are integers
// (8-bit samples: two columns per 32-bit add, in 16-bit halves that cannot
// carry, 16 * 255 < 2^16).
template <bool kVec>
__device__ __forceinline__ void add4(const uint8_t *p, int c, int w,
                                     uint32_t (&s)[4]) {
  if constexpr (kVec) {
    const uint32_t u = *reinterpret_cast<const uint32_t *>(p);
    s[0] += u & 0x00ff00ffu;        // columns 0 and 2
    s[1] += (u >> 8) & 0x00ff00ffu; // columns 1 and 3
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      s[j] += c + j < w ? static_cast<uint32_t>(p[j]) : 0u;
  }
}

template <bool kVec>
__device__ __forceinline__ void add4(const uint16_t *p, int c, int w,
                                     uint32_t (&s)[4]) {
  if constexpr (kVec) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    s[0] += u.x & 0xffffu;
    s[1] += u.x >> 16;
    s[2] += u.y & 0xffffu;
    s[3] += u.y >> 16;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      s[j] += c + j < w ? static_cast<uint32_t>(p[j]) : 0u;
  }
}

// Column sums of the 4 columns in natural order.
template <typename InT, bool kVec>
__device__ __forceinline__ void unpack4(const uint32_t (&s)[4],
                                        uint32_t (&o)[4]) {
  if constexpr (kVec && sizeof(InT) == 1) {
    o[0] = s[0] & 0xffffu;
    o[1] = s[1] & 0xffffu;
    o[2] = s[0] >> 16;
    o[3] = s[1] >> 16;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = s[j];
  }
}

template <typename InT, bool kVec, int F>
__global__ __launch_bounds__(kDecThreads) void decimate_pow2_kernel(
    FramePair in, int w, int h, float iscale, int ow, int oh, int xpb,
    float *__restrict__ dref_all, float *__restrict__ ddist_all, int y0) {
  constexpr int f = F;
  const int z = blockIdx.z; // frame of a batched launch
  const InT *__restrict__ ref = static_cast<const InT *>(in.a[z]);
  const InT *__restrict__ dist = static_cast<const InT *>(in.b[z]);
  const size_t plane = static_cast<size_t>(ow) * static_cast<size_t>(oh);
  float *__restrict__ dref = dref_all + z * plane;
  float *__restrict__ ddist = ddist_all + z * plane;
  __shared__ uint32_t cs[2][kDecSpan];
  const int t = threadIdx.x;
  const int y = y0 + static_cast<int>(blockIdx.y);
  const int half = f / 2;
  const int x0 = blockIdx.x * xpb;
  const int x1 = min(ow, x0 + xpb);
  const int lo = max(0, x0 * f - half - f);
  const int a = lo & ~3;
  const int hi = min(w - 1, (x1 - 1) * f - half + f - 1);
  const int c = a + 4 * t;
  uint32_t sr[4] = {0u, 0u, 0u, 0u};
  uint32_t sd[4] = {0u, 0u, 0u, 0u};
  if (c <= hi) {
    const int ry = y * f - half;
#pragma unroll
    for (int k = 0; k < F; ++k) {
      const size_t off = static_cast<size_t>(sym_index(ry + k, h)) *
                             static_cast<size_t>(w) +
                         static_cast<size_t>(c);
      add4<kVec>(ref + off, c, w, sr);
      add4<kVec>(dist + off, c, w, sd);
    }
  }
  uint32_t ur[4], ud[4];
  unpack4<InT, kVec>(sr, ur);
  unpack4<InT, kVec>(sd, ud);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    cs[0][4 * t + j] = ur[j];
    cs[1][4 * t + j] = ud[j];
  }
  __syncthreads();
  for (int xo = x0 + t; xo < x1; xo += kDecThreads) {
    const int cx = xo * f - half;
    uint32_t u = 0u, v = 0u;
#pragma unroll
    for (int dx = 0; dx < f; ++dx) {
      const int k = sym_index(cx + dx, w) - a;
      u += cs[0][k];
      v += cs[1][k];
    }
    const size_t o = static_cast<size_t>(y) * static_cast<size_t>(ow) +
                     static_cast<size_t>(xo);
    dref[o] = static_cast<float>(u) * iscale;
    ddist[o] = static_cast<float>(v) * iscale;
  }
}

// SSIM value of one pixel from its five window means: the combined formula
// of the published SSIM in fp32, in the order written, with a correctly
// rounded division (the library is built with IEEE fp32 division and no
// contraction).
__device__ __forceinline__ float ssim_value(float mu1, float mu2, float xx,
                                            float yy, float xy, float c1,
                                            float c2) {
  const float m11 = mu1 * mu1;
  const float m22 = mu2 * mu2;
  const float m12 = mu1 * mu2;
  const float s11 = xx - m11;
  const float s22 = yy - m22;
  const float s12 = xy - m12;
  const float num = (2.0f * m12 + c1) * (2.0f * s12 + c2);
  const float den = (m11 + m22 + c1) * (s11 + s22 + c2);
  return num / den;
}

// Tap k of the window: the taps are symmetric bit for bit (checked on the
// host), so t[k] and t[10-k] are read from one place and the products of a
// sample with both are one expression.
__device__ __forceinline__ float wtap(const SsimArgs &sa, int k) {
  return sa.t[k < kTaps - 1 - k ? k : kTaps - 1 - k];
}

// One block: a kTileW x kTileH tile of SSIM values.
//   1. the (kTileH+10) x (kTileW+10) input tile of both planes to LDS as
//      fp32, mirrored;
//   2. vertical passes of x, y, x*x, y*y, x*y: thread (column, half) owns
//      kTileH/2 rows; the five products of a sample are formed once per read;
//   3. the vertical results to LDS (the input tile's region);
//   4. horizontal passes, kTileW * kTileH / 256 pixels per thread, and the
//      SSIM value, stored at map[x * pitch + y].
// A window accumulator starts at its first product instead of 0 + product:
// every input is >= +0, so the product is never -0 and both are the same.
template <typename InT>
__global__ __launch_bounds__(256) void ssim_kernel(
    FramePair in, int w, int h, float in_scale, SsimArgs sa,
    float *__restrict__ map_all, int pitch, int ty0) {
  const int zf = blockIdx.z; // frame of a batched launch
  const InT *__restrict__ px = static_cast<const InT *>(in.a[zf]);
  const InT *__restrict__ py = static_cast<const InT *>(in.b[zf]);
  float *__restrict__ map =
      map_all + zf * static_cast<size_t>(w) * static_cast<size_t>(pitch);
  constexpr int R = kRadius;
  constexpr int IW = kTileW + 2 * R; // 74 columns
  constexpr int IH = kTileH + 2 * R; // 18 rows
  constexpr int P = IW + 1;          // odd pitch
  constexpr int VB = kTileH / 2;     // rows per thread, vertical pass
  constexpr int HB = kTileW * kTileH / 256; // pixels per thread, horizontal
  constexpr int SEGS = kTileW / HB;  // threads per tile row
  constexpr int kIn = 2 * IH * P;
  constexpr int kV = 5 * kTileH * P;
  static_assert(SEGS * kTileH == 256, "one horizontal segment per thread");
  __shared__ float lds[kIn > kV ? kIn : kV];

  const int tid = threadIdx.x;
  const int x0 = blockIdx.x * kTileW;
  const int y0 = (ty0 + static_cast<int>(blockIdx.y)) * kTileH;
  // all of a thread's loads are issued before the first LDS store
  {
    constexpr int kPer = (IH * IW + 255) / 256;
    InT vx[kPer], vy[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = tid + 256 * k;
      if (i < IH * IW) {
        const int r = i / IW;
        const int c = i - r * IW;
        const size_t off = static_cast<size_t>(sym_index(y0 - R + r, h)) *
                               static_cast<size_t>(w) +
                           static_cast<size_t>(sym_index(x0 - R + c, w));
        vx[k] = px[off];
        vy[k] = py[off];
      }
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = tid + 256 * k;
      if (i < IH * IW) {
        const int r = i / IW;
        const int c = i - r * IW;
        lds[r * P + c] = norm(vx[k], in_scale);
        lds[IH * P + r * P + c] = norm(vy[k], in_scale);
      }
    }
  }
  __syncthreads();

  const int vc = tid & 127;
  const int vb = tid >> 7;
  const bool vact = vc < IW;
  float acc[5][VB];
  if (vact) {
    const float *sx = lds + (vb * VB) * P + vc;
    const float *sy = sx + IH * P;
#pragma unroll
    for (int j = 0; j < VB + 2 * R; ++j) {
      const float x = sx[j * P];
      const float y = sy[j * P];
      const float xx = x * x;
      const float yy = y * y;
      const float xy = x * y;
#pragma unroll
      for (int i = 0; i < VB; ++i) {
        const int k = j - i;
        if (k >= 0 && k < kTaps) {
          const float tk = wtap(sa, k);
          if (k == 0) {
            acc[0][i] = tk * x;
            acc[1][i] = tk * y;
            acc[2][i] = tk * xx;
            acc[3][i] = tk * yy;
            acc[4][i] = tk * xy;
          } else {
            acc[0][i] = acc[0][i] + tk * x;
            acc[1][i] = acc[1][i] + tk * y;
            acc[2][i] = acc[2][i] + tk * xx;
            acc[3][i] = acc[3][i] + tk * yy;
            acc[4][i] = acc[4][i] + tk * xy;
          }
        }
      }
    }
  }
  __syncthreads(); // the input tile is dead
  if (vact) {
#pragma unroll
    for (int q = 0; q < 5; ++q)
#pragma unroll
      for (int i = 0; i < VB; ++i)
        lds[(q * kTileH + vb * VB + i) * P + vc] = acc[q][i];
  }
  __syncthreads();

  const int ty = tid / SEGS;
  const int seg = tid % SEGS;
  float fq[5][HB];
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    const float *row = lds + (q * kTileH + ty) * P + seg * HB;
    float v[HB + 2 * R];
#pragma unroll
    for (int j = 0; j < HB + 2 * R; ++j)
      v[j] = row[j];
#pragma unroll
    for (int i = 0; i < HB; ++i) {
      float s = wtap(sa, 0) * v[i];
#pragma unroll
      for (int k = 1; k < kTaps; ++k)
        s = s + wtap(sa, k) * v[i + k];
      fq[q][i] = s;
    }
  }
  const int y = y0 + ty;
#pragma unroll
  for (int i = 0; i < HB; ++i) {
    const int x = x0 + seg * HB + i;
    if (x < w && y < h)
      map[static_cast<size_t>(x) * static_cast<size_t>(pitch) +
          static_cast<size_t>(y)] =
          ssim_value(fq[0][i], fq[1][i], fq[2][i], fq[3][i], fq[4][i], sa.c1,
                     sa.c2);
  }
}

// Ordered row sums.  A block owns 64 rows; wave 0's lane r adds
// map[x * pitch + y0 + r] for x = 0 .. w-1 into an fp64 sum from 0.0, in
// that order (a serial loop over the row).  The block stages the map in
// chunks of kSumCols columns x 64 rows through LDS: all four waves issue
// every load of a chunk at once (float4, 64 consecutive rows of a column are
// one 256-byte run), then wave 0 adds the chunk from LDS while the other
// waves load the next chunk into the second buffer.  Rows beyond h (up to
// the pitch, inside the buffer) are computed and dropped.
constexpr int kSumCols = 96;
constexpr int kSumF4 = kSumCols * 16;  // 4-float vectors per chunk
constexpr int kSumPer = kSumF4 / 192;  // per loading thread
static_assert(kSumF4 % 192 == 0, "three waves load a chunk evenly");
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load_chunk(f32x4 (&v)[kSumPer],
                                           const float *__restrict__ map,
                                           int pitch, int y0, int x0, int w,
                                           int lt) {
#pragma unroll
  for (int k = 0; k < kSumPer; ++k) {
    const int i = lt + 192 * k;
    const int col = min(x0 + i / 16, w - 1); // in bounds; extras unused
    v[k] = *reinterpret_cast<const f32x4 *>(
        map + static_cast<size_t>(col) * static_cast<size_t>(pitch) + y0 +
        4 * (i % 16));
  }
}

__device__ __forceinline__ void store_chunk(float *buf,
                                            const f32x4 (&v)[kSumPer],
                                            int lt) {
#pragma unroll
  for (int k = 0; k < kSumPer; ++k)
    *reinterpret_cast<f32x4 *>(buf + 4 * (lt + 192 * k)) = v[k];
}

__global__ __launch_bounds__(256) void rowsum_kernel(
    const float *__restrict__ map_all, int w, int h, int pitch,
    double *__restrict__ rows_all) {
  __shared__ float buf[2][kSumCols * 64];
  const int zf = blockIdx.y; // frame of a batched launch
  const float *__restrict__ map =
      map_all + zf * static_cast<size_t>(w) * static_cast<size_t>(pitch);
  double *__restrict__ rows = rows_all + zf * static_cast<size_t>(pitch);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int y0 = blockIdx.x * 64;
  const int chunks = (w + kSumCols - 1) / kSumCols;
  const int lt = tid - 64; // loading thread index of waves 1..3
  if (wave > 0) {
    f32x4 v[kSumPer];
    load_chunk(v, map, pitch, y0, 0, w, lt);
    store_chunk(buf[0], v, lt);
  }
  __syncthreads();
  double acc = 0.0;
  for (int ch = 0; ch < chunks; ++ch) {
    const int x0 = ch * kSumCols;
    if (wave == 0) {
      const float *b = buf[ch & 1] + lane;
      const int n = min(kSumCols, w - x0);
      int x = 0;
      for (; x + 16 <= n; x += 16) {
        float t[16];
#pragma unroll
        for (int k = 0; k < 16; ++k)
          t[k] = b[(x + k) * 64];
#pragma unroll
        for (int k = 0; k < 16; ++k)
          acc = acc + static_cast<double>(t[k]);
      }
      for (; x < n; ++x)
        acc = acc + static_cast<double>(b[x * 64]);
    } else if (ch + 1 < chunks) {
      f32x4 v[kSumPer];
      load_chunk(v, map, pitch, y0, x0 + kSumCols, w, lt);
      store_chunk(buf[(ch + 1) & 1], v, lt);
    }
    __syncthreads();
  }
  if (wave == 0 && y0 + lane < h)
    rows[y0 + lane] = acc;
}

// ------------------------------------------------------------------ launch

namespace {

template <typename InT>
hipError_t launch_decimate_t(const FramePair &in, int n, int w, int h, int f,
                             float tap, float in_scale, int ow, int oh,
                             float *dref, float *ddist, hipStream_t stream) {
  const int xpb = outputs_per_block(f);
  const uintptr_t align = 4 * sizeof(InT);
  bool vec = w % 4 == 0;
  for (int z = 0; z < n; ++z)
    vec = vec && ((reinterpret_cast<uintptr_t>(in.a[z]) |
                   reinterpret_cast<uintptr_t>(in.b[z])) % align) == 0;
  // in_scale and tap are powers of two for these factors, so is their
  // product
  const float iscale = in_scale * tap;
  const dim3 blk(kDecThreads);
  // grid y holds at most kMaxGridY output rows per launch
  for (int y0 = 0; y0 < oh; y0 += kMaxGridY) {
    const dim3 grid(static_cast<unsigned>((ow + xpb - 1) / xpb),
                    static_cast<unsigned>(std::min(kMaxGridY, oh - y0)),
                    static_cast<unsigned>(n));
#define FSSIM_POW2(F)                                                          \
  if (vec)                                                                     \
    decimate_pow2_kernel<InT, true, F><<<grid, blk, 0, stream>>>(              \
        in, w, h, iscale, ow, oh, xpb, dref, ddist, y0);                       \
  else                                                                         \
    decimate_pow2_kernel<InT, false, F><<<grid, blk, 0, stream>>>(             \
        in, w, h, iscale, ow, oh, xpb, dref, ddist, y0)
    if (f == 2) {
      FSSIM_POW2(2);
    } else if (f == 4) {
      FSSIM_POW2(4);
    } else if (f == 8) {
      FSSIM_POW2(8);
    } else if (f == 16) {
      FSSIM_POW2(16);
    } else if (vec) {
      decimate_kernel<InT, true><<<grid, blk, 0, stream>>>(
          in, w, h, f, tap, in_scale, ow, oh, xpb, dref, ddist, y0);
    } else {
      decimate_kernel<InT, false><<<grid, blk, 0, stream>>>(
          in, w, h, f, tap, in_scale, ow, oh, xpb, dref, ddist, y0);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
      return e;
  }
#undef FSSIM_POW2
  return hipSuccess;
}

template <typename InT>
hipError_t launch_ssim_t(const FramePair &in, int n, int w, int h,
                         float in_scale, const SsimArgs &sa, float *map,
                         hipStream_t stream) {
  const int tiles_y = (h + kTileH - 1) / kTileH;
  // grid y holds at most kMaxGridY rows of tiles per launch
  for (int t0 = 0; t0 < tiles_y; t0 += kMaxGridY) {
    const dim3 grid(static_cast<unsigned>((w + kTileW - 1) / kTileW),
                    static_cast<unsigned>(std::min(kMaxGridY, tiles_y - t0)),
                    static_cast<unsigned>(n));
    ssim_kernel<InT><<<grid, dim3(256), 0, stream>>>(in, w, h, in_scale, sa,
                                                     map, map_pitch(h), t0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
      return e;
  }
  return hipSuccess;
}

} // namespace

hipError_t launch_decimate(int bpc, const FramePair &in, int n, int w, int h,
                           int f, float tap, float in_scale, int ow, int oh,
                           float *dref, float *ddist, hipStream_t stream) {
  if (f < 2 || outputs_per_block(f) < 1 || ow < 1 || oh < 1 || n < 1 ||
      n > kMaxBatch)
    return hipErrorInvalidValue;
  if (bpc == 8)
    return launch_decimate_t<uint8_t>(in, n, w, h, f, tap, in_scale, ow, oh,
                                      dref, ddist, stream);
  return launch_decimate_t<uint16_t>(in, n, w, h, f, tap, in_scale, ow, oh,
                                     dref, ddist, stream);
}

hipError_t launch_ssim(int bpc, const FramePair &in, int n, int w, int h,
                       float in_scale, const SsimArgs &sa, float *map,
                       hipStream_t stream) {
  if (w < 1 || h < 1 || n < 1 || n > kMaxBatch)
    return hipErrorInvalidValue;
  if (bpc == 0)
    return launch_ssim_t<float>(in, n, w, h, 1.0f, sa, map, stream);
  if (bpc == 8)
    return launch_ssim_t<uint8_t>(in, n, w, h, in_scale, sa, map, stream);
  return launch_ssim_t<uint16_t>(in, n, w, h, in_scale, sa, map, stream);
}

hipError_t launch_ssim_rowsum(const float *map, int n, int w, int h,
                              double *rows, hipStream_t stream) {
  if (w < 1 || h < 1 || n < 1 || n > kMaxBatch)
    return hipErrorInvalidValue;
  const int pitch = map_pitch(h);
  rowsum_kernel<<<dim3(static_cast<unsigned>(pitch / 64),
                       static_cast<unsigned>(n)),
                  dim3(256), 0, stream>>>(map, w, h, pitch, rows);
  return hipGetLastError();
}

} // namespace fssimk
