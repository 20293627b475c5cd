// fssim_internal.h -- host-side declarations of the float SSIM kernels
// (not part of the public ABI).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace fssimk {

constexpr int kTaps = 11; // SSIM window, radius 5
constexpr int kRadius = 5;

// Decimation: a block of kDecThreads threads covers one decimated row and
// up to kDecSpan plane columns (4 per thread), i.e. outputs_per_block(f)
// decimated pixels.
constexpr int kDecThreads = 256;
constexpr int kDecSpan = 4 * kDecThreads;

// Widest run of decimated pixels whose windows, together with the columns
// their mirrored indices reach, fit in one block's kDecSpan columns after
// the start is rounded down to a multiple of 4.
inline int outputs_per_block(int f) { return (kDecSpan - 3 - 2 * f) / f; }

// SSIM stage: tiles of 64 x 8 pixels (small tiles: the decimated planes are
// small, and more blocks keep more waves busy).
constexpr int kTileW = 64;
constexpr int kTileH = 8;

// Map layout: column-major, pitch rounded up to whole 64-row groups, so the
// row-sum waves (one lane per row) read 64 consecutive floats per column.
inline int map_pitch(int h) { return (h + 63) / 64 * 64; }

// Constants of the SSIM stage, passed to its kernel by value.
struct SsimArgs {
  float t[kTaps];
  float c1, c2;
};

// Host generators (fssim_taps.cpp): the 11 window taps, the box tap of a
// factor, C1 and C2, the factor and the decimated size.
void window_taps(float t[kTaps]);
float box_tap(int f);
SsimArgs make_ssim_args();
int factor(int w, int h);
int decimated_size(int n, int f);

// Frames one launch may carry (blockIdx.z of the decimation and SSIM
// kernels, blockIdx.y of the row sums).
constexpr int kMaxBatch = 16;
// Blocks per launch in grid dimension y (the runtime allows 65536; planes
// with more rows of blocks take several launches).
constexpr int kMaxGridY = 65535;

// Per-frame planes of a launch: frame z reads a[z] and b[z].
struct FramePair {
  const void *a[kMaxBatch];
  const void *b[kMaxBatch];
};

// Decimates both planes of n frames (samples of bpc bits, 1 or 2 bytes) by
// f into dref / ddist + z * ow * oh (ow x oh fp32, row-major, pitch ow).
hipError_t launch_decimate(int bpc, const FramePair &in, int n, int w, int h,
                           int f, float tap, float in_scale, int ow, int oh,
                           float *dref, float *ddist, hipStream_t stream);

// SSIM stage of n w x h pairs into map + z * w * map_pitch(h) (column-major,
// pitch map_pitch(h)).  bpc 0 means fp32 planes (the decimated ones); 8..16
// the samples.
hipError_t launch_ssim(int bpc, const FramePair &in, int n, int w, int h,
                       float in_scale, const SsimArgs &sa, float *map,
                       hipStream_t stream);

// Ordered fp64 sums of the rows of n maps into rows + z * map_pitch(h).
hipError_t launch_ssim_rowsum(const float *map, int n, int w, int h,
                              double *rows, hipStream_t stream);

} // namespace fssimk
