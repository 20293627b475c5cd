// vif_internal.h -- host-side declarations shared by the library's
// translation units (not part of the public ABI).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace vifk {

constexpr int kScales = 4;
constexpr int kMaxTaps = 17;
constexpr int kWidths[kScales] = {17, 9, 5, 3};

// Tile of the per-scale kernel: 112 output columns x 16 output rows, and
// the row strip of the term layout (16 rows).
constexpr int kTileW = 112;
constexpr int kTileH = 16;

struct TapArgs {
  float t[kMaxTaps];
};

// Host tap generator (vif_taps.cpp).
int gaussian_taps(int scale, float *taps);

// Geometry of one scale.
struct ScaleGeom {
  int w, h;
  int strips;        // ceil(h / kTileH)
  size_t term_elems; // floats in the term buffer: strips * w * 32
};

// Per-scale filter + statistic + decimation kernel.  in_* are the scale's
// planes (native samples at scale 0, fp32 planes above); next_* receive the
// next scale's planes (unused at scale 3).
hipError_t launch_scale(int scale, int bpc, const void *in_ref,
                        const void *in_dist, const ScaleGeom &g,
                        const TapArgs &taps, const TapArgs &next_taps,
                        float *terms, float *next_ref, float *next_dist,
                        hipStream_t stream);

// Ordered per-row sums of one scale's term buffer into rows[2*y + c].
hipError_t launch_rowsum(const float *terms, const ScaleGeom &g, float *rows,
                         hipStream_t stream);

}  // namespace vifk
