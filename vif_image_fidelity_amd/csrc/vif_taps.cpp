// vif_taps.cpp -- host Gaussian tap generator (ADR-1422 "float_vif_sycl
// computes the CPU's arithmetic ...", Decision: the taps come from the
// CPU's run-time routine for each scale and every launch receives its
// scale's taps by value; no kernel holds a tap literal).
//
// Scale s has N = 17, 9, 5, 3 taps and sigma = N / 5 (the published
// pixel-domain VIF window).  In fp64: sigma = N / 5.0, denom = (2.0 * sigma)
// * sigma, g_k = exp(-(d*d) / denom) for d = k - (N-1)/2, S = the sum of g_k
// in ascending k from 0.0; each tap is (float)(g_k / S), one rounding.
// Built without -ffast-math and with contraction off, so each fp64
// operation rounds once, as written.
#include <cmath>

#include "vif_internal.h"

namespace vifk {

int gaussian_taps(int scale, float *taps) {
  if (scale < 0 || scale >= kScales || taps == nullptr)
    return -1;
  const int n = kWidths[scale];
  const int r = (n - 1) / 2;
  const double sigma = static_cast<double>(n) / 5.0;
  const double denom = 2.0 * sigma * sigma;
  double g[kMaxTaps];
  for (int k = 0; k < n; ++k) {
    const double d = static_cast<double>(k - r);
    g[k] = std::exp(-(d * d) / denom);
  }
  double sum = 0.0;
  for (int k = 0; k < n; ++k)
    sum = sum + g[k];
  for (int k = 0; k < n; ++k)
    taps[k] = static_cast<float>(g[k] / sum);
  return n;
}

} // namespace vifk
