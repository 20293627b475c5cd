// fssim_taps.cpp -- host constants of the float SSIM feature, passed to the
// kernels by value.
//
// Decimation (Research-2130 "float_ssim decimation on the SYCL device",
// Question and Sources): the factor max(1, round(min(w, h) / 256)) with C's
// round (halves away from zero), the box tap 1.0f / (f * f) in fp32 and the
// decimated size n / f + (n & 1).
//
// SSIM stage (the published SSIM; the pages print no window): 11 taps of a
// Gaussian with sigma 1.5, each exp() in fp64, normalised by their fp64 sum
// in ascending order and rounded once to fp32; C1 = (0.01 * 255)^2 and
// C2 = (0.03 * 255)^2 formed in fp64 and rounded to fp32.  Built without
// -ffast-math and with contraction off, so every operation rounds once.
#include <cmath>

#include "fssim_internal.h"

namespace fssimk {

void window_taps(float t[kTaps]) {
  const double sigma = 1.5;
  const double denom = 2.0 * sigma * sigma;
  double g[kTaps];
  for (int k = 0; k < kTaps; ++k) {
    const double d = static_cast<double>(k - kRadius);
    g[k] = std::exp(-(d * d) / denom);
  }
  double sum = 0.0;
  for (int k = 0; k < kTaps; ++k)
    sum = sum + g[k];
  for (int k = 0; k < kTaps; ++k)
    t[k] = static_cast<float>(g[k] / sum);
}

float box_tap(int f) { return 1.0f / static_cast<float>(f * f); }

SsimArgs make_ssim_args() {
  SsimArgs a{};
  window_taps(a.t);
  const double k1 = 0.01 * 255.0;
  const double k2 = 0.03 * 255.0;
  a.c1 = static_cast<float>(k1 * k1);
  a.c2 = static_cast<float>(k2 * k2);
  return a;
}

int factor(int w, int h) {
  const int m = w < h ? w : h;
  const int f = static_cast<int>(std::round(static_cast<double>(m) / 256.0));
  return f < 1 ? 1 : f;
}

int decimated_size(int n, int f) { return n / f + (n & 1); }

} // namespace fssimk
