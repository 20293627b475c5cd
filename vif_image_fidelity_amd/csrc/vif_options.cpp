// vif_options.cpp -- checks of the feature's options and the constants of
// the per-pixel statistic built from them.
//
// The pages name the options (ADR-1422 "float_vif_sycl computes the CPU's
// arithmetic ...", Decision and Consequences: vif_sigma_nsq,
// vif_enhn_gain_limit, vif_skip_scale0, vif_scale1..3_min_val with default
// 0, and the tap generator's vif_kernelscale) without their arithmetic; the
// meaning taken for each is stated in include/vif.h.
#include <cmath>

#include "../../include/vif.h"
#include "vif_internal.h"

namespace vifk {

bool options_valid(const OptionValues &o) {
  if (!(o.sigma_nsq >= 0.0) || std::isinf(o.sigma_nsq))
    return false;
  if (!(o.enhn_gain_limit >= 0.0))
    return false;
  if (o.kernelscale != 1.0)
    return false;
  for (double v : o.scale_min_val)
    if (std::isnan(v))
      return false;
  return o.skip_scale0 == 0 || o.skip_scale0 == 1;
}

bool options_ok(const vif_options &o) {
  OptionValues v{};
  v.sigma_nsq = o.sigma_nsq;
  v.enhn_gain_limit = o.enhn_gain_limit;
  v.kernelscale = o.kernelscale;
  for (int i = 0; i < 3; ++i)
    v.scale_min_val[i] = o.scale_min_val[i];
  v.skip_scale0 = o.skip_scale0;
  return o.reserved == 0 && options_valid(v);
}

StatArgs make_stat_args(double nsq, double gain_limit) {
  StatArgs a{};
  a.nsq = nsq;
  a.inv_nsq = 0.0;
  int e = 0;
  // nsq = 2^(e-1) exactly when its frexp fraction is 1/2; the reciprocal
  // is then exact, and so is the product with any fp32 value (no overflow or
  // underflow in fp64).  The range 2^-20 .. 2^20 also keeps the numerator
  // ratio's quotient inside the domain of its shorter division (the kernels
  // for a power-of-two nsq use it; other values take the general kernels).
  if (nsq > 0.0 && std::frexp(nsq, &e) == 0.5 && e >= -19 && e <= 21) {
    a.inv_nsq = std::ldexp(1.0, 1 - e);
    a.nsq_f = static_cast<float>(nsq);
    a.inv_nsq_f = static_cast<float>(a.inv_nsq);
  }
  a.gain = static_cast<float>(gain_limit);
  return a;
}

} // namespace vifk
